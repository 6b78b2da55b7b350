// append.hip -- project each sequence's new token to its per-head latents and
// write them into the latent caches.
//
// Per head h the cache row is x . A_Kh with A_Kh in R^{E x r} ("WSVD:
// Weighted Low-Rank Approximation for Fast and Efficient Execution of
// Low-Precision Vision-Language Models", Arabic page section 2a, German page
// section 2A, Japanese page section 2.1).  Stacking all heads gives one skinny
// GEMM  P[nb, 2 nh r] = x[nb, E] . [A_K | A_V][E, 2 nh r]  (nb = 64, E = 4096,
// 2 nh r = 3072 for the LLaVA-7B-shaped step): about 62 flop per byte of A,
// under the MFMA ridge, so it is bound by streaming A from HBM.  It runs on
// matrix cores (v_mfma_f32_16x16x32_bf16) so the arithmetic hides under
// that stream.
//
// One launch.  Block = 64 rows of x  x  64 columns of A  x  one E-slice;
// enough E-slices (KS) are used to put >= 1.5 blocks on each CU.
//  * A block requests two LDS stages (2 x 256 E rows of A and x) at once,
//    one register buffer per stage.  With E = 4096 the split makes every
//    slice exactly two stages, so the whole A stream is in flight at once
//    and never waits on a dependent round trip.
//  * A arrives row-major (columns contiguous) but the MFMA B operand wants 8
//    consecutive k per lane, so each thread loads an 8 x 8 (k x n) bf16
//    block with eight 16-byte loads (a wave covers 8 full 128-byte rows per
//    load), transposes it in registers and stores 8 k-contiguous vectors
//    into LDS.  The LDS tile is [64 n][256 k] with a 16-byte row pad and the
//    k-block index xor-swizzled by n/8, so both the transposed stores and
//    the fragment reads are free of bank conflicts.
//  * x is read with whole-row loads (a wave covers two 512-byte row pieces
//    per load) into a second padded LDS tile [64 m][256 k]; gathering the
//    MFMA A fragments (16 rows x 16 bytes) straight from memory instead
//    cost several times more L2 requests for the same bytes.
//  * Each wave owns 16 rows of x and all 64 columns: 4 accumulators of
//    16 x 16.
//  * With KS > 1 each block writes its fp32 partial tile to the workspace
//    (device-coherent 16-byte stores, in the accumulator's own lane order,
//    so a wave writes 1 KB contiguous per store) and bumps
//    the tile's arrival counter; the block that arrives last sums the KS
//    partials in slice order (so the result does not depend on which block
//    finished last), resets the counter, rounds once to the cache dtype and
//    writes row pos[b] of every head's K and V cache.
//
// W8A8 variant (w8): x arrives as int8 codes of the Hadamard-rotated token
// with one fp32 scale per token, A as int8 codes of the rotated factor,
// stored transposed ([nh r, E], k-contiguous) with one fp32 scale per
// column (the pages' W8A8 setting with S1 outlier smoothing: German page
// section 2C, Italian page section 2C, Arabic page section 2c).  Both
// operands are k-contiguous, so both tiles are staged with whole-row loads
// and no transpose, and v_mfma_i32_16x16x64_i8 accumulates exact int32
// sums; the partial tiles are int32 (their sum is exact in any order).
// The latent is acc * sx[b] * sA[n] in fp32, then stored as above.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

#ifndef WSVD_APPEND_TARGET_BLOCKS
#define WSVD_APPEND_TARGET_BLOCKS 384
#endif

namespace wsvd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int AP_NT = 64;           // columns per block
constexpr int AP_MT = 64;           // rows of x per block
constexpr int AP_EC = 256;          // E rows per LDS stage
constexpr int AP_PITCH = AP_EC + 8; // bf16 elements per LDS row (16-byte pad)
constexpr int AP_TILE_VALS = AP_NT * AP_MT;  // fp32 values in one partial tile

union V16 {
    u32x4 u;
    bf16x8 b;
};

// One stage of operands in registers: this thread's 8 x 8 block of A and
// its eight 16-byte pieces of x rows.
struct Stage {
    u32x4 a[8];
    u32x4 x[8];
};

// Raw buffer descriptor over `bytes` bytes at p (gfx9 word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;     // cache-policy bit nt: streamed once
constexpr int kCoherentAgent = 16;  // cache-policy bit sc1: device-coherent

// Buffer loads keep one 32-bit lane offset per stream and put the uniform
// part (stage start, row step) in a scalar offset, instead of a 64-bit
// address per load.
struct TileCtx {
    __amdgpu_buffer_rsrc_t ra, rx;
    uint32_t a_voff;     // bytes: (kblk * 8 * N1 + ncol) * 2
    uint32_t a_row;      // bytes per row of A: N1 * 2
    uint32_t x_voff[8];  // bytes: (xrow_i * E + xcol) * 2
};

__device__ __forceinline__ void load_stage(Stage& s, const TileCtx& c, int es) {
    // Columns past N1 read column 0 and rows past nb read row nb - 1 instead
    // (in bounds); those outputs are never written, and an output column
    // (row) depends only on its own column of A (row of x).
#pragma unroll
    for (int i = 0; i < 8; ++i)
        s.a[i] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, c.a_voff, (es + i) * c.a_row, kNonTemporal);
#pragma unroll
    for (int i = 0; i < 8; ++i) s.x[i] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_voff[i], es * 2, 0);
}

// Transpose the stage's A block into LDS, stage x rows beside it, and run
// the stage's MFMAs.
__device__ __forceinline__ void mma_stage(const Stage& s, uint16_t* sB, uint16_t* sX, f32x4 (&acc)[4], int tid,
                                          int lane, int wave) {
    const int nblk = tid & 7;
    const int kblk = tid >> 3;
    // 8 x 8 transpose: tr[n'] holds k = 0..7 of column n'.
    u32x4 tr[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t r0 = s.a[2 * p][w], r1 = s.a[2 * p + 1][w];
            tr[2 * w][p] = (r0 & 0xffffu) | (r1 << 16);
            tr[2 * w + 1][p] = (r0 >> 16) | (r1 & 0xffff0000u);
        }
    }
    __syncthreads();  // the previous stage's fragment reads are done
#pragma unroll
    for (int np = 0; np < 8; ++np) {
        const int n = nblk * 8 + np;
        const int kb = kblk ^ (nblk & 7);
        *reinterpret_cast<u32x4*>(&sB[n * AP_PITCH + kb * 8]) = tr[np];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(&sX[((tid >> 5) + 8 * i) * AP_PITCH + (tid & 31) * 8]) = s.x[i];
    __syncthreads();
    const uint16_t* xr = sX + (wave * 16 + (lane & 15)) * AP_PITCH + (lane >> 4) * 8;
#pragma unroll
    for (int st = 0; st < AP_EC / 32; ++st) {
        V16 xf;
        xf.u = *reinterpret_cast<const u32x4*>(xr + st * 32);
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            const int n = jn * 16 + (lane & 15);
            const int kb = (st * 4 + (lane >> 4)) ^ ((n >> 3) & 7);
            V16 bf;
            bf.u = *reinterpret_cast<const u32x4*>(&sB[n * AP_PITCH + kb * 8]);
            acc[jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf.b, bf.b, acc[jn], 0, 0, 0);
        }
    }
}


// ---- W8A8 operands: 512 k (bytes) per stage ---------------------------------
constexpr int AP_ECB = 512;                 // int8 k per stage
constexpr int AP_PITCHB = AP_ECB + 16;      // bytes per LDS row (same 528 as bf16)
static_assert(AP_PITCHB == AP_PITCH * 2, "both variants share the LDS tiles");

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct TileCtxW8 {
    __amdgpu_buffer_rsrc_t ra, rx;
    uint32_t a_voff[8];  // bytes: row n_i of A^T (clamped to N1 - 1) * E + 16 * (tid & 31)
    uint32_t x_voff[8];  // bytes: row m_i of x (clamped to nb - 1) * E + 16 * (tid & 31)
};

__device__ __forceinline__ void load_stage_w8(Stage& s, const TileCtxW8& c, int es) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s.a[i] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, c.a_voff[i], es, kNonTemporal);
#pragma unroll
    for (int i = 0; i < 8; ++i) s.x[i] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_voff[i], es, 0);
}

// Rows (tid >> 5) + 8 i of both tiles, 16 bytes at 16 (tid & 31); then
// 8 k-steps of 64: lane l reads 16 bytes of row l % 16 at k 16 (l / 16) of
// the step, for x (the wave's 16 rows) and for A (each 16-column group).
__device__ __forceinline__ void mma_stage_w8(const Stage& s, uint8_t* sB, uint8_t* sX, i32x4 (&acc)[4], int tid,
                                             int lane, int wave) {
    __syncthreads();  // the previous stage's fragment reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 5) + 8 * i;
        *reinterpret_cast<u32x4*>(&sB[row * AP_PITCHB + (tid & 31) * 16]) = s.a[i];
        *reinterpret_cast<u32x4*>(&sX[row * AP_PITCHB + (tid & 31) * 16]) = s.x[i];
    }
    __syncthreads();
    const uint8_t* xr = sX + (wave * 16 + (lane & 15)) * AP_PITCHB + (lane >> 4) * 16;
    const uint8_t* br = sB + (lane & 15) * AP_PITCHB + (lane >> 4) * 16;
#pragma unroll
    for (int st = 0; st < AP_ECB / 64; ++st) {
        const i32x4 xf = __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4*>(xr + st * 64));
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            const i32x4 bf =
                __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4*>(br + jn * 16 * AP_PITCHB + st * 64));
            acc[jn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf, bf, acc[jn], 0, 0, 0);
        }
    }
}

// int8 cache rows (r in 16, 32, 64, so a head's r columns are whole
// 16-column groups of one tile): per (row, head) the absmax over the head's
// columns -- 16 lanes by DPP, then the head's column groups in registers --
// gives the fp16 scale fp16(absmax / 127); codes are
// clamp(round_half_even(v / scale), -127, 127), a zero row stores scale 0.
// Rows m0r .. m0r + 3 of this lane, columns n0 + jn * 16 + (lane & 15).
__device__ __forceinline__ void store_int8_rows(const AppendArgs& a, const f32x4 (&acc)[4], void* C, uint16_t* S,
                                                const int (&prow)[4], int n0, int m0r, int lane) {
    const int N1 = a.nh * a.r;
    const int gj = a.r >> 4;  // column groups per head: 1, 2 or 4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float mx[4];
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) mx[jn] = group_max<16>(fabsf(acc[jn][i]));
        // combine the groups of each head (heads start at a multiple of gj)
        if (gj >= 2) {
            const float m01 = fmaxf(mx[0], mx[1]), m23 = fmaxf(mx[2], mx[3]);
            mx[0] = mx[1] = m01;
            mx[2] = mx[3] = m23;
        }
        if (gj == 4) mx[0] = mx[1] = mx[2] = mx[3] = fmaxf(mx[0], mx[2]);
        const int m = m0r + i;
        const int p = prow[i];
        if (m >= a.nb || p < 0 || p >= a.L_cap) continue;
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            const int n = n0 + jn * 16 + (lane & 15);
            if (n >= N1) continue;
            const int h = n / a.r;
            const int col = n - h * a.r;
            const uint16_t sb = f32_to_f16(mx[jn] / 127.f);
            const float sc = f16_to_f32(sb);
            float code = 0.f;
            if (sc > 0.f) code = fminf(fmaxf(__builtin_rintf(acc[jn][i] / sc), -127.f), 127.f);
            const size_t row = ((size_t)m * a.nh + h) * a.L_cap + p;
            __builtin_nontemporal_store((int8_t)(int)code, static_cast<int8_t*>(C) + row * a.r + col);
            if (col == 0)
                __hip_atomic_store(S + row, sb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <bool W8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sB[AP_NT * AP_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sX[AP_MT * AP_PITCH];
    __shared__ int sh_last;

    const int N1 = a.nh * a.r;
    const int n0 = blockIdx.x * AP_NT;
    const int kv = blockIdx.y & 1;
    const int m0 = (blockIdx.y >> 1) * AP_MT;
    const int ks = blockIdx.z;
    const int e_len = a.E / a.KS;
    const int e_beg = ks * e_len;
    const int ns = e_len / (W8 ? AP_ECB : AP_EC);
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // acc holds fp32 sums, or (W8) the bits of exact int32 sums until the
    // scales are applied after the split-E reduction.
    f32x4 acc[4];
    Stage s0, s1;
    if constexpr (!W8) {
        TileCtx c;
        c.ra = make_rsrc(kv ? a.A_V : a.A_K, (uint32_t)((size_t)a.E * N1 * 2));
        c.rx = make_rsrc(a.x, (uint32_t)((size_t)a.nb * a.E * 2));
        int ncol = n0 + (tid & 7) * 8;
        if (ncol >= N1) ncol = 0;  // N1 is a multiple of 16, chunks are 8 wide
        c.a_row = (uint32_t)N1 * 2u;
        c.a_voff = ((uint32_t)(tid >> 3) * 8u * (uint32_t)N1 + (uint32_t)ncol) * 2u;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c.x_voff[i] = ((uint32_t)min(m0 + (tid >> 5) + 8 * i, a.nb - 1) * (uint32_t)a.E + (tid & 31) * 8u) * 2u;
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[jn] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Two stages (512 E rows) requested together; the split factor keeps
        // a block's slice at one or two stages, so one pass normally covers it.
        // Pairs are requested without a branch between them (an odd last
        // stage goes alone): behind a branch, the waits for the first stage
        // would also wait for the second, so its MFMAs could not overlap the
        // second stage's flight.
        int st = 0;
        for (; st + 1 < ns; st += 2) {
            load_stage(s0, c, e_beg + st * AP_EC);
            load_stage(s1, c, e_beg + (st + 1) * AP_EC);
            mma_stage(s0, sB, sX, acc, tid, lane, wave);
            mma_stage(s1, sB, sX, acc, tid, lane, wave);
        }
        if (st < ns) {
            load_stage(s0, c, e_beg + st * AP_EC);
            mma_stage(s0, sB, sX, acc, tid, lane, wave);
        }
    } else {
        TileCtxW8 c;
        c.ra = make_rsrc(kv ? a.A_V : a.A_K, (uint32_t)((size_t)a.E * N1));
        c.rx = make_rsrc(a.x, (uint32_t)((size_t)a.nb * a.E));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = (tid >> 5) + 8 * i;
            c.a_voff[i] = (uint32_t)min(n0 + row, N1 - 1) * (uint32_t)a.E + (tid & 31) * 16u;
            c.x_voff[i] = (uint32_t)min(m0 + row, a.nb - 1) * (uint32_t)a.E + (tid & 31) * 16u;
        }
        i32x4 iacc[4];
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) iacc[jn] = i32x4{0, 0, 0, 0};
        uint8_t* bB = reinterpret_cast<uint8_t*>(sB);
        uint8_t* bX = reinterpret_cast<uint8_t*>(sX);
        int st = 0;
        for (; st + 1 < ns; st += 2) {
            load_stage_w8(s0, c, e_beg + st * AP_ECB);
            load_stage_w8(s1, c, e_beg + (st + 1) * AP_ECB);
            mma_stage_w8(s0, bB, bX, iacc, tid, lane, wave);
            mma_stage_w8(s1, bB, bX, iacc, tid, lane, wave);
        }
        if (st < ns) {
            load_stage_w8(s0, c, e_beg + st * AP_ECB);
            mma_stage_w8(s0, bB, bX, iacc, tid, lane, wave);
        }
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[jn] = __builtin_bit_cast(f32x4, iacc[jn]);
    }

    // Rows of the caches this lane's accumulator entries go to (requested
    // only once the tile is complete, beside the last round of loads).
    int prow[4];
    float xs[4], as[4];  // W8: this lane's row and column scales
    auto load_pos = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wave * 16 + (lane >> 4) * 4 + i;
            prow[i] = (m < a.nb) ? a.pos[m] : -1;
            if constexpr (W8) xs[i] = a.sx[min(m, a.nb - 1)];
        }
        if constexpr (W8) {
            const float* sA = kv ? a.sA_V : a.sA_K;
#pragma unroll
            for (int jn = 0; jn < 4; ++jn) as[jn] = sA[min(n0 + jn * 16 + (lane & 15), N1 - 1)];
        }
    };

    if (a.KS > 1) {
        // Partial tile in accumulator lane order: accumulator jn of thread t
        // is the 16 bytes at float index ((ks * 4 + jn) * 256 + t) * 4 of the
        // tile's KS-slice area.
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(a.part + (size_t)tile * a.KS * AP_TILE_VALS, (uint32_t)(a.KS * AP_TILE_VALS * sizeof(float)));
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[jn]), rs,
                                                   ((ks * 4 + jn) * 256 + tid) * 16, 0, kCoherentAgent);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            sh_last = (__hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (unsigned)(a.KS - 1));
        __syncthreads();
        if (!sh_last) return;
        load_pos();

        // Last arrival: ordered sum over the KS slices, 8 slices per round
        // trip (all loads of a round are issued before any is used).
        f32x4 sum[4];
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) sum[jn] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < a.KS; k0 += 8) {
            f32x4 v[8][4];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = min(k0 + u, a.KS - 1);
#pragma unroll
                for (int jn = 0; jn < 4; ++jn)
                    v[u][jn] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((k * 4 + jn) * 256 + tid) * 16, 0,
                                                                     kCoherentAgent));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k0 + u < a.KS) {
#pragma unroll
                    for (int jn = 0; jn < 4; ++jn) {
                        if constexpr (W8)
                            sum[jn] = __builtin_bit_cast(f32x4, __builtin_bit_cast(i32x4, sum[jn]) +
                                                                    __builtin_bit_cast(i32x4, v[u][jn]));
                        else
                            sum[jn] += v[u][jn];
                    }
                }
            }
        }
        if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[jn] = sum[jn];
    } else {
        load_pos();
    }
    if constexpr (W8) {  // exact integer sums -> latent values
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            const i32x4 q = __builtin_bit_cast(i32x4, acc[jn]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[jn][i] = (float)q[i] * xs[i] * as[jn];
        }
    }

    void* C = kv ? a.C_V : a.C_K;
    if (a.C_dt == WSVD_I8) {
        store_int8_rows(a, acc, C, kv ? a.s_V : a.s_K, prow, n0, m0 + wave * 16 + (lane >> 4) * 4, lane);
        return;
    }
    // Round once and scatter into the caches.
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
        const int n = n0 + jn * 16 + (lane & 15);
        if (n >= N1) continue;
        const int h = n / a.r;
        const int col = n - h * a.r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wave * 16 + (lane >> 4) * 4 + i;
            const int p = prow[i];
            if (m >= a.nb || p < 0 || p >= a.L_cap) continue;
            const size_t off = (((size_t)m * a.nh + h) * a.L_cap + p) * a.r + col;
            store_elem_wt(C, a.C_dt, off, acc[jn][i]);
        }
    }
}

int append_num_esplits(int nb, int E, int nh, int r) {
    const long ntile = append_num_tiles(nb, nh, r);
    int ks = 1;
    // >= 1.5 blocks per CU (256 CUs); every E-slice a whole number of the
    // larger (int8, 512 k) stage, so both variants split the same way and
    // share one workspace size.
    while (ntile * ks < WSVD_APPEND_TARGET_BLOCKS && E % (2 * ks * AP_ECB) == 0) ks *= 2;
    return ks;
}

// The int8 operands' slices: the same split halved while a slice would hold
// a single 512-k stage, so each block requests a pair of stages at once
// (measured on MI355X at the 64 x 4096 -> 32 x 48 shape: 17.5 against
// 18.5 us with the quantiser).  Never more slices than the bf16 split, so
// the workspace sized for that split covers it.
int append_num_esplits_w8(int nb, int E, int nh, int r) {
    int ks = append_num_esplits(nb, E, nh, r);
    while (ks > 1 && E / ks < 2 * AP_ECB) ks /= 2;
    return ks;
}

long append_num_tiles(int nb, int nh, int r) {
    return (long)((nh * r + AP_NT - 1) / AP_NT) * 2 * ((nb + AP_MT - 1) / AP_MT);
}

size_t append_partial_bytes(int nb, int E, int nh, int r) {
    const int ks = append_num_esplits(nb, E, nh, r);
    if (ks <= 1) return 0;
    return (size_t)append_num_tiles(nb, nh, r) * ks * AP_TILE_VALS * sizeof(float);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
    const int N1 = a.nh * a.r;
    dim3 g((N1 + AP_NT - 1) / AP_NT, 2 * ((a.nb + AP_MT - 1) / AP_MT), a.KS);
    if (a.w8)
        hipLaunchKernelGGL(append_kernel<true>, g, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(append_kernel<false>, g, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace wsvd
