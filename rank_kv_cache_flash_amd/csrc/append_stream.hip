// append_stream.hip -- the new token's per-head latents, bf16 operands:
// C_K[b, h, pos[b], :] = x[b] . A_Kh and the same for V ("WSVD: Weighted
// Low-Rank Approximation for Fast and Efficient Execution of Low-Precision
// Vision-Language Models", Arabic page section 2a, German page section 2A,
// Japanese page section 2.1: A_Kh in R^{E x r}, the cache keeps x A_Kh per
// head).  Stacking the heads gives P[nb, nh r] = x[nb, E] . A[E, nh r] for K
// and for V: a skinny GEMM that is bound by streaming A from HBM (about 62
// flop per byte of A at 64 tokens, under the matrix-core ridge), so the
// design goal is to keep A's bytes flowing and to add as little traffic as
// possible around them.
//
// Block = 8 waves; output tile = 64 rows of x  x  64 columns of one factor
// (128-byte rows of A); E is cut into KS slices, the fewest (halving) that
// give about 160+ blocks: 4 slices and 192 blocks at the LLaVA-7B step shape.
//  * Stage = 256 rows of A (64 columns) and the matching 256 k of x.  The
//    8 waves are 4 k-groups x 2 column halves: a wave owns a 64-k slice of
//    every stage and the 64 x 32 outputs of its half, so each byte of A is
//    read from LDS once per block and each byte of x twice.  (8 k-groups of
//    32 k, every wave computing all 64 x 64 outputs, read x once but sum
//    twice as many partial tiles at the end: 0.44 us slower at the LLaVA-7B
//    step shape; 2 k-groups x 4 column quarters, reading x four times, as
//    slow as 8.)  x is loaded as whole 512-byte row pieces and staged in LDS
//    beside A (reading the operand layout straight from memory, 16 rows x
//    64 bytes per load, measured 1.2 us slower at the LLaVA-7B step shape).
//  * A arrives n-contiguous; its stage is stored to LDS row-major (rows
//    padded by 32 bytes against bank conflicts) and the B
//    operands are read with gfx950's transposing LDS read
//    (ds_read_b64_tr_b16): in each group of 16 lanes, lane i receives element
//    i % 4 of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12,
//    so when those 16 lanes address 4 rows x 16 columns, lane i holds four
//    consecutive k of column i -- half a B fragment.
//  * Four stages of A and x are in flight in registers (at the step shape a
//    slice is exactly four stages, so a block requests its whole share in the
//    prologue); the steady-state loop of longer slices requests stage s + 4
//    right after consuming stage s, with no branch around the request.
//  * Blocks are placed so that each XCD runs one E slice (its L2 then holds
//    a quarter of x).
//  * The 4 k-groups' partial tiles are summed in LDS in k order; each thread
//    then owns 8 consecutive outputs of one row, i.e. of one head.  With
//    KS > 1 each block stores its sum write-through and takes a ticket; the
//    last of the KS blocks of a tile adds the others' sums in slice order
//    (own slice from registers), so the result does not depend on which
//    block finished last, resets the counter and writes the rows.  The
//    hand-off relies on the same gfx950 ordering as the decode merge
//    (split_merge.hpp): write-through device-scope stores acknowledged
//    before a relaxed device-scope ticket.
//  * Rows are rounded once to the cache dtype; int8 caches store absmax
//    codes with an fp16 scale per (row, head) (max over the head's lanes by
//    DPP).
// Where the time goes (MI355X, 64 x 4096 -> 2 x 1536, timing copies with
// parts removed, taken with 8 k-groups): launch 1.8 us, result stores 1.5,
// the stage loop 1.5, the sum across waves 1.9 (0.44 us less with the 4
// k-groups above), the split-E exchange 3.7 (three dependent device-scope
// round trips), and about 5 us of loads on top.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

namespace {

typedef __bf16 as_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 as_bf16x8 __attribute__((ext_vector_type(8)));
typedef float as_f32x4 __attribute__((ext_vector_type(4)));
#define WSVD_LDS __attribute__((address_space(3)))

constexpr int kStageK = 256;   // rows of A per stage
constexpr int kWaves = 8;
constexpr int kKGroups = 4;                   // waves = k-groups x column groups
constexpr int kCGroups = kWaves / kKGroups;
constexpr int kKSteps = kStageK / 32 / kKGroups;  // 32-k MFMA steps per wave per stage
constexpr int kDepth = 4;      // stages in flight (registers)
constexpr int kRows = 64;      // rows of x per block
constexpr int kTargetBlocks = 160;

template <int NT>
struct Tile {
    static constexpr int CPR = NT / 8;                       // 16-byte chunks per A row
    static constexpr int NA = kStageK * CPR / 512;           // A chunks per thread per stage
    static constexpr int PITCH = NT * 2 + 32;                // LDS bytes per A row
    static constexpr int NJ = NT / 16;                       // 16-column groups
    static constexpr int OPT = NT * kRows / 512;             // outputs per thread at the end
    static constexpr int STAGE_BYTES = kStageK * PITCH;
    static constexpr int XPITCH = kStageK * 2 + 32;          // LDS bytes per x row of a stage (see below)
    static constexpr int XSTAGE_BYTES = kRows * XPITCH;
    static constexpr int BUF_BYTES = STAGE_BYTES + XSTAGE_BYTES;  // one stage of A and x
    static constexpr int RED_PITCH = NT + 4;                 // floats per reduction row (bank spread)
    static constexpr int RED_BYTES = kKGroups * kRows * RED_PITCH * 4;
    static constexpr int LDS_BYTES = (2 * BUF_BYTES > RED_BYTES) ? 2 * BUF_BYTES : RED_BYTES;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int kNt = 2;       // cache policy: streamed once
constexpr int kSc1 = 16;     // cache policy: device-coherent (written through)

__device__ __forceinline__ as_bf16x4 tr_read(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((WSVD_LDS as_bf16x4*)(WSVD_LDS unsigned char*)p);
}

template <int N>
__device__ __forceinline__ float lane_group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    return v;
}

// The 8 consecutive cache elements a thread owns, rounded once: one
// 16-byte store for bf16, two for f32.  Plain stores: the threads of a
// (row, head) segment fill whole L2 lines, which then go to memory once
// (write-through stores of the pieces measured the same time and twice
// the write traffic).
__device__ __forceinline__ void store_row_values(const AppendArgs& a, void* C, size_t off, const float (&v)[8]) {
    if (a.C_dt == WSVD_BF16) {
        u32x4 w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = (uint32_t)f32_to_bf16(v[2 * c]) | ((uint32_t)f32_to_bf16(v[2 * c + 1]) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(C) + off) = w;
    } else {  // F32
#pragma unroll
        for (int c = 0; c < 8; c += 4)
            *reinterpret_cast<u32x4*>(static_cast<float*>(C) + off + c) =
                u32x4{__float_as_uint(v[c]), __float_as_uint(v[c + 1]), __float_as_uint(v[c + 2]),
                      __float_as_uint(v[c + 3])};
    }
}

}  // namespace

// Block id -> (output tile, E slice).  Blocks are dealt to the 8 XCDs round
// robin; when KS divides 8 and the grid is a multiple of 8, XCD x only runs
// slice x % KS, so each XCD's L2 holds one slice of x instead of all of it.
__device__ __forceinline__ void block_tile(int id, int ntiles, int KS, int& tile, int& ks) {
    const int total = ntiles * KS;
    if (KS <= 8 && (8 % KS) == 0 && (total % 8) == 0) {
        const int xcd = id & 7;
        tile = (id >> 3) * (8 / KS) + xcd / KS;
        ks = xcd % KS;
    } else {
        tile = id % ntiles;
        ks = id / ntiles;
    }
}

template <int NT>
__global__ __launch_bounds__(512) void append_bf16_kernel(AppendArgs a) {
    using T = Tile<NT>;
    static_assert(T::OPT == 8, "the epilogue stores 8 outputs per thread");
    __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS_BYTES];
    __shared__ int sh_last;

    const int N1 = a.nh * a.r;
    const int ntile_n = (N1 + NT - 1) / NT;
    int tile, ks;
    block_tile(blockIdx.x, ntile_n * 2 * ((a.nb + kRows - 1) / kRows), a.KS, tile, ks);
    const int n0 = (tile % ntile_n) * NT;
    const int kv = (tile / ntile_n) & 1;
    const int m0 = (tile / ntile_n / 2) * kRows;
    const int e_len = a.E / a.KS;
    const int e_beg = ks * e_len;
    const int ns = e_len / kStageK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- operand addressing ---------------------------------------------------
    // A chunk c = tid + 512 i of a stage: row c / CPR, 8 columns at 8 (c % CPR).
    // Columns past N1 (a ragged last tile) read column 0: those outputs are
    // never written, and an output column depends only on its own column.
    const __amdgpu_buffer_rsrc_t ra = rsrc(kv ? a.A_V : a.A_K, (uint32_t)((size_t)a.E * N1 * 2));
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, (uint32_t)((size_t)a.nb * a.E * 2));
    uint32_t a_voff[T::NA], a_lds[T::NA];
#pragma unroll
    for (int i = 0; i < T::NA; ++i) {
        const int c = tid + 512 * i;
        const int row = c / T::CPR;
        int col = n0 + 8 * (c % T::CPR);
        if (col >= N1) col = 0;
        a_voff[i] = ((uint32_t)(e_beg + row) * (uint32_t)N1 + (uint32_t)col) * 2u;
        a_lds[i] = (uint32_t)(row * T::PITCH + (c % T::CPR) * 16);
    }
    const uint32_t a_stage_bytes = (uint32_t)kStageK * (uint32_t)N1 * 2u;
    // x chunk c = tid + 512 i of a stage: row c / 32, 8 k at 8 (c % 32), so a
    // wave-wide load reads two whole 512-byte row pieces (reading the operand
    // layout directly -- 16 rows x 64 bytes per load -- measured 1.2 us slower
    // at the LLaVA-7B step shape).  Rows past nb start past the end of x, where
    // buffer loads return zeros.  The stage goes to LDS (rows padded by 32
    // bytes: 0.2 us faster than a 16-byte pad at the LLaVA-7B step shape, 48
    // no better; the pad of A's rows, 16 to 48 bytes, made no difference) and each
    // wave reads back its fragments of 16-row group t: row 16 t + lane % 16,
    // k = the start of the wave's k-group slice (+ 32 per MFMA step),
    // 8 (lane / 16) onwards.
    uint32_t x_voff[4], x_lds[4], x_frag[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 512 * i;
        x_voff[i] = ((uint32_t)(m0 + c / 32) * (uint32_t)a.E + (uint32_t)(e_beg + 8 * (c % 32))) * 2u;
        x_lds[i] = (uint32_t)(T::STAGE_BYTES + (c / 32) * T::XPITCH + (c % 32) * 16);
        x_frag[i] = (uint32_t)(T::STAGE_BYTES + (16 * i + (lane & 15)) * T::XPITCH + 64 * kKSteps * (wave / kCGroups) +
                               16 * (lane >> 4));
    }

    u32x4 ar[kDepth][T::NA], xr[kDepth][4];
    auto load = [&](int d, int s) {
#pragma unroll
        for (int i = 0; i < T::NA; ++i)
            ar[d][i] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff[i], s * a_stage_bytes, kNt);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            xr[d][t] = __builtin_amdgcn_raw_buffer_load_b128(rx, x_voff[t], s * kStageK * 2, 0);
    };

    constexpr int NJW = T::NJ / kCGroups;  // 16-column groups of the wave's columns
    as_f32x4 acc[4][NJW];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < NJW; ++j) acc[t][j] = as_f32x4{0.f, 0.f, 0.f, 0.f};

    // B operand addresses inside a stage: lane s of each 16-lane group points
    // at row (its group's 8-k block of the wave's k-group slice) + s / 4 and
    // columns (the wave's column group) + 16 j + 4 (s % 4).
    const int brow = 32 * kKSteps * (wave / kCGroups) + 8 * (lane >> 4) + ((lane & 15) >> 2);
    const int bcol_bytes = 8 * (lane & 3) + 32 * NJW * (wave % kCGroups);

    auto consume = [&](int d, int s) {
        unsigned char* sa = smem + (s & 1) * T::BUF_BYTES;
#pragma unroll
        for (int i = 0; i < T::NA; ++i) *reinterpret_cast<u32x4*>(sa + a_lds[i]) = ar[d][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(sa + x_lds[i]) = xr[d][i];
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
            as_bf16x8 bf[NJW];
#pragma unroll
            for (int j = 0; j < NJW; ++j) {
                const unsigned char* p = sa + (brow + 32 * kk) * T::PITCH + 32 * j + bcol_bytes;
                const as_bf16x4 lo = tr_read(p);
                const as_bf16x4 hi = tr_read(p + 4 * T::PITCH);
                bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const as_bf16x8 xf =
                    __builtin_bit_cast(as_bf16x8, *reinterpret_cast<const u32x4*>(sa + x_frag[t] + 64 * kk));
#pragma unroll
                for (int j = 0; j < NJW; ++j)
                    acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, bf[j], acc[t][j], 0, 0, 0);
            }
        }
    };

    // Prologue: the first kDepth stages, requested unconditionally (a slice
    // shorter than kDepth stages re-requests its last stage).
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load(d, d < ns ? d : ns - 1);
    int s = 0;
    // Steady state: consume stage s + d from buffer d, refill it with stage
    // s + d + kDepth; no branch around any request.
    for (; s + 2 * kDepth <= ns; s += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            consume(d, s + d);
            load(d, s + d + kDepth);
        }
    }
    // Tail: fewer than 2 kDepth stages left.
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        if (s + d < ns) {
            consume(d, s + d);
            if (s + d + kDepth < ns) load(d, s + d + kDepth);
        }
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        if (s + kDepth + d < ns) consume(d, s + kDepth + d);

    // ---- sum the k-groups' partial tiles in LDS, in k order -------------------
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < NJW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((wave / kCGroups) * kRows + 16 * t + 4 * (lane >> 4) + i) * T::RED_PITCH +
                    16 * (NJW * (wave % kCGroups) + j) + (lane & 15)] = acc[t][j][i];
    __syncthreads();
    const int row = tid / (NT / T::OPT);          // 8 threads per row
    const int c0 = (tid % (NT / T::OPT)) * T::OPT;
    float v[T::OPT];
#pragma unroll
    for (int c = 0; c < T::OPT; ++c) v[c] = 0.f;
#pragma unroll
    for (int w = 0; w < kKGroups; ++w) {
#pragma unroll
        for (int c = 0; c < T::OPT; c += 4) {
            const as_f32x4 q = *reinterpret_cast<const as_f32x4*>(&red[(w * kRows + row) * T::RED_PITCH + c0 + c]);
            v[c] += q[0];
            v[c + 1] += q[1];
            v[c + 2] += q[2];
            v[c + 3] += q[3];
        }
    }

    // ---- split-E exchange -------------------------------------------------------
    if (a.KS > 1) {
        // A partial tile is stored lane-major -- 16-byte piece k of thread t
        // at (k * 512 + t) * 16 -- so each store instruction writes 1 KB
        // contiguous; only the same thread positions read it back.
        constexpr int TV = kRows * NT;  // floats per partial tile
        const __amdgpu_buffer_rsrc_t rp =
            rsrc(a.part + (size_t)tile * a.KS * TV, (uint32_t)((size_t)a.KS * TV * sizeof(float)));
        const uint32_t my_off = (uint32_t)tid * 16u;
#pragma unroll
        for (int c = 0; c < T::OPT; c += 4)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, as_f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]}),
                                                   rp, my_off + (c / 4) * 512u * 16u, ks * TV * 4, kSc1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            sh_last = (__hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (unsigned)(a.KS - 1));
        __syncthreads();
        if (!sh_last) return;
        // Sum in slice order; this block's own slice comes from registers.
        float sum[T::OPT];
#pragma unroll
        for (int c = 0; c < T::OPT; ++c) sum[c] = 0.f;
        for (int k = 0; k < a.KS; ++k) {
            if (k == ks) {
#pragma unroll
                for (int c = 0; c < T::OPT; ++c) sum[c] += v[c];
            } else {
#pragma unroll
                for (int c = 0; c < T::OPT; c += 4) {
                    const as_f32x4 q = __builtin_bit_cast(
                        as_f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, my_off + (c / 4) * 512u * 16u, k * TV * 4,
                                                                        kSc1));
                    sum[c] += q[0];
                    sum[c + 1] += q[1];
                    sum[c + 2] += q[2];
                    sum[c + 3] += q[3];
                }
            }
        }
        if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int c = 0; c < T::OPT; ++c) v[c] = sum[c];
    }

    // ---- round once and write row pos[m] of the head's cache --------------------
    const int m = m0 + row;
    const int n = n0 + c0;
    void* C = kv ? a.C_V : a.C_K;
    if (a.C_dt == WSVD_I8) {
        // absmax over the head's r columns: r / OPT consecutive lanes
        float mx = 0.f;
#pragma unroll
        for (int c = 0; c < T::OPT; ++c) mx = fmaxf(mx, fabsf(v[c]));
        const int g = a.r / T::OPT;   // 2, 4 or 8 lanes (heads never straddle a tile here)
        mx = (g == 2) ? lane_group_max<2>(mx) : (g == 4) ? lane_group_max<4>(mx) : lane_group_max<8>(mx);
        if (m >= a.nb || n >= N1) return;
        const int p = a.pos[m];
        if (p < 0 || p >= a.L_cap) return;
        const int h = n / a.r;
        const int col = n - h * a.r;
        const uint16_t sb = f32_to_f16(mx / 127.f);
        const float sc = f16_to_f32(sb);
        uint64_t codes = 0;
#pragma unroll
        for (int c = 0; c < T::OPT; ++c) {
            float q = 0.f;
            if (sc > 0.f) q = fminf(fmaxf(__builtin_rintf(v[c] / sc), -127.f), 127.f);
            codes |= (uint64_t)(uint8_t)(int8_t)(int)q << (8 * c);
        }
        const size_t rowi = ((size_t)m * a.nh + h) * a.L_cap + p;
        *reinterpret_cast<uint64_t*>(static_cast<int8_t*>(C) + rowi * a.r + col) = codes;
        if (col == 0) (kv ? a.s_V : a.s_K)[rowi] = sb;
        return;
    }
    if (m >= a.nb || n >= N1) return;
    const int p = a.pos[m];
    if (p < 0 || p >= a.L_cap) return;
    const int h = n / a.r;
    const size_t off = (((size_t)m * a.nh + h) * a.L_cap + p) * a.r + (n - h * a.r);
    store_row_values(a, C, off, v);
}

// Column tile: 64 columns (128-byte rows of A; whole heads of every rank but
// 48, as int8 caches need).  Measured on MI355X at the 64 x 4096 -> 2 x 1536
// shape: 32-column tiles with 2 slices double the x reads (each tile reads
// all of x over its slice) and ran 20.8 us, 64-column tiles with 2, 4 and 8
// slices 21.9, 16.1 and 28.7 us.
int append_bf16_tile_cols(int C_dt, int r) { (void)C_dt; (void)r; return 64; }

long append_bf16_num_tiles(int nb, int nh, int r, int NT) {
    return (((long)nh * r + NT - 1) / NT) * 2 * (((long)nb + kRows - 1) / kRows);
}

// Fewest E slices (whole 256-row stages, halving) that give >= 160 blocks.
int append_bf16_num_esplits(int nb, int E, int nh, int r, int NT) {
    const long nt = append_bf16_num_tiles(nb, nh, r, NT);
    int ks = 1;
    while (nt * ks < kTargetBlocks && E % (2L * ks * kStageK) == 0) ks *= 2;
    return ks;
}

size_t append_bf16_partial_bytes(int nb, int E, int nh, int r, int NT) {
    const int ks = append_bf16_num_esplits(nb, E, nh, r, NT);
    if (ks <= 1) return 0;
    return (size_t)append_bf16_num_tiles(nb, nh, r, NT) * ks * kRows * NT * sizeof(float);
}

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t st) {
    const int NT = append_bf16_tile_cols(a.C_dt, a.r);
    const int N1 = a.nh * a.r;
    const unsigned blocks = (unsigned)(((N1 + NT - 1) / NT) * 2 * ((a.nb + kRows - 1) / kRows) * a.KS);
    dim3 g(blocks);
    if (NT != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_bf16_kernel<64>, g, dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace wsvd
