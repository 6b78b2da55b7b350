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
// Kernel 1 (gemm): block = 64 rows of x  x  64 columns of A  x  one E-slice of
// EC rows.  Enough E-slices are used to put >= 1.5 blocks on each CU.  A
// arrives row-major (columns contiguous) but the MFMA B operand wants 8
// consecutive k per lane, so each thread loads an 8 x 8 (k x n) bf16 block
// with eight 16-byte loads (a wave covers 8 full 128-byte rows per load),
// transposes it in registers and stores 8 k-contiguous vectors into LDS.
// The LDS tile is [64 n][EC k] with a 16-byte row pad and the k-block index
// xor-swizzled by n/8, so both the transposed stores and the fragment reads
// are free of bank conflicts.  Each wave owns 16 rows of x and all 64
// columns: 4 accumulators of 16 x 16.  The fp32 partial tile goes to the
// workspace.
// Kernel 2 (reduce + scatter): sums the E-slices in index order (so the
// result is deterministic), rounds once to the cache dtype and writes row
// pos[b] of every head's K and V cache.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int AP_NT = 64;           // columns per block
constexpr int AP_MT = 64;           // rows of x per block
constexpr int AP_EC = 256;          // E rows per LDS stage
constexpr int AP_PITCH = AP_EC + 8; // bf16 elements per LDS row (16-byte pad)

union V16 {
    u32x4 u;
    bf16x8 b;
};

__global__ __launch_bounds__(256) void append_gemm_kernel(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sB[AP_NT * AP_PITCH];

    const int N1 = a.nh * a.r;
    const int n0 = blockIdx.x * AP_NT;
    const int kv = blockIdx.y & 1;
    const int m0 = (blockIdx.y >> 1) * AP_MT;
    const int ks = blockIdx.z;
    const int e_len = a.E / a.KS;
    const int e_beg = ks * e_len;
    const uint16_t* A = kv ? a.A_V : a.A_K;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // loader role: 8 x 8 block (k rows kblk*8.., n cols nblk*8..)
    const int nblk = tid & 7;
    const int kblk = tid >> 3;  // 0..31
    const int ncol = n0 + nblk * 8;
    const bool col_ok = ncol < N1;  // N1 is a multiple of 16

    // MFMA role
    const int mrow = m0 + wave * 16 + (lane & 15);
    const bool row_ok = mrow < a.nb;
    const int kq = (lane >> 4) * 8;  // this lane's k offset inside a 32-wide step

    f32x4 acc[4];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[jn] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int es = e_beg; es < e_beg + e_len; es += AP_EC) {
        // ---- global -> registers -------------------------------------------
        u32x4 blk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const size_t e = (size_t)es + kblk * 8 + i;
            blk[i] = col_ok ? load16_stream(A + e * N1 + ncol) : u32x4{0u, 0u, 0u, 0u};
        }
        V16 xf[AP_EC / 32];
#pragma unroll
        for (int st = 0; st < AP_EC / 32; ++st) {
            xf[st].u = row_ok ? *reinterpret_cast<const u32x4*>(a.x + (size_t)mrow * a.E + es + st * 32 + kq)
                              : u32x4{0u, 0u, 0u, 0u};
        }
        // ---- 8 x 8 transpose: out[n'] holds k = 0..7 of column n' ------------
        u32x4 tr[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t r0 = blk[2 * p][w], r1 = blk[2 * p + 1][w];
                tr[2 * w][p] = (r0 & 0xffffu) | (r1 << 16);
                tr[2 * w + 1][p] = (r0 >> 16) | (r1 & 0xffff0000u);
            }
        }
        __syncthreads();  // previous stage's readers are done
#pragma unroll
        for (int np = 0; np < 8; ++np) {
            const int n = nblk * 8 + np;
            const int kb = kblk ^ (nblk & 7);
            *reinterpret_cast<u32x4*>(&sB[n * AP_PITCH + kb * 8]) = tr[np];
        }
        __syncthreads();
        // ---- MFMA over the stage ----------------------------------------------
#pragma unroll
        for (int st = 0; st < AP_EC / 32; ++st) {
#pragma unroll
            for (int jn = 0; jn < 4; ++jn) {
                const int n = jn * 16 + (lane & 15);
                const int kb = (st * 4 + (lane >> 4)) ^ ((n >> 3) & 7);
                V16 bf;
                bf.u = *reinterpret_cast<const u32x4*>(&sB[n * AP_PITCH + kb * 8]);
                acc[jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[st].b, bf.b, acc[jn], 0, 0, 0);
            }
        }
    }

    // ---- partial tile -> workspace: part[ks][m][kv*N1 + n] ------------------
    const int N2 = 2 * N1;
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
        const int n = n0 + jn * 16 + (lane & 15);
        if (n >= N1) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wave * 16 + (lane >> 4) * 4 + i;
            if (m < a.nb) a.part[((size_t)ks * a.nb + m) * N2 + kv * N1 + n] = acc[jn][i];
        }
    }
}

__global__ __launch_bounds__(256) void append_scatter_kernel(AppendArgs a) {
    const int N1 = a.nh * a.r;
    const int N2 = 2 * N1;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.nb * N2) return;
    const int b = (int)(idx / N2);
    const int n = (int)(idx % N2);
    const int p = a.pos[b];
    if (p < 0 || p >= a.L_cap) return;
    float v = 0.f;
    for (int ks = 0; ks < a.KS; ++ks) v += a.part[((size_t)ks * a.nb + b) * N2 + n];
    const int kv = n >= N1;
    const int nn = n - kv * N1;
    const int h = nn / a.r;
    const int i = nn % a.r;
    void* C = kv ? a.C_V : a.C_K;
    const size_t off = (((size_t)b * a.nh + h) * a.L_cap + p) * a.r + i;
    store_elem(C, a.C_dt, off, v);
}

int append_num_esplits(int nb, int E, int nh, int r) {
    // Blocks without E-splitting: column tiles x {K, V} x row tiles.
    const long ntile = (long)((nh * r + AP_NT - 1) / AP_NT) * 2 * ((nb + AP_MT - 1) / AP_MT);
    int ks = 1;
    // >= 1.5 blocks per CU (256 CUs), E-slices a multiple of the LDS stage.
    while (ntile * ks < 384 && E % (2 * ks * AP_EC) == 0) ks *= 2;
    return ks;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
    const int N1 = a.nh * a.r;
    dim3 g1((N1 + AP_NT - 1) / AP_NT, 2 * ((a.nb + AP_MT - 1) / AP_MT), a.KS);
    hipLaunchKernelGGL(append_gemm_kernel, g1, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t tot = (size_t)a.nb * 2 * N1;
    hipLaunchKernelGGL(append_scatter_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace wsvd
