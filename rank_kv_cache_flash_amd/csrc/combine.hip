// combine.hip -- log-sum-exp merge of split partials (the merge step of the
// Flash-Decoding pass named on the WSVD page, German page section 2D and
// Japanese page section 2.4).
//
//   out[b,h,:] = sum_s w_s o_s / sum_s w_s,   w_s = exp(lse_s - max_s lse_s)
//
// Empty splits (lse = -inf) weigh nothing; a row whose splits are all empty
// is zero.  The sum runs over s in index order, so the result does not
// depend on scheduling.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

// One block of 256 threads merges 256 / H rows (H = 64 or 128); lanes read
// o_part with unit stride, so every access is coalesced.
__global__ __launch_bounds__(256) void combine_kernel(int nbh, int H, int S, const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, void* out, int out_dt) {
    const int rows_per_block = 256 / H;
    const int row = blockIdx.x * rows_per_block + threadIdx.x / H;
    const int t = threadIdx.x % H;
    if (row >= nbh) return;
    const float* ls = lse_part + (size_t)row * S;
    const float* op = o_part + (size_t)row * S * H + t;
    float M = kNegInf;
    float acc = 0.f, wsum = 0.f;
    constexpr int kFew = 8;
    if (S <= kFew) {
        // Every lse value and this lane's o_part column requested at once (one
        // round trip); the sum below runs in the same order as the loop form.
        float lv[kFew], ov[kFew];
#pragma unroll
        for (int s = 0; s < kFew; ++s) {
            lv[s] = s < S ? ls[s] : kNegInf;
            ov[s] = s < S ? op[(size_t)s * H] : 0.f;
        }
#pragma unroll
        for (int s = 0; s < kFew; ++s) M = fmaxf(M, lv[s]);
        if (M != kNegInf) {
#pragma unroll
            for (int s = 0; s < kFew; ++s) {
                if (s < S) {
                    const float w = (lv[s] == kNegInf) ? 0.f : fast_exp2((lv[s] - M) * kLog2e);
                    wsum += w;
                    acc = fmaf(w, ov[s], acc);
                }
            }
        }
    } else {
        for (int s = 0; s < S; ++s) M = fmaxf(M, ls[s]);
        if (M != kNegInf) {
            for (int s = 0; s < S; ++s) {
                const float lv = ls[s];
                const float w = (lv == kNegInf) ? 0.f : fast_exp2((lv - M) * kLog2e);
                wsum += w;
                acc = fmaf(w, op[(size_t)s * H], acc);
            }
        }
    }
    const float v = (wsum > 0.f) ? acc / wsum : 0.f;
    store_elem_wt(out, out_dt, (size_t)row * H + t, v);
}

// Zero n uint32 words with vector stores (a kernel rather than a memset, so
// it can sit in a captured graph like the calls around it).
__global__ __launch_bounds__(256) void fill_zero_u32_kernel(unsigned* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_fill_zero_u32(unsigned* p, size_t n, hipStream_t st) {
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_zero_u32_kernel, dim3((unsigned)(blocks < 1024 ? (blocks ? blocks : 1) : 1024)),
                       dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_combine(int nb, int nh, int H, int S, const float* o_part, const float* lse_part, void* out,
                          int out_dt, hipStream_t st) {
    const int nbh = nb * nh;
    const int rows_per_block = 256 / H;
    const unsigned nblk = (unsigned)((nbh + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(combine_kernel, dim3(nblk), dim3(256), 0, st, nbh, H, S, o_part, lse_part, out, out_dt);
    return hipGetLastError();
}

}  // namespace wsvd
