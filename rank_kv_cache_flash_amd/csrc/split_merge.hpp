// split_merge.hpp -- the in-kernel merge of split partials, shared by the
// split decode kernels.
//
// Flash-Decoding's merge ("WSVD: Weighted Low-Rank Approximation for Fast
// and Efficient Execution of Low-Precision Vision-Language Models", German
// page section 2D, Japanese page section 2.4): out = sum_s w_s o_s / sum_s
// w_s with w_s = exp(lse_s - max lse).  The partials were stored
// write-through at device scope; once every wave has seen its stores
// complete, one relaxed device-scope increment publishes them.  The split
// that brings the count to S reads them back with device-scope loads (not
// served from a stale L2 line), merges them in split order (so the result
// does not depend on which split finished last), writes out[b, h, :] and
// resets the counter.  No cache-wide writeback or invalidate is needed.
//
// Ordering assumption.  The partials and the counter are all relaxed
// device-scope atomics, so the language memory model alone does not order
// the partial stores before the increment.  The order comes from gfx950
// itself: a device-scope store is written through to memory (it does not
// stay in this XCD's L2), the s_waitcnt(0) below returns only once every
// such store of the wave has been acknowledged, and the barrier then holds
// the increment back until all waves got there; the reader's device-scope
// loads bypass the non-coherent L2 copies.  The portable form -- a release
// increment and an acquire on the last split -- compiles to a full L2
// writeback before the increment and an L2 invalidate after it; measured on
// MI355X it made the 1 x 32-head, 1088-token step 1.2 us slower (6.87 ->
// 8.10 us), so it is not used.  The cross-XCD repeated-merge test guards
// this assumption.
#pragma once

#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

// Call with every thread of the block after its partial and lse stores;
// sh_proj is 256 floats of LDS, sh_last one int of LDS.
template <int H>
__device__ __forceinline__ void merge_if_last_split(const DecodeArgs& a, size_t bh, int S, float* sh_proj,
                                                    int& sh_last) {
    const int tid = threadIdx.x;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        sh_last = (__hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(S - 1));
    __syncthreads();
    if (!sh_last) return;
    const float* lsp = a.lse_part + bh * S;
    const float* opp = a.o_part + bh * S * H;
    // Up to kFewSplits splits: every lane requests all lse values and its
    // o_part column in one round trip, then sums in split order exactly as
    // the chunked path below does for a single chunk.
    constexpr int kFewSplits = 8;
    if (S <= kFewSplits) {
        if (tid < H) {
            float lv[kFewSplits], ov[kFewSplits];
#pragma unroll
            for (int u = 0; u < kFewSplits; ++u) {
                lv[u] = u < S ? load_coherent(lsp + u) : kNegInf;
                ov[u] = u < S ? load_coherent(opp + (size_t)u * H + tid) : 0.f;
            }
            float M = kNegInf;
#pragma unroll
            for (int u = 0; u < kFewSplits; ++u) M = fmaxf(M, lv[u]);
            float accm = 0.f, wsum = 0.f;
            if (M != kNegInf) {
#pragma unroll
                for (int u = 0; u < kFewSplits; ++u) {
                    if (u < S) {
                        const float w = (lv[u] == kNegInf) ? 0.f : fast_exp2((lv[u] - M) * kLog2e);
                        wsum += w;
                        accm = fmaf(w, ov[u], accm);
                    }
                }
            }
            store_elem_wt(a.out, a.out_dt, bh * H + tid, wsum > 0.f ? accm / wsum : 0.f);
        }
        if (tid == 0) __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // Online merge over chunks of up to 256 splits: one parallel load of the
    // chunk's lse values into LDS, then each output lane issues its o_part
    // loads eight at a time before consuming them.
    float Mrun = kNegInf, accm = 0.f, wsum = 0.f;
    for (int k0 = 0; k0 < S; k0 += 256) {
        const int n = min(256, S - k0);
        __syncthreads();
        if (tid < n) sh_proj[tid] = load_coherent(lsp + k0 + tid);
        __syncthreads();
        float cm = kNegInf;
        for (int k = 0; k < n; ++k) cm = fmaxf(cm, sh_proj[k]);
        const float Mn = fmaxf(Mrun, cm);
        if (Mn == kNegInf) continue;
        const float rs = (Mrun == kNegInf) ? 0.f : fast_exp2((Mrun - Mn) * kLog2e);
        accm *= rs;
        wsum *= rs;
        Mrun = Mn;
        if (tid < H) {
            for (int k = 0; k < n; k += 8) {
                float ov[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    ov[u] = (k + u < n) ? load_coherent(opp + (size_t)(k0 + k + u) * H + tid) : 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (k + u < n) {
                        const float lv = sh_proj[k + u];
                        const float w = (lv == kNegInf) ? 0.f : fast_exp2((lv - Mn) * kLog2e);
                        wsum += w;
                        accm = fmaf(w, ov[u], accm);
                    }
                }
            }
        }
    }
    if (tid < H) store_elem_wt(a.out, a.out_dt, bh * H + tid, wsum > 0.f ? accm / wsum : 0.f);
    if (tid == 0) __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace wsvd
