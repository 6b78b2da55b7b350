// shared_decode.hip -- decoding over a conventional (whole-matrix) low-rank
// factorisation, the scheme the per-head kernel replaces.
//
// The usual SVD compression factors the whole K (V) projection with one
// latent of global rank R shared by all heads, and every head rebuilds its
// keys and values from that shared latent while decoding (Japanese page
// section 1, German page section 1, Italian page section 1, Arabic page
// section 1); per-head factors cut the latent from L x R to L x r and the
// rebuild cost by r / R (Arabic page section 2a, Italian page section 2A).
// Head h's keys are C_K[b] B_K[:, hH:(h+1)H] with C_K[b] in R^{L x R} and
// B_K in R^{R x nh H}; values likewise.
//
// The same fold as the per-head kernel applies -- s_t = C_K[b, t] . q'_h
// with q'_h = B_K[:, hH:(h+1)H] q_h -- so nothing of size L x H is ever
// formed; what remains is the defining cost of the scheme: every head
// streams the whole R-wide shared latent.  Four launches:
//   shared_fold_kernel   q'[b, h, :] (fp32), B_K read once per step;
//   shared_split_kernel  one block per (b, h, split): the shared latent
//                        rows of the split, one row per wave-wide pass
//                        (R / 64 elements per lane), online softmax, and the
//                        R-wide value accumulation; partials are R wide;
//   shared_merge_kernel  per (h, chunk of 128 latent columns, group of 8
//                        sequences): merge the partials on those columns and
//                        multiply by the same rows of B_V[:, hH:(h+1)H];
//   shared_sum_kernel    adds the chunk contributions in order.
// The latent is read with ordinary (cached) loads: the nh blocks of one
// sequence and split read the same rows, and they are placed on one XCD so
// that the repeats can be served from its L2.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {
namespace {

constexpr int kFoldRows = 4;      // rows of B_K per fold block
constexpr int kMergeSeqs = 8;     // sequences per merge block
constexpr int kMergeRows = 128;   // latent columns per merge block
constexpr int kXcds = 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(group_sum<16>(v))); }

// ---------------------------------------------------------------------------
// q'[b, h, k] = scale_log2 * sum_j B_K[k, hH + j] q[b, h, j].  Block (x, y):
// rows [kFoldRows x, +kFoldRows) and columns [2048 y, 2048 y + 2048) of B_K;
// each thread holds 8 consecutive columns (one 16-byte load per row), so the
// H / 8 threads of a head reduce over DPP.  A thread's slice of q[b, h] is
// loaded once per sequence and used for all of the block's rows.
template <int H>
__global__ __launch_bounds__(256) void shared_fold_kernel(int nb, int nh, int R, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ B_K, float scale_log2,
                                                          float* __restrict__ qp) {
    constexpr int GL = H / 8;  // lanes per head
    const int tid = threadIdx.x;
    const size_t ld = (size_t)nh * H;
    const size_t col = (size_t)blockIdx.y * 2048 + (size_t)tid * 8;
    const bool live_c = col < ld;
    const int h = (int)(col / H);
    const int e0 = (int)(col % H);
    const int k0 = blockIdx.x * kFoldRows;
    u32x4 bk[kFoldRows];
#pragma unroll
    for (int i = 0; i < kFoldRows; ++i) {
        bk[i] = u32x4{0u, 0u, 0u, 0u};
        if (live_c && k0 + i < R) bk[i] = *reinterpret_cast<const u32x4*>(B_K + (size_t)(k0 + i) * ld + col);
    }
    for (int b = 0; b < nb; ++b) {
        u32x4 qw = u32x4{0u, 0u, 0u, 0u};
        if (live_c) qw = *reinterpret_cast<const u32x4*>(q + ((size_t)b * nh + h) * H + e0);
#pragma unroll
        for (int i = 0; i < kFoldRows; ++i) {
            float p = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                p = fmaf(bf16_lo(bk[i][w]), bf16_lo(qw[w]), p);
                p = fmaf(bf16_hi(bk[i][w]), bf16_hi(qw[w]), p);
            }
            p = group_sum<GL>(p);
            if (live_c && (tid % GL) == 0 && k0 + i < R) qp[((size_t)b * nh + h) * R + k0 + i] = p * scale_log2;
        }
    }
}

// ---------------------------------------------------------------------------
// Split attention over the shared latent.  Blocks are laid out so that the
// nh heads of one (sequence, split) stream share an XCD: bid % 8 picks the
// XCD, streams are dealt to XCDs round-robin, heads fastest inside.
template <int R, int U>
__global__ __launch_bounds__(256) void shared_split_kernel(int nb, int nh, int S, int L_cap,
                                                           const int32_t* __restrict__ Ls,
                                                           const uint16_t* __restrict__ C_K,
                                                           const uint16_t* __restrict__ C_V,
                                                           const float* __restrict__ qp, float* __restrict__ o_part,
                                                           float* __restrict__ lse_part) {
    constexpr int EPL = R / 64;      // elements per lane of a row
    constexpr int NC = EPL / 8;      // 16-byte chunks per lane
    constexpr int NW = 4;
    static_assert(NC >= 1, "R >= 512");
    __shared__ float sh_acc[NW][R];
    __shared__ float sh_m[NW], sh_l[NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;
    const int x = bid % kXcds, slot = bid / kXcds;
    const int g = x + kXcds * (slot / nh);  // stream = b * S + s
    const int h = slot % nh;
    if (g >= nb * S) return;  // padding block (uniform)
    const int b = g / S, s = g % S;

    int ell = Ls[b];
    ell = min(max(ell, 0), L_cap);
    const int chunk = (ell + S - 1) / S;
    const int t0 = min(ell, s * chunk);
    const int t1 = min(ell, t0 + chunk);
    const int ntok = t1 - t0;
    const size_t bh = (size_t)b * nh + h;

    float qv[EPL];
    {
        const float4* src = reinterpret_cast<const float4*>(qp + bh * R + lane * EPL);
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c) {
            const float4 v = src[c];
            qv[4 * c + 0] = v.x;
            qv[4 * c + 1] = v.y;
            qv[4 * c + 2] = v.z;
            qv[4 * c + 3] = v.w;
        }
    }
    const char* kb = reinterpret_cast<const char*>(C_K + ((size_t)b * L_cap + t0) * R) + lane * EPL * 2;
    const char* vb = reinterpret_cast<const char*>(C_V + ((size_t)b * L_cap + t0) * R) + lane * EPL * 2;
    constexpr size_t RB = (size_t)R * 2;  // bytes per latent row

    u32x4 kA[U][NC], vA[U][NC], kB[U][NC], vB[U][NC];
    auto load_tile = [&](int tb, u32x4 (*kr)[NC], u32x4 (*vr)[NC]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t row = (size_t)min(tb + u, ntok - 1);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                kr[u][c] = *reinterpret_cast<const u32x4*>(kb + row * RB + 16 * c);
                vr[u][c] = *reinterpret_cast<const u32x4*>(vb + row * RB + 16 * c);
            }
        }
    };
    constexpr int STEP = NW * U;
    const int tb = wave * U;
    if (tb < ntok) load_tile(tb, kA, vA);
    if (tb + STEP < ntok) load_tile(tb + STEP, kB, vB);

    float m = kNegInf, l = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    auto consume = [&](int tbc, u32x4 (*kr)[NC], u32x4 (*vr)[NC]) {
        float sc[U];
        float mloc = kNegInf;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float p = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    p = fmaf(bf16_lo(kr[u][c][w]), qv[8 * c + 2 * w], p);
                    p = fmaf(bf16_hi(kr[u][c][w]), qv[8 * c + 2 * w + 1], p);
                }
            const float d = wave_sum(p);
            sc[u] = (tbc + u) < ntok ? d : kNegInf;
            mloc = fmaxf(mloc, sc[u]);
        }
        const float mn = fmaxf(m, mloc);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = fast_exp2(sc[u] - mu);
            l += p;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[8 * c + 2 * w] = fmaf(p, bf16_lo(vr[u][c][w]), acc[8 * c + 2 * w]);
                    acc[8 * c + 2 * w + 1] = fmaf(p, bf16_hi(vr[u][c][w]), acc[8 * c + 2 * w + 1]);
                }
        }
        m = mn;
    };

    const int nt = (ntok > tb) ? (ntok - tb + STEP - 1) / STEP : 0;
    int k = 0;
    for (; k + 3 < nt; k += 2) {
        consume(tb + k * STEP, kA, vA);
        load_tile(tb + (k + 2) * STEP, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        consume(tb + (k + 1) * STEP, kB, vB);
        load_tile(tb + (k + 3) * STEP, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int rem = nt - k;
    if (rem >= 1) consume(tb + k * STEP, kA, vA);
    if (rem >= 3) load_tile(tb + (k + 2) * STEP, kA, vA);
    if (rem >= 2) consume(tb + (k + 1) * STEP, kB, vB);
    if (rem >= 3) consume(tb + (k + 2) * STEP, kA, vA);

    // ---- merge the waves, normalise, store the R-wide partial -----------------
#pragma unroll
    for (int e = 0; e < EPL; ++e) sh_acc[wave][lane * EPL + e] = acc[e];
    if (lane == 0) {
        sh_m[wave] = m;
        sh_l[wave] = l;
    }
    __syncthreads();
    float M = sh_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sh_m[w]);
    float wt[NW];
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wt[w] = (sh_m[w] == kNegInf) ? 0.f : fast_exp2(sh_m[w] - M);
        Lt += sh_l[w] * wt[w];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    float* op = o_part + (bh * S + s) * R;
    for (int i = tid; i < R; i += 256) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) o = fmaf(sh_acc[w][i], wt[w], o);
        op[i] = o * inv;
    }
    if (tid == 0) lse_part[bh * S + s] = Lt > 0.f ? (M + fast_log2(Lt)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// Merge + projection, split over chunks of kMergeRows latent columns.  Block
// (h, c, y): for sequences [8y, 8y + 8) it merges the split partials on
// columns [128c, 128c + 128) only, then multiplies them by the same rows of
// B_V[:, hH:(h+1)H] (thread (kl, cg): 8 output columns cg, rows kl, kl + NKL,
// ..., 16-byte loads) and stores the chunk's contribution; shared_sum_kernel
// adds the chunks in order.
template <int H>
__global__ __launch_bounds__(256) void shared_merge_kernel(int nb, int nh, int S, int R,
                                                           const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           const uint16_t* __restrict__ B_V,
                                                           float* __restrict__ proj_part) {
    constexpr int GL = H / 8;        // threads per B_V row slice
    constexpr int NKL = 256 / GL;    // rows in flight
    __shared__ float sh_o[kMergeSeqs][kMergeRows];
    __shared__ float sh_w[64];
    __shared__ float sh_red[4][kMergeSeqs][H];
    const int tid = threadIdx.x;
    const int h = blockIdx.x, c = blockIdx.y;
    const int b0 = blockIdx.z * kMergeSeqs;
    const int nbg = min(kMergeSeqs, nb - b0);
    const int k0 = c * kMergeRows;

    // B_V rows of this chunk for the projection, requested first.
    static_assert(kMergeRows % NKL == 0, "projection rows per thread");
    const int cg = tid % GL, kl = tid / GL;
    const size_t ld = (size_t)nh * H;
    u32x4 bvr[kMergeRows / NKL];
#pragma unroll
    for (int it = 0; it < kMergeRows / NKL; ++it)
        bvr[it] = *reinterpret_cast<const u32x4*>(B_V + (size_t)(k0 + kl + it * NKL) * ld + (size_t)h * H + cg * 8);

    for (int u = 0; u < kMergeSeqs; ++u) {
        float acc = 0.f, wsum = 0.f;
        if (u < nbg) {
            const size_t bh = (size_t)(b0 + u) * nh + h;
            const float* lsp = lse_part + bh * S;
            // Loads eight at a time, issued before any is used.
            float Mx = kNegInf;
            for (int s0 = 0; s0 < S; s0 += 8) {
                float lv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) lv[i] = s0 + i < S ? lsp[s0 + i] : kNegInf;
#pragma unroll
                for (int i = 0; i < 8; ++i) Mx = fmaxf(Mx, lv[i]);
            }
            for (int s0 = 0; s0 < S; s0 += 64) {
                const int n = min(64, S - s0);
                __syncthreads();
                if (tid < n) {
                    const float lv = lsp[s0 + tid];
                    sh_w[tid] = (lv == kNegInf) ? 0.f : fast_exp2((lv - Mx) * kLog2e);
                }
                __syncthreads();
                if (tid < kMergeRows) {
                    for (int s1 = 0; s1 < n; s1 += 8) {
                        float ov[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            ov[i] = s1 + i < n ? o_part[(bh * S + s0 + s1 + i) * R + k0 + tid] : 0.f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            if (s1 + i < n) {
                                const float w = sh_w[s1 + i];
                                wsum += w;
                                acc = fmaf(w, ov[i], acc);
                            }
                        }
                    }
                }
            }
        }
        if (tid < kMergeRows) sh_o[u][tid] = wsum > 0.f ? acc / wsum : 0.f;
    }
    __syncthreads();

    float o[kMergeSeqs][8];
#pragma unroll
    for (int u = 0; u < kMergeSeqs; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[u][e] = 0.f;
    // This thread's kMergeRows / NKL rows of B_V, all requested before any is
    // used (the chunk's B_V was also requested before the merge above).
    constexpr int NIT = kMergeRows / NKL;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int k = kl + it * NKL;
        const u32x4 bv = bvr[it];
#pragma unroll
        for (int u = 0; u < kMergeSeqs; ++u) {
            const float ov = sh_o[u][k];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                o[u][2 * w] = fmaf(ov, bf16_lo(bv[w]), o[u][2 * w]);
                o[u][2 * w + 1] = fmaf(ov, bf16_hi(bv[w]), o[u][2 * w + 1]);
            }
        }
    }
    // Rows kl of one wave: lanes that differ in the bits above log2(GL).
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int u = 0; u < kMergeSeqs; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[u][e];
            for (int m = GL; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
            o[u][e] = v;
        }
    if (lane < GL) {
#pragma unroll
        for (int u = 0; u < kMergeSeqs; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) sh_red[wave][u][cg * 8 + e] = o[u][e];
    }
    __syncthreads();
    for (int i = tid; i < nbg * H; i += 256) {
        const int u = i / H, j = i % H;
        const float v = sh_red[0][u][j] + sh_red[1][u][j] + sh_red[2][u][j] + sh_red[3][u][j];
        proj_part[(((size_t)c * nb + b0 + u) * nh + h) * H + j] = v;
    }
}

// out[b, h, :] = sum over the R / kMergeRows chunk contributions, in order.
__global__ __launch_bounds__(256) void shared_sum_kernel(long n, int nc, const float* __restrict__ proj_part,
                                                         void* out, int out_dt) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    // nc <= 16 (R / 128): every contribution requested at once, summed in order.
    float pv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) pv[c] = c < nc ? proj_part[(size_t)c * n + i] : 0.f;
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        if (c < nc) v += pv[c];
    store_elem_wt(out, out_dt, (size_t)i, v);
}

template <int H, int R>
hipError_t launch_shared_hr(const SharedArgs& a, hipStream_t st) {
    constexpr int U = R >= 2048 ? 2 : 4;
    const long cols = (long)a.nh * H;
    hipLaunchKernelGGL((shared_fold_kernel<H>), dim3(R / kFoldRows, (unsigned)((cols + 2047) / 2048)), dim3(256), 0,
                       st, a.nb, a.nh, R, a.q, a.B_K, a.scale_log2, a.qp);
    const long streams = (long)a.nb * a.S;
    const long padded = (streams + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((shared_split_kernel<R, U>), dim3((unsigned)(padded * a.nh)), dim3(256), 0, st, a.nb, a.nh,
                       a.S, a.L_cap, a.L, a.C_K, a.C_V, a.qp, a.o_part, a.lse_part);
    hipLaunchKernelGGL((shared_merge_kernel<H>), dim3(a.nh, R / kMergeRows, (a.nb + kMergeSeqs - 1) / kMergeSeqs),
                       dim3(256), 0, st, a.nb, a.nh, a.S, R, a.o_part, a.lse_part, a.B_V, a.proj_part);
    const long n = (long)a.nb * a.nh * H;
    hipLaunchKernelGGL(shared_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, R / kMergeRows,
                       a.proj_part, a.out, a.out_dt);
    return hipGetLastError();
}

template <int H>
hipError_t launch_shared_h(const SharedArgs& a, hipStream_t st) {
    switch (a.R) {
        case 512: return launch_shared_hr<H, 512>(a, st);
        case 1024: return launch_shared_hr<H, 1024>(a, st);
        case 2048: return launch_shared_hr<H, 2048>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_shared_decode(const SharedArgs& a, hipStream_t st) {
    switch (a.H) {
        case 64: return launch_shared_h<64>(a, st);
        case 128: return launch_shared_h<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wsvd
