// decode.hip -- split-L low-rank flash decoding over a per-head latent cache.
//
// One workgroup handles one (sequence b, head h, split s).  What it computes
// is the fused pass described for WSVD on the page "WSVD: Weighted Low-Rank
// Approximation for Fast and Efficient Execution of Low-Precision
// Vision-Language Models" (German page section 2D, Italian page section 2D,
// Arabic page section 2c, Japanese page section 2.4): latent rows are
// streamed from HBM and consumed on chip by qK^T, softmax and the V product;
// neither K nor V is ever written to memory.
//
// The factor is applied without per-token reconstruction:
//   score_t = sigma q . (c_t B_K) = c_t . (B_K q)      (q' folded once)
//   o       = sum_t p_t (v_t B_V) = (sum_t p_t v_t) B_V (projected once)
// so the hot loop is an r-long dot and an r-long scaled add per token, and
// the only bytes per token are the two latent rows (plus two fp16 scales for
// an int8 cache).  That is what keeps the kernel on the HBM roof.
//
// Hot-loop layout (gfx950, wave64).  A lane owns a 16-byte chunk of a latent
// row: EPC = 16 / sizeof(element) consecutive dims.  G = r / EPC lanes hold
// one row; rows sit in slots of GP = next_pow2(G) lanes (lanes j >= G of a
// slot are idle and contribute zeros), so one wave-wide 16-byte load reads
// RW = 64 / GP consecutive rows -- one contiguous block of HBM.  The score
// of a row is reduced inside its slot with DPP row operations.  Each slot
// keeps its own running max / sum (online softmax); slots, waves and then
// splits are merged by log-sum-exp weights.
//
// int8 rows are converted with the byte-to-float instructions after an
// xor with 0x80 (value = byte - 128); the -128 offset is folded into a
// per-lane constant for the scores and into a running sum of weights for V,
// so each code costs one convert and one FMA.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

template <int CT> struct CacheTraits;
template <> struct CacheTraits<WSVD_F32> { static constexpr int EPC = 4; static constexpr int SZ = 4; };
template <> struct CacheTraits<WSVD_BF16> { static constexpr int EPC = 8; static constexpr int SZ = 2; };
template <> struct CacheTraits<WSVD_I8> { static constexpr int EPC = 16; static constexpr int SZ = 1; };

constexpr int next_pow2(int x) { return x <= 1 ? 1 : 2 * next_pow2((x + 1) / 2); }

// Dot of one 16-byte chunk with the lane's slice of q'.
template <int CT>
__device__ __forceinline__ float chunk_dot(const u32x4& d, const float* qp) {
    float acc = 0.f;
    if constexpr (CT == WSVD_F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = fmaf(qp[k], __uint_as_float(d[k]), acc);
    } else if constexpr (CT == WSVD_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc = fmaf(qp[2 * k], bf16_lo(d[k]), acc);
            acc = fmaf(qp[2 * k + 1], bf16_hi(d[k]), acc);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t u = d[k] ^ 0x80808080u;
#pragma unroll
            for (int c = 0; c < 4; ++c) acc = fmaf(qp[4 * k + c], float((u >> (8 * c)) & 0xffu), acc);
        }
    }
    return acc;
}

// acc += w * chunk (int8: w * (byte + 128); the offset is removed later).
template <int CT>
__device__ __forceinline__ void chunk_axpy(const u32x4& d, float w, float* acc) {
    if constexpr (CT == WSVD_F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = fmaf(w, __uint_as_float(d[k]), acc[k]);
    } else if constexpr (CT == WSVD_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] = fmaf(w, bf16_lo(d[k]), acc[2 * k]);
            acc[2 * k + 1] = fmaf(w, bf16_hi(d[k]), acc[2 * k + 1]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t u = d[k] ^ 0x80808080u;
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[4 * k + c] = fmaf(w, float((u >> (8 * c)) & 0xffu), acc[4 * k + c]);
        }
    }
}

template <int H, int R, int CT, int U>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    using T = CacheTraits<CT>;
    constexpr int EPC = T::EPC;
    constexpr int G = R / EPC;
    static_assert(R % EPC == 0, "rank must fill whole 16-byte chunks");
    constexpr int GP = next_pow2(G);
    static_assert(GP <= 16, "a row must fit one DPP row of 16 lanes");
    constexpr int RW = 64 / GP;
    constexpr int NW = 4;
    constexpr int TILE = U * RW;
    constexpr bool I8 = (CT == WSVD_I8);

    __shared__ float sh_q[H];
    __shared__ float sh_qp[R];
    __shared__ float sh_red_o[NW][R];
    __shared__ float sh_red_m[NW];
    __shared__ float sh_red_l[NW];
    __shared__ float sh_on[R];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Block -> (b, s, h) with h fastest: consecutive blocks land on different
    // XCDs round-robin, so with nh a multiple of 8 each head always runs on
    // the same XCD and its factors stay in that XCD's L2.
    const int bid = blockIdx.x;
    const int h = bid % a.nh;
    const int rest = bid / a.nh;
    const int s = rest % a.S;
    const int b = rest / a.S;

    int ell = a.L[b];
    ell = min(max(ell, 0), a.L_cap);
    const int chunk = (ell + a.S - 1) / a.S;
    const int t0 = min(ell, s * chunk);
    const int t1 = min(ell, t0 + chunk);

    const size_t bh = (size_t)b * a.nh + h;
    float* o_out = a.o_part + (bh * a.S + s) * H;
    if (t0 >= t1) {  // empty split: uniform over the block
        for (int i = tid; i < H; i += 256) o_out[i] = 0.f;
        if (tid == 0) a.lse_part[bh * a.S + s] = kNegInf;
        return;
    }

    // ---- prologue: q' = (sigma log2 e) B_K[h] q ---------------------------
    for (int i = tid; i < H; i += 256) sh_q[i] = load_elem(a.q, a.q_dt, bh * H + i);
    __syncthreads();
    {
        const int i = tid >> 2, qq = tid & 3;
        float acc = 0.f;
        if (i < R) {
            const size_t base = ((size_t)h * R + i) * H + qq * (H / 4);
#pragma unroll 8
            for (int j = 0; j < H / 4; ++j) acc = fmaf(load_elem(a.B_K, a.B_dt, base + j), sh_q[qq * (H / 4) + j], acc);
        }
        acc = group_sum<4>(acc);
        if (i < R && qq == 0) sh_qp[i] = acc * a.scale_log2;
    }
    __syncthreads();

    const int g = lane / GP;
    const int j = lane % GP;
    const bool act = j < G;
    float qp[EPC];
#pragma unroll
    for (int c = 0; c < EPC; ++c) qp[c] = act ? sh_qp[min(j, G - 1) * EPC + c] : 0.f;
    float qoff = 0.f;  // int8: sum of the lane's q' slice, times 128
    if constexpr (I8) {
#pragma unroll
        for (int c = 0; c < EPC; ++c) qoff += qp[c];
        qoff *= 128.f;
    }

    // ---- hot loop ----------------------------------------------------------
    const size_t row_bytes = (size_t)R * T::SZ;
    const char* kbase = static_cast<const char*>(a.C_K) + (bh * a.L_cap + t0) * row_bytes + j * 16;
    const char* vbase = static_cast<const char*>(a.C_V) + (bh * a.L_cap + t0) * row_bytes + j * 16;
    const uint16_t* skb = I8 ? a.s_K + bh * a.L_cap + t0 : nullptr;
    const uint16_t* svb = I8 ? a.s_V + bh * a.L_cap + t0 : nullptr;
    const int ntok = t1 - t0;

    float m = kNegInf, l = 0.f, pw = 0.f;
    float acc[EPC];
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] = 0.f;

    for (int tb = wave * TILE; tb < ntok; tb += NW * TILE) {
        u32x4 kr[U], vr[U];
        float sk[U], sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = tb + u * RW + g;
            const bool rv = row < ntok;
            if (rv && act) {
                kr[u] = load16_stream(kbase + (size_t)row * row_bytes);
                vr[u] = load16_stream(vbase + (size_t)row * row_bytes);
            } else {
                kr[u] = u32x4{0u, 0u, 0u, 0u};
                vr[u] = u32x4{0u, 0u, 0u, 0u};
            }
            if constexpr (I8) {
                sk[u] = rv ? f16_to_f32(skb[row]) : 0.f;
                sv[u] = rv ? f16_to_f32(svb[row]) : 0.f;
            }
        }
        float sc[U];
        float mloc = kNegInf;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float part = chunk_dot<CT>(kr[u], qp);
            if constexpr (I8) part -= qoff;  // zero chunks (idle lane / past the end) cancel too
            float d = group_sum<GP>(part);
            if constexpr (I8) d *= sk[u];
            sc[u] = (tb + u * RW + g) < ntok ? d : kNegInf;
            mloc = fmaxf(mloc, sc[u]);
        }
        const float mn = fmaxf(m, mloc);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        l *= alpha;
        if constexpr (I8) pw *= alpha;
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = fast_exp2(sc[u] - mu);
            l += p;
            float w = p;
            if constexpr (I8) {
                w *= sv[u];
                pw += w;
            }
            chunk_axpy<CT>(vr[u], w, acc);
        }
        m = mn;
    }

    // ---- merge slots inside the wave ---------------------------------------
    float Mw = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) Mw = fmaxf(Mw, shfl_xor_f(Mw, off));
    const float f = (m == kNegInf) ? 0.f : fast_exp2(m - Mw);
    l *= f;
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] *= f;
    if constexpr (I8) {
        pw *= f;
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] -= 128.f * pw;
    }
#pragma unroll
    for (int off = GP; off < 64; off <<= 1) {
        l += shfl_xor_f(l, off);
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] += shfl_xor_f(acc[c], off);
    }
    if (g == 0 && act) {
#pragma unroll
        for (int c = 0; c < EPC; ++c) sh_red_o[wave][j * EPC + c] = acc[c];
    }
    if (lane == 0) {
        sh_red_m[wave] = Mw;
        sh_red_l[wave] = l;
    }
    __syncthreads();

    // ---- merge waves, normalise, project through B_V ------------------------
    float M = sh_red_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sh_red_m[w]);
    float wt[NW];
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wt[w] = (sh_red_m[w] == kNegInf) ? 0.f : fast_exp2(sh_red_m[w] - M);
        Lt += sh_red_l[w] * wt[w];
    }
    if (tid < R) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) o = fmaf(sh_red_o[w][tid], wt[w], o);
        sh_on[tid] = o / Lt;
    }
    __syncthreads();
    for (int jj = tid; jj < H; jj += 256) {
        float o = 0.f;
        const size_t base = (size_t)h * R * H + jj;
#pragma unroll 8
        for (int i = 0; i < R; ++i) o = fmaf(sh_on[i], load_elem(a.B_V, a.B_dt, base + (size_t)i * H), o);
        o_out[jj] = o;
    }
    if (tid == 0) a.lse_part[bh * a.S + s] = (M + fast_log2(Lt)) * kLn2;
}

template <int H, int R, int CT>
static hipError_t launch_hrc(const DecodeArgs& a, hipStream_t st) {
    constexpr int U = 4;
    const unsigned nblk = (unsigned)((size_t)a.nb * a.nh * a.S);
    hipLaunchKernelGGL((decode_split_kernel<H, R, CT, U>), dim3(nblk), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int H, int R>
static hipError_t launch_hr(const DecodeArgs& a, int C_dt, hipStream_t st) {
    switch (C_dt) {
        case WSVD_F32: return launch_hrc<H, R, WSVD_F32>(a, st);
        case WSVD_BF16: return launch_hrc<H, R, WSVD_BF16>(a, st);
        case WSVD_I8: return launch_hrc<H, R, WSVD_I8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int H>
static hipError_t launch_h(const DecodeArgs& a, int r, int C_dt, hipStream_t st) {
    switch (r) {
        case 16: return launch_hr<H, 16>(a, C_dt, st);
        case 32: return launch_hr<H, 32>(a, C_dt, st);
        case 48: return launch_hr<H, 48>(a, C_dt, st);
        case 64: return launch_hr<H, 64>(a, C_dt, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_split(const DecodeArgs& a, int H, int r, int C_dt, hipStream_t st) {
    switch (H) {
        case 64: return launch_h<64>(a, r, C_dt, st);
        case 128: return launch_h<128>(a, r, C_dt, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wsvd
