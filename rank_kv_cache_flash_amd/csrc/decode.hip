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
// slot repeat chunk G-1 with a zero q' slice), so one wave-wide 16-byte load
// reads RW = 64 / GP consecutive rows -- one contiguous block of HBM.  The
// score of a row is reduced inside its slot with DPP row operations.  Each
// slot keeps its own running max / sum (online softmax); slots, waves and
// then splits are merged by log-sum-exp weights.  Each wave double-buffers U
// row batches in registers (tiles), so the next tile is in flight while the
// current one is consumed.  The steady-state loop has no branch around a
// load (rows past the end of the split re-read its last row and score
// -inf), its buffers stay in fixed registers, and the tail requests only
// tiles that exist.  Loads use a wave-uniform 64-bit base plus a 32-bit lane
// offset (the scalar-base load form).
//
// Prologue: q and both factors, then the first two latent tiles of every
// wave, are requested before anything waits, all without a branch: vector
// loads complete in order, so a wait for q placed after a conditional tile
// request would also wait for the tiles.  q' = B_K q is formed from the
// factor chunks held in registers while the tiles are in flight; B_V stays in
// LDS for the projection at the end.  The in-wave merge uses VALU cross-lane
// operations (DPP row rotations and the gfx950 permlane16/32 swaps), not LDS
// round trips.
//
// Merge: with one split and an output the block writes out directly.  With
// more splits and an output (and a grid small enough for the host to keep
// the merge in this launch), each split stores its partial, then the last
// split of a (b, h) to finish (a per-(b, h) counter in the workspace, reset
// by that split) merges all of them in split order, so the result is
// deterministic.  Larger grids leave the merge to a second launch.
//
// The online softmax moves its reference max only when a score passes it by
// 2^8, so the accumulators are not rescaled on every tile.
//
// int8 rows: after an xor with 0x80, one byte permute turns two codes into
// two exact fp16 values 1024 + 128 + code, and each code then costs one
// mixed-precision FMA (fp16 operand, fp32 accumulate); the offset is folded
// into a per-lane constant for the scores and into a running sum of weights
// for V.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"
#include "split_merge.hpp"

namespace wsvd {

template <int CT> struct CacheTraits;
template <> struct CacheTraits<WSVD_F32> { static constexpr int EPC = 4; static constexpr int SZ = 4; };
template <> struct CacheTraits<WSVD_BF16> { static constexpr int EPC = 8; static constexpr int SZ = 2; };
template <> struct CacheTraits<WSVD_I8> { static constexpr int EPC = 16; static constexpr int SZ = 1; };

constexpr int next_pow2(int x) { return x <= 1 ? 1 : 2 * next_pow2((x + 1) / 2); }

// Element e of a 16-byte chunk of a factor of dtype BT, as float.
template <int BT>
__device__ __forceinline__ float chunk_elem(const u32x4& d, int e) {
    if constexpr (BT == WSVD_F32) {
        return __uint_as_float(d[e]);
    } else if constexpr (BT == WSVD_BF16) {
        return (e & 1) ? bf16_hi(d[e >> 1]) : bf16_lo(d[e >> 1]);
    } else {
        return f16_to_f32((e & 1) ? uint16_t(d[e >> 1] >> 16) : uint16_t(d[e >> 1] & 0xffffu));
    }
}

template <int BT>
__device__ __forceinline__ float raw_elem(const void* base, int idx) {
    if constexpr (BT == WSVD_F32) {
        return static_cast<const float*>(base)[idx];
    } else if constexpr (BT == WSVD_BF16) {
        return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    } else {
        return f16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    }
}

// int8 codes as exact fp16 values: byte c + 128 placed in the mantissa of
// 1024 (fp16 0x6400 | u = 1024 + u), two codes per dword by one byte
// permute, so each code then costs one mixed-precision FMA (fp16 operand,
// fp32 accumulate) instead of a conversion and an FMA.  Every value carries
// an offset of kI8Offset = 1024 + 128, removed once per row (scores) and once
// per split (values).
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
constexpr float kI8Offset = 1152.f;
__device__ __forceinline__ h2 i8_pair_lo(uint32_t w) {
    return __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, 0x04010400u));
}
__device__ __forceinline__ h2 i8_pair_hi(uint32_t w) {
    return __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, 0x04030402u));
}

// Dot of one 16-byte latent chunk with the lane's slice of q'.
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
            const h2 lo = i8_pair_lo(d[k]), hi = i8_pair_hi(d[k]);
            acc = fmaf(qp[4 * k + 0], (float)lo.x, acc);
            acc = fmaf(qp[4 * k + 1], (float)lo.y, acc);
            acc = fmaf(qp[4 * k + 2], (float)hi.x, acc);
            acc = fmaf(qp[4 * k + 3], (float)hi.y, acc);
        }
    }
    return acc;
}

// acc += w * chunk (int8: w * (code + kI8Offset); the offset is removed later).
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
            const h2 lo = i8_pair_lo(d[k]), hi = i8_pair_hi(d[k]);
            acc[4 * k + 0] = fmaf(w, (float)lo.x, acc[4 * k + 0]);
            acc[4 * k + 1] = fmaf(w, (float)lo.y, acc[4 * k + 1]);
            acc[4 * k + 2] = fmaf(w, (float)hi.x, acc[4 * k + 2]);
            acc[4 * k + 3] = fmaf(w, (float)hi.y, acc[4 * k + 3]);
        }
    }
}

// DENSE = true is the comparison baseline: ordinary Flash-Decoding over full
// K / V rows (r = H, no factors): q' is q itself and the partial is o / l.
//
// Rank-48 instances are held to 3 waves per SIMD (3 resident blocks per CU):
// measured on MI355X over the ragged 64 x 32-head step, a 4th resident block
// per CU made the split kernel about 2.5 us slower.
template <int H, int R, int CT, int BT, int U, bool DENSE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, (R == 48) ? 3 : 8)))
void decode_split_kernel(DecodeArgs a) {
    static_assert(!DENSE || R == H, "dense rows are H wide");
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
    constexpr int BES = (BT == WSVD_F32) ? 4 : 2;  // factor element bytes
    constexpr int BEPC = 16 / BES;                 // factor elements per chunk
    constexpr int NBC = DENSE ? 1 : R * H / BEPC;  // chunks per factor
    constexpr int NBT = (NBC + 255) / 256;         // chunks per thread
    constexpr int CPR = H / BEPC;                  // chunks per factor row
    constexpr int NPART = 256 / H;                 // projection: threads per output
    static_assert(R % NPART == 0, "projection split");

    __shared__ float sh_q[256];  // q in [0, H); every thread stores its word
    __shared__ float sh_qpart[NBC];
    __shared__ float sh_qp[R];
    __shared__ u32x4 sh_bv[NBC];
    __shared__ float sh_red_o[NW][R];
    __shared__ float sh_red_m[NW];
    __shared__ float sh_red_l[NW];
    __shared__ float sh_on[R];
    __shared__ float sh_proj[256];
    __shared__ int sh_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index through readfirstlane: the compiler then treats it (and the
    // token loop bounds derived from it) as wave-uniform scalar values.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Block -> (b, s, h) with h fastest: consecutive blocks land on different
    // XCDs round-robin, so with nh a multiple of 8 each head always runs on
    // the same XCD and its factors stay in that XCD's L2.
    const int bid = blockIdx.x;
    const int h = bid % a.nh;
    const int rest = bid / a.nh;
    const int s = rest % a.S;
    const int b = rest / a.S;
    const int S = a.S;

    const size_t bh = (size_t)b * a.nh + h;
    int ell = a.L[b];

    // ---- requests: q, B_K, B_V (independent of the length, so they travel
    // together with the L[b] read instead of after it) ----------------------
    const size_t q_idx = bh * H + (tid < H ? tid : 0);
    const uint32_t q_word = load_q_word(a.q, a.q_dt, q_idx);
    const char* bk_base = static_cast<const char*>(a.B_K) + (size_t)h * R * H * BES;
    const char* bv_base = static_cast<const char*>(a.B_V) + (size_t)h * R * H * BES;
    // int8 caches: B_V (needed only after the token loop) is requested after
    // the fold, so the first burst of requests -- which every block of the
    // large int8 grids issues at once -- carries only q, B_K and latent tiles.
    constexpr bool LATE_BV = I8;
    u32x4 bk[NBT], bv[NBT];
#pragma unroll
    for (int k = 0; k < NBT; ++k) {
        const int c = tid + 256 * k;
        if (!DENSE && (NBC % 256 == 0 || c < NBC)) {
            bk[k] = *reinterpret_cast<const u32x4*>(bk_base + (size_t)c * 16);
            if constexpr (!LATE_BV) bv[k] = *reinterpret_cast<const u32x4*>(bv_base + (size_t)c * 16);
        }
    }
    // Keep the q and factor requests ahead of the latent tiles below.
    __builtin_amdgcn_sched_barrier(0);

    ell = min(max(ell, 0), a.L_cap);
    const int chunk = (ell + S - 1) / S;
    const int t0 = min(ell, s * chunk);
    const int t1 = min(ell, t0 + chunk);
    const int ntok = t1 - t0;

    float* o_out = a.o_part + (bh * S + s) * H;
    float lse_out = kNegInf;
    // One split with an output: the result goes straight to out and no
    // partial is written (measured on MI355X: the 512-block, 4096-token batch
    // ran 1.6 us faster without those stores).
    const bool direct = (S == 1) && a.out;

    // No branch on ntok: every block runs the same code, so nothing keeps the
    // factor and q requests above from being issued before L[b] lands.  An
    // empty range (ntok == 0) consumes no latent tile and ends with a zero
    // partial and lse = -inf.
    {
        // ---- first latent batches ---------------------------------------------
        const int g = lane / GP;
        const int j = lane % GP;
        const bool act = j < G;
        constexpr uint32_t row_bytes = (uint32_t)R * T::SZ;
        const char* kseq = static_cast<const char*>(a.C_K) + bh * a.L_cap * row_bytes;
        const char* vseq = static_cast<const char*>(a.C_V) + bh * a.L_cap * row_bytes;
        const char* skseq = I8 ? reinterpret_cast<const char*>(a.s_K + bh * a.L_cap) : nullptr;
        const char* svseq = I8 ? reinterpret_cast<const char*>(a.s_V + bh * a.L_cap) : nullptr;
        const uint32_t lane_off = (uint32_t)min(j, G - 1) * 16u;
        // Requested rows are clamped to the split's last row (for an empty
        // split: row t0, kept inside the cache), so every request is in bounds
        // and rows past the split re-read valid data.  Offsets stay 32-bit:
        // the host bounds L_cap * row bytes below 2^31.
        const int rlast = min(t0 + max(ntok, 1) - 1, a.L_cap - 1);

        // int8 scales are kept as raw fp16 bits, one per 32-bit register:
        // two halves packed into one register would need the loads to land
        // before the next requests go out.
        u32x4 kA[U], vA[U], kB[U], vB[U];
        uint32_t skA[U], svA[U], skB[U], svB[U];

        auto load_tile = [&](int tb, u32x4* kr, u32x4* vr, uint32_t* sk, uint32_t* sv) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t row = (uint32_t)min(t0 + tb + u * RW + g, rlast);
                const uint32_t off = row * row_bytes + lane_off;
                kr[u] = load16_stream(kseq + off);
                vr[u] = load16_stream(vseq + off);
                if constexpr (I8) {  // raw fp16 bits: converted when consumed, so no wait here
                    sk[u] = *reinterpret_cast<const uint16_t*>(skseq + row * 2u);
                    sv[u] = *reinterpret_cast<const uint16_t*>(svseq + row * 2u);
                }
            }
        };

        // This wave's tiles start at tb + k * STEP; the first two are requested
        // before the prologue waits for anything, unconditionally (a wave with
        // fewer rows re-reads the split's last row): with a branch around them
        // the waits for q and the factors below would have to assume the
        // tiles were not requested and so wait for them as well.
        constexpr int STEP = NW * TILE;
        int tb = wave * TILE;
        load_tile(tb, kA, vA, skA, svA);
        load_tile(tb + STEP, kB, vB, skB, svB);

        // ---- q' = (sigma log2 e) B_K q from the chunks in registers ------------
        const float qv = q_word_value(q_word, a.q_dt, q_idx);
        sh_q[tid] = qv;  // unconditional, so the q request is not sunk below the tiles
        if (DENSE && tid < H) sh_qp[tid] = qv * a.scale_log2;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NBT; ++k) {
            const int c = tid + 256 * k;
            if (!DENSE && (NBC % 256 == 0 || c < NBC)) {
                const int col = (c % CPR) * BEPC;
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < BEPC; ++e) p = fmaf(chunk_elem<BT>(bk[k], e), sh_q[col + e], p);
                sh_qpart[c] = p;
                if constexpr (!LATE_BV) sh_bv[c] = bv[k];
            }
        }
        __syncthreads();
        if (!DENSE && tid < R) {
            float p = 0.f;
#pragma unroll
            for (int c = 0; c < CPR; ++c) p += sh_qpart[tid * CPR + c];
            sh_qp[tid] = p * a.scale_log2;
        }
        __syncthreads();

        float qp[EPC];
#pragma unroll
        for (int c = 0; c < EPC; ++c) qp[c] = act ? sh_qp[min(j, G - 1) * EPC + c] : 0.f;
        float qoff = 0.f;  // int8: kI8Offset * sum of the lane's q' slice
        if constexpr (I8) {
#pragma unroll
            for (int c = 0; c < EPC; ++c) qoff += qp[c];
            qoff *= kI8Offset;
        }

        if constexpr (LATE_BV) {
#pragma unroll
            for (int k = 0; k < NBT; ++k) {
                const int c = tid + 256 * k;
                if (!DENSE && (NBC % 256 == 0 || c < NBC))
                    bv[k] = *reinterpret_cast<const u32x4*>(bv_base + (size_t)c * 16);
            }
        }

        // ---- hot loop ----------------------------------------------------------
        float m = kNegInf, l = 0.f, pw = 0.f;
        float acc[EPC];
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] = 0.f;

        auto consume = [&](int tbc, const u32x4* kr, const u32x4* vr, const uint32_t* sk, const uint32_t* sv) {
            float sc[U];
            float mloc = kNegInf;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float part = chunk_dot<CT>(kr[u], qp);
                if constexpr (I8) part -= qoff;
                float d = group_sum<GP>(part);
                if constexpr (I8) d *= f16_to_f32(uint16_t(sk[u]));
                sc[u] = (tbc + u * RW + g) < ntok ? d : kNegInf;
                mloc = fmaxf(mloc, sc[u]);
            }
            // The reference max moves only when some lane's new scores pass it
            // by 2^8 (log2 units): the weights exp2(s - m) then stay below 256
            // and the accumulators are not rescaled on every tile.
            if (__builtin_amdgcn_ballot_w64(mloc > m + 8.f) != 0) {
                const float mn = fmaxf(m, mloc);
                const float alpha = fast_exp2(m - ((mn == kNegInf) ? 0.f : mn));
                l *= alpha;
                if constexpr (I8) pw *= alpha;
#pragma unroll
                for (int c = 0; c < EPC; ++c) acc[c] *= alpha;
                m = mn;
            }
            const float mu = (m == kNegInf) ? 0.f : m;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = fast_exp2(sc[u] - mu);
                l += p;
                float w = p;
                if constexpr (I8) {
                    w *= f16_to_f32(uint16_t(sv[u]));
                    pw += w;
                }
                chunk_axpy<CT>(vr[u], w, acc);
            }
        };

        // Even tiles live in buffer A, odd tiles in B.  The steady-state loop
        // consumes a pair and requests the next pair unconditionally; the tail
        // requests only tiles that exist (only the first pair may hold rows
        // nobody consumes).
        const int nt = (ntok > tb) ? (ntok - tb + STEP - 1) / STEP : 0;
        int k = 0;
        // The scheduling barriers pin each refill between the two consumes:
        // sunk below the second consume, the refill left that consume
        // waiting for every load in flight (vmcnt(0)) instead of its own.
        for (; k + 3 < nt; k += 2) {
            consume(tb + k * STEP, kA, vA, skA, svA);
            load_tile(tb + (k + 2) * STEP, kA, vA, skA, svA);
            __builtin_amdgcn_sched_barrier(0);
            consume(tb + (k + 1) * STEP, kB, vB, skB, svB);
            load_tile(tb + (k + 3) * STEP, kB, vB, skB, svB);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int rem = nt - k;
        if (rem >= 1) consume(tb + k * STEP, kA, vA, skA, svA);
        if (rem >= 3) load_tile(tb + (k + 2) * STEP, kA, vA, skA, svA);
        if (rem >= 2) consume(tb + (k + 1) * STEP, kB, vB, skB, svB);
        if (rem >= 3) consume(tb + (k + 2) * STEP, kA, vA, skA, svA);

        // ---- merge slots inside the wave (VALU cross-lane operations) ----------
        const float Mw = wave_max(m);
        const float f = (m == kNegInf) ? 0.f : fast_exp2(m - Mw);
        l *= f;
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] *= f;
        if constexpr (I8) {
            pw *= f;
#pragma unroll
            for (int c = 0; c < EPC; ++c) acc[c] -= kI8Offset * pw;
        }
        l = sum_over_slots<GP>(l);
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] = sum_over_slots<GP>(acc[c]);
        if (g == 0 && act) {
#pragma unroll
            for (int c = 0; c < EPC; ++c) sh_red_o[wave][j * EPC + c] = acc[c];
        }
        if (lane == 0) {
            sh_red_m[wave] = Mw;
            sh_red_l[wave] = l;
        }
        if constexpr (LATE_BV) {
#pragma unroll
            for (int k = 0; k < NBT; ++k) {
                const int c = tid + 256 * k;
                if (!DENSE && (NBC % 256 == 0 || c < NBC)) sh_bv[c] = bv[k];
            }
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
            sh_on[tid] = Lt > 0.f ? o / Lt : 0.f;
        }
        __syncthreads();
        if constexpr (!DENSE) {
            const int jj = tid % H;
            const int part = tid / H;
            constexpr int RP = R / NPART;
            const void* bvr = static_cast<const void*>(sh_bv);
            float o = 0.f;
#pragma unroll
            for (int i = part * RP; i < (part + 1) * RP; ++i) o = fmaf(sh_on[i], raw_elem<BT>(bvr, i * H + jj), o);
            sh_proj[tid] = o;
        }
        __syncthreads();
        if (tid < H) {
            float o = 0.f;
            if constexpr (DENSE) {
                o = sh_on[tid];
            } else {
#pragma unroll
                for (int p = 0; p < NPART; ++p) o += sh_proj[p * H + tid];
            }
            if (direct) {
                store_elem_wt(a.out, a.out_dt, bh * H + tid, o);
            } else {
                store_coherent(o_out + tid, o);
            }
        }
        lse_out = Lt > 0.f ? (M + fast_log2(Lt)) * kLn2 : kNegInf;
    }
    if (direct) return;
    if (tid == 0) store_coherent(a.lse_part + bh * S + s, lse_out);

    // ---- last split of (b, h) merges all partials ------------------------------
    if (!a.out) return;
    merge_if_last_split<H>(a, bh, S, sh_proj, sh_last);
}

template <int H, int R, int CT, int BT>
static hipError_t launch_hrcb(const DecodeArgs& a, hipStream_t st) {
    // Row batches per buffer: int8 chunks carry 16 codes per lane, so two
    // batches (double-buffered) keep the kernel under 128 VGPRs -- four
    // blocks per CU.
    constexpr int U = (CT == WSVD_I8) ? 2 : 4;
    const unsigned nblk = (unsigned)((size_t)a.nb * a.nh * a.S);
    hipLaunchKernelGGL((decode_split_kernel<H, R, CT, BT, U>), dim3(nblk), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int H, int R, int CT>
static hipError_t launch_hrc(const DecodeArgs& a, hipStream_t st) {
    switch (a.B_dt) {
        case WSVD_F32: return launch_hrcb<H, R, CT, WSVD_F32>(a, st);
        case WSVD_BF16: return launch_hrcb<H, R, CT, WSVD_BF16>(a, st);
        case WSVD_F16: return launch_hrcb<H, R, CT, WSVD_F16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int H, int R>
static hipError_t launch_hr(const DecodeArgs& a, int C_dt, hipStream_t st) {
    switch (C_dt) {
        case WSVD_F32: return launch_hrc<H, R, WSVD_F32>(a, st);
        case WSVD_BF16:
            // The bf16 rank-32 instances live in decode_bf16_r32.hip.
            if constexpr (R == 32) return launch_decode_bf16_r32(a, H, st);
            else return launch_hrc<H, R, WSVD_BF16>(a, st);
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

#ifdef WSVD_DECODE_BF16_R32_UNIT
// The bf16-cache, rank-32 instances (every factor dtype, H 64 and 128),
// compiled in a translation unit of their own; see decode_bf16_r32.hip.
hipError_t launch_decode_bf16_r32(const DecodeArgs& a, int H, hipStream_t st) {
    switch (H) {
        case 64: return launch_hrc<64, 32, WSVD_BF16>(a, st);
        case 128: return launch_hrc<128, 32, WSVD_BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}
#else
hipError_t launch_dense_split(const DecodeArgs& a, int H, hipStream_t st) {
    const unsigned nblk = (unsigned)((size_t)a.nb * a.nh * a.S);
    switch (H) {
        case 64:
            hipLaunchKernelGGL((decode_split_kernel<64, 64, WSVD_BF16, WSVD_BF16, 4, true>), dim3(nblk), dim3(256), 0,
                               st, a);
            break;
        case 128:
            hipLaunchKernelGGL((decode_split_kernel<128, 128, WSVD_BF16, WSVD_BF16, 4, true>), dim3(nblk), dim3(256),
                               0, st, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int H, int r, int C_dt, hipStream_t st) {
    switch (H) {
        case 64: return launch_h<64>(a, r, C_dt, st);
        case 128: return launch_h<128>(a, r, C_dt, st);
        default: return hipErrorInvalidValue;
    }
}
#endif

}  // namespace wsvd
