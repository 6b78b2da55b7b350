// decode_rope.hip -- split decode with a rotary position step on every
// reconstructed key row.
//
// The pages' fused kernel loads latent tiles, rebuilds them on chip through
// the head's factor and uses them at once for qK^T, softmax and the V
// product ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
// Execution of Low-Precision Vision-Language Models": German page section
// 2D, Italian page section 2D, Japanese page section 2.4, Arabic page
// section 2c).  With rotary position embeddings the key of token t is
// R(t) (c_t B_Kh), so the fold q' = B_Kh q no longer applies: this kernel
// rebuilds each key tile on matrix cores and rotates it in registers.
//
// Per (b, h, split) workgroup of 4 waves; a wave takes 16-row tiles (tile
// k of wave w starts at row 16 w + 64 k of the split), two tiles in flight.
//  * K tile: v_mfma_f32_16x16x32_bf16 with the 16 latent rows as the A
//    operand (lane l: row l % 16, 8 consecutive ranks at 8 (l / 16)), read
//    straight from the cache, and B_Kh as the B operand: staged transposed
//    in LDS once, then each lane keeps its fragments of the whole factor in
//    registers for the split (r H / 512 u32x4 per lane), so tiles do not
//    re-read LDS.  The result (lane l: rows 4 (l / 16) .. +3, column l % 16
//    of each 16-column group) holds both members of every rotation pair
//    (column c and c + H/2) in one lane.
//  * Rotation: pair (c, c + H/2) of row t turns by t theta_c.  Since
//    <q, R(t) k> = <R(-t) q, k>, the lane turns its slice of q instead: to
//    its first row's position with cos / sin from the caller's tables, then
//    back by theta_c per following row (cos theta_c, sin theta_c are table
//    row 1) -- four operations per pair and row instead of rotating the key
//    and stepping the angle separately.
//  * Scores: the lane's key columns times the turned q (sigma log2 e folded
//    in), summed over the 16 lanes of a DPP row; each lane then takes the
//    score of its own A-operand row with one shuffle per row slot.
//  * Values stay in latent space: the lane accumulates p c_V of its row and
//    rank chunk (online softmax per lane), and the split's r-vector is
//    projected through B_Vh once, as in the folded kernel.
//  * Prologue: q, both factors and the cos / sin of one position step are
//    requested first, then the wave's first two tiles without a branch, so
//    staging B_Kh into LDS overlaps the tiles' flight.
//  * Partials, workspace layout and the merge are the folded kernel's (with
//    one split and an output, out is written directly).
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"
#include "split_merge.hpp"

namespace wsvd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

union R16 {
    u32x4 u;
    bf16x8 b;
};

template <int H, int R>
__global__ __launch_bounds__(256) void decode_rope_kernel(DecodeArgs a, const float* rcos, const float* rsin) {
    constexpr int NW = 4;
    constexpr int NJ = H / 16;     // 16-column groups of a key row
    constexpr int NP = H / 32;     // groups holding the first member of each pair
    constexpr int KS = R / 32;     // MFMA k-steps
    constexpr int TR = 16;         // rows per wave tile
    constexpr int STEP = NW * TR;  // rows per workgroup iteration
    constexpr int BP = R + 8;      // bf16 per LDS row of B_K^T (16-byte pad)
    constexpr int NBC = R * H / 8; // 16-byte chunks per factor
    constexpr int NPART = 256 / H;
    constexpr int RP = R / NPART;
    constexpr int HH = H / 2;

    __shared__ __attribute__((aligned(16))) uint16_t sBkT[H * BP];
    __shared__ u32x4 sh_bv[NBC];
    __shared__ float sh_q[256];  // q in [0, H); every thread stores its value
    __shared__ float sh_red_o[NW][R];
    __shared__ float sh_red_m[NW];
    __shared__ float sh_red_l[NW];
    __shared__ float sh_on[R];
    __shared__ float sh_proj[256];
    __shared__ int sh_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;   // k-group (A operand) / row quad (result)
    const int rr = lane & 15;  // row (A operand) / column (result)

    const int bid = blockIdx.x;
    const int h = bid % a.nh;
    const int rest = bid / a.nh;
    const int s = rest % a.S;
    const int b = rest / a.S;
    const int S = a.S;

    int ell = a.L[b];

    // q and both factors are requested first, ahead of the latent tiles, so
    // that staging them below waits only for these requests.
    static_assert(NBC % 256 == 0, "factor chunks per thread");
    constexpr int NBT = NBC / 256;
    const size_t bh = (size_t)b * a.nh + h;
    const size_t q_idx = bh * H + (tid < H ? tid : 0);
    const uint32_t q_word = load_q_word(a.q, a.q_dt, q_idx);
    const u32x4* bkc = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.B_K) + (size_t)h * R * H);
    const u32x4* bvc = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.B_V) + (size_t)h * R * H);
    u32x4 bkr[NBT], bvr[NBT];
#pragma unroll
    for (int k = 0; k < NBT; ++k) {
        bkr[k] = bkc[tid + 256 * k];
        bvr[k] = bvc[tid + 256 * k];
    }
    float c1[NP], s1[NP];  // cos / sin of theta_c, c = 16 p + rr (table row 1)
    const int row1 = (a.L_cap > 1) ? HH : 0;  // a one-row table: row 0 (angle 0)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        c1[p] = rcos[row1 + 16 * p + rr];
        s1[p] = rsin[row1 + 16 * p + rr];
    }
    __builtin_amdgcn_sched_barrier(0);

    ell = min(max(ell, 0), a.L_cap);
    const int chunk = (ell + S - 1) / S;
    const int t0 = min(ell, s * chunk);
    const int t1 = min(ell, t0 + chunk);
    const int ntok = t1 - t0;

    float* o_out = a.o_part + (bh * S + s) * H;
    float lse_out = kNegInf;
    const bool direct = (S == 1) && a.out;  // one split with an output: no partial

    if (ntok > 0) {  // uniform over the block
        // ---- first two tiles of the wave, then q and the factors staged ------------
        const uint16_t* kbase = static_cast<const uint16_t*>(a.C_K) + (bh * a.L_cap + t0) * R + 8 * g;
        const uint16_t* vbase = static_cast<const uint16_t*>(a.C_V) + (bh * a.L_cap + t0) * R + 8 * g;

        R16 kA[KS], vA[KS], kB[KS], vB[KS];
        float cA[NP], sA[NP], cB[NP], sB[NP];

        auto load_tile = [&](int tb, R16* kr, R16* vr, float* cr, float* sr) {
            const int row = min(tb + rr, ntok - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kr[ks].u = load16_stream(kbase + (size_t)row * R + 32 * ks);
                vr[ks].u = load16_stream(vbase + (size_t)row * R + 32 * ks);
            }
            const int ta = min(t0 + tb + 4 * g, a.L_cap - 1);  // position of the lane's first result row
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                cr[p] = rcos[(size_t)ta * HH + 16 * p + rr];
                sr[p] = rsin[(size_t)ta * HH + 16 * p + rr];
            }
        };

        // Both tiles are requested unconditionally (a wave with fewer rows
        // re-reads the split's last row): with a branch around them the waits
        // for the factors below would also wait for the tiles.
        const int tb0 = wave * TR;
        load_tile(tb0, kA, vA, cA, sA);
        load_tile(tb0 + STEP, kB, vB, cB, sB);

#pragma unroll
        for (int kk = 0; kk < NBT; ++kk) {
            const int c = tid + 256 * kk;
            const int k = c / (H / 8);
            const int n0 = (c % (H / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) sBkT[(n0 + e) * BP + k] = uint16_t(bkr[kk][e >> 1] >> ((e & 1) * 16));
            sh_bv[c] = bvr[kk];
        }
        sh_q[tid] = q_word_value(q_word, a.q_dt, q_idx);
        __syncthreads();

        float qv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) qv[j] = sh_q[16 * j + rr] * a.scale_log2;

        R16 breg[NJ * KS];  // this lane's B operand fragments of B_Kh
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                breg[ks * NJ + j].u = *reinterpret_cast<const u32x4*>(&sBkT[(16 * j + rr) * BP + 32 * ks + 8 * g]);
        float m = kNegInf, l = 0.f;
        float acc[8 * KS];
#pragma unroll
        for (int c = 0; c < 8 * KS; ++c) acc[c] = 0.f;

        auto consume = [&](int tb, const R16* kr, const R16* vr, const float* cr, const float* sr) {
            f32x4 kt[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) kt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    R16 bf;
                    bf = breg[ks * NJ + j];
                    kt[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks].b, bf.b, kt[j], 0, 0, 0);
                }
            }
            // rows 4 g + i sit at positions t0 + tb + 4 g + i: q turned back
            // to the first of them, then back by one step per row
            float q1[NP], q2[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                q1[p] = fmaf(qv[p], cr[p], qv[p + NP] * sr[p]);
                q2[p] = fmaf(qv[p + NP], cr[p], -(qv[p] * sr[p]));
            }
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d = 0.f;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    d = fmaf(kt[p][i], q1[p], d);
                    d = fmaf(kt[p + NP][i], q2[p], d);
                    if (i < 3) {
                        const float n1 = fmaf(q1[p], c1[p], q2[p] * s1[p]);
                        q2[p] = fmaf(q2[p], c1[p], -(q1[p] * s1[p]));
                        q1[p] = n1;
                    }
                }
                d = group_sum<16>(d);
                sc[i] = (tb + 4 * g + i < ntok) ? d : kNegInf;
            }
            // the score of this lane's own row (A-operand row rr lives in quad rr / 4)
            const int src = 16 * (rr >> 2);
            const float y0 = __shfl(sc[0], src, 64), y1 = __shfl(sc[1], src, 64);
            const float y2 = __shfl(sc[2], src, 64), y3 = __shfl(sc[3], src, 64);
            const int q4 = rr & 3;
            const float my = q4 == 0 ? y0 : (q4 == 1 ? y1 : (q4 == 2 ? y2 : y3));
            // The running max moves only when some lane's score grows past it by
            // more than 2^8 (or is first set): below that, exp2(score - m) stays
            // under 256 and the accumulators need no rescaling.
            if (__builtin_amdgcn_ballot_w64(my > m + 8.f)) {
                const float mn = (my > m + 8.f) ? my : m;
                const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int c = 0; c < 8 * KS; ++c) acc[c] *= alpha;
                m = mn;
            }
            const float pr = fast_exp2(my - ((m == kNegInf) ? 0.f : m));
            l += pr;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t w = vr[ks].u[c >> 1];
                    const float vc = (c & 1) ? bf16_hi(w) : bf16_lo(w);
                    acc[8 * ks + c] = fmaf(pr, vc, acc[8 * ks + c]);
                }
            }
        };

        const int nt = (ntok > tb0) ? (ntok - tb0 + STEP - 1) / STEP : 0;
        int k = 0;
        for (; k + 3 < nt; k += 2) {
            consume(tb0 + k * STEP, kA, vA, cA, sA);
            load_tile(tb0 + (k + 2) * STEP, kA, vA, cA, sA);
            __builtin_amdgcn_sched_barrier(0);
            consume(tb0 + (k + 1) * STEP, kB, vB, cB, sB);
            load_tile(tb0 + (k + 3) * STEP, kB, vB, cB, sB);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int rem = nt - k;
        if (rem >= 1) consume(tb0 + k * STEP, kA, vA, cA, sA);
        if (rem >= 3) load_tile(tb0 + (k + 2) * STEP, kA, vA, cA, sA);
        if (rem >= 2) consume(tb0 + (k + 1) * STEP, kB, vB, cB, sB);
        if (rem >= 3) consume(tb0 + (k + 2) * STEP, kA, vA, cA, sA);

        // ---- merge the wave's rows (lanes of one DPP row hold different rows) --
        const float Mw = wave_max(m);
        const float f = (m == kNegInf) ? 0.f : fast_exp2(m - Mw);
        l = group_sum<16>(l * f);
#pragma unroll
        for (int c = 0; c < 8 * KS; ++c) acc[c] = group_sum<16>(acc[c] * f);
        if (rr == 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int c = 0; c < 8; ++c) sh_red_o[wave][32 * ks + 8 * g + c] = acc[8 * ks + c];
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
        {
            const int jj = tid % H;
            const int part = tid / H;
            const uint16_t* bvr = reinterpret_cast<const uint16_t*>(sh_bv);
            float o = 0.f;
#pragma unroll
            for (int i = part * RP; i < (part + 1) * RP; ++i) o = fmaf(sh_on[i], bf16_to_f32(bvr[i * H + jj]), o);
            sh_proj[tid] = o;
        }
        __syncthreads();
        if (tid < H) {
            float o = 0.f;
#pragma unroll
            for (int p = 0; p < NPART; ++p) o += sh_proj[p * H + tid];
            if (direct) {
                store_elem_wt(a.out, a.out_dt, bh * H + tid, o);
            } else {
                store_coherent(o_out + tid, o);
            }
        }
        lse_out = (M + fast_log2(Lt)) * kLn2;
    } else {
        for (int i = tid; i < H; i += 256) {
            if (direct) {
                store_elem_wt(a.out, a.out_dt, bh * H + i, 0.f);
            } else {
                store_coherent(o_out + i, 0.f);
            }
        }
    }
    if (direct) return;
    if (tid == 0) store_coherent(a.lse_part + bh * S + s, lse_out);

    if (!a.out) return;
    merge_if_last_split<H>(a, bh, S, sh_proj, sh_last);
}

// cos / sin tables of the rotation: entry [t][i] for angle t * base^(-2 i / H)
// (i < H / 2), computed in double and rounded once to fp32.
__global__ void rope_tables_kernel(int L_cap, int H, double base, float* rcos, float* rsin) {
    const int HH = H / 2;
    const size_t n = (size_t)L_cap * HH;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx / HH);
        const int i = (int)(idx - (size_t)t * HH);
        const double ang = (double)t * pow(base, -2.0 * (double)i / (double)H);
        rcos[idx] = (float)cos(ang);
        rsin[idx] = (float)sin(ang);
    }
}

hipError_t launch_decode_rope(const DecodeArgs& a, int H, int r, const float* rcos, const float* rsin,
                              hipStream_t st) {
    const unsigned nblk = (unsigned)((size_t)a.nb * a.nh * a.S);
    if (H == 128 && r == 32)
        hipLaunchKernelGGL((decode_rope_kernel<128, 32>), dim3(nblk), dim3(256), 0, st, a, rcos, rsin);
    else if (H == 128 && r == 64)
        hipLaunchKernelGGL((decode_rope_kernel<128, 64>), dim3(nblk), dim3(256), 0, st, a, rcos, rsin);
    else if (H == 64 && r == 32)
        hipLaunchKernelGGL((decode_rope_kernel<64, 32>), dim3(nblk), dim3(256), 0, st, a, rcos, rsin);
    else if (H == 64 && r == 64)
        hipLaunchKernelGGL((decode_rope_kernel<64, 64>), dim3(nblk), dim3(256), 0, st, a, rcos, rsin);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_rope_tables(int L_cap, int H, double base, float* rcos, float* rsin, hipStream_t st) {
    const size_t n = (size_t)L_cap * (H / 2);
    const size_t want = (n + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(rope_tables_kernel, dim3(blocks), dim3(256), 0, st, L_cap, H, base, rcos, rsin);
    return hipGetLastError();
}

}  // namespace wsvd
