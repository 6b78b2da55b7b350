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
// k of wave w starts at row 16 w + 64 k of the split), D = 2 tiles in flight.
//  * Loads: each wave-wide 16-byte load reads whole latent rows, 1 KB
//    contiguous (8 rows at rank 64).  The matrix-core operand wants a lane
//    per row instead, so each tile is staged through the wave's own LDS
//    buffer: stored row-wise with the 16-byte chunks of row t xor-swizzled by
//    t % (chunks per row), which keeps the stores, the operand reads and the
//    transposing reads below free of bank conflicts.  Loading the operand
//    layout straight from the cache (half of each of 16 rows per load)
//    measured about 20% slower on MI355X, with or without the arithmetic.
//  * K tile: v_mfma_f32_16x16x32_bf16 with the 16 latent rows as the A
//    operand (lane l: row l % 16, 8 consecutive ranks at 8 (l / 16)), read
//    from the staged tile, and B_Kh as the B operand: staged transposed in
//    LDS once, then each lane keeps its fragments of the whole factor in
//    registers for the split (r H / 512 u32x4 per lane), so tiles do not
//    re-read it.  The result (lane l: rows 4 (l / 16) .. +3, column l % 16
//    of each 16-column group) holds both members of every rotation pair
//    (column c and c + H/2) in one lane.  B_Kh's columns are permuted as
//    they are staged, so a lane's NP = H / 32 pairs are consecutive pair
//    indices and their cos / sin are one 16-byte (H = 64: 8-byte) load of a
//    table row.
//  * Rotation: pair (c, c + H/2) of row t turns by t theta_c.  Since
//    <q, R(t) k> = <R(-t) q, k>, the lane turns its slice of q instead.  A
//    lane's first result row in every tile sits at the same offset
//    16 w + 4 (l / 16) from the tile's start, so q is turned back by that
//    offset once per split; each tile then turns it back by the tile's own
//    offset (one table row, the same for the whole wave), and by theta_c per
//    following row (cos theta_c, sin theta_c are table row 1) -- four
//    operations per pair and row instead of rotating the key and stepping
//    the angle separately.  Measured on MI355X, a table row per row quad
//    (2 KB of cos / sin per 4 KB tile) cost about 8% of the kernel's time.
//  * Scores: the lane's key columns times the turned q (sigma log2 e folded
//    in), summed over the 16 lanes of a DPP row: every lane of row quad
//    l / 16 then holds the scores of tile rows 4 (l / 16) .. +3.
//  * Values stay in latent space and go through the matrix cores:
//    o += V^T p with v_mfma_f32_16x16x16_bf16, where the A operand (rank
//    l % 16, rows 4 (l / 16) ..) comes from the staged value tile through
//    gfx950's transposing LDS read and the B operand is the lane's own four
//    weights -- exactly the rows whose scores it holds, so no shuffle is
//    needed.  The weights are rounded once to bf16 and the softmax sum counts
//    them as rounded.  One running max serves the whole wave (an MFMA sums
//    rows of all four row quads), moved only when a score passes it by 2^8.
//    The split's r-vector is projected through B_Vh once, as in the folded
//    kernel.
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
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define WSVD_LDS_AS __attribute__((address_space(3)))

// gfx950's transposing LDS read: in each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8,
// i/4+12 -- so when those 16 lanes address 4 rows x 16 columns of a row-major
// bf16 tile, lane i holds the 4 rows of column i.
__device__ __forceinline__ bf16x4 tr_read_b64(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((WSVD_LDS_AS bf16x4*)(WSVD_LDS_AS unsigned char*)p);
}

union R16 {
    u32x4 u;
    bf16x8 b;
};

// Key column carried by column group j (of 16) and result lane rr.  Columns
// are permuted so that the NP pairs a lane owns are consecutive pair indices
// NP rr .. NP rr + NP - 1: its cos / sin then come from one vector load of a
// table row.  Group p < NP holds the first member of pair NP rr + p, group
// p + NP the second (column + H / 2), so both members stay in one lane.
template <int H>
__device__ __forceinline__ constexpr int rope_key_col(int j, int rr) {
    constexpr int NP = H / 32;
    return (j / NP) * (H / 2) + NP * rr + (j % NP);
}

template <int NP>
__device__ __forceinline__ void load_pairs(const float* p, float* v) {
    if constexpr (NP == 4) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        static_assert(NP == 2, "H is 64 or 128");
        const float2 x = *reinterpret_cast<const float2*>(p);
        v[0] = x.x; v[1] = x.y;
    }
}

template <int H, int R>
__global__ __launch_bounds__(256) void decode_rope_kernel(DecodeArgs a, const float* rcos, const float* rsin) {
    // Tiles in flight per wave (measured on MI355X: 3 or 4 were no faster on
    // the 16 x 32-head, 4096-token rank-64 decode).
    constexpr int D = 2;
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
    constexpr int NG = R / 16;            // 16-rank groups of the value product
    constexpr int RB = 2 * R;             // bytes per latent row
    constexpr int CPR = R / 8;            // 16-byte chunks per latent row
    constexpr int RPI = 64 / CPR;         // rows per wave-wide 16-byte load (1 KB, contiguous)
    static_assert(RPI * KS == TR, "a tile is KS contiguous loads per cache");
    __shared__ __attribute__((aligned(16))) unsigned char sKV[NW * 2 * TR * RB];
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
    float c1[NP], s1[NP];  // cos / sin of theta_c for the lane's pairs c = NP rr + p (table row 1)
    const int row1 = (a.L_cap > 1) ? HH : 0;  // a one-row table: row 0 (angle 0)
    load_pairs<NP>(rcos + row1 + NP * rr, c1);
    load_pairs<NP>(rsin + row1 + NP * rr, s1);
    // cos / sin of the lane's first result row inside a tile, 16 wave + 4 g
    // (a row past the table belongs to no token, so any angle serves there)
    float cw[NP], sw[NP];
    {
        const int rw = min(TR * wave + 4 * g, a.L_cap - 1) * HH;
        load_pairs<NP>(rcos + rw + NP * rr, cw);
        load_pairs<NP>(rsin + rw + NP * rr, sw);
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
        const uint16_t* kbase = static_cast<const uint16_t*>(a.C_K) + (bh * a.L_cap + t0) * R + 8 * (lane % CPR);
        const uint16_t* vbase = static_cast<const uint16_t*>(a.C_V) + (bh * a.L_cap + t0) * R + 8 * (lane % CPR);

        R16 kb[D][KS], vb[D][KS];
        float cb[D][NP], sb[D][NP];

        const int tb0 = wave * TR;
        auto load_tile = [&](int tb, R16* kr, R16* vr, float* cr, float* sr) {
            // Load ks covers tile rows RPI ks .. RPI ks + RPI - 1 whole (lane: row
            // lane / CPR, chunk lane % CPR): every wave load is 1 KB contiguous.
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int row = min(tb + RPI * ks + lane / CPR, ntok - 1);
                kr[ks].u = load16_stream(kbase + (size_t)row * R);
                vr[ks].u = load16_stream(vbase + (size_t)row * R);
            }
            const int ta = min(t0 + tb - tb0, a.L_cap - 1);  // the tile's offset in the split; see qv
            load_pairs<NP>(rcos + (size_t)ta * HH + NP * rr, cr);
            load_pairs<NP>(rsin + (size_t)ta * HH + NP * rr, sr);
        };

        // Both tiles are requested unconditionally (a wave with fewer rows
        // re-reads the split's last row): with a branch around them the waits
        // for the factors below would also wait for the tiles.
#pragma unroll
        for (int d = 0; d < D; ++d) load_tile(tb0 + d * STEP, kb[d], vb[d], cb[d], sb[d]);

#pragma unroll
        for (int kk = 0; kk < NBT; ++kk) {
            const int c = tid + 256 * kk;
            const int k = c / (H / 8);
            const int n0 = (c % (H / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // key column n0 + e sits in column group j, lane rr' (see rope_key_col)
                const int col = n0 + e;
                const int hi = col / HH, ch = col % HH;
                const int nn = 16 * ((ch % NP) + NP * hi) + ch / NP;
                sBkT[nn * BP + k] = uint16_t(bkr[kk][e >> 1] >> ((e & 1) * 16));
            }
            sh_bv[c] = bvr[kk];
        }
        sh_q[tid] = q_word_value(q_word, a.q_dt, q_idx);
        __syncthreads();

        float qv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) qv[j] = sh_q[rope_key_col<H>(j, rr)] * a.scale_log2;
        // q turned back once by the lane's fixed row offset in a tile: each tile
        // then needs the angle of its offset in the split only -- one table row
        // for the whole wave instead of one per row quad.
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float x = qv[p], y = qv[p + NP];
            qv[p] = fmaf(x, cw[p], y * sw[p]);
            qv[p + NP] = fmaf(y, cw[p], -(x * sw[p]));
        }

        R16 breg[NJ * KS];  // this lane's B operand fragments of B_Kh
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                breg[ks * NJ + j].u = *reinterpret_cast<const u32x4*>(&sBkT[(16 * j + rr) * BP + 32 * ks + 8 * g]);
        // m is shared by the whole wave: one value-product MFMA sums rows of all
        // four row quads, so their weights need one reference.
        float m = kNegInf, l = 0.f;
        f32x4 oacc[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // The wave's tile in LDS, swizzled: 16-byte chunk c of row t sits at
        // t RB + 16 (c ^ (t % CPR)), so the row-wise stores, the operand reads
        // (16 rows, one chunk) and the transposing reads are free of bank conflicts.
        unsigned char* sKw = sKV + wave * 2 * TR * RB;
        unsigned char* sVw = sKw + TR * RB;
        auto swz = [](int t, int c) { return t * RB + 16 * (c ^ (t % CPR)); };
        int woff[KS], koff[KS], voff[NG];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            woff[ks] = swz(RPI * ks + lane / CPR, lane % CPR);
            koff[ks] = swz(rr, g + 4 * ks);  // A operand: row rr, ranks 8 g + 32 ks ..
        }
#pragma unroll
        for (int j = 0; j < NG; ++j)  // transposing read: rows 4 g + rr / 4, 8-byte chunk rr % 4 of rank group j
            voff[j] = swz(4 * g + (rr >> 2), 2 * j + ((rr & 3) >> 1)) + 8 * (rr & 1);

        auto consume = [&](int tb, const R16* kr, const R16* vr, const float* cr, const float* sr) {
            // Stage the tile in LDS and read the key tile back in the matrix-core
            // operand layout (lane: row rr, 8 ranks at 8 g + 32 ks).
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                *reinterpret_cast<u32x4*>(sKw + woff[ks]) = kr[ks].u;
                *reinterpret_cast<u32x4*>(sVw + woff[ks]) = vr[ks].u;
            }
            R16 ka[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[ks].u = *reinterpret_cast<const u32x4*>(sKw + koff[ks]);
            f32x4 kt[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) kt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    R16 bf;
                    bf = breg[ks * NJ + j];
                    kt[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks].b, bf.b, kt[j], 0, 0, 0);
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
            // The running max moves only when some score grows past it by more
            // than 2^8 (or is first set): below that, exp2(score - m) stays under
            // 256 and the accumulators need no rescaling.
            const float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            if (__builtin_amdgcn_ballot_w64(mloc > m + 8.f)) {
                const float mn = fmaxf(m, wave_max(mloc));
                const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int j = 0; j < NG; ++j) oacc[j] *= alpha;
                m = mn;
            }
            const float mu = (m == kNegInf) ? 0.f : m;
            // Weights of this lane's rows 4 g .. 4 g + 3, rounded once to bf16 and
            // counted in l as rounded, so the numerator and the denominator use the
            // same weights: the B operand of the value product (every column alike).
            f32x4 pw;
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[i] = fast_exp2(sc[i] - mu);
            const bf16x4 pb = __builtin_convertvector(pw, bf16x4);
#pragma unroll
            for (int i = 0; i < 4; ++i) l += (float)pb[i];
            // o += V^T p on matrix cores: the A operand (rank l % 16, rows 4 g ..)
            // comes from the transposing LDS read of the tile just stored.
#pragma unroll
            for (int j = 0; j < NG; ++j)
                oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, tr_read_b64(sVw + voff[j])),
                                                                     __builtin_bit_cast(s16x4, pb), oacc[j], 0, 0, 0);
        };

        const int nt = (ntok > tb0) ? (ntok - tb0 + STEP - 1) / STEP : 0;
        int k = 0;
        for (; k + 2 * D - 1 < nt; k += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                consume(tb0 + (k + d) * STEP, kb[d], vb[d], cb[d], sb[d]);
                load_tile(tb0 + (k + d + D) * STEP, kb[d], vb[d], cb[d], sb[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (k + d < nt) consume(tb0 + (k + d) * STEP, kb[d], vb[d], cb[d], sb[d]);
            if (k + d + D < nt) load_tile(tb0 + (k + d + D) * STEP, kb[d], vb[d], cb[d], sb[d]);
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (k + D + d < nt) consume(tb0 + (k + D + d) * STEP, kb[d], vb[d], cb[d], sb[d]);

        // ---- merge the wave's row quads (one running max for the wave) ---------
        // l: every lane of a DPP row holds its quad's sum; oacc: lane 16 g holds
        // ranks 16 j + 4 g .. + 3 (the MFMA already summed over all 16 rows).
        l = sum_over_slots<16>(l);
        if (rr == 0) {
#pragma unroll
            for (int j = 0; j < NG; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) sh_red_o[wave][16 * j + 4 * g + i] = oacc[j][i];
        }
        if (lane == 0) {
            sh_red_m[wave] = m;
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
