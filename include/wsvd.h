/*
 * wsvd.h -- C ABI of libwsvd.so: WSVD per-head low-rank flash decoding on
 * AMD MI355X (gfx950).
 *
 * Citations refer to the page "WSVD: Weighted Low-Rank Approximation for
 * Fast and Efficient Execution of Low-Precision Vision-Language Models"
 * (gist.science, paper 2604.02570) by language and section.
 *
 * Notation (Arabic page section 2a; German page section 2A): head h of an
 * attention layer factors its key projection as W_Kh ~ A_Kh B_Kh with
 * A_Kh in R^{E x r} and B_Kh in R^{r x H}; E is the embedding width, H the
 * head dimension and r the per-head rank.  The cache keeps, per head and
 * per token, only the r-dim latent C_Kh = x A_Kh (L x r per head).  Values
 * are factored the same way (A_Vh, B_Vh, C_Vh).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer is a caller-owned DEVICE buffer unless stated otherwise.
 *   The library allocates nothing and keeps no state: calls are reentrant
 *   and may be issued from several host threads on different streams.
 * - Tensors are dense and row-major with the shapes given below.  Every
 *   tensor base pointer must be 16-byte aligned (torch allocations are).
 * - Calls only enqueue work on `stream` and return; nothing synchronises.
 *   Outputs are valid once the stream reaches that point.
 * - Every argument problem that the host can see is reported by a negative
 *   wsvd_status before anything is launched: NULL pointers, non-positive
 *   sizes, r > H, an (H, r, dtype) combination that is not compiled,
 *   misaligned pointers, a workspace that is too small.  A failed launch
 *   returns WSVD_ERR_HIP.  There is no fallback path.
 * - Values held in device memory (L[b], pos[b]) cannot be checked by the
 *   host; their documented handling is below.
 * - Compiled shapes: H in {64, 128}; r in {16, 32, 48, 64} with r <= H.
 */
#ifndef WSVD_H_
#define WSVD_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wsvd_dtype {
    WSVD_F32 = 0,   /* IEEE binary32                                  */
    WSVD_BF16 = 1,  /* bfloat16 (upper half of a binary32)            */
    WSVD_F16 = 2,   /* IEEE binary16 (only for q, B, x, A and out)    */
    WSVD_I8 = 3     /* signed 8-bit codes (latent caches only)        */
} wsvd_dtype;

typedef enum wsvd_status {
    WSVD_OK = 0,
    WSVD_ERR_NULL = -1,         /* a required pointer is NULL                      */
    WSVD_ERR_SHAPE = -2,        /* non-positive size, r > H, inconsistent sizes    */
    WSVD_ERR_DTYPE = -3,        /* dtype not allowed for that argument             */
    WSVD_ERR_UNSUPPORTED = -4,  /* (H, r, dtype) combination not compiled          */
    WSVD_ERR_ALIGN = -5,        /* a base pointer is not 16-byte aligned           */
    WSVD_ERR_WORKSPACE = -6,    /* workspace NULL or smaller than required         */
    WSVD_ERR_HIP = -7           /* the HIP runtime reported a launch error         */
} wsvd_status;

/*
 * wsvd_decode_attn -- one decode step of attention over a per-head latent
 * cache, without materialising K or V.
 *
 * Defines (German page section 2D; Italian page section 2D; Arabic page
 * section 2c; Japanese page section 2.4): latent tiles are streamed from
 * memory, combined on chip with the head's factor, and used at once for
 * qK^T, softmax and the V product inside a Flash-Decoding pass.  The result
 * equals, for every sequence b and head h with l = L[b]:
 *
 *     K = C_K[b,h,:l,:] B_K[h],  V = C_V[b,h,:l,:] B_V[h]     (l x H)
 *     out[b,h,:] = softmax(sigma * K q[b,h,:]) V
 *
 * computed here as q' = B_K[h] q (folded once), scores = C_K q', and an
 * r-dim V accumulation projected through B_V[h] once per split.
 *
 * Arguments
 *   nb, nh, H, r     batch, heads, head dim, per-head rank (> 0, r <= H)
 *   L_cap            cache capacity in tokens (> 0); one sequence's rows of
 *                    one head, L_cap * r elements, must stay below 2 GiB
 *                    (WSVD_ERR_SHAPE otherwise)
 *   L                int32 [nb]: tokens attended per sequence.  Device
 *                    values are clamped to [0, L_cap]; L[b] == 0 yields a
 *                    zero output row.
 *   q, q_dt          [nb, nh, H]   F32 | BF16 | F16
 *   C_K, C_V, C_dt   [nb, nh, L_cap, r]   F32 | BF16 | I8.  Rows at or past
 *                    L[b] may hold any bits: they never enter the result.
 *   s_K, s_V         fp16 [nb, nh, L_cap] per-token scales, required iff
 *                    C_dt == WSVD_I8 (value = code * scale); else ignored
 *   B_K, B_V, B_dt   [nh, r, H]    F32 | BF16 | F16
 *   softmax_scale    sigma; <= 0 selects 1/sqrt(H)
 *   n_splits         splits of each sequence (0 = automatic, see
 *                    wsvd_decode_num_splits).  Split s of a sequence with
 *                    l tokens covers [s*ceil(l/S), min(l, (s+1)*ceil(l/S))).
 *   workspace        device scratch of at least wsvd_decode_workspace_bytes
 *                    bytes, 256-byte aligned.  Layout, each region 256-byte
 *                    aligned:
 *                      counters uint32 [nb, nh] at byte offset 0, in the
 *                               first wsvd_decode_counter_bytes(nb, nh)
 *                               bytes (same place for every split count);
 *                      o_part   float [nb, nh, S, H] at byte offset
 *                               wsvd_decode_opart_offset(...): each split's
 *                               attention normalised over its own tokens
 *                               (zeros for an empty split);
 *                      lse_part float [nb, nh, S] at byte offset
 *                               wsvd_decode_lse_offset(...): natural-log
 *                               log-sum-exp of the split's scaled scores
 *                               (-inf for an empty split).
 *                    Zero-counter rule: when a call that passes an output
 *                    starts, the counter bytes [0, wsvd_decode_counter_bytes
 *                    (nb, nh)) must be zero, and the call leaves them zero;
 *                    bytes past them need no initial contents and may be
 *                    overwritten.  So a workspace zero-filled once serves
 *                    any run of calls in stream order whose nb * nh never
 *                    grows (a call with a larger nb * nh than an earlier one
 *                    needs its counter bytes zero-filled again first).  The
 *                    library cannot check this: with non-zero counters the
 *                    last-split test misfires, so rows of out may be left
 *                    unwritten or merged from partials that are not yet
 *                    complete, and no error is returned.  Calls in flight at
 *                    the same time need separate workspaces.  On return
 *                    (stream order) the workspace holds the split partials,
 *                    except with an output and S == 1: then each row goes
 *                    straight to out and the partial area is left as it
 *                    was.
 *   out, out_dt      [nb, nh, H] F32 | BF16 | F16, or NULL to stop after the
 *                    partials (e.g. to merge partials from several devices
 *                    with wsvd_combine_splits).  With an output and up to
 *                    2047 split blocks (nb*nh*S) the whole step is one
 *                    kernel launch: the last split of each (b, h) to finish
 *                    merges that row's partials.  Larger grids write the
 *                    partials and merge them in a second launch (the
 *                    wsvd_combine_splits kernel).  Either way partials are
 *                    merged in split order, so the result is the same and
 *                    does not depend on scheduling.
 *   stream           HIP stream to enqueue on (0 = null stream).
 */
int wsvd_decode_attn(int nb, int nh, int H, int r, int L_cap,
                     const int32_t* L,
                     const void* q, wsvd_dtype q_dt,
                     const void* C_K, const void* C_V, wsvd_dtype C_dt,
                     const uint16_t* s_K, const uint16_t* s_V,
                     const void* B_K, const void* B_V, wsvd_dtype B_dt,
                     float softmax_scale, int n_splits,
                     void* workspace, size_t workspace_bytes,
                     void* out, wsvd_dtype out_dt,
                     hipStream_t stream);

/*
 * wsvd_decode_attn_noalloc -- wsvd_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and the call
 * allocates nothing.  Arguments, results and kernels are those of
 * wsvd_decode_attn with an output (out must not be NULL: the partials stay
 * in the library's scratch).
 *
 * Scratch: one static device array per GPU, held from the library's load
 * until the process ends: merge counters for up to 65536 (b, h) pairs in a
 * region of their own (256 KiB, zero at start, and every call leaves them
 * zero), then 16 MiB for the split partials, laid out as in the decode
 * workspace.  Calls whose nb * nh exceeds 65536, or whose partials
 * (wsvd_decode_workspace_bytes(...) - wsvd_decode_counter_bytes(nb, nh))
 * exceed 16 MiB, return WSVD_ERR_WORKSPACE with nothing launched.  The
 * first call on a device looks the array up and zero-fills the counter
 * region on `stream`.  The scratch of the current device is used; `stream`
 * must belong to it.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams, or several host
 * threads without ordering) race on it and give wrong results.  Calls
 * ordered on one stream are safe.
 */
int wsvd_decode_attn_noalloc(int nb, int nh, int H, int r, int L_cap,
                             const int32_t* L,
                             const void* q, wsvd_dtype q_dt,
                             const void* C_K, const void* C_V, wsvd_dtype C_dt,
                             const uint16_t* s_K, const uint16_t* s_V,
                             const void* B_K, const void* B_V, wsvd_dtype B_dt,
                             float softmax_scale, int n_splits,
                             void* out, wsvd_dtype out_dt,
                             hipStream_t stream);

/*
 * wsvd_combine_splits -- merge per-split partials into the attention output.
 *
 * The Flash-Decoding pass named on the German page section 2D (and the
 * Japanese page section 2.4) splits the cached tokens; this is its merge:
 * out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max_s lse_s).
 * Splits with lse = -inf carry no weight; if every split of a row is empty
 * the row is zero.  Rounding to out_dt is to nearest, ties to even.
 *
 *   o_part   float [nb, nh, S, H]  (S = n_splits > 0)
 *   lse_part float [nb, nh, S]
 *   out      [nb, nh, H] in out_dt (F32 | BF16 | F16)
 */
int wsvd_combine_splits(int nb, int nh, int H, int n_splits,
                        const float* o_part, const float* lse_part,
                        void* out, wsvd_dtype out_dt,
                        hipStream_t stream);

/*
 * wsvd_append_latent -- project the new token of each sequence to its
 * per-head latents and write them into the caches.
 *
 * Per head, the cached latent is the token activation times the head's
 * factor A_Kh in R^{E x r} (Arabic page section 2a; German page section 2A;
 * Japanese page section 2.1).  For every b and h:
 *
 *     C_K[b, h, pos[b], :] = x[b, :] A_K[:, h*r:(h+1)*r]
 *     C_V[b, h, pos[b], :] = x[b, :] A_V[:, h*r:(h+1)*r]
 *
 * accumulated in fp32 on matrix cores and rounded once to C_dt (nearest,
 * ties to even).
 *
 * Int8 caches (the 8-bit latent storage of the pages' W8A8 setting, German
 * page section 2C, Arabic page section 2c) store each new (b, h) row as
 * symmetric absmax codes: scale = fp16(max_i |c_i| / 127) goes to
 * s_K / s_V[b, h, pos[b]], code_i = clamp(round_half_even(c_i / scale),
 * -127, 127); a row whose scale is 0 stores zeros.  The decode reads such
 * rows as code * scale.  Int8 caches need r in {16, 32, 64} (a head must be
 * whole 16-column groups of one 64-column tile; r = 48 returns
 * WSVD_ERR_UNSUPPORTED).
 *
 *   nb, E, nh, r     batch, embedding width, heads, rank (r as above)
 *   L_cap            cache capacity in tokens
 *   x, x_dt          [nb, E]         BF16
 *   A_K, A_V, A_dt   [E, nh*r]       BF16 (column block h is A_Kh)
 *   pos              int32 [nb] device: row to write; rows with pos[b]
 *                    outside [0, L_cap) are skipped
 *   C_K, C_V, C_dt   [nb, nh, L_cap, r]   BF16 | F32 | I8
 *   s_K, s_V         fp16 [nb, nh, L_cap] row scales, required (16-byte
 *                    aligned) iff C_dt == WSVD_I8; must be NULL otherwise
 *   workspace        device scratch of wsvd_append_workspace_bytes(...)
 *                    bytes, 256-byte aligned: one arrival counter per output
 *                    tile in the first wsvd_append_counter_bytes(nb, nh, r)
 *                    bytes, then fp32 split-E partial tiles.  The counter
 *                    bytes must be zero when a call starts and every call
 *                    leaves them zero (the same rule, and the same silent
 *                    failure when it is broken, as the decode workspace's
 *                    counters), so calls issued one after another on a
 *                    stream may share a workspace zero-filled once as long
 *                    as the counter area does not grow; concurrent calls on
 *                    different streams need separate workspaces.  When the
 *                    size function returns 0 no split is used and
 *                    workspace may be NULL.
 */
int wsvd_append_latent(int nb, int E, int nh, int r, int L_cap,
                       const void* x, wsvd_dtype x_dt,
                       const void* A_K, const void* A_V, wsvd_dtype A_dt,
                       const int32_t* pos,
                       void* C_K, void* C_V, wsvd_dtype C_dt,
                       uint16_t* s_K, uint16_t* s_V,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * wsvd_decode_attn_rope -- wsvd_decode_attn with a rotary position step on
 * every reconstructed key row.
 *
 * The pages' fused kernel rebuilds latent tiles through the head's factor
 * on chip and uses them at once (German page section 2D, Italian page
 * section 2D, Japanese page section 2.4, Arabic page section 2c); they name
 * no position encoding.  With rotary embeddings the key of cached token t
 * is R(t) (C_K[b,h,t,:] B_K[h]), which cannot be folded into q, so each key
 * tile is rebuilt on matrix cores and rotated before the scores:
 *
 *     K_t = R(t) (C_K[b,h,t,:] B_K[h]),  V_t = C_V[b,h,t,:] B_V[h]
 *     out[b,h,:] = softmax(sigma * K q[b,h,:]) V,   t = 0 .. L[b]-1
 *
 * R(t) rotates each pair (i, i + H/2) of a key by angle t * theta_i (the
 * half-split convention); q must arrive already rotated to its own
 * position.  cos / sin come from the tables below (row t, column i).
 *
 *   rope_cos, rope_sin  fp32 [L_cap, H/2], e.g. from wsvd_rope_tables
 *   C_dt, B_dt          BF16 only; H in {64, 128}; r in {32, 64}
 *   other arguments, the split rule, partials, workspace and merge exactly
 *   as for wsvd_decode_attn (int8 caches are not supported here).
 */
int wsvd_decode_attn_rope(int nb, int nh, int H, int r, int L_cap,
                          const int32_t* L,
                          const void* q, wsvd_dtype q_dt,
                          const void* C_K, const void* C_V, wsvd_dtype C_dt,
                          const void* B_K, const void* B_V, wsvd_dtype B_dt,
                          const float* rope_cos, const float* rope_sin,
                          float softmax_scale, int n_splits,
                          void* workspace, size_t workspace_bytes,
                          void* out, wsvd_dtype out_dt,
                          hipStream_t stream);

/*
 * wsvd_rope_tables -- rope_cos[t, i] = cos(t * base^(-2 i / H)), rope_sin
 * likewise, for t < L_cap and i < H/2 (fp32 [L_cap, H/2], computed in double
 * and rounded once).  H even, base > 1 (e.g. 10000).
 */
int wsvd_rope_tables(int L_cap, int H, float base, float* rope_cos, float* rope_sin,
                     hipStream_t stream);

/*
 * W8A8 projection of the new token (German page section 2C, Italian page
 * section 2C, Japanese page section 2.3, Arabic page section 2c: the
 * low-rank layers run with 8-bit weights and activations, and an
 * orthogonal Hadamard rotation S1 smooths activation outliers before
 * quantisation).  Readings: S1 = H_E / sqrt(E), the Sylvester Walsh-Hadamard
 * matrix of order E (a power of two), which is symmetric and orthogonal, so
 * x A = (x S1)(S1 A) and the factor side is rotated once, offline; codes are
 * symmetric absmax int8 with one fp32 scale per row (token) or per column
 * (factor output): s = max|v| / 127, code = clamp(round_half_even(v / s),
 * -127, 127), zero codes when s == 0.  Supported E: powers of two from 256
 * to 8192.
 *
 * wsvd_w8a8_prepare_factor -- offline: rotate a factor A [E, N] (F32 | BF16
 * | F16, column block h of width r is A_Kh) down its columns and quantise
 * each column: AqT int8 [N, E] (row n holds column n's codes, k-contiguous)
 * and sA fp32 [N].
 */
int wsvd_w8a8_prepare_factor(int E, int N, const void* A, wsvd_dtype A_dt,
                             int8_t* AqT, float* sA, hipStream_t stream);

/*
 * wsvd_w8a8_quantize_activations -- per step: rotate each token x[b, :]
 * (F32 | BF16 | F16, [nb, E]) by S1 and quantise it: xq int8 [nb, E],
 * sx fp32 [nb].
 */
int wsvd_w8a8_quantize_activations(int nb, int E, const void* x, wsvd_dtype x_dt,
                                   int8_t* xq, float* sx, hipStream_t stream);

/*
 * wsvd_append_latent_w8a8 -- wsvd_append_latent with integer operands:
 *
 *     c[b, h*r + i] = (sum_e xq[b, e] AqT_K[h*r + i, e]) * sx[b] * sA_K[h*r + i]
 *
 * (the sum is exact: int32 on matrix cores), then c is stored in row pos[b]
 * of C_K exactly as wsvd_append_latent stores it (BF16 | F32 rounded once;
 * I8 as absmax codes with fp16 s_K); the same for V.  E must be a multiple
 * of 512.  Workspace: wsvd_append_workspace_bytes(nb, E, nh, r), with the
 * same zero-counter rule.  Other arguments as for wsvd_append_latent.
 */
int wsvd_append_latent_w8a8(int nb, int E, int nh, int r, int L_cap,
                            const int8_t* xq, const float* sx,
                            const int8_t* AqT_K, const int8_t* AqT_V,
                            const float* sA_K, const float* sA_V,
                            const int32_t* pos,
                            void* C_K, void* C_V, wsvd_dtype C_dt,
                            uint16_t* s_K, uint16_t* s_V,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * wsvd_dense_decode_attn -- the speed baseline the pages compare WSVD with:
 * ordinary Flash-Decoding attention over full K and V (Japanese page
 * section 4, German page section 4: decode latency against Flash Decoding).
 * Same split rule, partial format, merge (in-kernel or second launch) and workspace as
 * wsvd_decode_attn; it exists so both can be timed on the same device.
 *
 *     out[b,h,:] = softmax(sigma * K[b,h,:l,:] q[b,h,:]) V[b,h,:l,:],  l = L[b]
 *
 *   K, V, kv_dt   [nb, nh, L_cap, H] BF16 (H in {64, 128}); L_cap * H below 2^30
 *   workspace     wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits)
 *                 bytes, same layout and zero-counter rule as above
 *   other arguments as for wsvd_decode_attn.
 */
int wsvd_dense_decode_attn(int nb, int nh, int H, int L_cap,
                           const int32_t* L,
                           const void* q, wsvd_dtype q_dt,
                           const void* K, const void* V, wsvd_dtype kv_dt,
                           float softmax_scale, int n_splits,
                           void* workspace, size_t workspace_bytes,
                           void* out, wsvd_dtype out_dt,
                           hipStream_t stream);

/* Splits wsvd_decode_attn uses for these sizes (n_splits > 0 is returned
 * unchanged; 0 selects the automatic choice).  Pure host function.
 * Returns a negative wsvd_status for invalid sizes. */
int wsvd_decode_num_splits(int nb, int nh, int L_cap, int n_splits);

/* Workspace bytes wsvd_decode_attn needs (0 on invalid sizes).  Pure host. */
size_t wsvd_decode_workspace_bytes(int nb, int nh, int H, int L_cap, int n_splits);

/* Bytes of the decode workspace's merge-counter area (offset 0): nb*nh
 * uint32 rounded up to 256 (0 on invalid sizes).  Pure host. */
size_t wsvd_decode_counter_bytes(int nb, int nh);

/* Byte offsets of o_part and lse_part inside the decode workspace (0 on
 * invalid sizes).  Pure host. */
size_t wsvd_decode_opart_offset(int nb, int nh, int H, int L_cap, int n_splits);
size_t wsvd_decode_lse_offset(int nb, int nh, int H, int L_cap, int n_splits);

/* Workspace bytes wsvd_append_latent needs: 0 on invalid sizes, and 0 when
 * the sizes need no E split (then the workspace argument may be NULL).
 * Pure host. */
size_t wsvd_append_workspace_bytes(int nb, int E, int nh, int r);

/* Bytes of the append workspace's arrival-counter area (offset 0, one
 * uint32 per output tile, rounded up to 256).  Pure host. */
size_t wsvd_append_counter_bytes(int nb, int nh, int r);

/*
 * Offline per-head factorisation (Arabic page section 2a, German page
 * section 2A, Japanese page section 2.1: every head's E x H slice W_h of a
 * projection is factored on its own at rank r, W_h ~ A_h B_h).  Readings:
 * W fp32 [E, nh*H] holds the heads side by side (columns [h H, (h + 1) H)
 * are W_h); the unweighted factors are the rank-r truncated SVD W_h =
 * U S V^T, split as A_h = U_r S_r and B_h = V_r^T, so the latent keeps the
 * singular values and the rows of B_h are orthonormal.  Offline work: run
 * once per layer, nothing here is on the decode path.
 *
 * wsvd_factorize_svd -- A fp32 [E, nh*r] (column block h is A_h), B fp32
 * [nh, r, H] (B_h = B[h]), sigma fp32 [nh, H] (all H singular values of
 * each head, descending), sweeps int32 [nh] or NULL (Jacobi sweeps used per
 * head, negative when the iteration stopped at its cap without converging).
 * Computed in fp64 through G_h = W_h^T W_h (its eigenvectors are the right
 * singular vectors); rows of B_h are orthonormal with their largest-
 * magnitude entry positive; where W_h has rank below r the missing rows
 * complete an orthonormal set (their A columns are then zero to rounding).
 * A_h = W_h B_h^T with the returned fp32 B.  H in {64, 128}; 1 <= r <= H.
 * Workspace: wsvd_factorize_svd_workspace_bytes(E, nh, H) bytes, 16-byte
 * aligned, no initial contents required.  Non-finite W gives non-finite
 * outputs.
 */
size_t wsvd_factorize_svd_workspace_bytes(int E, int nh, int H);
int wsvd_factorize_svd(int E, int nh, int H, int r, const float* W,
                       float* A, float* B, float* sigma, int32_t* sweeps,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * Weighted refinement (Arabic page section 2b, German page section 2B,
 * Japanese page section 2.2: factors are fitted to minimise
 * sum F (.) (W - A B)^2 with importance weights F).  Reading: alternating
 * least squares with F given (fp32 [E, nh*H], laid out like W, entries > 0
 * and finite); each call is one exact half-step, solved in fp64:
 *
 * wsvd_weighted_update_A -- every row a of A_h (output fp32 [E, nh*r])
 *   minimises sum_j F[e, hH + j] (W[e, hH + j] - a . B_h[:, j])^2 for the
 *   given B fp32 [nh, r, H];
 * wsvd_weighted_update_B -- every column b of B_h (output fp32 [nh, r, H])
 *   minimises sum_e F[e, hH + j] (W[e, hH + j] - A_h[e, :] . b)^2 for the
 *   given A fp32 [E, nh*r].
 *
 * H in {64, 128}; r in {16, 32, 48, 64}.  The r x r normal matrix of every
 * row (column) must be positive definite (B_h of full row rank, A_h of full
 * column rank over the rows with weight); a singular one yields non-finite
 * values in that row (column).  No workspace.
 */
int wsvd_weighted_update_A(int E, int nh, int H, int r, const float* W,
                           const float* F, const float* B, float* A,
                           hipStream_t stream);
int wsvd_weighted_update_B(int E, int nh, int H, int r, const float* W,
                           const float* F, const float* A, float* B,
                           hipStream_t stream);

/*
 * Ablation: decoding over a conventional (whole-matrix) factorisation, the
 * scheme the per-head path replaces.  One latent of global rank R is shared
 * by all heads and every head rebuilds its keys and values from it
 * (Japanese page section 1, German page section 1, Italian page section 1,
 * Arabic page section 1; per-head factors cut the latent to L x r and the
 * rebuild cost by r / R, Arabic page section 2a).  Reading: head h's keys
 * are C_K[b] B_K[:, hH:(h+1)H], values likewise.
 *
 *   q        BF16 [nb, nh, H]
 *   C_K, C_V BF16 [nb, L_cap, R]   shared latent rows of each sequence
 *   B_K, B_V BF16 [R, nh*H]        column block h maps the latent to head h
 *   L        int32 [nb] (device), clamped to [0, L_cap]; 0 gives a zero row
 *   out      F32 | BF16 [nb, nh, H]
 * H in {64, 128}; R in {512, 1024, 2048}.  softmax_scale <= 0 means
 * 1/sqrt(H); n_splits 0 = the same automatic rule as wsvd_decode_attn.
 * Four launches: the q' = B_K-block fold, split attention over the shared
 * latent (every head streams the whole R-wide rows), merge + projection in
 * chunks of 128 latent columns, and the sum of the chunks.
 * Workspace: wsvd_shared_decode_workspace_bytes(...), 256-byte aligned, no
 * initial contents required.
 */
size_t wsvd_shared_decode_workspace_bytes(int nb, int nh, int R, int L_cap, int n_splits);
int wsvd_shared_decode_attn(int nb, int nh, int H, int R, int L_cap,
                            const int32_t* L, const void* q,
                            const void* C_K, const void* C_V,
                            const void* B_K, const void* B_V,
                            float softmax_scale, int n_splits,
                            void* workspace, size_t workspace_bytes,
                            void* out, wsvd_dtype out_dt, hipStream_t stream);

/*
 * wsvd_floor_probe -- measurement aid, not part of the decode path: the
 * floor a decode launch of `blocks` workgroups of 256 threads cannot beat on
 * this device.  mode 0 launches an empty kernel (sink: float [blocks], read
 * and possibly written); mode 1 streams `bytes` of src (16-byte aligned,
 * split evenly into whole 16-byte chunks per block, at most 4096 chunks per
 * block), every request issued before any is used, and stores one value per
 * block into sink.  A small decode step (for example 5 MB for one 32-head
 * layer of 1088 tokens) is bound by these, not by HBM bandwidth.
 * WSVD_ERR_SHAPE for a bad mode, grid or byte count.
 */
int wsvd_floor_probe(int mode, int blocks, const void* src, size_t bytes, float* sink, hipStream_t stream);

/* Static description of a status code.  Pure host; never NULL. */
const char* wsvd_status_string(int status);

/* Library version, e.g. "wsvd 0.1 gfx950".  Pure host. */
const char* wsvd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WSVD_H_ */
