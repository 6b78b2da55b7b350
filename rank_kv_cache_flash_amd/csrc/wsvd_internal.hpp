// wsvd_internal.hpp -- argument blocks and launchers shared by the C ABI
// (abi.hip) and the kernel files.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wsvd {

// Everything the split decode kernel reads, passed by value as kernargs.
struct DecodeArgs {
    int nb, nh, L_cap, S;
    const int32_t* L;
    const void* q;
    int q_dt;
    const void* C_K;
    const void* C_V;
    const uint16_t* s_K;
    const uint16_t* s_V;
    const void* B_K;
    const void* B_V;
    int B_dt;
    float scale_log2;  // softmax scale times log2(e)
    float* o_part;     // [nb, nh, S, H]
    float* lse_part;   // [nb, nh, S]
    unsigned* counters;  // [nb, nh] arrival counters (zero between calls)
    void* out;         // [nb, nh, H] or null (partials only)
    int out_dt;
};

hipError_t launch_decode_split(const DecodeArgs& a, int H, int r, int C_dt, hipStream_t st);
// The bf16-cache, rank-32 split-kernel instances (decode_bf16_r32.hip).
hipError_t launch_decode_bf16_r32(const DecodeArgs& a, int H, hipStream_t st);

// Decode with a rotary position step on every reconstructed key row
// (bf16 caches and factors; H in 64, 128; r in 32, 64).
hipError_t launch_decode_rope(const DecodeArgs& a, int H, int r, const float* rcos, const float* rsin,
                              hipStream_t st);
hipError_t launch_rope_tables(int L_cap, int H, double base, float* rcos, float* rsin, hipStream_t st);

// Dense Flash-Decoding baseline (bf16 K / V rows of H values, no factors).
hipError_t launch_dense_split(const DecodeArgs& a, int H, hipStream_t st);

hipError_t launch_combine(int nb, int nh, int H, int S, const float* o_part, const float* lse_part,
                          void* out, int out_dt, hipStream_t st);
// Measurement floors (probe.hip): mode 0 an empty launch, mode 1 a stream of
// `bytes` from src split evenly over `blocks` blocks of 256 threads.
hipError_t launch_probe(int mode, int blocks, const void* src, size_t bytes, float* sink, hipStream_t st);

// p[0 .. n) = 0 (uint32 words), one small launch.
hipError_t launch_fill_zero_u32(unsigned* p, size_t n, hipStream_t st);

struct AppendArgs {
    int nb, E, nh, r, L_cap;
    int w8;               // 0: bf16 x [nb, E], A [E, nh*r]
                          // 1: int8 x codes [nb, E] + sx, int8 A^T codes [nh*r, E] + sA
    const void* x;
    const void* A_K;
    const void* A_V;
    const float* sx;      // fp32 [nb]      (w8 only)
    const float* sA_K;    // fp32 [nh*r]    (w8 only)
    const float* sA_V;
    const int32_t* pos;
    void* C_K;
    void* C_V;
    int C_dt;
    uint16_t* s_K;        // fp16 [nb, nh, L_cap] row scales (int8 caches only)
    uint16_t* s_V;
    float* part;          // split-E partial tiles (KS > 1 only): fp32, or int32 for w8
    unsigned* counters;   // per-tile arrival counters, zero between calls
    int KS;               // number of E splits
};

// bf16 operands (append_stream.hip): x [nb, E] and A [E, nh*r] bf16.
hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t st);
// Its column tile (32, or 64 for int8 caches of rank 64), tile count, E
// slices and partial-tile bytes (0 when E is not split) (host).
int append_bf16_tile_cols(int C_dt, int r);
long append_bf16_num_tiles(int nb, int nh, int r, int NT);
int append_bf16_num_esplits(int nb, int E, int nh, int r, int NT);
size_t append_bf16_partial_bytes(int nb, int E, int nh, int r, int NT);

// int8 operands (append.hip): x codes [nb, E] + sx, A^T codes [nh*r, E] + sA.
hipError_t launch_append_w8(const AppendArgs& a, hipStream_t st);
long append_w8_num_tiles(int nb, int nh, int r);
int append_w8_num_esplits(int nb, int E, int nh, int r);
size_t append_w8_partial_bytes(int nb, int E, int nh, int r);

// W8A8 helpers (w8a8.hip): S1 rotation + per-row int8 codes of activations,
// and the offline rotation + per-column int8 codes of a factor.
hipError_t launch_w8a8_quantize_rows(int nb, int E, const void* x, int x_dt, int8_t* xq, float* sx,
                                     hipStream_t st);
hipError_t launch_w8a8_prepare(int E, int N, const void* A, int A_dt, int8_t* AqT, float* sA, hipStream_t st);
// Columns of A one prepare block rotates at once (LDS holds cols * E floats).
int w8a8_prepare_cols(int E);

// Offline per-head factorisation (factorize.hip).  Truncated SVD: Gram
// partials into Gpart ([chunks, nh, H, H] fp64), Jacobi per head, then
// A = W B^T.  Weighted refinement: one alternating least squares half-step,
// rows = true solves the rows of A from B, false the columns of B from A.
int svd_num_chunks(int E, int nh);
hipError_t launch_factorize_svd(const float* W, int E, int nh, int H, int r, float* A, float* B, float* sigma,
                                int* sweeps, double* Gpart, hipStream_t st);
hipError_t launch_factorize_weighted(bool rows, const float* W, const float* F, const float* in, int E, int nh,
                                     int H, int r, float* out, hipStream_t st);

// Decode over a conventional shared rank-R latent (shared_decode.hip):
// bf16 q [nb, nh, H], C_K / C_V [nb, L_cap, R], B_K / B_V [R, nh*H].
struct SharedArgs {
    int nb, nh, H, R, L_cap, S;
    const int32_t* L;
    const uint16_t* q;
    const uint16_t* C_K;
    const uint16_t* C_V;
    const uint16_t* B_K;
    const uint16_t* B_V;
    float scale_log2;
    float* qp;        // fp32 [nb, nh, R]
    float* o_part;    // fp32 [nb, nh, S, R]
    float* lse_part;  // fp32 [nb, nh, S]
    float* proj_part; // fp32 [R / 128, nb, nh, H]
    void* out;        // [nb, nh, H]
    int out_dt;
};

hipError_t launch_shared_decode(const SharedArgs& a, hipStream_t st);

}  // namespace wsvd
