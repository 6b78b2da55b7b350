// w8a8.hip -- the integer operands of the W8A8 append.
//
// The pages run the projections at W8A8 and smooth activation outliers with
// an orthogonal Hadamard rotation S1 before quantising ("WSVD: Weighted
// Low-Rank Approximation for Fast and Efficient Execution of Low-Precision
// Vision-Language Models": German page section 2C, Italian page section 2C,
// Japanese page section 2.3, Arabic page section 2c).  S1 here is the
// normalised Walsh-Hadamard matrix H = H_E / sqrt(E) (Sylvester order, E a
// power of two); it is symmetric and orthogonal, so x . A = (x H) . (H A)
// and the rotation of A is folded offline.
//
//  * quantize_rows: per token, x~ = x H by a fast Walsh-Hadamard transform
//    (log2 E butterfly passes, fp32: in registers, across lanes with DPP and
//    the gfx950 row swaps, then once through LDS), then symmetric absmax codes
//    with one fp32 scale:
//    s = max|x~| / 127, code = clamp(round_half_even(x~ / s), -127, 127),
//    all zero if s == 0.
//  * prepare: offline, per output column n of a factor A [E, N]: the same
//    transform down the column, the same codes with one fp32 scale per
//    column, written transposed (A^T codes [N, E], k-contiguous) so the
//    append's integer MFMA reads both operands without a transpose.
//
// Both are small, one-off passes (the activations are nb x E values); one
// workgroup owns whole rows so the transform needs no cross-block traffic.
#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {

// In-place unnormalised Walsh-Hadamard transform of `cols` length-E vectors
// (the offline factor pass)
// stored back to back in LDS (E a power of two): pass h pairs element i
// with i + h inside each block of 2h and writes (a + b, a - b).
__device__ __forceinline__ void fwht_lds(float* L, int E, int cols) {
    const int half = E >> 1;
    for (int h = 1; h < E; h <<= 1) {
        __syncthreads();
        for (int p = threadIdx.x; p < cols * half; p += blockDim.x) {
            const int c = p / half;
            const int q = p - c * half;
            const int i = ((q & ~(h - 1)) << 1) | (q & (h - 1));
            float* v = L + (size_t)c * E;
            const float x0 = v[i], x1 = v[i + h];
            v[i] = x0 + x1;
            v[i + h] = x0 - x1;
        }
    }
    __syncthreads();
}

// Maximum over the workgroup (256 threads); every thread gets it.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ int8_t code_of(float v, float s) {
    if (!(s > 0.f)) return 0;
    return (int8_t)(int)fminf(fmaxf(__builtin_rintf(v / s), -127.f), 127.f);
}

// One token per workgroup.  Thread t holds EPT = E / 256 consecutive
// elements, so the transform's passes split by distance: inside a thread's
// registers (distance < EPT), across the lanes of a wave (DPP and row swaps,
// not LDS shuffles: the same results, and the W8A8 append with this step
// measured 17.5 -> 17.0 us on MI355X), and the
// last two passes (distances E/4 and E/2, between the 4 waves) as one 4-point
// transform per column after a single trip through LDS.
// Element i of a tensor of compile-time dtype DT, as float (straight-line
// loads: a runtime dtype switch per element serialised them).
template <int DT>
__device__ __forceinline__ float elem(const void* p, size_t i) {
    if constexpr (DT == WSVD_F32) return static_cast<const float*>(p)[i];
    else if constexpr (DT == WSVD_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Value of lane l ^ D (D = 1 .. 32) in every lane l.
template <int D>
__device__ __forceinline__ float lane_xor(float v, int lane) {
    if constexpr (D == 1) {
        return dpp_f<kDppQuadXor1>(v);
    } else if constexpr (D == 2) {
        return dpp_f<kDppQuadXor2>(v);
    } else if constexpr (D == 4) {
        const float from_below = dpp_f<0x114>(v);  // row_shr:4, lane l - 4
        const float from_above = dpp_f<0x104>(v);  // row_shl:4, lane l + 4
        return (lane & 4) ? from_below : from_above;
    } else if constexpr (D == 8) {
        return dpp_f<0x128>(v);  // row_ror:8 inside 16 lanes is l ^ 8
    } else {
        const uint32_t u = __float_as_uint(v);
        const auto r = (D == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                 : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(r[0] == u ? r[1] : r[0]);  // the element that is not this lane's
    }
}

// One transform pass over lane pairs (l, l ^ D): (a + b, a - b), the lower
// lane keeping the sum.
template <int D, int EPT>
__device__ __forceinline__ void butterfly_lanes(float (&v)[EPT], int lane) {
    const bool upper = (lane & D) != 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const float y = lane_xor<D>(v[k], lane);
        v[k] = upper ? (y - v[k]) : (v[k] + y);
    }
}

template <int EPT, int DT>
__global__ __launch_bounds__(256) void w8a8_quantize_rows_kernel(const void* x, float inv_sqrt_e, int8_t* xq,
                                                                 float* sx) {
    constexpr int E = EPT * 256;
    constexpr int Q = E / 4;  // one wave's span
    __shared__ float L[E];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const size_t b = blockIdx.x;
    float v[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) v[k] = elem<DT>(x, b * E + (size_t)tid * EPT + k);
    // passes inside the thread
#pragma unroll
    for (int h = 1; h < EPT; h <<= 1) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            if (k & h) continue;
            const float a0 = v[k], a1 = v[k + h];
            v[k] = a0 + a1;
            v[k + h] = a0 - a1;
        }
    }
    // passes across lanes: element distance EPT * d, partner lane l ^ d
    // through DPP and the gfx950 row swaps (no LDS round trips)
    butterfly_lanes<1>(v, lane);
    butterfly_lanes<2>(v, lane);
    butterfly_lanes<4>(v, lane);
    butterfly_lanes<8>(v, lane);
    butterfly_lanes<16>(v, lane);
    butterfly_lanes<32>(v, lane);
#pragma unroll
    for (int k = 0; k < EPT; ++k) L[tid * EPT + k] = v[k];
    __syncthreads();
    // last two passes: column j of the four wave spans, j = tid + 256 i
    constexpr int NJ = (Q + 255) / 256;
    float o[NJ][4];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
        const int j = tid + 256 * i;
        if (j >= Q) break;
        const float a0 = L[j], a1 = L[j + Q], a2 = L[j + 2 * Q], a3 = L[j + 3 * Q];
        const float s01 = a0 + a1, d01 = a0 - a1, s23 = a2 + a3, d23 = a2 - a3;
        o[i][0] = (s01 + s23) * inv_sqrt_e;
        o[i][1] = (d01 + d23) * inv_sqrt_e;
        o[i][2] = (s01 - s23) * inv_sqrt_e;
        o[i][3] = (d01 - d23) * inv_sqrt_e;
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, fabsf(o[i][c]));
    }
    const float s = block_max(m, red) / 127.f;
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
        const int j = tid + 256 * i;
        if (j >= Q) break;
#pragma unroll
        for (int c = 0; c < 4; ++c) xq[b * E + j + c * Q] = code_of(o[i][c], s);
    }
    if (tid == 0) sx[b] = s;
}

__global__ __launch_bounds__(256) void w8a8_prepare_kernel(const void* A, int A_dt, int E, int N, int cols,
                                                           float inv_sqrt_e, int8_t* AqT, float* sA) {
    extern __shared__ float L[];  // [cols][E]
    __shared__ float red[4];
    const int n0 = blockIdx.x * cols;
    for (int idx = threadIdx.x; idx < cols * E; idx += 256) {
        const int e = idx / cols;
        const int c = idx - e * cols;
        L[(size_t)c * E + e] = (n0 + c < N) ? load_elem(A, A_dt, (size_t)e * N + n0 + c) : 0.f;
    }
    fwht_lds(L, E, cols);
    for (int c = 0; c < cols && n0 + c < N; ++c) {
        float* v = L + (size_t)c * E;
        float m = 0.f;
        for (int e = threadIdx.x; e < E; e += 256) {
            const float t = v[e] * inv_sqrt_e;
            v[e] = t;
            m = fmaxf(m, fabsf(t));
        }
        const float s = block_max(m, red) / 127.f;
        int8_t* out = AqT + (size_t)(n0 + c) * E;
        for (int e = threadIdx.x; e < E; e += 256) out[e] = code_of(v[e], s);
        if (threadIdx.x == 0) sA[n0 + c] = s;
    }
}

// At most 32 KB of LDS per workgroup: cols * E floats.
int w8a8_prepare_cols(int E) { return E >= 8192 ? 1 : min(8, 8192 / E); }

template <int EPT>
static void launch_qr(int nb, const void* x, int x_dt, float inv, int8_t* xq, float* sx, hipStream_t st) {
    if (x_dt == WSVD_F32)
        hipLaunchKernelGGL((w8a8_quantize_rows_kernel<EPT, WSVD_F32>), dim3(nb), dim3(256), 0, st, x, inv, xq, sx);
    else if (x_dt == WSVD_BF16)
        hipLaunchKernelGGL((w8a8_quantize_rows_kernel<EPT, WSVD_BF16>), dim3(nb), dim3(256), 0, st, x, inv, xq, sx);
    else
        hipLaunchKernelGGL((w8a8_quantize_rows_kernel<EPT, WSVD_F16>), dim3(nb), dim3(256), 0, st, x, inv, xq, sx);
}

hipError_t launch_w8a8_quantize_rows(int nb, int E, const void* x, int x_dt, int8_t* xq, float* sx,
                                     hipStream_t st) {
    const float inv = (float)(1.0 / __builtin_sqrt((double)E));
    switch (E) {
        case 256: launch_qr<1>(nb, x, x_dt, inv, xq, sx, st); break;
        case 512: launch_qr<2>(nb, x, x_dt, inv, xq, sx, st); break;
        case 1024: launch_qr<4>(nb, x, x_dt, inv, xq, sx, st); break;
        case 2048: launch_qr<8>(nb, x, x_dt, inv, xq, sx, st); break;
        case 4096: launch_qr<16>(nb, x, x_dt, inv, xq, sx, st); break;
        case 8192: launch_qr<32>(nb, x, x_dt, inv, xq, sx, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_w8a8_prepare(int E, int N, const void* A, int A_dt, int8_t* AqT, float* sA, hipStream_t st) {
    const int cols = w8a8_prepare_cols(E);
    const float inv = (float)(1.0 / __builtin_sqrt((double)E));
    const size_t lds = (size_t)cols * E * sizeof(float);
    hipLaunchKernelGGL(w8a8_prepare_kernel, dim3((N + cols - 1) / cols), dim3(256), lds, st, A, A_dt, E, N, cols,
                       inv, AqT, sA);
    return hipGetLastError();
}

}  // namespace wsvd
