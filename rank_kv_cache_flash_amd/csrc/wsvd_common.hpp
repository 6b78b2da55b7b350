// wsvd_common.hpp -- shared device helpers for the gfx950 kernels.
//
// Only what several kernels need: dtype conversions, DPP row reductions
// and small vector types.  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wsvd.h"

namespace wsvd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}

// float -> bf16, round to nearest, ties to even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // nearest, ties to even
}

// Element `i` of a q / B / x / A style tensor of runtime dtype `dt`, as float.
__device__ __forceinline__ float load_elem(const void* p, int dt, size_t i) {
    switch (dt) {
        case WSVD_F32: return static_cast<const float*>(p)[i];
        case WSVD_BF16: return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
        default: return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
}

// q element idx: the dword holding it (one unconditional load, any dtype)
// and, separately, its value.  Converting only after every other prologue
// request is out keeps the first requests from waiting on this one.
__device__ __forceinline__ uint32_t load_q_word(const void* q, int q_dt, size_t idx) {
    const size_t word = (q_dt == WSVD_F32) ? idx : (idx >> 1);
    return static_cast<const uint32_t*>(q)[word];
}
__device__ __forceinline__ float q_word_value(uint32_t w, int q_dt, size_t idx) {
    const uint16_t half = (idx & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xffffu);
    const float fb = bf16_to_f32(half);
    const float fh = f16_to_f32(half);
    return (q_dt == WSVD_F32) ? __uint_as_float(w) : (q_dt == WSVD_BF16 ? fb : fh);
}

// Store `v` as element i of a tensor of runtime dtype `dt`, written through
// to memory at device scope.  Results a kernel leaves behind go out this
// way: a plain store leaves a dirty L2 line for the end-of-kernel release
// to write back, which measured slower than storing through.
__device__ __forceinline__ void store_elem_wt(void* p, int dt, size_t i, float v) {
    switch (dt) {
        case WSVD_F32:
            __hip_atomic_store(static_cast<float*>(p) + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        case WSVD_BF16:
            __hip_atomic_store(static_cast<uint16_t*>(p) + i, f32_to_bf16(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            break;
        default:
            __hip_atomic_store(static_cast<uint16_t*>(p) + i, f32_to_f16(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            break;
    }
}

// ---------------------------------------------------------------------------
// cross-lane sums inside rows of 16 lanes (DPP: no LDS traffic)
// ---------------------------------------------------------------------------
// DPP control words (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane j of 8 <-> 7-j
constexpr int kDppRowMirror = 0x140;   // lane j of 16 <-> 15-j

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N in 1, 2, 4, 8, 16); every lane of a
// group ends with the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_f<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_f<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
    return v;
}

// Maximum over aligned groups of N lanes, like group_sum.
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return v;
}

// Lane l combined with lane l^16 (l^32): gfx950 permlane swaps exchange rows
// of two registers; with both operands equal, the two results hold v_l and
// v_(l^16) (v_(l^32)) in every lane.  VALU only, no LDS round trip.
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum over the whole wave, in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return xor32_max(xor16_max(v));
}

// Sum over the lanes that share (lane % GP) -- one lane of every row slot of
// GP lanes -- in every lane: rotations by GP, 2GP, .. inside each 16-lane
// row (DPP row_ror), then across rows.
template <int GP>
__device__ __forceinline__ float sum_over_slots(float v) {
    if constexpr (GP <= 1) v += dpp_f<0x121>(v);
    if constexpr (GP <= 2) v += dpp_f<0x122>(v);
    if constexpr (GP <= 4) v += dpp_f<0x124>(v);
    if constexpr (GP <= 8) v += dpp_f<0x128>(v);
    return xor32_sum(xor16_sum(v));
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) {
    return __shfl_xor(v, m, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Device-scope (all XCDs) coherent store / load: written through to memory,
// read past any L2 copy, so partials written by one XCD can be merged on
// another without a cache-wide writeback or invalidate.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load marked non-temporal: the latent stream is read once,
// so it should not evict the factor lines that many workgroups reuse.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

}  // namespace wsvd
