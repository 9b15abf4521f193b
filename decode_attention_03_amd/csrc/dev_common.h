// dev_common.h -- small device helpers for the gfx950 kernels of libfd:
// element conversion, 128-bit loads, wave64 DPP row reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fd_internal.h"

namespace fd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element conversion.  Storage is raw bits; arithmetic is fp32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Unpack one 32-bit word into 1 (f32) or 2 (16-bit types) floats.
template <int DT>
__device__ __forceinline__ void unpack_word(uint32_t w, float *out) {
    if constexpr (DT == kF32) {
        out[0] = __builtin_bit_cast(float, w);
    } else if constexpr (DT == kBF16) {
        out[0] = bf16_lo(w);
        out[1] = bf16_hi(w);
    } else {
        out[0] = f16_lo(w);
        out[1] = f16_hi(w);
    }
}

// Two-wide dot product of packed 16-bit pairs accumulated in fp32
// (v_dot2c_f32_bf16 / v_dot2c_f32_f16): acc + a.lo*b.lo + a.hi*b.hi.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), acc, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), acc, false);
}

template <int DT>
struct ElemInfo {
    static constexpr int bytes = DT == kF32 ? 4 : 2;
    static constexpr int per_word = 4 / bytes;
};

// fp32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> binary16 bits (hardware conversion, round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Store one fp32 value into an output array of dtype `out_dtype`.
__device__ __forceinline__ void store_out(void *base, size_t idx, float val, int out_dtype) {
    if (out_dtype == kF32)
        static_cast<float *>(base)[idx] = val;
    else if (out_dtype == kBF16)
        static_cast<uint16_t *>(base)[idx] = f32_to_bf16_rne(val);
    else
        static_cast<uint16_t *>(base)[idx] = f32_to_f16_rne(val);
}

// ---------------------------------------------------------------------------
// Loads.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 128-/64-bit loads; NT = 1 marks them non-temporal (data read once).
template <int NT = 0>
__device__ __forceinline__ u32x4 ld128(const void *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    else
        return *static_cast<const u32x4 *>(p);
}
template <int NT = 0>
__device__ __forceinline__ u32x2 ld64(const void *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(static_cast<const u32x2 *>(p));
    else
        return *static_cast<const u32x2 *>(p);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions inside one 16-lane DPP row of a wave64.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same
// bits (each step adds a lane and its partner in both orders, and fp32
// addition is commutative).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: quads
    v += dpp_mov<0x141>(v);  // row_half_mirror: the two quads of each half-row
    v += dpp_mov<0x140>(v);  // row_mirror: the two half-rows
    return v;
}

// Sum over groups of N = 4, 8 or 16 consecutive lanes (N divides a DPP row);
// every lane of a group receives the same bits.
template <int N>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16, "unsupported group size");
    v += dpp_mov<0xB1>(v);       // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);       // quad_perm [2,3,0,1]
    if constexpr (N >= 8)
        v += dpp_mov<0x141>(v);  // row_half_mirror
    if constexpr (N >= 16)
        v += dpp_mov<0x140>(v);  // row_mirror
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace fd
