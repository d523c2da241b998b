// rt_common.hpp -- device helpers shared by the gfx950 kernels of the routed
// attention library.  Only this library includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWave = 64;

// ---- bfloat16 <-> float32 ----------------------------------------------------
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ u16 f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u16)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

// 8 bf16 values packed in a uint4 (16 bytes) <-> MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Unpack the i-th bf16 of a uint4 to float.
__device__ __forceinline__ float u4_elem(const uint4& v, int i) {
    uint32_t word = (i < 2) ? v.x : (i < 4) ? v.y : (i < 6) ? v.z : v.w;
    return bf2f((u16)((i & 1) ? (word >> 16) : (word & 0xffffu)));
}

__device__ __forceinline__ uint32_t pack2(u16 lo, u16 hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// ---- MFMA --------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l (g = l / 16) supplies A[row = l % 16][k = 8g .. 8g+7] and
// B[k = 8g .. 8g+7][col = l % 16]; it receives D[row = 4g + i][col = l % 16],
// i = 0..3.  Since k is summed over, any permutation of k applied to both
// operands alike gives the same product.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- wave helpers --------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float xor_max_16_32(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float xor_sum_16_32(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ int clamp_pos(int t, int n) { return t < 0 ? 0 : (t >= n ? n - 1 : t); }

// Typed loads of one token element for the float32 and bf16 variants.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, long i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, long i, float v) { p[i] = v; }
};
template <> struct Elem<u16> {
    static __device__ __forceinline__ float load(const u16* p, long i) { return bf2f(p[i]); }
    static __device__ __forceinline__ void store(u16* p, long i, float v) { p[i] = f2bf(v); }
};

}  // namespace rt
