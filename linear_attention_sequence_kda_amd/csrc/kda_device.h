// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFloor = -5.0f;   // lower bound of every step's log-decay

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Floored, clamped log-decay in log2 units: log2(exp(min(0, max(-5, g)))).
__device__ __forceinline__ float log2_decay(float g) {
  return fminf(0.0f, fmaxf(kFloor, g)) * kLog2e;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
}

// Load 4 consecutive elements of a bf16 or fp32 array as floats (16/8-byte aligned).
template <bool BF16>
__device__ __forceinline__ float4 load4(const void *p, size_t idx) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *p, size_t idx) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[idx]);
  else return static_cast<const float *>(p)[idx];
}

template <bool BF16>
__device__ __forceinline__ void store4(void *p, size_t idx, float4 x) {
  if constexpr (BF16) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16_bits(x.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16_bits(x.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + idx) = w;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(p) + idx) = x;
  }
}

}  // namespace kda
