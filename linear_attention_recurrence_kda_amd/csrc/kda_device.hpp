// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// bf16 values travel as raw 16-bit patterns; conversions are explicit.
struct bf16raw {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16raw x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Round to nearest even; NaN stays NaN (gfx950's v_cvt_pk_bf16_f32, no
// branches).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// The same rounding in integer arithmetic (NaN handled by a branch).  The
// single decode step measured faster with it than with the conversion
// instruction.
__device__ __forceinline__ uint16_t f32_to_bf16_bits_int(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16raw from_f32<bf16raw>(float x) { return bf16raw{f32_to_bf16_bits(x)}; }

template <typename T>
__device__ __forceinline__ T from_f32_int(float x);
template <>
__device__ __forceinline__ float from_f32_int<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16raw from_f32_int<bf16raw>(float x) { return bf16raw{f32_to_bf16_bits_int(x)}; }

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// 1/x by v_rcp_f32 (about 1 ulp), in place of the correctly rounded division
// (a scale, a reciprocal, four FMAs and a fix-up per element).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace kda
