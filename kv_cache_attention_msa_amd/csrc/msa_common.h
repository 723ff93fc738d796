// Device helpers shared by the MSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_internal.h"

namespace msa {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round-to-nearest-even float -> bfloat16 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Pool block id of a device-side block entry (resolved by the upload kernel).
__device__ __forceinline__ int entry_block(const BlockEntry& e) {
  return (int)((uint32_t)e.bt_valid & ((1u << kBtIndexBits) - 1u));
}
__device__ __forceinline__ int entry_valid(const BlockEntry& e) {
  return (int)((uint32_t)e.bt_valid >> kBtIndexBits) + 1;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace msa
