// bf16 <-> fp32 conversions of the kernels (bf16 is the upper half of an fp32 bit pattern).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ngram {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace ngram
