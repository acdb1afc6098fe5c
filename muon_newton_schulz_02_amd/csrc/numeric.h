// Scalar helpers of the HIP kernels: bfloat16 bit conversions and the
// update scale of the write-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float((h & 0xFFFFu) << 16);
}

// Round a binary32 value to bfloat16, nearest with ties to even; NaN stays a
// (quiet) NaN, overflow goes to infinity.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// t = fl32(lr * s) with s from the scale rule: 0 none (s = 1),
// 1 sqrt(max(1, rows/cols)), 2 0.2*sqrt(max(rows, cols)); s and the
// product in binary64, one rounding to binary32.
__device__ __forceinline__ float update_scale(float lr, int rule, int rows, int cols) {
  double s = 1.0;
  if (rule == 1) {
    const double r = double(rows) / double(cols);
    s = sqrt(r > 1.0 ? r : 1.0);
  } else if (rule == 2) {
    s = 0.2 * sqrt(double(rows > cols ? rows : cols));
  }
  return float(double(lr) * s);
}

}  // namespace muon
