// Scalar helpers of the HIP kernels: bfloat16 bit conversions and the
// update scale of the write-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Global-memory view of a pointer: accesses through it compile to global_*
// instructions, counted by vmcnt only.  Through a generic pointer they become
// flat instructions, which also count in lgkmcnt, so that every wait for LDS
// results would wait for the global traffic in flight as well.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float((h & 0xFFFFu) << 16);
}

// Round two binary32 values to bfloat16, nearest with ties to even (overflow
// to infinity, NaN stays NaN), with the converter of the CDNA4 vector unit
// (v_cvt_pk_bf16_f32); returns lo | hi << 16.  A test of every binary32 bit
// pattern found it equal to the explicit rounding (add 0x7FFF plus the
// lowest kept bit, truncate) on all non-NaN inputs.
__device__ __forceinline__ uint32_t float2_to_bf16x2_bits(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) { return uint16_t(float2_to_bf16x2_bits(f, 0.f)); }

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
