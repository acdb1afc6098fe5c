// Measurement aid: the dense bf16 MFMA rate the chip sustains.
//
// Every wave runs CHAINS independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 with operands in registers (no memory traffic in
// the loop), two waves per SIMD.  The operands change every round (a lane
// pattern xor-ed into their mantissas) so that the matrix cores switch bits
// as they do on real data, which sets the power draw and with it the clock
// the chip holds under MFMA load.  Timing the launch gives the achievable
// rate against which the Newton-Schulz products can be read, beside the
// vendor's 2.4 GHz figure.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int PROBE_THREADS = 512;  // 8 waves: two per SIMD
constexpr int CHAINS = 4;
}  // namespace

__global__ __launch_bounds__(PROBE_THREADS) void mfma_probe_kernel(int64_t iterations, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  // bf16 values in [1, 2) with lane-dependent mantissas
  u32x4 a = {0x3F803F80u ^ (lane * 0x00070005u), 0x3F813F82u ^ (lane * 0x00030001u),
             0x3F833F84u ^ (lane * 0x00050003u), 0x3F853F86u ^ (lane * 0x00010007u)};
  u32x4 b = {0x3F873F88u ^ (lane * 0x00020003u), 0x3F893F8Au ^ (lane * 0x00060001u),
             0x3F8B3F8Cu ^ (lane * 0x00040005u), 0x3F8D3F8Eu ^ (lane * 0x00010002u)};
  const u32x4 flip = {0x00150015u, 0x002A002Au, 0x00330033u, 0x004C004Cu};
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  for (int64_t it = 0; it < iterations; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc[c], 0, 0, 0);
    a ^= flip;
    b ^= flip.yzwx;
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  // never true for finite sums; keeps the chains live
  if (s == -1.0f) sink[0] = s;
}

hipError_t launch_mfma_probe(int64_t iterations, int32_t cus, float* sink, double* flops, hipStream_t stream) {
  const int64_t waves = int64_t(cus) * (PROBE_THREADS / 64);
  *flops = double(waves) * double(iterations) * CHAINS * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(uint32_t(cus)), dim3(PROBE_THREADS), 0, stream, iterations, sink);
  return hipGetLastError();
}

}  // namespace muon
