// Measurement aid: the dense bf16 MFMA rate the chip sustains on real data.
//
// Every wave runs CHAINS independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 with operands in registers (no memory traffic in
// the loop), two waves per SIMD.  The operands are NSET fragments of random
// bits per lane (random sign and mantissa, exponents within a factor of 2^7),
// taken in turn, so that the matrix cores switch as many bits as they do on
// the products' data.  That matters: under MFMA load the clock the chip holds
// depends on the data, and constant or zero operands run near the nominal
// 2.4 GHz while random ones hold it far lower.  Timing the launch gives the
// achievable rate against which the Newton-Schulz products can be read,
// beside the vendor's 2.4 GHz figure.
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
constexpr int NSET = 8;             // operand fragments per lane, taken in turn

// integer hash (two multiply-xorshift rounds)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// two bf16 values from 32 random bits: sign and 7 mantissa bits kept,
// exponent field 124 + 3 random bits (magnitudes in [2^-3, 2^5))
__device__ __forceinline__ uint32_t random_bf16x2(uint32_t h) {
  const uint32_t lo = (h & 0x807Fu) | ((124u + ((h >> 7) & 7u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807Fu) | ((124u + ((h >> 23) & 7u)) << 7);
  return lo | (hi << 16);
}
}  // namespace

__global__ __launch_bounds__(PROBE_THREADS) void mfma_probe_kernel(int64_t iterations, float* __restrict__ sink) {
  const uint32_t gid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  u32x4 a[NSET], b[NSET];
#pragma unroll
  for (int s = 0; s < NSET; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[s][e] = random_bf16x2(mix32(gid * 64u + uint32_t(s * 4 + e)));
      b[s][e] = random_bf16x2(mix32(gid * 64u + uint32_t(32 + s * 4 + e) + 0x9E3779B9u));
    }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  // round r takes fragment pair (r % NSET, (r + c) % NSET) in chain c
  const int64_t full = iterations / NSET;
  for (int64_t it = 0; it < full; ++it) {
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                         __builtin_bit_cast(bf16x8, b[(s + c) % NSET]), acc[c], 0, 0, 0);
  }
  for (int64_t it = full * NSET; it < iterations; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                       __builtin_bit_cast(bf16x8, b[c % NSET]), acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  // the operands are finite and bounded, so the sums are never NaN; the
  // test keeps the chains live
  if (__builtin_isnan(s)) sink[0] = s;
}

hipError_t launch_mfma_probe(int64_t iterations, int32_t cus, float* sink, double* flops, hipStream_t stream) {
  const int64_t waves = int64_t(cus) * (PROBE_THREADS / 64);
  *flops = double(waves) * double(iterations) * CHAINS * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(uint32_t(cus)), dim3(PROBE_THREADS), 0, stream, iterations, sink);
  return hipGetLastError();
}

}  // namespace muon
