// Elementwise and reduction kernels of the Muon step on gfx950.
//
//  * momentum_kernel: per element, in binary32 with one rounding per
//    operation, M <- beta*M + G and U <- G + beta*M (Nesterov) or U <- M;
//    stores U into the workspace in the wide orientation X (m x n, m <= n;
//    through an LDS transpose for tall matrices) in the Newton-Schulz storage
//    format, zero-filling the padding; writes one binary32 sum of u^2 per
//    64x64 tile (wavefront shuffles, then LDS across the four waves).
//    G and M are touched once per step, so their vector loads and the M
//    store carry the nontemporal hint (measured 4 % faster); U is read
//    again by the Newton-Schulz products and is stored normally.
//  * norm_finalize_kernel: sums a matrix's tile partials in a fixed order
//    and forms 1/(||U||_F + eps).
//  * writeback_direct_kernel: the write-back when no Newton-Schulz step is
//    asked for (O = U / (||U||_F + eps)).
//
// Momentum is the heavy-ball buffer of the Muon optimizer ("把 GPT-2 的训练
// 租金估算从 4.3 万美元压到 40 美元…", table 符号与约定, row "Muon": an
// orthogonalised-momentum optimizer for matrix parameters).  The heavy-ball
// form, the Nesterov variant and eps = 1e-7 are readings; the pages print
// no formula.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"
#include "numeric.h"

#pragma clang fp contract(off)

namespace muon {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

__device__ inline int find_matrix(const int32_t* __restrict__ off, int count, int tile) {
  int lo = 0, hi = count;  // off[lo] <= tile < off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline float load_elem(const void* p, int64_t idx, int bf16) {
  return bf16 ? bf16_bits_to_float(gmem(reinterpret_cast<const uint16_t*>(p))[idx])
              : gmem(reinterpret_cast<const float*>(p))[idx];
}

// Store four consecutive values of the Newton-Schulz working format.
__device__ inline void store4_ws(void* base, int64_t plane, int prec, int64_t idx, const float v[4]) {
  if (is_f32(prec)) {
    *gmem(reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx)) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base);
    const uint32_t h01 = float2_to_bf16x2_bits(v[0], v[1]), h23 = float2_to_bf16x2_bits(v[2], v[3]);
    *gmem(reinterpret_cast<u32x2*>(p + idx)) = u32x2{h01, h23};
    if (prec == PREC_BF16X3) {
      const uint32_t l01 = float2_to_bf16x2_bits(v[0] - bf16_bits_to_float(h01), v[1] - bf16_bits_to_float(h01 >> 16));
      const uint32_t l23 = float2_to_bf16x2_bits(v[2] - bf16_bits_to_float(h23), v[3] - bf16_bits_to_float(h23 >> 16));
      *gmem(reinterpret_cast<u32x2*>(p + plane + idx)) = u32x2{l01, l23};
    }
  }
}

__device__ inline float load_ws(const void* base, int64_t plane, int prec, int64_t idx) {
  if (is_f32(prec)) return gmem(reinterpret_cast<const float*>(base))[idx];
  auto p = gmem(reinterpret_cast<const uint16_t*>(base));
  float v = bf16_bits_to_float(p[idx]);
  if (prec == PREC_BF16X3) v = v + bf16_bits_to_float(p[plane + idx]);
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace

// mode 0: momentum step; mode 1: U = G (Newton-Schulz only); mode 2: norms
// only (no workspace stores).
__global__ __launch_bounds__(256) void momentum_kernel(const MatDev* __restrict__ mats,
                                                       const int32_t* __restrict__ etile_off,
                                                       int32_t count, float beta, int32_t nesterov,
                                                       int32_t ema, int32_t mode, float* __restrict__ partials) {
  __shared__ float tile[ETILE][ETILE + 1];
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int mi = find_matrix(etile_off, count, b);
  const MatDev& md = mats[mi];
  const int local = b - etile_off[mi];
  const int tr0 = (local / md.etile_cols) * ETILE;   // natural row of the tile
  const int tc0 = (local % md.etile_cols) * ETILE;   // natural col of the tile
  const int tid = threadIdx.x;
  const int cg = tid & 15;
  const int rg = tid >> 4;
  const int rows = md.rows, cols = md.cols;
  const int prec = md.prec;
  const bool tr = md.transposed != 0;
  // X = U (wide) or X = U^T (tall), row stride ldx
  void* xw = md.X[0];
  const int64_t ldx = md.ldx;
  float ss = 0.f;

#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int rl = rg + 16 * p;
    const int row = tr0 + rl;
    const int col = tc0 + 4 * cg;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (row < rows && col < cols) {
      float g[4] = {0.f, 0.f, 0.f, 0.f}, m[4] = {0.f, 0.f, 0.f, 0.f};
      const bool full = md.vec_ok && (col + 3 < cols);
      const int64_t gi = int64_t(row) * md.ld_grad + col;
      if (full) {
        if (md.grad_bf16) {
          const u32x2 raw = __builtin_nontemporal_load(
              gmem(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(md.grad) + gi)));
          g[0] = bf16_bits_to_float(raw[0] & 0xFFFFu);
          g[1] = bf16_bits_to_float(raw[0] >> 16);
          g[2] = bf16_bits_to_float(raw[1] & 0xFFFFu);
          g[3] = bf16_bits_to_float(raw[1] >> 16);
        } else {
          const f32x4 raw = __builtin_nontemporal_load(
              gmem(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(md.grad) + gi)));
          g[0] = raw[0]; g[1] = raw[1]; g[2] = raw[2]; g[3] = raw[3];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < cols) g[e] = load_elem(md.grad, gi + e, md.grad_bf16);
      }
      if (mode == 0) {
        const int64_t mi64 = int64_t(row) * md.ld_mom + col;
        if (full) {
          const f32x4 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4*>(md.mom + mi64)));
          m[0] = raw[0]; m[1] = raw[1]; m[2] = raw[2]; m[3] = raw[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < cols) m[e] = gmem(md.mom)[mi64 + e];
        }
        float mn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // binary32, one rounding per operation (contraction is off here);
          // EMA form: the gradient enters as fl32((1 - beta) * g)
          const float gi = ema ? (1.f - beta) * g[e] : g[e];
          const float bm = beta * m[e];
          mn[e] = bm + gi;
          const float bn = beta * mn[e];
          u[e] = nesterov ? (gi + bn) : mn[e];
        }
        if (full) {
          __builtin_nontemporal_store(f32x4{mn[0], mn[1], mn[2], mn[3]},
                                      gmem(reinterpret_cast<f32x4*>(md.mom + mi64)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < cols) gmem(md.mom)[mi64 + e] = mn[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = g[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) if (col + e >= cols) u[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += u[e] * u[e];
    if (mode != 2) {
      if (!tr) {
        store4_ws(xw, md.plane_X, prec, int64_t(row) * ldx + col, u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[rl][4 * cg + e] = u[e];
      }
    }
  }

  if (mode != 2 && tr) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j = rg + 16 * p;          // natural column within the tile
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[4 * cg + e][j];
      store4_ws(xw, md.plane_X, prec, int64_t(tc0 + j) * ldx + tr0 + 4 * cg, v);
    }
  }

  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) partials[b] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void norm_finalize_kernel(const int32_t* __restrict__ etile_off,
                                                            const float* __restrict__ partials,
                                                            MatScal* __restrict__ scal,
                                                            float* __restrict__ norms_out) {
  __shared__ float red[4];
  const int mi = blockIdx.x;
  const int beg = etile_off[mi], end = etile_off[mi + 1];
  float s = 0.f;
  for (int i = beg + threadIdx.x; i < end; i += 256) s += partials[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float nrm = sqrtf(tot);
    const float inv = 1.0f / (nrm + 1e-7f);
    MatScal o;
    o.inv = inv;
    o.inv2 = inv * inv;
    o.norm = nrm;
    o.pad = 0.f;
    scal[mi] = o;
    if (norms_out) norms_out[mi] = nrm;
  }
}

__global__ __launch_bounds__(256) void writeback_direct_kernel(const MatDev* __restrict__ mats,
                                                               const int32_t* __restrict__ etile_off,
                                                               int32_t count,
                                                               const MatScal* __restrict__ scal,
                                                               float lr, int32_t scale_rule,
                                                               const float2* __restrict__ wb) {
  const int b = blockIdx.x;
  const int mi = find_matrix(etile_off, count, b);
  const MatDev& md = mats[mi];
  const int local = b - etile_off[mi];
  const int tr0 = (local / md.etile_cols) * ETILE;
  const int tc0 = (local % md.etile_cols) * ETILE;
  const bool tr = md.transposed != 0;
  const void* xw = md.X[0];
  const float inv = scal[mi].inv;
  const float t = wb ? wb[mi].x : update_scale(lr, scale_rule, md.rows, md.cols);
  const float d = wb ? wb[mi].y : 1.f;
  for (int e = threadIdx.x; e < ETILE * ETILE; e += 256) {
    const int row = tr0 + e / ETILE, col = tc0 + e % ETILE;
    if (row >= md.rows || col >= md.cols) continue;
    const int64_t xi = tr ? int64_t(col) * md.ldx + row : int64_t(row) * md.ldx + col;
    const float o = inv * load_ws(xw, md.plane_X, md.prec, xi);
    if (md.param) {
      const int64_t pi = int64_t(row) * md.ld_param + col;
      if (md.param_bf16) {
        auto pw = gmem(reinterpret_cast<uint16_t*>(md.param));
        const float w = bf16_bits_to_float(pw[pi]);
        pw[pi] = float_to_bf16_bits(w * d - t * o);
      } else {
        auto pw = gmem(reinterpret_cast<float*>(md.param));
        pw[pi] = pw[pi] * d - t * o;
      }
    }
    if (md.upd) gmem(md.upd)[int64_t(row) * md.ld_upd + col] = o;
  }
}

hipError_t launch_momentum(const MatDev* mats, const int32_t* etile_off, int32_t count,
                           int64_t total_tiles, float beta, int32_t nesterov, int32_t ema, int32_t mode,
                           float* partials, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(momentum_kernel, dim3(unsigned(total_tiles)), dim3(256), 0, stream, mats,
                     etile_off, count, beta, nesterov, ema, mode, partials);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const int32_t* etile_off, int32_t count, const float* partials,
                                MatScal* scal, float* norms_out, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(unsigned(count)), dim3(256), 0, stream, etile_off,
                     partials, scal, norms_out);
  return hipGetLastError();
}

hipError_t launch_writeback_direct(const MatDev* mats, const int32_t* etile_off, int32_t count,
                                   int64_t total_tiles, const MatScal* scal, float lr,
                                   int32_t scale_rule, const float2* wb, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(writeback_direct_kernel, dim3(unsigned(total_tiles)), dim3(256), 0, stream,
                     mats, etile_off, count, scal, lr, scale_rule, wb);
  return hipGetLastError();
}

}  // namespace muon
