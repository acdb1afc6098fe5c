// Elementwise and reduction kernels of the Muon step on gfx950.
//
//  * momentum_kernel: per element, in binary32 with one rounding per
//    operation, M <- beta*M + G and U <- G + beta*M (Nesterov) or U <- M;
//    stores U into the workspace in the wide orientation X (m x n, m <= n;
//    through an LDS transpose for tall matrices) in the Newton-Schulz storage
//    format, zero-filling the padding; writes one binary32 sum of u^2 per
//    tile (wavefront shuffles, then LDS across the four waves).
//    Tall matrices go through an LDS transpose, in 64 x 128 tiles staged as
//    bf16 for the bf16 working format (two 128-element row runs per wave and
//    load) and in 64 x 64 binary32 tiles for the others; the rest in 16 x 256
//    tiles, one 256-element row run per wave and instruction.
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
    if (is_split(prec)) {
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
  if (is_split(prec)) v = v + bf16_bits_to_float(p[plane + idx]);
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Momentum of four consecutive elements: M' = beta M + g_in, U = Nesterov ?
// g_in + beta M' : M', g_in = g (heavy ball) or fl32((1 - beta) g) (EMA), each
// operation rounded once in binary32 (contraction is off in this file).
__device__ inline void momentum4(const float* g, const float* m, float* mn, float* u, float beta, int nesterov,
                                 int ema) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float gi = ema ? (1.f - beta) * g[e] : g[e];
    const float bm = beta * m[e];
    mn[e] = bm + gi;
    const float bn = beta * mn[e];
    u[e] = nesterov ? (gi + bn) : mn[e];
  }
}

// The RTILE_R x RTILE_C tile (tr0, tc0) of a matrix iterated untransposed:
// wave w takes rows w, w + 4, w + 8, w + 12 and lane l the four columns from
// tc0 + 4 l, so every load and store instruction of a wave covers one
// contiguous run of a row (1 KB of M).  All four rows' loads are issued
// before any store.  Returns this thread's sum of u^2.
__device__ inline float momentum_rows(const MatDev& md, int tr0, int tc0, float beta, int32_t nesterov, int32_t ema,
                                      int32_t mode) {
  static_assert(RTILE_C == 4 * 64 && RTILE_R == 4 * 4, "four rows of one wave-wide run per wave");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = tc0 + 4 * lane;
  const int rows = md.rows, cols = md.cols;
  float g[4][4], m[4][4];
  bool live[4], full[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = tr0 + w + 4 * q;
    live[q] = row < rows && col < cols;
    full[q] = live[q] && md.vec_ok && col + 3 < cols;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[q][e] = m[q][e] = 0.f;
    const int64_t gi = int64_t(row) * md.ld_grad + col;
    const int64_t mi = int64_t(row) * md.ld_mom + col;
    if (full[q]) {
      if (md.grad_bf16) {
        const u32x2 raw = __builtin_nontemporal_load(
            gmem(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(md.grad) + gi)));
        g[q][0] = bf16_bits_to_float(raw[0] & 0xFFFFu);
        g[q][1] = bf16_bits_to_float(raw[0] >> 16);
        g[q][2] = bf16_bits_to_float(raw[1] & 0xFFFFu);
        g[q][3] = bf16_bits_to_float(raw[1] >> 16);
      } else {
        const f32x4 raw = __builtin_nontemporal_load(
            gmem(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(md.grad) + gi)));
        g[q][0] = raw[0]; g[q][1] = raw[1]; g[q][2] = raw[2]; g[q][3] = raw[3];
      }
      if (mode == 0) {
        const f32x4 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4*>(md.mom + mi)));
        m[q][0] = raw[0]; m[q][1] = raw[1]; m[q][2] = raw[2]; m[q][3] = raw[3];
      }
    } else if (live[q]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < cols) {
          g[q][e] = load_elem(md.grad, gi + e, md.grad_bf16);
          if (mode == 0) m[q][e] = gmem(md.mom)[mi + e];
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = tr0 + w + 4 * q;
    float mn[4], u[4];
    if (mode == 0) {
      momentum4(g[q], m[q], mn, u, beta, nesterov, ema);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = g[q][e];
    }
    // elements outside the matrix loaded as zero and stay zero: they fill
    // the workspace padding
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += u[e] * u[e];
    if (mode == 0 && live[q]) {
      const int64_t mi = int64_t(row) * md.ld_mom + col;
      if (full[q]) {
        __builtin_nontemporal_store(f32x4{mn[0], mn[1], mn[2], mn[3]}, gmem(reinterpret_cast<f32x4*>(md.mom + mi)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < cols) gmem(md.mom)[mi + e] = mn[e];
      }
    }
    if (mode != 2) store4_ws(md.X[0], md.plane_X, md.prec, ws_index(md.prec, row, col, md.ldx), u);
  }
  return ss;
}

// The TBF_R x TBF_C tile (tr0, tc0) of a tall matrix in the bf16 working
// format: thread (rg, cg) takes rows rg + RSTEP p (p = 0 .. 7, four at a
// time, loads before stores) and the four columns from tc0 + 4 cg (for
// 64 x 128, each wave load covers two 128-element row runs); u goes to LDS
// as bf16 (the rounding the workspace stores), then each X row (a natural
// column) leaves as one run of the tile's TBF_R natural rows, TBF_R / 4
// threads per row.  Returns this thread's sum of u^2.
__device__ inline float momentum_tall_bf16(const MatDev& md, int tr0, int tc0, float beta, int32_t nesterov,
                                           int32_t ema, int32_t mode, uint16_t (*t16)[TBF_C + 4]) {
  constexpr int CG = TBF_C / 4, RSTEP = 256 / CG;   // column groups of 4; row step between a thread's rows
  constexpr int CGO = TBF_R / 4, JSTEP = 256 / CGO;  // store side: groups of 4 natural rows; X-row step
  static_assert(TBF_R * TBF_C == 8 * 1024 && 8 * RSTEP == TBF_R && 8 * JSTEP == TBF_C, "8 rows, 8 stores a thread");
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int col = tc0 + 4 * cg;
  const int rows = md.rows, cols = md.cols;
  float ss = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float g[4][4], m[4][4];
    bool live[4], full[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = tr0 + rg + RSTEP * (4 * half + q);
      live[q] = row < rows && col < cols;
      full[q] = live[q] && md.vec_ok && col + 3 < cols;
#pragma unroll
      for (int e = 0; e < 4; ++e) g[q][e] = m[q][e] = 0.f;
      const int64_t gi = int64_t(row) * md.ld_grad + col;
      const int64_t mi = int64_t(row) * md.ld_mom + col;
      if (full[q]) {
        if (md.grad_bf16) {
          const u32x2 raw = __builtin_nontemporal_load(
              gmem(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(md.grad) + gi)));
          g[q][0] = bf16_bits_to_float(raw[0] & 0xFFFFu);
          g[q][1] = bf16_bits_to_float(raw[0] >> 16);
          g[q][2] = bf16_bits_to_float(raw[1] & 0xFFFFu);
          g[q][3] = bf16_bits_to_float(raw[1] >> 16);
        } else {
          const f32x4 raw = __builtin_nontemporal_load(
              gmem(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(md.grad) + gi)));
          g[q][0] = raw[0]; g[q][1] = raw[1]; g[q][2] = raw[2]; g[q][3] = raw[3];
        }
        if (mode == 0) {
          const f32x4 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4*>(md.mom + mi)));
          m[q][0] = raw[0]; m[q][1] = raw[1]; m[q][2] = raw[2]; m[q][3] = raw[3];
        }
      } else if (live[q]) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < cols) {
            g[q][e] = load_elem(md.grad, gi + e, md.grad_bf16);
            if (mode == 0) m[q][e] = gmem(md.mom)[mi + e];
          }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = rg + RSTEP * (4 * half + q);
      const int row = tr0 + rl;
      float u[4] = {0.f, 0.f, 0.f, 0.f};
      if (live[q]) {
        if (mode == 0) {
          float mn[4];
          momentum4(g[q], m[q], mn, u, beta, nesterov, ema);
          const int64_t mi = int64_t(row) * md.ld_mom + col;
          if (full[q]) {
            __builtin_nontemporal_store(f32x4{mn[0], mn[1], mn[2], mn[3]}, gmem(reinterpret_cast<f32x4*>(md.mom + mi)));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < cols) gmem(md.mom)[mi + e] = mn[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = g[q][e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) if (col + e >= cols) u[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += u[e] * u[e];
      if (mode != 2)
        *reinterpret_cast<u32x2*>(&t16[rl][4 * cg]) =
            u32x2{float2_to_bf16x2_bits(u[0], u[1]), float2_to_bf16x2_bits(u[2], u[3])};
    }
  }
  if (mode != 2) {
    __syncthreads();
    const int cgo = tid % CGO, jo = tid / CGO;
    uint16_t* xw = reinterpret_cast<uint16_t*>(md.X[0]);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int j = jo + JSTEP * p;       // natural column within the tile: X row tc0 + j
      const uint32_t v0 = t16[4 * cgo][j], v1 = t16[4 * cgo + 1][j], v2 = t16[4 * cgo + 2][j],
                     v3 = t16[4 * cgo + 3][j];
      *gmem(reinterpret_cast<u32x2*>(xw + ws_index(md.prec, tc0 + j, tr0 + 4 * cgo, md.ldx))) =
          u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
    }
  }
  return ss;
}

}  // namespace

// mode 0: momentum step; mode 1: U = G (Newton-Schulz only); mode 2: norms
// only (no workspace stores).
__global__ __launch_bounds__(256) void momentum_kernel(const MatDev* __restrict__ mats,
                                                       const int32_t* __restrict__ etile_off,
                                                       int32_t count, float beta, int32_t nesterov,
                                                       int32_t ema, int32_t mode, float* __restrict__ partials) {
  // the LDS of one tall tile: a 64 x 64 binary32 tile or a 64 x 128 bf16 one
  constexpr int TILE_LDS = TBF_R * (TBF_C + 4) * 2 > ETILE * (ETILE + 1) * 4 ? TBF_R * (TBF_C + 4) * 2
                                                                            : ETILE * (ETILE + 1) * 4;
  __shared__ __attribute__((aligned(16))) char tile_lds[TILE_LDS];
  float (*tile)[ETILE + 1] = reinterpret_cast<float (*)[ETILE + 1]>(tile_lds);
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int mi = find_matrix(etile_off, count, b);
  const MatDev& md = mats[mi];
  const int local = b - etile_off[mi];
  const int tid = threadIdx.x;
  if (!md.transposed) {
    const float ssr = wave_sum(momentum_rows(md, (local / md.etile_cols) * RTILE_R,
                                             (local % md.etile_cols) * RTILE_C, beta, nesterov, ema, mode));
    if ((tid & 63) == 0) red[tid >> 6] = ssr;
    __syncthreads();
    if (tid == 0) partials[b] = (red[0] + red[1]) + (red[2] + red[3]);
    return;
  }
  if (md.prec == PREC_BF16) {
    const float ssr = wave_sum(momentum_tall_bf16(md, (local / md.etile_cols) * TBF_R,
                                                  (local % md.etile_cols) * TBF_C, beta, nesterov, ema, mode,
                                                  reinterpret_cast<uint16_t (*)[TBF_C + 4]>(tile_lds)));
    if ((tid & 63) == 0) red[tid >> 6] = ssr;
    __syncthreads();
    if (tid == 0) partials[b] = (red[0] + red[1]) + (red[2] + red[3]);
    return;
  }
  const int tr0 = (local / md.etile_cols) * ETILE;   // natural row of the tile
  const int tc0 = (local % md.etile_cols) * ETILE;   // natural col of the tile
  const int cg = tid & 15;
  const int rg = tid >> 4;
  const int rows = md.rows, cols = md.cols;
  const int prec = md.prec;
  const bool tr = md.transposed != 0;
  // X = U (wide) or X = U^T (tall), row stride ldx
  void* xw = md.X[0];
  const int64_t ldx = md.ldx;
  float ss = 0.f;

  // all four rows' loads before any store (the stores would otherwise hold
  // back the next row's loads)
  float g[4][4], m[4][4];
  bool live[4], full[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = tr0 + rg + 16 * p;
    const int col = tc0 + 4 * cg;
    live[p] = row < rows && col < cols;
    full[p] = live[p] && md.vec_ok && (col + 3 < cols);
#pragma unroll
    for (int e = 0; e < 4; ++e) g[p][e] = m[p][e] = 0.f;
    const int64_t gi = int64_t(row) * md.ld_grad + col;
    const int64_t mi64 = int64_t(row) * md.ld_mom + col;
    if (full[p]) {
      if (md.grad_bf16) {
        const u32x2 raw = __builtin_nontemporal_load(
            gmem(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(md.grad) + gi)));
        g[p][0] = bf16_bits_to_float(raw[0] & 0xFFFFu);
        g[p][1] = bf16_bits_to_float(raw[0] >> 16);
        g[p][2] = bf16_bits_to_float(raw[1] & 0xFFFFu);
        g[p][3] = bf16_bits_to_float(raw[1] >> 16);
      } else {
        const f32x4 raw = __builtin_nontemporal_load(
            gmem(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(md.grad) + gi)));
        g[p][0] = raw[0]; g[p][1] = raw[1]; g[p][2] = raw[2]; g[p][3] = raw[3];
      }
      if (mode == 0) {
        const f32x4 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4*>(md.mom + mi64)));
        m[p][0] = raw[0]; m[p][1] = raw[1]; m[p][2] = raw[2]; m[p][3] = raw[3];
      }
    } else if (live[p]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < cols) {
          g[p][e] = load_elem(md.grad, gi + e, md.grad_bf16);
          if (mode == 0) m[p][e] = gmem(md.mom)[mi64 + e];
        }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int rl = rg + 16 * p;
    const int row = tr0 + rl;
    const int col = tc0 + 4 * cg;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (live[p]) {
      if (mode == 0) {
        float mn[4];
        momentum4(g[p], m[p], mn, u, beta, nesterov, ema);
        const int64_t mi64 = int64_t(row) * md.ld_mom + col;
        if (full[p]) {
          __builtin_nontemporal_store(f32x4{mn[0], mn[1], mn[2], mn[3]},
                                      gmem(reinterpret_cast<f32x4*>(md.mom + mi64)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < cols) gmem(md.mom)[mi64 + e] = mn[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = g[p][e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) if (col + e >= cols) u[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += u[e] * u[e];
    if (mode != 2) {
      if (!tr) {
        store4_ws(xw, md.plane_X, prec, ws_index(prec, row, col, ldx), u);
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
      store4_ws(xw, md.plane_X, prec, ws_index(prec, tc0 + j, tr0 + 4 * cg, ldx), v);
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
  const bool tr = md.transposed != 0;
  const bool tbf = tr && md.prec == PREC_BF16;
  const int th = tr ? (tbf ? TBF_R : ETILE) : RTILE_R, tw = tr ? (tbf ? TBF_C : ETILE) : RTILE_C;
  const int tr0 = (local / md.etile_cols) * th;
  const int tc0 = (local % md.etile_cols) * tw;
  const void* xw = md.X[0];
  const float inv = scal[mi].inv;
  const float t = wb ? wb[mi].x : update_scale(lr, scale_rule, md.rows, md.cols);
  const float d = wb ? wb[mi].y : 1.f;
  for (int e = threadIdx.x; e < th * tw; e += 256) {
    const int row = tr0 + e / tw, col = tc0 + e % tw;
    if (row >= md.rows || col >= md.cols) continue;
    const int64_t xi = tr ? ws_index(md.prec, col, row, md.ldx) : ws_index(md.prec, row, col, md.ldx);
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
