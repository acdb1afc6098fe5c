// Newton-Schulz matrix products on gfx950 MFMA, one grouped launch per
// phase over every matrix of the call.
//
// A polynomial Newton-Schulz step (N. J. Higham, Functions of Matrices,
// ch. 8; the Muon optimizer's orthogonalisation in "开发者千美元训3.8B模型
// 击败GPT-2", paragraph 影响) on a wide matrix X (m x n, m <= n) is three
// products, each written here as C = P Q^T with both operands read along
// their contiguous (K) dimension:
//
//   GRAM  A = s^2 * X X^T          P = Q = X (m x n), K = n; symmetric, so only
//                                  tiles on or above the diagonal run and each
//                                  stores itself and its mirror.
//   POLY  B = b A + c A A^T        P = Q = A (A is symmetric, A A = A A^T);
//                                  symmetric like GRAM; b A added in the
//                                  epilogue.  Skipped when c == 0.
//   COMB  X' = s (a X + B X)       P = B (or A when c == 0, with B X -> b A X),
//                                  Q = X^T (n x m), K = m.  The epilogue adds
//                                  a X and stores X' in both layouts (X' for
//                                  the next GRAM, X'^T for the next COMB); on
//                                  the last step it writes the update back
//                                  into the weight instead.
//
// s = 1/(||U||_F + eps) on the first step (the momentum kernel stores U
// unscaled) and 1 afterwards.
//
// Tiles: NS_TILE x NS_TILE outputs per 256-thread workgroup (four waves,
// 2 x 2, each NS_TILE/2 square), K staged 128 bytes per row at a time through
// double-buffered LDS with a 16-byte row pad.  Operands are zero-padded to a
// multiple of 256 in the workspace, so no load is predicated.  Tile lists
// are split into one contiguous, cost-balanced segment per XCD; workgroup b
// runs on XCD b % 8 and takes entry b / 8 of that XCD's segment, so tiles
// that share operand panels share an L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"
#include "numeric.h"

#pragma clang fp contract(off)

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KB = 128;     // bytes of K per operand row per stage
constexpr int PITCH = 144;  // LDS row pitch in bytes

template <int PREC> struct Fmt;
template <> struct Fmt<PREC_BF16> { static constexpr int esz = 2, npl = 1; };
template <> struct Fmt<PREC_BF16X3> { static constexpr int esz = 2, npl = 2; };
template <> struct Fmt<PREC_F32> { static constexpr int esz = 4, npl = 1; };

template <int PREC>
__device__ __forceinline__ float ld1(const void* base, int64_t plane, int64_t idx) {
  if constexpr (PREC == PREC_F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base);
    float v = bf16_bits_to_float(p[idx]);
    if constexpr (PREC == PREC_BF16X3) v = v + bf16_bits_to_float(p[plane + idx]);
    return v;
  }
}

template <int PREC>
__device__ __forceinline__ void st1(void* base, int64_t plane, int64_t idx, float v) {
  if constexpr (PREC == PREC_F32) {
    reinterpret_cast<float*>(base)[idx] = v;
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base);
    const uint16_t h = float_to_bf16_bits(v);
    p[idx] = h;
    if constexpr (PREC == PREC_BF16X3) p[plane + idx] = float_to_bf16_bits(v - bf16_bits_to_float(h));
  }
}

// four consecutive elements, idx a multiple of 4
template <int PREC>
__device__ __forceinline__ void st4(void* base, int64_t plane, int64_t idx, const float* v) {
  if constexpr (PREC == PREC_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base);
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = float_to_bf16_bits(v[e]);
    *reinterpret_cast<uint2*>(p + idx) =
        make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
    if constexpr (PREC == PREC_BF16X3) {
      uint16_t l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) l[e] = float_to_bf16_bits(v[e] - bf16_bits_to_float(h[e]));
      *reinterpret_cast<uint2*>(p + plane + idx) =
          make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
    }
  }
}

// eight consecutive elements, idx a multiple of 8
template <int PREC>
__device__ __forceinline__ void ld8(const void* base, int64_t plane, int64_t idx, float* v) {
  if constexpr (PREC == PREC_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
    const f32x4 a = p[0], b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base);
    const u32x4 h = *reinterpret_cast<const u32x4*>(p + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_bits_to_float(h[e] & 0xFFFFu);
      v[2 * e + 1] = bf16_bits_to_float(h[e] >> 16);
    }
    if constexpr (PREC == PREC_BF16X3) {
      const u32x4 l = *reinterpret_cast<const u32x4*>(p + plane + idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = v[2 * e] + bf16_bits_to_float(l[e] & 0xFFFFu);
        v[2 * e + 1] = v[2 * e + 1] + bf16_bits_to_float(l[e] >> 16);
      }
    }
  }
}

template <int PREC>
__device__ __forceinline__ void st8(void* base, int64_t plane, int64_t idx, const float* v) {
  if constexpr (PREC == PREC_F32) {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx);
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base);
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = float_to_bf16_bits(v[e]);
    u32x4 hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = uint32_t(h[2 * e]) | (uint32_t(h[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(p + idx) = hv;
    if constexpr (PREC == PREC_BF16X3) {
      u32x4 lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t l0 = float_to_bf16_bits(v[2 * e] - bf16_bits_to_float(h[2 * e]));
        const uint32_t l1 = float_to_bf16_bits(v[2 * e + 1] - bf16_bits_to_float(h[2 * e + 1]));
        lv[e] = l0 | (l1 << 16);
      }
      *reinterpret_cast<u32x4*>(p + plane + idx) = lv;
    }
  }
}

// W[row][c0 .. c0+7] <- rnd(W - t*o) for the columns below `ncols`, and the
// optional binary32 export of o.
__device__ __forceinline__ void write_back8(const MatDev& md, int row, int c0, int ncols, const float* o,
                                            float t) {
  const int cnt = ncols - c0;
  if (cnt <= 0) return;
  if (md.param) {
    const int64_t pi = int64_t(row) * md.ld_param + c0;
    if (md.param_bf16) {
      uint16_t* pw = reinterpret_cast<uint16_t*>(md.param) + pi;
      if (cnt >= 8 && md.wvec_ok) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(pw);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w0 = bf16_bits_to_float(raw[e] & 0xFFFFu);
          const float w1 = bf16_bits_to_float(raw[e] >> 16);
          raw[e] = uint32_t(float_to_bf16_bits(w0 - t * o[2 * e])) |
                   (uint32_t(float_to_bf16_bits(w1 - t * o[2 * e + 1])) << 16);
        }
        *reinterpret_cast<u32x4*>(pw) = raw;
      } else {
        for (int e = 0; e < 8 && e < cnt; ++e) pw[e] = float_to_bf16_bits(bf16_bits_to_float(pw[e]) - t * o[e]);
      }
    } else {
      float* pw = reinterpret_cast<float*>(md.param) + pi;
      if (cnt >= 8 && md.wvec_ok) {
        f32x4* q = reinterpret_cast<f32x4*>(pw);
        f32x4 a = q[0], b = q[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = a[e] - t * o[e];
          b[e] = b[e] - t * o[4 + e];
        }
        q[0] = a;
        q[1] = b;
      } else {
        for (int e = 0; e < 8 && e < cnt; ++e) pw[e] = pw[e] - t * o[e];
      }
    }
  }
  if (md.upd) {
    float* pu = md.upd + int64_t(row) * md.ld_upd + c0;
    if (cnt >= 8 && md.uvec_ok) {
      f32x4* q = reinterpret_cast<f32x4*>(pu);
      q[0] = f32x4{o[0], o[1], o[2], o[3]};
      q[1] = f32x4{o[4], o[5], o[6], o[7]};
    } else {
      for (int e = 0; e < 8 && e < cnt; ++e) pu[e] = o[e];
    }
  }
}

template <int PREC>
__device__ __forceinline__ void mfma_step(f32x16& acc, const u32x4* a, const u32x4* b) {
  if constexpr (PREC == PREC_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
  } else if constexpr (PREC == PREC_BF16X3) {
    // small cross terms first, then hi*hi
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[1]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
  } else {
    const f32x4 fa = __builtin_bit_cast(f32x4, a[0]);
    const f32x4 fb = __builtin_bit_cast(f32x4, b[0]);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc, 0, 0, 0);
  }
}

// Global -> registers: one stage (KB bytes of K) of BT rows, 16 bytes per
// chunk, eight chunks per row, chunk c = tid + 256*q.
template <int NPL, int CH, int ESZ>
__device__ __forceinline__ void load_tile(u32x4 (&r)[NPL][CH], const char* g, int64_t plane, int64_t ld,
                                          int kt, int tid) {
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int c = tid + 256 * q;
    const int64_t off = int64_t(c >> 3) * ld * ESZ + int64_t(kt) * KB + (c & 7) * 16;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      r[pl][q] = *reinterpret_cast<const u32x4*>(g + pl * plane * ESZ + off);
  }
}

// Registers -> LDS (row pitch PITCH; the planes of one operand follow each other).
template <int NPL, int CH>
__device__ __forceinline__ void store_tile(const u32x4 (&r)[NPL][CH], char* lds, int tid) {
  constexpr int OPB = CH * 32 * PITCH;  // CH*256/8 rows
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int c = tid + 256 * q;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      *reinterpret_cast<u32x4*>(lds + pl * OPB + (c >> 3) * PITCH + (c & 7) * 16) = r[pl][q];
  }
}

template <int PREC, int PHASE, int BT>
__global__ __launch_bounds__(256) void ns_gemm_kernel(const MatDev* __restrict__ mats,
                                                      const MatScal* __restrict__ scal,
                                                      const int2* __restrict__ tiles, PhaseArgs pa) {
  constexpr int ESZ = Fmt<PREC>::esz;
  constexpr int NPL = Fmt<PREC>::npl;
  constexpr int WT = BT / 2;               // wave tile edge
  constexpr int F = WT / 32;               // 32x32 MFMA blocks per wave edge
  constexpr int CH = BT * (KB / 16) / 256; // 16-byte chunks per thread, per operand plane
  constexpr int OPB = BT * PITCH;          // LDS bytes of one operand plane
  constexpr int STAGE = 2 * NPL * OPB;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int bid = blockIdx.x;
  const int2 te = tiles[(bid % NUM_XCD) * pa.per_xcd + bid / NUM_XCD];
  if (te.x < 0) return;
  const MatDev& md = mats[te.x];
  const int ti = te.y >> 16, tj = te.y & 0xFFFF;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;

  const char* Pg;
  const char* Qg;
  int64_t ldP, ldQ, planeP, planeQ;
  int K;
  if constexpr (PHASE == PH_GRAM) {
    Pg = Qg = reinterpret_cast<const char*>(md.X[pa.cur]);
    ldP = ldQ = md.Np;
    planeP = planeQ = md.plane_X;
    K = md.Np;
  } else if constexpr (PHASE == PH_POLY) {
    Pg = Qg = reinterpret_cast<const char*>(md.A);
    ldP = ldQ = md.Mp;
    planeP = planeQ = md.plane_A;
    K = md.Mp;
  } else {
    Pg = reinterpret_cast<const char*>(pa.c != 0.f ? md.B : md.A);
    Qg = reinterpret_cast<const char*>(md.Xt[pa.cur]);
    ldP = ldQ = md.Mp;
    planeP = md.plane_A;
    planeQ = md.plane_X;
    K = md.Mp;
  }
  Pg += int64_t(ti) * BT * ldP * ESZ;
  Qg += int64_t(tj) * BT * ldQ * ESZ;
  const int nk = K * ESZ / KB;

  u32x4 rP[NPL][CH], rQ[NPL][CH];
  f32x16 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  load_tile<NPL, CH, ESZ>(rP, Pg, planeP, ldP, 0, tid);
  load_tile<NPL, CH, ESZ>(rQ, Qg, planeQ, ldQ, 0, tid);
  store_tile<NPL, CH>(rP, smem, tid);
  store_tile<NPL, CH>(rQ, smem + NPL * OPB, tid);
  __syncthreads();

  const int frag_off = (lane & 31) * PITCH + (lane >> 5) * 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) {
      load_tile<NPL, CH, ESZ>(rP, Pg, planeP, ldP, kt + 1, tid);
      load_tile<NPL, CH, ESZ>(rQ, Qg, planeQ, ldQ, kt + 1, tid);
    }
    const char* sP = smem + s * STAGE;
    const char* sQ = sP + NPL * OPB;
#pragma unroll
    for (int ks = 0; ks < KB / 32; ++ks) {
      u32x4 af[F][NPL], bf[F][NPL];
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          af[f][pl] = *reinterpret_cast<const u32x4*>(sP + pl * OPB + (wm * WT + f * 32) * PITCH + ks * 32 + frag_off);
          bf[f][pl] = *reinterpret_cast<const u32x4*>(sQ + pl * OPB + (wn * WT + f * 32) * PITCH + ks * 32 + frag_off);
        }
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j) mfma_step<PREC>(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) {
      store_tile<NPL, CH>(rP, smem + (s ^ 1) * STAGE, tid);
      store_tile<NPL, CH>(rQ, smem + (s ^ 1) * STAGE + NPL * OPB, tid);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // The accumulators go through LDS (the loop above ended with a barrier, so
  // the operand tiles are dead) and leave in two passes of 16-byte accesses:
  // a row pass (tile rows, contiguous in the row-major output) and, where a
  // transposed copy is needed, a column pass (tile columns, contiguous in
  // the transposed output).
  constexpr int SP = BT + 4;              // staging pitch in floats
  static_assert(BT * SP * 4 <= 2 * STAGE, "staging tile does not fit");
  constexpr int TPR = BT / 8;             // threads per row, 8 elements each
  constexpr int RPP = 256 / TPR;          // rows per pass
  float* stg = reinterpret_cast<float*>(smem);
  {
    const int half = lane >> 5;
    const int lc = lane & 31;
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          stg[(wm * WT + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3)) * SP + wn * WT + j * 32 + lc] =
              acc[i][j][v];
  }
  __syncthreads();
  const int pr = tid / TPR;
  const int pc = (tid % TPR) * 8;
  const int gi_base = ti * BT, gj_base = tj * BT;

  if constexpr (PHASE == PH_GRAM || PHASE == PH_POLY) {
    const float gs = (PHASE == PH_GRAM && pa.first) ? scal[te.x].inv2 : 1.f;
    void* out = (PHASE == PH_GRAM) ? md.A : md.B;
    const int64_t ld = md.Mp;
    const bool mirror = ti != tj;
#pragma unroll 2
    for (int r = pr; r < BT; r += RPP) {
      float* sp = stg + r * SP + pc;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sp[e];
      const int64_t idx = int64_t(gi_base + r) * ld + gj_base + pc;
      if constexpr (PHASE == PH_GRAM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gs * v[e];
      } else {
        float av[8];
        ld8<PREC>(md.A, md.plane_A, idx, av);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = pa.b * av[e] + pa.c * v[e];
      }
      st8<PREC>(out, md.plane_A, idx, v);
      if (mirror) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sp[e] = v[e];
      }
    }
    if (mirror) {
      __syncthreads();
#pragma unroll 2
      for (int jl = pr; jl < BT; jl += RPP) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stg[(pc + e) * SP + jl];
        st8<PREC>(out, md.plane_A, int64_t(gj_base + jl) * ld + gi_base + pc, v);
      }
    }
  } else {
    const float s = pa.first ? scal[te.x].inv : 1.f;
    const float cb = (pa.c != 0.f) ? 1.f : pa.b;
    const void* xc = md.X[pa.cur];
    const int64_t ldx = md.Np, ldt = md.Mp;
    const bool tr = md.transposed != 0;
    const float t = update_scale(pa.lr, pa.scale_rule, md.rows, md.cols);
#pragma unroll 2
    for (int r = pr; r < BT; r += RPP) {
      float* sp = stg + r * SP + pc;
      const int gi = gi_base + r, gj = gj_base + pc;
      const int64_t idx = int64_t(gi) * ldx + gj;
      float xv[8], v[8];
      ld8<PREC>(xc, md.plane_X, idx, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = s * (pa.a * xv[e] + cb * sp[e]);
      if (!pa.last) {
        st8<PREC>(md.X[pa.cur ^ 1], md.plane_X, idx, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sp[e] = v[e];
      } else if (!tr) {
        if (gi < md.m) write_back8(md, gi, gj, md.n, v, t);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sp[e] = v[e];
      }
    }
    if (!pa.last || tr) {
      __syncthreads();
#pragma unroll 2
      for (int jl = pr; jl < BT; jl += RPP) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stg[(pc + e) * SP + jl];
        const int gj = gj_base + jl, gi = gi_base + pc;
        if (!pa.last) {
          st8<PREC>(md.Xt[pa.cur ^ 1], md.plane_X, int64_t(gj) * ldt + gi, v);
        } else if (gj < md.n) {
          // tall matrix: natural row gj, natural columns gi .. gi+7
          write_back8(md, gj, gi, md.m, v, t);
        }
      }
    }
  }
}

template <int PREC, int PHASE>
hipError_t launch_one(const MatDev* mats, const MatScal* scal, const int2* tiles,
                      const PhaseArgs& pa, hipStream_t stream) {
  const unsigned grid = unsigned(NUM_XCD) * unsigned(pa.per_xcd);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((ns_gemm_kernel<PREC, PHASE, NS_TILE>), dim3(grid), dim3(256), 0, stream,
                     mats, scal, tiles, pa);
  return hipGetLastError();
}

template <int PREC>
hipError_t launch_prec(int phase, const MatDev* mats, const MatScal* scal, const int2* tiles,
                       const PhaseArgs& pa, hipStream_t stream) {
  switch (phase) {
    case PH_GRAM: return launch_one<PREC, PH_GRAM>(mats, scal, tiles, pa, stream);
    case PH_POLY: return launch_one<PREC, PH_POLY>(mats, scal, tiles, pa, stream);
    case PH_COMB: return launch_one<PREC, PH_COMB>(mats, scal, tiles, pa, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ns_phase(int prec, int phase, const MatDev* mats, const MatScal* scal,
                           const int2* tiles, const PhaseArgs& args, hipStream_t stream) {
  switch (prec) {
    case PREC_BF16: return launch_prec<PREC_BF16>(phase, mats, scal, tiles, args, stream);
    case PREC_BF16X3: return launch_prec<PREC_BF16X3>(phase, mats, scal, tiles, args, stream);
    case PREC_F32: return launch_prec<PREC_F32>(phase, mats, scal, tiles, args, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
