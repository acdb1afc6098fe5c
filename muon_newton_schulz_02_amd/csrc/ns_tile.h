// Tile code of the Newton-Schulz products shared by the per-phase grids
// (ns_gemm.hip) and the persistent chain (ns_chain.hip): operand staging,
// the MFMA k-loop and the epilogues of one output tile.  Each including
// file gets its own copy (anonymous namespace), so the per-phase kernels
// are compiled exactly as if the chain did not exist.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "muon_internal.h"
#include "numeric.h"

#pragma clang fp contract(off)

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Loads through address space 1 compile to global_load (counted by vmcnt
// only); generic pointers give flat loads, which also count in lgkmcnt and
// so make every LDS wait also wait for the in-flight global loads.
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;

constexpr int KB = 128;     // bytes of K per operand row per stage
constexpr int PITCH = 144;  // LDS row pitch in bytes

// Element size and the number of planes a k-step stages together: the
// pipelined split-bf16 tiles stage one plane at a time (each product is three
// bf16 products over K, one per pair of planes), the one-stage split-bf16
// tiles both planes of a k-step.
template <int PREC> struct Fmt;
template <> struct Fmt<PREC_BF16> { static constexpr int esz = 2, spl = 1; };
template <> struct Fmt<PREC_BF16X3> { static constexpr int esz = 2, spl = 1; };
template <> struct Fmt<PREC_F32> { static constexpr int esz = 4, spl = 1; };
template <> struct Fmt<PREC_BF16S> { static constexpr int esz = 2, spl = 1; };
template <> struct Fmt<PREC_F32S> { static constexpr int esz = 4, spl = 1; };
template <> struct Fmt<PREC_BF16X3S> { static constexpr int esz = 2, spl = 2; };

// Tile shape per format: T x T tile, WP x WQ waves (rows x columns), NT threads.
// bf16 and split-bf16: 256 x 256 over eight waves (two per SIMD, each
// 128 x 64, 128 accumulator registers), so one wave's barrier or LDS wait
// overlaps the other's matrix-core work.  float32 and the small-stack tiles
// use 128 x 128 over four waves (small-stack float32: 64 x 64 over two).
// The 256 x 256 tiles run the software-pipelined k-loop with their own LDS
// layout (and transposed-operand block order); the others stage one k-step
// at a time in the swizzled layout.
constexpr bool pipelined(int prec) { return prec == PREC_BF16 || prec == PREC_BF16X3; }

template <int PREC> struct Cfg;
template <> struct Cfg<PREC_BF16> { static constexpr int BT = 256, WP = 2, WQ = 4, NT = 512; };
template <> struct Cfg<PREC_BF16X3> { static constexpr int BT = 256, WP = 2, WQ = 4, NT = 512; };
template <> struct Cfg<PREC_BF16X3S> { static constexpr int BT = 128, WP = 2, WQ = 2, NT = 256; };
template <> struct Cfg<PREC_F32> { static constexpr int BT = 128, WP = 2, WQ = 2, NT = 256; };
template <> struct Cfg<PREC_BF16S> { static constexpr int BT = 128, WP = 2, WQ = 2, NT = 256; };
// small-stack binary32: 64 x 64 over two waves of 32 x 64
template <> struct Cfg<PREC_F32S> { static constexpr int BT = 64, WP = 2, WQ = 1, NT = 128; };

// LDS operand layout of the one-stage tiles: row r at r * PITCH, 16-byte
// chunk ch at 16 (ch ^ ((r >> 4) & 7)).  (The pipelined tiles use their own,
// unswizzled layout.)
__device__ __forceinline__ int lds_off(int r, int ch) { return r * PITCH + ((ch ^ ((r >> 4) & 7)) << 4); }

// Workgroup barrier for LDS reuse only: this wave's LDS accesses complete,
// then s_barrier.  Unlike __syncthreads it does not wait for global stores
// in flight, so a tile's output drains while the next tile loads; no tile of
// a launch reads what another tile of that launch writes.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ storage

// Four consecutive values of the working format at element idx (a multiple
// of 4); the split-bf16 format keeps its lo plane `plane` elements further.
template <int PREC>
__device__ __forceinline__ void st4(void* base, int64_t plane, int64_t idx, const float* v) {
  if constexpr (is_f32(PREC)) {
    *gmem(reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx)) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base);
    const uint32_t h01 = float2_to_bf16x2_bits(v[0], v[1]), h23 = float2_to_bf16x2_bits(v[2], v[3]);
    *gmem(reinterpret_cast<u32x2*>(p + idx)) = u32x2{h01, h23};
    if constexpr (is_split(PREC)) {
      const uint32_t l01 = float2_to_bf16x2_bits(v[0] - bf16_bits_to_float(h01), v[1] - bf16_bits_to_float(h01 >> 16));
      const uint32_t l23 = float2_to_bf16x2_bits(v[2] - bf16_bits_to_float(h23), v[3] - bf16_bits_to_float(h23 >> 16));
      *gmem(reinterpret_cast<u32x2*>(p + plane + idx)) = u32x2{l01, l23};
    }
  }
}

// W[row][col] <- rnd(W*d - t*o) (each operation rounded to binary32; d = 1
// without weight decay, and W*1 = W exactly), and the optional binary32
// export of o.
__device__ __forceinline__ void write_back1(const MatDev& md, int row, int col, float o, float t, float d) {
  if (md.param) {
    const int64_t pi = int64_t(row) * md.ld_param + col;
    if (md.param_bf16) {
      auto pw = gmem(reinterpret_cast<uint16_t*>(md.param) + pi);
      *pw = float_to_bf16_bits(bf16_bits_to_float(*pw) * d - t * o);
    } else {
      auto pw = gmem(reinterpret_cast<float*>(md.param) + pi);
      *pw = *pw * d - t * o;
    }
  }
  if (md.upd) *gmem(md.upd + int64_t(row) * md.ld_upd + col) = o;
}

// The same for W[row][c0 .. c0+NE-1] (NE = 4 or 8, c0 a multiple of NE),
// columns below ncols only.  wvec_ok promises 16-byte aligned rows.
template <int NE>
__device__ __forceinline__ void write_back_n(const MatDev& md, int row, int c0, int ncols, const float* o,
                                             float t, float d) {
  const int cnt = ncols - c0;
  if (cnt <= 0) return;
  if (cnt >= NE && md.wvec_ok) {
    const int64_t pi = int64_t(row) * md.ld_param + c0;
    if (md.param) {
      if (md.param_bf16) {
        auto pw = gmem(reinterpret_cast<uint16_t*>(md.param) + pi);
        uint32_t raw[NE / 2];
        if constexpr (NE == 8) {
          const u32x4 r4 = *reinterpret_cast<__attribute__((address_space(1))) const u32x4*>(pw);
          raw[0] = r4[0]; raw[1] = r4[1]; raw[2] = r4[2]; raw[3] = r4[3];
        } else {
          const u32x2 r2 = *reinterpret_cast<__attribute__((address_space(1))) const u32x2*>(pw);
          raw[0] = r2[0]; raw[1] = r2[1];
        }
#pragma unroll
        for (int e = 0; e < NE / 2; ++e) {
          const float w0 = bf16_bits_to_float(raw[e] & 0xFFFFu), w1 = bf16_bits_to_float(raw[e] >> 16);
          raw[e] = float2_to_bf16x2_bits(w0 * d - t * o[2 * e], w1 * d - t * o[2 * e + 1]);
        }
        if constexpr (NE == 8) {
          *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(pw) = u32x4{raw[0], raw[1], raw[2], raw[3]};
        } else {
          *reinterpret_cast<__attribute__((address_space(1))) u32x2*>(pw) = u32x2{raw[0], raw[1]};
        }
      } else {
        auto pw = gmem(reinterpret_cast<f32x4*>(reinterpret_cast<float*>(md.param) + pi));
#pragma unroll
        for (int h = 0; h < NE / 4; ++h) {
          f32x4 w = pw[h];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = w[e] * d - t * o[4 * h + e];
          pw[h] = w;
        }
      }
    }
    if (md.upd) {
      auto pu = gmem(md.upd + int64_t(row) * md.ld_upd + c0);
      if (md.uvec_ok) {
#pragma unroll
        for (int h = 0; h < NE / 4; ++h)
          reinterpret_cast<__attribute__((address_space(1))) f32x4*>(pu)[h] = f32x4{o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) pu[e] = o[e];
      }
    }
    return;
  }
  for (int e = 0; e < NE && e < cnt; ++e) write_back1(md, row, c0 + e, o[e], t, d);
}

// Read-modify-write of PER 8-element runs of W per thread (run k: chunk
// tid + NT k), their binary32 update values in LDS.  run(q, so, row, col,
// rok, ncols) names run q: LDS float offset, W row and first column, whether
// the row exists, and the column count.  For bf16 W with 16-byte aligned rows
// and no update export, the loads of B runs go out before their stores, so
// their latencies overlap (a load is not moved above an earlier store to the
// same array by the compiler).
template <int PER, int B, int NT, class Run>
__device__ __forceinline__ void write_back_runs(const MatDev& md, const float* stg, int tid, float t, float d, Run run) {
  static_assert(PER % B == 0, "batches");
  const bool fast = md.param != nullptr && md.param_bf16 && md.wvec_ok && md.upd == nullptr;
#pragma unroll 1
  for (int k0 = 0; k0 < PER; k0 += B) {
    u32x4 w[B];
    bool full[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      int so, row, col, ncols;
      bool rok;
      run(tid + NT * (k0 + k), so, row, col, rok, ncols);
      full[k] = fast && rok && col + 8 <= ncols;
      if (full[k])
        w[k] = *gmem(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(md.param) +
                                                    int64_t(row) * md.ld_param + col));
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      int so, row, col, ncols;
      bool rok;
      run(tid + NT * (k0 + k), so, row, col, rok, ncols);
      if (!rok) continue;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(stg + so);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(stg + so + 4);
      const float o[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      if (full[k]) {
        uint32_t raw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w0 = bf16_bits_to_float(w[k][e] & 0xFFFFu), w1 = bf16_bits_to_float(w[k][e] >> 16);
          raw[e] = float2_to_bf16x2_bits(w0 * d - t * o[2 * e], w1 * d - t * o[2 * e + 1]);
        }
        *gmem(reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(md.param) + int64_t(row) * md.ld_param + col)) =
            u32x4{raw[0], raw[1], raw[2], raw[3]};
      } else {
        write_back_n<8>(md, row, col, ncols, o, t, d);
      }
    }
  }
}

// ------------------------------------------------------------------ MFMA

// acc += A operand (Q side) x B operand (P side) over one k-slab.
template <int PREC>
__device__ __forceinline__ void mfma_step(f32x16& acc, const u32x4* q, const u32x4* p) {
  if constexpr (bf16_single(PREC)) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[0]),
                                                   __builtin_bit_cast(bf16x8, p[0]), acc, 0, 0, 0);
  } else if constexpr (is_split(PREC)) {
    // small cross terms first, then hi*hi
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[1]),
                                                   __builtin_bit_cast(bf16x8, p[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[0]),
                                                   __builtin_bit_cast(bf16x8, p[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[0]),
                                                   __builtin_bit_cast(bf16x8, p[0]), acc, 0, 0, 0);
  } else {
    const f32x4 fq = __builtin_bit_cast(f32x4, q[0]);
    const f32x4 fp = __builtin_bit_cast(f32x4, p[0]);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fq.x, fp.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fq.y, fp.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fq.z, fp.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fq.w, fp.w, acc, 0, 0, 0);
  }
}

// A P-side fragment of alpha * I for one k-slab: this lane's values are the
// k-values of one row; `pos` is the index of the diagonal entry among them
// (outside the range: none).  For the bf16 formats alpha is split into
// hi + lo bf16 values: out[0] carries hi, out[1] lo.
template <int PREC>
__device__ __forceinline__ void identity_frag(u32x4* out, int pos, float alpha) {
  if constexpr (is_f32(PREC)) {
    const uint32_t bits = __float_as_uint(alpha);
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (pos == e) ? bits : 0u;
    out[0] = v;
  } else {
    const uint32_t hi = float_to_bf16_bits(alpha);
    const uint32_t lo = float_to_bf16_bits(alpha - bf16_bits_to_float(hi));
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      const uint32_t bits = pl == 0 ? hi : lo;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (pos == 2 * e ? bits : 0u) | (pos == 2 * e + 1 ? (bits << 16) : 0u);
      out[pl] = v;
    }
  }
}

template <int PREC>
__device__ __forceinline__ void mfma_identity(f32x16& acc, const u32x4* q, const u32x4* id) {
  if constexpr (bf16_single(PREC)) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[0]),
                                                   __builtin_bit_cast(bf16x8, id[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[0]),
                                                   __builtin_bit_cast(bf16x8, id[0]), acc, 0, 0, 0);
  } else {
    mfma_step<PREC>(acc, q, id);
  }
}

// ------------------------------------------------------------------ staging

// Staging geometry of one operand of a T x T tile for one stage (KB bytes of K).
//   direct: the operand's rows are K-contiguous; chunk c = tid + NT q is
//           row c / 8, 16-byte chunk c % 8.  CH chunks per thread.
//   trans:  the operand's element (row r, k) sits at memory (k, r), row
//           stride ld.  A block is 4 consecutive k-values of RPB = 16 / esz
//           consecutive rows: four 16-byte loads, transposed in registers into
//           4 k-values per row (8 bytes for bf16: half an LDS chunk; 16 bytes
//           for float32: a whole chunk).  NB blocks per stage, PER per thread.
template <int ESZ, int BT, int NT>
struct Geo {
  static constexpr int CH = BT * (KB / 16) / NT;
  static constexpr int RPB = 16 / ESZ;
  static constexpr int RB = BT / RPB;
  static constexpr int KG = KB / ESZ / 4;
  static constexpr int NB = RB * KG;
  static constexpr int PER = (NB + NT - 1) / NT;
  static constexpr int NREG = (CH > PER * 4) ? CH : PER * 4;
};

// Where one operand of one tile comes from.
struct OpSrc {
  const char* direct;      // its row 0, k = 0 (direct layout); null if never direct
  const char* trans;       // memory element (k = 0, its row 0) of the transposed layout
  int64_t ld_b;            // row stride in bytes (both layouts)
  int64_t plane_b;         // bytes between the hi and lo planes
  int sym_tile;            // symmetric operand: its tile-row index; -1: fixed layout
  int always_trans;        // COMB's X operand
  // tiled bf16 (one buffer resource at `direct`, the matrix): byte offsets
  // of the direct and transposed origins, and from one 256-k block of the
  // transposed layout to the next
  int org_d, org_t, kblk_t;
};

// Buffer resources over the two layouts of an operand: loads then take a
// 32-bit per-thread offset (the same every stage) and a scalar stage offset,
// with no per-load address arithmetic.  Word 3 = 0x00020000: raw 32-bit
// data, no swizzle; the record count covers any workspace matrix.
struct OpRsrc {
  __amdgpu_buffer_rsrc_t direct, trans;
};
__device__ __forceinline__ OpRsrc op_rsrc(const OpSrc& s) {
  constexpr int RECORDS = 0x7FFFFFFF;
  return {__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(s.direct), 0, RECORDS, 0x00020000),
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(s.trans), 0, RECORDS, 0x00020000)};
}

template <int ESZ, int BT>
__device__ __forceinline__ bool stage_is_trans(const OpSrc& s, int kt) {
  if (s.always_trans) return true;
  if (s.sym_tile < 0) return false;
  return (kt * (KB / ESZ)) / BT < s.sym_tile;  // below the diagonal: read the mirror block
}

// The same choice for operand OPD (0: P, 1: Q) of a product, with what the
// phase fixes decided at compile time: GRAM reads rows of X only, COMBINE's
// iterate is read along its columns only.
template <int PHASE, int OPD, int ESZ, int BT>
__device__ __forceinline__ bool op_trans(const OpSrc& s, int kt) {
  if constexpr (PHASE == PH_GRAM) return false;
  else if constexpr (PHASE == PH_COMB && OPD == 1) return true;
  else return (kt * (KB / ESZ)) / BT < s.sym_tile;
}

// The pipelined split-bf16 tiles run a product as three bf16 products over
// K, one per segment of the k-loop: segment 0 pairs the lo plane of Q with
// the hi plane of P, segment 1 hi with lo, segment 2 hi with hi (the small
// cross terms first).  The plane (0: hi, 1: lo) operand OPD takes in segment seg.
constexpr int split_plane(int opd, int seg) { return opd == 0 ? (seg == 1 ? 1 : 0) : (seg == 0 ? 1 : 0); }

// Loads number I0 .. I1 - 1 of this thread's loads of one operand of stage kt
// (numbered q * 4 + e for the transposed layout, q for the direct one).  Both
// layouts take NREG loads per thread; the layout is selected per load (buffer
// resource, scalar and per-thread offset), not branched on: loads issued in
// two branches into the same registers make the compiler wait for them at the
// join.
template <int ESZ, int BT, int NT, int NPL, int NREG, int I0 = 0, int I1 = 1 << 20>
__device__ __forceinline__ void load_stage(u32x4 (&r)[NPL][NREG], const OpSrc& s, const OpRsrc& rs, int kt,
                                           int tid) {
  using G = Geo<ESZ, BT, NT>;
  static_assert(G::PER == 1 && G::CH == 4 && NREG == 4 && G::NB == NT, "one block or four chunks per thread");
  const bool tr = stage_is_trans<ESZ, BT>(s, kt);
  const __amdgpu_buffer_rsrc_t rsrc = tr ? rs.trans : rs.direct;
  const int ld = int(s.ld_b);
  // transposed: block (row block rb, k-group kg), loads e = 0..3 are memory
  // rows 4 kg + e, 16 bytes at row block rb (consecutive threads, consecutive
  // row blocks); direct: chunk tid + NT i is row tid / 8 + (NT / 8) i,
  // 16-byte chunk tid % 8
  const int rb = tid % G::RB, kg = tid / G::RB;
  const int off = tr ? (kg * 4) * ld + rb * 16 : (tid >> 3) * ld + (tid & 7) * 16;
  const int step = tr ? ld : (NT / 8) * ld;
  const int sbase = tr ? kt * (KB / ESZ) * ld : kt * KB;
#pragma unroll
  for (int i = 0; i < NREG; ++i) {
    if (i < I0 || i >= I1) continue;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      r[pl][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, sbase + i * step + pl * int(s.plane_b), 0));
  }
}

// Operand OPD (0: P, 1: Q) of stage kt into registers, in the form the
// tile's k-loop stages it; the pipelined split-bf16 tiles take plane pl of it
// (0: hi, 1: lo; the other formats stage every plane and ignore pl).
template <int PREC, int PHASE, int OPD>
__device__ __forceinline__ void load_operand(u32x4 (&r)[Fmt<PREC>::spl][4], const OpSrc& s, const OpRsrc& rs, int kt,
                                             int tid, int pl) {
  constexpr int ESZ = Fmt<PREC>::esz, BT = Cfg<PREC>::BT, NT = Cfg<PREC>::NT;
  if constexpr (pipelined(PREC)) {
    // row form (chunk tid + NT i: row tid / 8 + (NT / 8) i, 16 bytes at 16 (tid % 8))
    // or k-row form (k-row tid / 32 + (NT / 32) i, 16 bytes at 16 (tid % 32))
    static_assert(ESZ == 2 && BT * 2 == 32 * 16, "bf16 256-wide stages");
    // tiled buffers (ws_index): 512-byte rows; stage kt is quarter kt % 4 of
    // k-block kt / 4, the next tile of a direct operand's tile row or the
    // next tile row (kblk_t bytes on) of a transposed one
    const bool tr = op_trans<PHASE, OPD, ESZ, BT>(s, kt);
    constexpr int ld = 512;
    const int off = tr ? (tid >> 5) * ld + (tid & 31) * 16 : (tid >> 3) * ld + (tid & 7) * 16;
    const int step = tr ? (NT / 32) * ld : (NT / 8) * ld;
    int sbase = tr ? s.org_t + (kt >> 2) * s.kblk_t + (kt & 3) * ((KB / 2) * ld)
                   : s.org_d + (kt >> 2) * WS_TILE_STRIDE + (kt & 3) * KB;
    if constexpr (PREC == PREC_BF16X3) sbase += pl ? int(s.plane_b) : 0;
    const __amdgpu_buffer_rsrc_t rsrc = rs.direct;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[0][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, sbase + i * step, 0));
  } else {
    load_stage<ESZ, BT, NT, Fmt<PREC>::spl, 4>(r, s, rs, kt, tid);
  }
}

// 4 x 8 transpose of 16-bit values: in[e] holds k-value e of 8 consecutive
// rows (two rows per dword); out[c] holds the 4 k-values of row c.
__device__ __forceinline__ void transpose4x8_b16(const u32x4* in, u32x2* out) {
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) {
    const uint32_t k0 = in[0][c2], k1 = in[1][c2], k2 = in[2][c2], k3 = in[3][c2];
    out[2 * c2] = u32x2{__builtin_amdgcn_perm(k1, k0, 0x05040100u), __builtin_amdgcn_perm(k3, k2, 0x05040100u)};
    out[2 * c2 + 1] = u32x2{__builtin_amdgcn_perm(k1, k0, 0x07060302u), __builtin_amdgcn_perm(k3, k2, 0x07060302u)};
  }
}

template <int ESZ, int BT, int NT, int NPL, int NREG, int OPB>
__device__ __forceinline__ void store_stage(const u32x4 (&r)[NPL][NREG], const OpSrc& s, int kt, char* lds,
                                            int tid) {
  using G = Geo<ESZ, BT, NT>;
  if (stage_is_trans<ESZ, BT>(s, kt)) {
#pragma unroll
    for (int q = 0; q < G::PER; ++q) {
      const int blk = tid + NT * q;
      if (G::NB % NT != 0 && blk >= G::NB) break;
      const int rb = blk % G::RB, kg = blk / G::RB;
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        if constexpr (ESZ == 2) {
          u32x2 t[8];
          transpose4x8_b16(&r[pl][q * 4], t);
#pragma unroll
          for (int c = 0; c < 8; ++c)
            *reinterpret_cast<u32x2*>(lds + pl * OPB + lds_off(rb * 8 + c, kg >> 1) + ((kg & 1) << 3)) = t[c];
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4*>(lds + pl * OPB + lds_off(rb * 4 + c, kg)) =
                u32x4{r[pl][q * 4 + 0][c], r[pl][q * 4 + 1][c], r[pl][q * 4 + 2][c], r[pl][q * 4 + 3][c]};
        }
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < G::CH; ++q) {
      const int c = tid + NT * q;
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) *reinterpret_cast<u32x4*>(lds + pl * OPB + lds_off(c >> 3, c & 7)) = r[pl][q];
    }
  }
}

// Store a bf16 output tile (BT x BT at `out`, row stride ld bytes) through
// LDS: every lane's four consecutive columns go to LDS as 8 bytes, then each
// 32 lanes write 512 contiguous bytes of one row (stores straight from the
// accumulators would put 16 bytes into each of 32 rows per instruction).
// The k-loop has ended with a barrier, so the operand stages are free.
// Plane PL of two values in the bf16 working formats: 0 the bf16 rounding
// (hi), 1 the bf16 rounding of what hi leaves (lo).
template <int PL>
__device__ __forceinline__ uint32_t bf16x2_plane(float a, float b) {
  const uint32_t h = float2_to_bf16x2_bits(a, b);
  if constexpr (PL == 0) return h;
  else return float2_to_bf16x2_bits(a - bf16_bits_to_float(h), b - bf16_bits_to_float(h >> 16));
}

template <int FQ, int FP, int WTP, int WTQ, int BT, int NT, int LDSB, int PL = 0>
__device__ __forceinline__ void store_tile_bf16(const f32x16 (&acc)[FQ][FP], float sc, char* out, int64_t ld,
                                                char* smem, int wp, int wq, int lane, int tid) {
  constexpr int EP = BT * 2 + 16;  // staging pitch in bytes
  static_assert(BT * EP <= LDSB, "staging does not fit");
  // This thread's staging and store addresses are formed here, from a fresh
  // copy of its index: formed before the k-loop, they were kept in scratch
  // memory, and reloading them made the stores wait for every load in flight
  // (the next tile's first stage included).
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid));
  const int ln = t & 63, hsel = ln >> 5;
#pragma clang loop unroll(full)
  for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
    for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
      for (int g = 0; g < 4; ++g) {
        const int r = wp * WTP + 32 * i + (ln & 31), c = wq * WTQ + 32 * j + 8 * g + 4 * hsel;
        const f32x16& a = acc[j][i];
        *reinterpret_cast<u32x2*>(smem + r * EP + c * 2) =
            u32x2{bf16x2_plane<PL>(sc * a[4 * g], sc * a[4 * g + 1]),
                  bf16x2_plane<PL>(sc * a[4 * g + 2], sc * a[4 * g + 3])};
      }
  lds_barrier();
  constexpr int CPR = BT * 2 / 16;  // 16-byte chunks per row
  static_assert((BT * CPR) % NT == 0, "whole chunks per thread");
#pragma clang loop unroll(full)
  for (int k = 0; k < BT * CPR / NT; ++k) {
    const int q = t + k * NT;
    const int r = q / CPR, c16 = q % CPR;
    *gmem(reinterpret_cast<u32x4*>(out + int64_t(r) * ld + c16 * 16)) = *reinterpret_cast<const u32x4*>(smem + r * EP + c16 * 16);
  }
}

// ------------------------------------------------------------------ tile

// The two operand sources of tile (ti, tj) of one phase; returns K.
template <int PREC, int PHASE>
__device__ __forceinline__ int tile_ops(const MatDev& md, int ti, int tj, const PhaseArgs& pa, OpSrc& sp, OpSrc& sq) {
  constexpr int ESZ = Fmt<PREC>::esz;
  constexpr int BT = Cfg<PREC>::BT;
  if constexpr (pipelined(PREC)) {
    // tiled buffers (ws_index): rows of 512 bytes inside a tile; the k-blocks
    // of a direct operand are consecutive tiles of its tile row, those of a
    // transposed one consecutive tile rows of its tile column
    constexpr int TB = WS_TILE_STRIDE;
    const int tpx = md.ldx >> 8, tpa = md.lda >> 8;
    if constexpr (PHASE == PH_GRAM) {
      const char* x = reinterpret_cast<const char*>(md.X[pa.cur]);
      sp = {x, nullptr, 512, md.plane_X * 2, -1, 0, ti * tpx * TB, 0, 0};
      sq = {x, nullptr, 512, md.plane_X * 2, -1, 0, tj * tpx * TB, 0, 0};
      return md.Np;
    } else if constexpr (PHASE == PH_POLY) {
      const char* a = reinterpret_cast<const char*>(md.A);
      sp = {a, nullptr, 512, md.plane_A * 2, ti, 0, ti * tpa * TB, ti * TB, tpa * TB};
      sq = {a, nullptr, 512, md.plane_A * 2, tj, 0, tj * tpa * TB, tj * TB, tpa * TB};
      return md.Mp;
    } else {
      const char* b = reinterpret_cast<const char*>(md.B);
      const char* x = reinterpret_cast<const char*>(md.X[pa.cur]);
      sp = {b, nullptr, 512, md.plane_A * 2, ti, 0, ti * tpa * TB, ti * TB, tpa * TB};
      sq = {x, nullptr, 512, md.plane_X * 2, -1, 1, 0, tj * TB, tpx * TB};
      return md.Mp;
    }
  } else if constexpr (PHASE == PH_GRAM) {
    const char* x = reinterpret_cast<const char*>(md.X[pa.cur]);
    const int64_t ld = int64_t(md.ldx) * ESZ;
    sp = {x + int64_t(ti) * BT * ld, nullptr, ld, md.plane_X * ESZ, -1, 0, 0, 0, 0};
    sq = {x + int64_t(tj) * BT * ld, nullptr, ld, md.plane_X * ESZ, -1, 0, 0, 0, 0};
    return md.Np;
  } else if constexpr (PHASE == PH_POLY) {
    const char* a = reinterpret_cast<const char*>(md.A);
    const int64_t ld = int64_t(md.lda) * ESZ;
    // blocks below the diagonal are read through their mirror block
    sp = {a + int64_t(ti) * BT * ld, a + int64_t(ti) * BT * ESZ, ld, md.plane_A * ESZ, ti, 0, 0, 0, 0};
    sq = {a + int64_t(tj) * BT * ld, a + int64_t(tj) * BT * ESZ, ld, md.plane_A * ESZ, tj, 0, 0, 0, 0};
    return md.Mp;
  } else {
    const char* b = reinterpret_cast<const char*>(md.B);
    const char* x = reinterpret_cast<const char*>(md.X[pa.cur]);
    const int64_t lda = int64_t(md.lda) * ESZ, ldx = int64_t(md.ldx) * ESZ;
    sp = {b + int64_t(ti) * BT * lda, b + int64_t(ti) * BT * ESZ, lda, md.plane_A * ESZ, ti, 0, 0, 0, 0};
    sq = {nullptr, x + int64_t(tj) * BT * ESZ, ldx, md.plane_X * ESZ, -1, 1, 0, 0, 0};
    return md.Mp;
  }
}

// VAR: GRAM 1 = c != 0 (store A), 0 = c == 0 (store B = b A);
//      COMB 1 = last step (write-back), 0 = store the next iterate.
//
// rp / rq hold this thread's part of the tile's stage 0 on entry (loaded
// while the previous tile finished); during the last stage they receive the
// next tile's stage 0 (when has_next), whose operand sources are np / nq.
template <int PREC, int PHASE, int VAR, int NREG, typename NEXT>
__device__ __forceinline__ void ns_tile_body(const MatDev& md, const MatScal* __restrict__ scal, int mat,
                                             int ti, int tj, const PhaseArgs& pa, char* smem,
                                             u32x4 (&rp)[Fmt<PREC>::spl][NREG], u32x4 (&rq)[Fmt<PREC>::spl][NREG],
                                             const NEXT& next) {
  constexpr int ESZ = Fmt<PREC>::esz;
  constexpr int NPL = Fmt<PREC>::spl;
  constexpr int BT = Cfg<PREC>::BT, NT = Cfg<PREC>::NT, WQN = Cfg<PREC>::WQ;
  using G = Geo<ESZ, BT, NT>;
  constexpr int WTP = BT / Cfg<PREC>::WP;  // wave tile rows (P side)
  constexpr int WTQ = BT / WQN;            // wave tile columns (Q side)
  constexpr int FP = WTP / 32, FQ = WTQ / 32;  // 32x32 MFMA blocks per wave
  constexpr int OPB = BT * PITCH;          // LDS bytes of one operand plane
  constexpr int STAGE = 2 * NPL * OPB;
  constexpr int KE = KB / ESZ;             // k-values per stage
  constexpr int KS = ESZ == 2 ? 16 : 8;    // k-values per MFMA slab
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wq = w % WQN, wp = w / WQN;    // wave position: Q side (columns), P side (rows)

  OpSrc sp, sq;
  const int K = tile_ops<PREC, PHASE>(md, ti, tj, pa, sp, sq);
  const int nk = K / KE;
  const OpRsrc rsp = op_rsrc(sp), rsq = op_rsrc(sq);

  // additive term alpha * D on the tile's own rows (POLY: (b/c) A, COMB: a X)
  constexpr bool ADD = PHASE != PH_GRAM;
  const float alpha = PHASE == PH_POLY ? pa.b / pa.c : pa.a;
  const int prow0 = ti * BT + wp * WTP;    // first P-side (output) row of this wave

  static_assert(NREG == G::NREG, "staging registers");
  f32x16 acc[FQ][FP];                       // [fj][fi]
#pragma clang loop unroll(full)
  for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
    for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

  const int hsel = lane >> 5;
  // 256 x 256 tiles: software-pipelined k-loop (below); the others: one stage at a time.
  constexpr bool PIPE = pipelined(PREC);
  static_assert(!PIPE || (KE / KS == 4 && G::NREG == 4 && G::PER == 1 && G::CH == 4 && NPL == 1), "pipelined geometry");
  if constexpr (PIPE) {
    // Per stage kt (LDS buffer kt & 1), four k-slabs; slab s runs its MFMAs on
    // fragment set F[s & 1] while the LDS reads of slab s + 1 fill the other
    // set, so matrix-core and LDS work overlap inside each wave.  Stage kt + 1
    // goes into the other buffer from registers during slabs 0-2 (P: halves in
    // slabs 0 and 1, Q: slabs 1 and 2), the registers then take stage kt + 2
    // from memory (P after slab 1, Q after slab 2), and one barrier after slab
    // 2 publishes stage kt + 1, whose first slab is read during slab 3.  The
    // barrier also ends every read of this stage's buffer before the next
    // stage starts overwriting it.  The last two stages load the next tile's
    // stage 0 instead (or, without a next tile, this tile's again, unused).
    //
    // LDS: P buffer b at b OPB, Q buffer b at (2 + b) OPB, so that with the
    // buffer fixed at compile time (stages unrolled by two; nk is a multiple
    // of 4) every fragment address is one per-lane register plus an
    // immediate.  Operand row r sits at r * PITCH, its 16-byte k-chunk ch at
    // 16 ch, unswizzled: the LDS serves a ds_read_b128 in four groups of 16
    // lanes (lanes 0-31 and 32-63 apart; within each half, the lanes whose
    // index bits 2-4 have even parity, then odd), and a fragment read (32
    // consecutive rows, one chunk per half-wave) at this 144-byte pitch puts
    // every group on 16 distinct bank quads: 4.5 clk per instruction, against
    // 8 when rows 16-31 take other chunks than rows 0-15 (measured).
    //
    // Operands read along their memory columns (COMBINE's iterate, and the
    // blocks of A and B below the diagonal, read through their mirror block)
    // are staged in k-row form, chosen per stage: LDS row k holds the stage's
    // k-row as in memory (512 bytes) at a KP = 576-byte pitch, stored with
    // whole-row loads and ds_write_b128, and their fragments come from
    // ds_read_b64_tr_b16, which
    // gives lane j of each 16-lane group element j % 4 of the 8 bytes read by
    // lane 4 e + j / 4 of the group as its value e: with lane 4 e + m pointing
    // at k-row k0 + e, columns n0 + 4 m .. + 3, lane j receives k-values
    // k0 .. k0 + 3 of column n0 + j.  The 16 lanes of a read cover 4 rows x 32
    // bytes, the 32 lanes of a half-wave 4 rows x 64 bytes: distinct banks at
    // this pitch.
    constexpr int NF = FQ + FP;
    constexpr int QOFF = 2 * OPB;
    constexpr int KP = 576;
    static_assert(2 * QOFF <= 2 * STAGE && KE * KP <= OPB, "LDS layout");
    u32x4 F[2][NF];
    char* const lds = smem;
    // per-lane fragment offsets: row form (32 rows, one chunk per half-wave)
    // and k-row form (ds_read_b64_tr_b16: lane 4 e + m of each 16-lane group
    // points at k-row e, columns 4 m .. 4 m + 3 of its 16)
    const int kfr = (8 * hsel + ((lane & 15) >> 2)) * KP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    const int fragP = (wp * WTP + (lane & 31)) * PITCH + hsel * 16;
    const int fragPk = kfr + 2 * wp * WTP;
    // POLY, whose two operands both change form along k, derives Q's fragment
    // addresses from P's plus a wave-uniform offset at each use (an opaque
    // scalar copy keeps the sums out of registers): two vector registers fewer
    // kept its k-loop free of spills.  GRAM and COMBINE keep them precomputed.
    constexpr bool QDERIVED = PHASE == PH_POLY;
    const int qdr = __builtin_amdgcn_readfirstlane(QOFF + (wq * WTQ - wp * WTP) * PITCH);
    const int qdk = __builtin_amdgcn_readfirstlane(QOFF + 2 * (wq * WTQ - wp * WTP));
    const int fragQ0 = QOFF + (wq * WTQ + (lane & 31)) * PITCH + hsel * 16;
    const int fragQk0 = QOFF + kfr + 2 * wq * WTQ;
    const int stD = (tid >> 3) * PITCH + (tid & 7) * 16;               // row-form chunk tid, + q (NT / 8) rows
    const int stK = (tid >> 5) * KP + (tid & 31) * 16;                 // k-row piece tid, + i (NT / 32) k-rows
    auto read_frags = [&](u32x4 (&f)[NF], auto buf_c, int ks, bool ptr, bool qtr) {
      constexpr int BUF = decltype(buf_c)::value;
      int fragQ = fragQ0, fragQk = fragQk0;
      if constexpr (QDERIVED) {
        int qd, qk;
        asm volatile("s_mov_b32 %0, %2\n\ts_mov_b32 %1, %3" : "=s"(qd), "=s"(qk) : "s"(qdr), "s"(qdk));
        fragQ = fragP + qd;
        fragQk = fragPk + qk;
      }
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 ls16x4;
      typedef __attribute__((address_space(3))) char lchar;
      auto tr_pair = [&](int off) {
        lchar* a = (lchar*)(lds + off);
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)a));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)(a + 4 * KP)));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      if (qtr) {
#pragma clang loop unroll(full)
        for (int x = 0; x < FQ; ++x) f[x] = tr_pair(fragQk + BUF * OPB + x * 64 + ks * 16 * KP);
      } else {
#pragma clang loop unroll(full)
        for (int x = 0; x < FQ; ++x)
          f[x] = *reinterpret_cast<const u32x4*>(lds + fragQ + BUF * OPB + x * 32 * PITCH + ks * 32);
      }
      if (ptr) {
#pragma clang loop unroll(full)
        for (int x = 0; x < FP; ++x) f[FQ + x] = tr_pair(fragPk + BUF * OPB + x * 64 + ks * 16 * KP);
      } else {
#pragma clang loop unroll(full)
        for (int x = 0; x < FP; ++x)
          f[FQ + x] = *reinterpret_cast<const u32x4*>(lds + fragP + BUF * OPB + x * 32 * PITCH + ks * 32);
      }
    };
    auto mfma_half = [&](const u32x4 (&f)[NF], int h) {
#pragma clang loop unroll(full)
      for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
        for (int i = 2 * h; i < 2 * h + 2; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f[j]),
                                                              __builtin_bit_cast(bf16x8, f[FQ + i]), acc[j][i], 0, 0, 0);
    };
    // split-bf16: NSEG = 3 segments of nk stages each (split_plane); loop
    // stage g is stage kin(g) of segment segof(g)
    constexpr int NSEG = PREC == PREC_BF16X3 ? 3 : 1;
    const int NK = NSEG * nk;
    auto segof = [&](int g) { return NSEG == 1 ? 0 : (g >= 2 * nk ? 2 : (g >= nk ? 1 : 0)); };
    auto kin = [&](int g) { return g - segof(g) * nk; };
    // the additive term pairs alpha I with Q's hi plane and with its lo plane
    // once each: in segments 0 and 2, not in segment 1 (Q hi again)
    auto identity_add = [&](const u32x4 (&f)[NF], int g, int ks) {
      if constexpr (ADD) {
        if (NSEG > 1 && segof(g) == 1) return;
        const int kk = kin(g) * KE + ks * KS;
        const int d = kk - prow0;
        if (d >= 0 && d < WTP) {
          const int fi = d >> 5;
          const int pos = (lane & 31) - (d & 31) - (KS / 2) * hsel;
          u32x4 id[2];
          identity_frag<PREC>(id, pos, alpha);
#pragma clang loop unroll(full)
          for (int i = 0; i < FP; ++i)
            if (i == fi) {
#pragma clang loop unroll(full)
              for (int j = 0; j < FQ; ++j) mfma_identity<PREC_BF16>(acc[j][i], &f[j], id);
            }
        }
      }
    };
    // half H of one operand's part of stage kt, from registers to LDS at byte
    // offset BASE (the operand's buffer), in row or k-row form
    auto store_half = [&](const u32x4 (&r)[NPL][G::NREG], const OpSrc& src, int kt, auto base_c, auto h_c) {
      constexpr int BASE = decltype(base_c)::value;
      constexpr int H = decltype(h_c)::value;
      const bool tr = op_trans<PHASE, (BASE >= QOFF ? 1 : 0), ESZ, BT>(src, kin(kt));
#pragma unroll
      for (int i = 2 * H; i < 2 * H + 2; ++i) {
        const int off = tr ? stK + i * (NT / 32) * KP : stD + i * (NT / 8) * PITCH;
        *reinterpret_cast<u32x4*>(lds + BASE + off) = r[0][i];
      }
    };
    // the next tile's sources (or, without a next tile, this tile's), formed
    // just before the last two stages load from them
    OpSrc xp, xq;
    OpRsrc rxp, rxq;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    store_half(rp, sp, 0, I0{}, I0{});
    store_half(rp, sp, 0, I0{}, I1{});
    store_half(rq, sq, 0, std::integral_constant<int, QOFF>{}, I0{});
    store_half(rq, sq, 0, std::integral_constant<int, QOFF>{}, I1{});
    lds_barrier();
    load_operand<PREC, PHASE, 0>(rp, sp, rsp, kin(1), tid, split_plane(0, segof(1)));
    load_operand<PREC, PHASE, 1>(rq, sq, rsq, kin(1), tid, split_plane(1, segof(1)));
    auto ktrP = [&](int g) { return op_trans<PHASE, 0, ESZ, BT>(sp, kin(g)); };
    auto ktrQ = [&](int g) { return op_trans<PHASE, 1, ESZ, BT>(sq, kin(g)); };
    read_frags(F[0], I0{}, 0, ktrP(0), ktrQ(0));

    // MODE 0: store stage kt + 1, load stage kt + 2 of this tile; 1: store
    // stage kt + 1, load the next tile's stage 0; 2: the last stage.
    auto stage = [&](const int kt, auto buf_c, auto mode_c) {
      constexpr int BUF = decltype(buf_c)::value;
      constexpr int MODE = decltype(mode_c)::value;
      using CUR = std::integral_constant<int, BUF>;
      using NXT = std::integral_constant<int, BUF ^ 1>;
      using NP = std::integral_constant<int, (BUF ^ 1) * OPB>;
      using NQ = std::integral_constant<int, QOFF + (BUF ^ 1) * OPB>;
      // slab 0
      const bool ptr = ktrP(kt), qtr = ktrQ(kt);
      read_frags(F[1], CUR{}, 1, ptr, qtr);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[0], 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2) store_half(rp, sp, kt + 1, NP{}, I0{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[0], 1);
      identity_add(F[0], kt, 0);
      __builtin_amdgcn_sched_barrier(0);
      // slab 1
      read_frags(F[0], CUR{}, 2, ptr, qtr);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[1], 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2) {
        store_half(rp, sp, kt + 1, NP{}, I1{});
        store_half(rq, sq, kt + 1, NQ{}, I0{});
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[1], 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == 0) load_operand<PREC, PHASE, 0>(rp, sp, rsp, kin(kt + 2), tid, split_plane(0, segof(kt + 2)));
      if constexpr (MODE == 1) load_operand<PREC, PHASE, 0>(rp, xp, rxp, 0, tid, split_plane(0, 0));
      __builtin_amdgcn_sched_barrier(0);
      identity_add(F[1], kt, 1);
      __builtin_amdgcn_sched_barrier(0);
      // slab 2
      read_frags(F[1], CUR{}, 3, ptr, qtr);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[0], 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2) store_half(rq, sq, kt + 1, NQ{}, I1{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[0], 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == 0) load_operand<PREC, PHASE, 1>(rq, sq, rsq, kin(kt + 2), tid, split_plane(1, segof(kt + 2)));
      if constexpr (MODE == 1) load_operand<PREC, PHASE, 1>(rq, xq, rxq, 0, tid, split_plane(1, 0));
      __builtin_amdgcn_sched_barrier(0);
      identity_add(F[0], kt, 2);
      lds_barrier();
      // slab 3
      if constexpr (MODE != 2) read_frags(F[0], NXT{}, 0, ktrP(kt + 1), ktrQ(kt + 1));
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F[1], 0);
      mfma_half(F[1], 1);
      identity_add(F[1], kt, 3);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll 1
    for (int kt = 0; kt + 2 < NK; kt += 2) {
      stage(kt, I0{}, I0{});
      stage(kt + 1, I1{}, I0{});
    }
    if (!next(xp, xq)) {
      xp = sp;
      xq = sq;
    }
    rxp = op_rsrc(xp);
    rxq = op_rsrc(xq);
    stage(NK - 2, I0{}, I1{});
    stage(NK - 1, I1{}, std::integral_constant<int, 2>{});
    lds_barrier();
  } else {
    store_stage<ESZ, BT, NT, NPL, G::NREG, OPB>(rp, sp, 0, smem, tid);
    store_stage<ESZ, BT, NT, NPL, G::NREG, OPB>(rq, sq, 0, smem + NPL * OPB, tid);
    lds_barrier();

    // The loads of stage kt + 1 go out in two halves, P's before k-slab 0 and
    // Q's before k-slab 1 (bf16: four slabs), not in one burst: a burst of 64
    // loads per workgroup stalls every wave at issue, while loads issued in the
    // last slabs leave too little time before the stage's LDS stores.
    constexpr bool SPREAD = PREC == PREC_BF16 && KE / KS == 4 && G::NREG == 4;
    // One stage of the k-loop.  MORE: stage kt + 1 follows and is loaded; else
    // (the last stage) the loads fetch the next tile's stage 0, if any, which
    // then lands while this tile's epilogue runs.
    OpSrc np, nq;                            // the next tile's sources (last stage)
    OpRsrc rnp, rnq;
    bool has_next = false;
    auto stage = [&](const int kt, auto more_c) {
      constexpr bool MORE = decltype(more_c)::value;
      const int s = kt & 1;
      const bool ld = MORE || has_next;
      const int kl = MORE ? kt + 1 : 0;
      const OpSrc& lp_ = MORE ? sp : np;
      const OpSrc& lq_ = MORE ? sq : nq;
      const OpRsrc& rlp = MORE ? rsp : rnp;
      const OpRsrc& rlq = MORE ? rsq : rnq;
      if (!SPREAD && ld) {
        load_stage<ESZ, BT, NT, NPL, G::NREG>(rp, lp_, rlp, kl, tid);
        load_stage<ESZ, BT, NT, NPL, G::NREG>(rq, lq_, rlq, kl, tid);
      }
      const char* lP = smem + s * STAGE;
      const char* lQ = lP + NPL * OPB;
  #pragma clang loop unroll(full)
      for (int ks = 0; ks < KE / KS; ++ks) {
        if constexpr (SPREAD) {
          // the scheduling barriers keep the loads here: left free, the
          // scheduler sinks them to the LDS stores at the end of the stage
          if (ks == 0 && ld) load_stage<ESZ, BT, NT, NPL, G::NREG>(rp, lp_, rlp, kl, tid);
          if (ks == 1 && ld) load_stage<ESZ, BT, NT, NPL, G::NREG>(rq, lq_, rlq, kl, tid);
          if (ks < 2) __builtin_amdgcn_sched_barrier(0);
        }
        const int ch = 2 * ks + hsel;           // this lane's 16-byte chunk of the slab
        u32x4 qf[FQ][NPL], pf[FP][NPL];
  #pragma clang loop unroll(full)
        for (int f = 0; f < FQ; ++f) {
          const int rq_ = wq * WTQ + f * 32 + (lane & 31);
  #pragma clang loop unroll(full)
          for (int pl = 0; pl < NPL; ++pl)
            qf[f][pl] = *reinterpret_cast<const u32x4*>(lQ + pl * OPB + lds_off(rq_, ch));
        }
  #pragma clang loop unroll(full)
        for (int f = 0; f < FP; ++f) {
          const int rp_ = wp * WTP + f * 32 + (lane & 31);
  #pragma clang loop unroll(full)
          for (int pl = 0; pl < NPL; ++pl)
            pf[f][pl] = *reinterpret_cast<const u32x4*>(lP + pl * OPB + lds_off(rp_, ch));
        }
  #pragma clang loop unroll(full)
        for (int j = 0; j < FQ; ++j)
  #pragma clang loop unroll(full)
          for (int i = 0; i < FP; ++i) mfma_step<PREC>(acc[j][i], qf[j], pf[i]);
        if constexpr (ADD) {
          // the k-slab [kk, kk + KS) meets the output rows of this wave's block fi
          const int kk = kt * KE + ks * KS;
          const int d = kk - prow0;
          if (d >= 0 && d < WTP) {
            const int fi = d >> 5;
            // this lane's row within the block is lane & 31; its k-values are
            // kk + (KS / 2) h + e
            const int pos = (lane & 31) - (d & 31) - (KS / 2) * hsel;
            u32x4 id[2];
            identity_frag<PREC>(id, pos, alpha);
  #pragma clang loop unroll(full)
            for (int i = 0; i < FP; ++i)
              if (i == fi) {
  #pragma clang loop unroll(full)
                for (int j = 0; j < FQ; ++j) mfma_identity<PREC>(acc[j][i], qf[j], id);
              }
          }
        }
      }
      if constexpr (MORE) {
        store_stage<ESZ, BT, NT, NPL, G::NREG, OPB>(rp, sp, kt + 1, smem + (s ^ 1) * STAGE, tid);
        store_stage<ESZ, BT, NT, NPL, G::NREG, OPB>(rq, sq, kt + 1, smem + (s ^ 1) * STAGE + NPL * OPB, tid);
      }
      lds_barrier();
    };
  #pragma unroll 1
    for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, std::true_type{});
    has_next = next(np, nq);
    if (has_next) {
      rnp = op_rsrc(np);
      rnq = op_rsrc(nq);
    }
    stage(nk - 1, std::false_type{});
  }

  // ---------------------------------------------------------------- epilogue
  // acc[fj][fi][4g + e] is output row ti*BT + wp*WTP + 32 fi + (lane & 31),
  // output column tj*BT + wq*WTQ + 32 fj + 8g + 4h + e.
  const int orow = ti * BT + wp * WTP + (lane & 31);
  const int ocol = tj * BT + wq * WTQ + 4 * hsel;
  if constexpr ((PHASE == PH_GRAM || PHASE == PH_POLY) && pipelined(PREC)) {
    char* out = reinterpret_cast<char*>((PHASE == PH_GRAM && VAR == 1) ? md.A : md.B) +
                (int64_t(ti) * (md.lda >> 8) + tj) * WS_TILE_STRIDE;
    const float sc = PHASE == PH_POLY ? pa.c
                                      : (pa.first ? scal[mat].inv2 : 1.f) * (VAR == 1 ? 1.f : pa.b);
    store_tile_bf16<FQ, FP, WTP, WTQ, BT, NT, 2 * STAGE>(acc, sc, out, 512, smem, wp, wq, lane, tid);
    if constexpr (PREC == PREC_BF16X3) {    // the lo plane, staged through the same LDS
      lds_barrier();
      store_tile_bf16<FQ, FP, WTP, WTQ, BT, NT, 2 * STAGE, 1>(acc, sc, out + md.plane_A * 2, 512, smem, wp, wq, lane,
                                                              tid);
    }
  } else if constexpr (PHASE == PH_GRAM || PHASE == PH_POLY) {
    void* out = (PHASE == PH_GRAM && VAR == 1) ? md.A : md.B;
    const float sc = PHASE == PH_POLY ? pa.c
                                      : (pa.first ? scal[mat].inv2 : 1.f) * (VAR == 1 ? 1.f : pa.b);
#pragma clang loop unroll(full)
    for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
      for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma clang loop unroll(full)
          for (int e = 0; e < 4; ++e) v[e] = sc * acc[j][i][4 * g + e];
          st4<PREC>(out, md.plane_A, int64_t(orow + 32 * i) * md.lda + ocol + 32 * j + 8 * g, v);
        }
  } else {
    const float s = pa.first ? scal[mat].inv : 1.f;
    if constexpr (VAR == 0 && pipelined(PREC)) {
      char* xn = reinterpret_cast<char*>(md.X[pa.cur ^ 1]) + (int64_t(ti) * (md.ldx >> 8) + tj) * WS_TILE_STRIDE;
      store_tile_bf16<FQ, FP, WTP, WTQ, BT, NT, 2 * STAGE>(acc, s, xn, 512, smem, wp, wq, lane, tid);
      if constexpr (PREC == PREC_BF16X3) {
        lds_barrier();
        store_tile_bf16<FQ, FP, WTP, WTQ, BT, NT, 2 * STAGE, 1>(acc, s, xn + md.plane_X * 2, 512, smem, wp, wq, lane,
                                                                tid);
      }
    } else if constexpr (VAR == 0) {
      void* xn = md.X[pa.cur ^ 1];
#pragma clang loop unroll(full)
      for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
        for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma clang loop unroll(full)
            for (int e = 0; e < 4; ++e) v[e] = s * acc[j][i][4 * g + e];
            st4<PREC>(xn, md.plane_X, int64_t(orow + 32 * i) * md.ldx + ocol + 32 * j + 8 * g, v);
          }
    } else {
      // t = fl32(lr*s) and the decay factor d: per matrix from the host when
      // given (per-matrix lr or scale, weight decay), else from lr and the rule
      const float t = pa.wb ? pa.wb[mat].x : update_scale(pa.lr, pa.scale_rule, md.rows, md.cols);
      const float d = pa.wb ? pa.wb[mat].y : 1.f;
      if (md.transposed == 0) {
        // W = X': stage the binary32 update through LDS, one row of waves (RP
        // output rows = W rows) per pass, then read-modify-write 8-element
        // runs of W rows: 16-byte accesses, 512 bytes per 32 lanes.
        constexpr int RP = WTP;
        constexpr int NPASS = BT / RP;
        constexpr int SPN = BT + 4;           // staging pitch in floats: RP rows of BT floats
        static_assert(RP * SPN * 4 <= 2 * STAGE, "staging does not fit");
        float* stg = reinterpret_cast<float*>(smem);
#pragma unroll 1
        for (int pass = 0; pass < NPASS; ++pass) {
          if (wp == pass) {
#pragma clang loop unroll(full)
            for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
              for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
                for (int g = 0; g < 4; ++g) {
                  const int rl = 32 * i + (lane & 31), c = wq * WTQ + 32 * j + 8 * g + 4 * hsel;
                  const f32x16& a = acc[j][i];
                  *reinterpret_cast<f32x4*>(stg + rl * SPN + c) =
                      f32x4{s * a[4 * g], s * a[4 * g + 1], s * a[4 * g + 2], s * a[4 * g + 3]};
                }
          }
          lds_barrier();
          const int row_base = ti * BT + pass * RP;
          static_assert((RP * BT / 8) % NT == 0, "runs per thread");
          constexpr int PER = RP * BT / 8 / NT;
          write_back_runs<PER, (PER >= 4 ? 4 : PER), NT>(md, stg, tid, t, d,
                                                         [&](int q, int& so, int& row, int& col, bool& rok, int& ncols) {
            const int rl = q / (BT / 8), c8 = (q % (BT / 8)) * 8;
            so = rl * SPN + c8;
            row = row_base + rl;
            col = tj * BT + c8;
            rok = row < md.m;
            ncols = md.n;
          });
          lds_barrier();
        }
      } else {
        // W = X'^T: stage the binary32 update transposed through LDS, one row of
        // waves (RP output rows = W columns) per pass, then read-modify-write
        // 8-element runs of W rows: 16-byte accesses, 512 bytes per 32 lanes.
        constexpr int RP = WTP;               // output rows per pass
        constexpr int NPASS = BT / RP;
        constexpr int SPT = RP + 4;           // staging pitch in floats: BT rows of RP floats
        static_assert(BT * SPT * 4 <= 2 * STAGE, "staging does not fit");
        float* stg = reinterpret_cast<float*>(smem);
#pragma unroll 1
        for (int pass = 0; pass < NPASS; ++pass) {
          if (wp == pass) {
            const int rl = lane & 31;
#pragma clang loop unroll(full)
            for (int j = 0; j < FQ; ++j)
#pragma clang loop unroll(full)
              for (int i = 0; i < FP; ++i)
#pragma clang loop unroll(full)
                for (int g = 0; g < 4; ++g)
#pragma clang loop unroll(full)
                  for (int e = 0; e < 4; ++e) {
                    const int cl = wq * WTQ + 32 * j + 8 * g + 4 * hsel + e;
                    stg[cl * SPT + rl + 32 * i] = s * acc[j][i][4 * g + e];
                  }
          }
          lds_barrier();
          const int row_base = ti * BT + pass * RP;
          static_assert((BT * RP / 8) % NT == 0, "runs per thread");
          constexpr int PER = BT * RP / 8 / NT;
          write_back_runs<PER, (PER >= 4 ? 4 : PER), NT>(md, stg, tid, t, d,
                                                         [&](int q, int& so, int& row, int& col, bool& rok, int& ncols) {
            const int cl = q / (RP / 8), r8 = (q % (RP / 8)) * 8;
            so = cl * SPT + r8;
            row = tj * BT + cl;               // natural row = wide column
            col = row_base + r8;
            rok = row < md.n;
            ncols = md.m;
          });
          lds_barrier();
        }
      }
    }
  }
}

}  // namespace
}  // namespace muon
