// Newton-Schulz matrix products on gfx950 MFMA: one persistent, grouped
// launch per phase over every matrix of the call.
//
// A polynomial Newton-Schulz step (N. J. Higham, Functions of Matrices,
// ch. 8; the Muon optimizer's orthogonalisation in "开发者千美元训3.8B模型
// 击败GPT-2", paragraph 影响) on a wide matrix X (m x n, m <= n),
//
//     X' = a X + (b A + c A^2) X,   A = X X^T,
//
// is three products, each C[i][j] = sum_k P[i][k] Q[j][k] + alpha D[i][j]:
//
//   GRAM  A  = s^2 X X^T            P = Q = X (rows of X, K = n).  With c == 0
//                                   it stores B = b A instead and POLY is skipped.
//   POLY  B  = c (A A + (b/c) A)    P = Q = A (A symmetric), K = m.
//   COMB  X' = s (B X + a X)        P = B (symmetric), Q[j][k] = X[k][j], K = m.
//                                   The last step writes the update back into
//                                   the weight instead of storing X'.
//
// s = 1/(||U||_F + eps) on the first step (the momentum kernel stores U
// unscaled) and 1 afterwards.
//
// Design points:
//  * The MFMA A operand is the Q side and the B operand the P side, so each
//    lane's accumulators hold four consecutive output columns of one output
//    row: row-major outputs leave as 8-byte stores, and no transposed copy of
//    any matrix is kept.
//  * A and B are symmetric, so GRAM and POLY compute and store only the tiles
//    on or above the diagonal.  A consumer that needs a block below the
//    diagonal stages the mirror block transposed.
//  * Q in COMB reads X along its rows (the contraction index k is X's row
//    index), and so do the blocks of A and B below the diagonal, read through
//    their mirror block.  The 256 x 256 tiles (bf16 and split-bf16) stage
//    such operands in k-row form (each LDS row a k-row as in memory) and read
//    their fragments with ds_read_b64_tr_b16; the 128 x 128 and 64 x 64 tiles
//    load 4 k-values of 8 rows (4 rows for float32), transpose them in
//    registers and write 8 bytes (16 for float32) per row into LDS.
//  * The additive terms a X and (b/c) A run on the matrix cores: where the
//    k-slab meets the tile's own rows, extra MFMAs pair the Q fragment with
//    a scaled identity fragment (for bf16 the scale is split into hi + lo, so
//    the term carries about 17 significant bits, far inside the bf16 storage
//    error), and no epilogue reads memory.
//  * LDS rows hold 128 bytes of K at a pitch of 144 bytes.  The 256 x 256
//    tiles keep rows unswizzled (a fragment read of 32 consecutive rows then
//    puts each 16-lane group of the LDS on distinct banks) and k-row stages
//    at a 576-byte pitch; the smaller tiles put the 16-byte chunk ch of row r
//    at chunk position ch ^ ((r >> 4) & 7), so their fragment reads and
//    transposed writes are both free of bank conflicts.
//  * Tiles: 256 x 256 over eight waves (2 x 4, each 128 x 64) for bf16 and
//    split-bf16, with a software-pipelined k-loop (a split-bf16 product runs
//    as three bf16 products over K, one plane pair each); 128 x 128 over four
//    waves (2 x 2, each 64 x 64) for float32 and for small bf16 and
//    split-bf16 stacks; 64 x 64 over two waves for small float32 stacks.  K
//    is staged 128 bytes per row, double-buffered through LDS with register
//    staging.  Operands are zero-padded to a multiple of 256; the 256 x 256
//    formats keep their workspace tile by tile.
//  * Tile lists are split into one contiguous, cost-balanced segment per XCD;
//    a persistent grid walks them, workgroup b on XCD b % 8 taking entries
//    b/8, b/8 + grid/8, ... of that XCD's segment, so tiles that share
//    operand panels share an L2.

#include "ns_tile.h"

namespace muon {
namespace {

// Persistent grid: workgroup b serves XCD b % 8 and walks that XCD's tile
// list from entry b / 8 with a stride of (grid / 8).
template <int PREC, int PHASE, int VAR>
__global__ __launch_bounds__(Cfg<PREC>::NT) void ns_gemm_kernel(const MatDev* __restrict__ mats,
                                                                const MatScal* __restrict__ scal,
                                                                const int2* __restrict__ tiles, PhaseArgs pa) {
  constexpr int NPL = Fmt<PREC>::spl;
  constexpr int STAGE = 2 * NPL * Cfg<PREC>::BT * PITCH;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int xcd = blockIdx.x % NUM_XCD;
  const int stride = gridDim.x / NUM_XCD;
  const int2* list = tiles + int64_t(xcd) * pa.per_xcd;
  using G = Geo<Fmt<PREC>::esz, Cfg<PREC>::BT, Cfg<PREC>::NT>;
  u32x4 rp[NPL][G::NREG], rq[NPL][G::NREG];  // the next stage 0, carried across tiles
  int slot = blockIdx.x / NUM_XCD;
  // a walk ends at its first padding entry (workgroup slot, slot + stride, ...)
  int2 te = slot < pa.per_xcd ? list[slot] : int2{-1, 0};
  if (te.x >= 0) {
    OpSrc sp, sq;
    tile_ops<PREC, PHASE>(mats[te.x], te.y >> 16, te.y & 0xFFFF, pa, sp, sq);
    const OpRsrc rsp = op_rsrc(sp), rsq = op_rsrc(sq);
    load_operand<PREC, PHASE, 0>(rp, sp, rsp, 0, threadIdx.x, split_plane(0, 0));
    load_operand<PREC, PHASE, 1>(rq, sq, rsq, 0, threadIdx.x, split_plane(1, 0));
  }
#pragma unroll 1
  while (te.x >= 0) {
    const int nslot = slot + stride;
    const int2 tn = nslot < pa.per_xcd ? list[nslot] : int2{-1, 0};
    // the next tile's operand sources, formed when its first stage is loaded
    auto next = [&](OpSrc& np, OpSrc& nq) {
      if (tn.x < 0) return false;
      tile_ops<PREC, PHASE>(mats[tn.x], tn.y >> 16, tn.y & 0xFFFF, pa, np, nq);
      return true;
    };
    ns_tile_body<PREC, PHASE, VAR, G::NREG>(mats[te.x], scal, te.x, te.y >> 16, te.y & 0xFFFF, pa, smem, rp, rq, next);
    lds_barrier();
    slot = nslot;
    te = tn;
  }
}

template <int PREC, int PHASE, int VAR>
hipError_t launch_one(const MatDev* mats, const MatScal* scal, const int2* tiles,
                      const PhaseArgs& pa, hipStream_t stream) {
  if (pa.per_xcd <= 0) return hipSuccess;
  // resident workgroups per XCD: CUs per XCD times workgroups per CU (LDS-bound)
  constexpr int per_cu = (ns_tile(PREC) == 256 || is_split(PREC)) ? 1 : 2;
  const int per_xcd = std::min(pa.per_xcd, pa.cus_per_xcd * per_cu);
  const unsigned grid = unsigned(NUM_XCD) * unsigned(per_xcd);
  static_assert(Cfg<PREC>::BT == ns_tile(PREC), "tile size disagrees with the host's tile lists");
  hipLaunchKernelGGL((ns_gemm_kernel<PREC, PHASE, VAR>), dim3(grid), dim3(Cfg<PREC>::NT), 0, stream,
                     mats, scal, tiles, pa);
  return hipGetLastError();
}

template <int PREC>
hipError_t launch_prec(int phase, const MatDev* mats, const MatScal* scal, const int2* tiles,
                       const PhaseArgs& pa, hipStream_t stream) {
  switch (phase) {
    case PH_GRAM:
      return pa.c != 0.f ? launch_one<PREC, PH_GRAM, 1>(mats, scal, tiles, pa, stream)
                         : launch_one<PREC, PH_GRAM, 0>(mats, scal, tiles, pa, stream);
    case PH_POLY: return launch_one<PREC, PH_POLY, 0>(mats, scal, tiles, pa, stream);
    case PH_COMB:
      return pa.last ? launch_one<PREC, PH_COMB, 1>(mats, scal, tiles, pa, stream)
                     : launch_one<PREC, PH_COMB, 0>(mats, scal, tiles, pa, stream);
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
    case PREC_BF16S: return launch_prec<PREC_BF16S>(phase, mats, scal, tiles, args, stream);
    case PREC_F32S: return launch_prec<PREC_F32S>(phase, mats, scal, tiles, args, stream);
    case PREC_BF16X3S: return launch_prec<PREC_BF16X3S>(phase, mats, scal, tiles, args, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
