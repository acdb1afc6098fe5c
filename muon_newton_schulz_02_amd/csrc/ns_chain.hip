// The persistent Newton-Schulz chain: one launch for every phase of every
// step of a call (the per-phase grids are in ns_gemm.hip; both run the
// tile code of ns_tile.h).

#include "ns_tile.h"

namespace muon {
namespace {

// ------------------------------------------------------------------ chain
// One persistent launch for every phase of every Newton-Schulz step of a
// call.  Each XCD has a queue of work items (XCD-local runs of each phase's
// tile list, as in the per-phase grids, in the order phase instances follow
// one another); its workgroups take items in queue order from an atomic head.
// An item waits until every tile of the phase instance it reads (the previous
// phase of its matrix) has been counted done, runs as in the per-phase
// kernels, then counts itself done.
//
// Deadlock freedom: every queue is sorted by one global order in which an
// item comes after everything it waits for, and items leave a queue in that
// order.  The earliest unfinished item overall therefore either is being run
// (its inputs are complete) or waits at the head of its queue, whose
// workgroups hold only finished items; so it runs.  The wait is bounded all
// the same: after spin_limit polls it gives up, raises the abort word (every
// other wait then gives up at its next poll) and the host's failure flag,
// and skips the tile (the call's results are then invalid and the host
// reports it), so the launch always ends.
//
// Coherence across XCDs (each has its own L2): every phase instance writes
// buffers of its own (the host gives each step its own A, B and next
// iterate), so no L2 can hold an earlier version of data an item reads; the
// producer makes its stores visible with a release fence (L2 write-back)
// before its agent-scope count, and the consumer reads the count with an
// agent-scope atomic load before any load of the data.

template <int PREC, int PHASE, int VAR>
__device__ __forceinline__ void chain_tile(const MatDev& md, const MatScal* __restrict__ scal, int mat, int ti,
                                           int tj, const PhaseArgs& pa, char* smem) {
  using G = Geo<Fmt<PREC>::esz, Cfg<PREC>::BT, Cfg<PREC>::NT>;
  u32x4 rp[Fmt<PREC>::spl][G::NREG], rq[Fmt<PREC>::spl][G::NREG];
  OpSrc sp, sq;
  tile_ops<PREC, PHASE>(md, ti, tj, pa, sp, sq);
  const OpRsrc rsp = op_rsrc(sp), rsq = op_rsrc(sq);
  load_operand<PREC, PHASE, 0>(rp, sp, rsp, 0, threadIdx.x, split_plane(0, 0));
  load_operand<PREC, PHASE, 1>(rq, sq, rsq, 0, threadIdx.x, split_plane(1, 0));
  ns_tile_body<PREC, PHASE, VAR, G::NREG>(md, scal, mat, ti, tj, pa, smem, rp, rq,
                                          [](OpSrc&, OpSrc&) { return false; });
}

template <int PREC>
__global__ __launch_bounds__(Cfg<PREC>::NT) void ns_chain_kernel(const MatDev* __restrict__ imats,
                                                                 const MatScal* __restrict__ scal,
                                                                 const ChainItem* __restrict__ items,
                                                                 const int32_t* __restrict__ xcd_off,
                                                                 const PhaseArgs* __restrict__ steps,
                                                                 int32_t* __restrict__ sync, int32_t* fail,
                                                                 int64_t spin_limit) {
  constexpr int NPL = Fmt<PREC>::spl;
  constexpr int STAGE = 2 * NPL * Cfg<PREC>::BT * PITCH;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int s_item, s_ok;
  const int xcd = blockIdx.x % NUM_XCD;
  const int beg = xcd_off[xcd], end = xcd_off[xcd + 1];
  int32_t* heads = sync;                  // [0, NUM_XCD): queue heads
  int32_t* abort = sync + NUM_XCD;        // one word, then padding
  int32_t* done = sync + CHAIN_SYNC_HEAD; // completion counters
  // No control flow in this loop depends on a per-lane value: wave 0 (a
  // wave-uniform test) takes items, waits and counts with all its lanes, lane
  // 0 contributing the 1 of each atomic.  With a thread-0 branch around that
  // work, the compiler routed the other lanes back to the barrier on their
  // own, and the workgroup ran its first item for ever.
  const bool lead = __builtin_amdgcn_readfirstlane(threadIdx.x) == 0;
  const int one = (threadIdx.x & 63) == 0 ? 1 : 0;
#pragma unroll 1
  for (;;) {
    if (lead) {
      const int got = __hip_atomic_fetch_add(&heads[xcd], one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int i = beg + __builtin_amdgcn_readfirstlane(got);   // lane 0's value: the head before its add
      int ok = 1;
      if (i < end) {
        const ChainItem it = items[i];
        if (it.wait >= 0) {
#pragma unroll 1
          for (int64_t polls = 0;; ++polls) {
            const int d = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(&done[it.wait], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (d >= it.need) break;
            const int ab = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (ab != 0) {
              ok = 0;
              break;
            }
            if (polls >= spin_limit) {
              ok = 0;
              __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              break;
            }
            __builtin_amdgcn_s_sleep(10);
          }
        }
      }
      s_item = i < end ? i : -1;
      s_ok = ok;
    }
    __syncthreads();
    const int i = __builtin_amdgcn_readfirstlane(s_item);
    const int ok = __builtin_amdgcn_readfirstlane(s_ok);
    if (i < 0) break;
    const ChainItem it = items[i];
    if (ok) {
      const MatDev& md = imats[it.desc];
      const PhaseArgs pa = steps[it.step];
      const int ti = it.tile >> 16, tj = it.tile & 0xFFFF;
      switch (it.kind) {
        case CHAIN_GRAM_B: chain_tile<PREC, PH_GRAM, 0>(md, scal, it.mat, ti, tj, pa, smem); break;
        case CHAIN_GRAM_A: chain_tile<PREC, PH_GRAM, 1>(md, scal, it.mat, ti, tj, pa, smem); break;
        case CHAIN_POLY: chain_tile<PREC, PH_POLY, 0>(md, scal, it.mat, ti, tj, pa, smem); break;
        case CHAIN_COMB: chain_tile<PREC, PH_COMB, 0>(md, scal, it.mat, ti, tj, pa, smem); break;
        default: chain_tile<PREC, PH_COMB, 1>(md, scal, it.mat, ti, tj, pa, smem); break;
      }
    }
    // every store of the workgroup acknowledged, then one release and the count
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (lead) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(&done[it.signal], one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void chain_setup_kernel(int32_t* __restrict__ sync, int32_t nsync, PhaseArgs* __restrict__ steps,
                                   ChainArgs args) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nsync; i += gridDim.x * blockDim.x) sync[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < MAX_CHAIN_STEPS; ++k) {
      if (k < args.steps) {
        PhaseArgs pa;
        pa.a = args.a[k];
        pa.b = args.b[k];
        pa.c = args.c[k];
        pa.lr = args.lr;
        pa.cur = 0;                     // each step's descriptor names its own buffers
        pa.first = k == 0;
        pa.last = k == args.steps - 1;
        pa.scale_rule = args.scale_rule;
        pa.per_xcd = 0;
        pa.cus_per_xcd = args.cus_per_xcd;
        pa.wb = args.wb;
        steps[k] = pa;
      }
    }
  }
}

template <int PREC>
hipError_t launch_chain_prec(const MatDev* imats, const MatScal* scal, const ChainItem* items, const int32_t* xcd_off,
                             int32_t per_xcd_max, PhaseArgs* steps, int32_t* sync, int32_t nsync, int32_t* fail,
                             const ChainArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(chain_setup_kernel, dim3(std::max(1, std::min(64, (nsync + 255) / 256))), dim3(256), 0, stream,
                     sync, nsync, steps, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || per_xcd_max <= 0) return e;
  constexpr int per_cu = (ns_tile(PREC) == 256 || is_split(PREC)) ? 1 : 2;
  const int per_xcd = std::min(per_xcd_max, args.cus_per_xcd * per_cu);
  hipLaunchKernelGGL(ns_chain_kernel<PREC>, dim3(unsigned(NUM_XCD) * unsigned(per_xcd)), dim3(Cfg<PREC>::NT), 0,
                     stream, imats, scal, items, xcd_off, steps, sync, fail, args.spin_limit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_chain(int prec, const MatDev* imats, const MatScal* scal, const ChainItem* items,
                           const int32_t* xcd_off, int32_t per_xcd_max, PhaseArgs* steps, int32_t* sync,
                           int32_t nsync, int32_t* fail, const ChainArgs& args, hipStream_t stream) {
  switch (prec) {
    case PREC_BF16:
      return launch_chain_prec<PREC_BF16>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail, args,
                                          stream);
    case PREC_BF16X3:
      return launch_chain_prec<PREC_BF16X3>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail,
                                            args, stream);
    case PREC_F32:
      return launch_chain_prec<PREC_F32>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail, args,
                                         stream);
    case PREC_BF16S:
      return launch_chain_prec<PREC_BF16S>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail, args,
                                           stream);
    case PREC_F32S:
      return launch_chain_prec<PREC_F32S>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail, args,
                                          stream);
    case PREC_BF16X3S:
      return launch_chain_prec<PREC_BF16X3S>(imats, scal, items, xcd_off, per_xcd_max, steps, sync, nsync, fail,
                                             args, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
