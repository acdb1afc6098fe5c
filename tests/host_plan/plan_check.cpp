// CPU check of the library's host-side planning: muon_api.cpp compiled for
// the host with the HIP runtime calls replaced by host-memory stubs and the
// kernel launchers replaced by checkers that walk the device lists exactly as
// the kernels do.
//   - per-phase grids: every tile of every matrix visited exactly once, no
//     tile outside its matrix, GRAM/POLY only on or above the diagonal, and
//     the busiest workgroup's work against the mean (load balance);
//   - momentum pass: every matrix's elementwise tile count and row length
//     are those of the kernel's tile shape for its path, and its U stores
//     stay inside the X buffer;
//   - persistent chain: every wait names a counter that receives exactly the
//     awaited number of signals, every buffer an item uses lies inside a
//     workspace allocation, and a round-robin scheduler over the per-XCD
//     queues (a workgroup holding an item whose inputs are incomplete makes
//     no progress) finishes every item without deadlock.
// Exit status 0 when every case passes; one "CASE" line per case.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <string>
#include <tuple>
#include <vector>

static std::vector<std::pair<char*, size_t>> g_allocs;
static hipError_t s_malloc(void** p, size_t n) {
  const size_t m = (n + 255) / 256 * 256;
  *p = aligned_alloc(256, m);
  if (!*p) return hipErrorOutOfMemory;
  if (m <= (size_t(64) << 20)) memset(*p, 0, m);  // larger workspaces stay untouched (lazily mapped)
  g_allocs.push_back({static_cast<char*>(*p), m});
  return hipSuccess;
}
static hipError_t s_free(void* p) {
  for (auto it = g_allocs.begin(); it != g_allocs.end(); ++it)
    if (it->first == p) { g_allocs.erase(it); break; }
  free(p);
  return hipSuccess;
}
static hipError_t s_hostmalloc(void** p, size_t n, unsigned) { return s_malloc(p, n); }
static hipError_t s_memcpy(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) { memcpy(d, s, n); return hipSuccess; }
static hipError_t s_ok0() { return hipSuccess; }
static hipError_t s_ok1(hipStream_t) { return hipSuccess; }
static hipError_t s_getdev(int* d) { *d = 0; return hipSuccess; }
static hipError_t s_attr(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }  // 256 CUs
static hipError_t s_evc(hipEvent_t* e, unsigned) { *e = reinterpret_cast<hipEvent_t>(0x1); return hipSuccess; }
static hipError_t s_evc2(hipEvent_t* e) { *e = reinterpret_cast<hipEvent_t>(0x1); return hipSuccess; }
static hipError_t s_evr(hipEvent_t, hipStream_t) { return hipSuccess; }
static hipError_t s_ev1(hipEvent_t) { return hipSuccess; }
static hipError_t s_setdev(int) { return hipSuccess; }
static hipError_t s_wait(hipStream_t, hipEvent_t, unsigned) { return hipSuccess; }
static hipError_t s_elapsed(float* ms, hipEvent_t, hipEvent_t) { *ms = 0; return hipSuccess; }
static const char* s_errstr(hipError_t) { return "stub"; }
#define hipMalloc s_malloc
#define hipFree s_free
#define hipHostMalloc s_hostmalloc
#define hipHostFree s_free
#define hipMemcpyAsync s_memcpy
#define hipStreamSynchronize s_ok1
#define hipDeviceSynchronize s_ok0
#define hipGetDevice s_getdev
#define hipSetDevice s_setdev
#define hipDeviceGetAttribute s_attr
#define hipEventCreateWithFlags s_evc
#define hipEventCreate s_evc2
#define hipEventRecord s_evr
#define hipEventSynchronize s_ev1
#define hipEventQuery s_ev1
#define hipStreamWaitEvent s_wait
#define hipEventDestroy s_ev1
#define hipGetLastError s_ok0
#define hipEventElapsedTime s_elapsed
#define hipGetErrorString s_errstr
#include "muon_api.cpp"

static int g_fail = 0;
static int g_count = 0;              // matrices in the current call
static double g_max_imbalance = 0;   // worst makespan / mean over the current call's phases
static int g_phase_launches = 0, g_chain_launches = 0;

#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      printf("  FAIL: " __VA_ARGS__);      \
      printf("\n");                        \
      g_fail = 1;                          \
    }                                      \
  } while (0)

static bool in_alloc(const void* p) {
  for (auto& a : g_allocs)
    if (static_cast<const char*>(p) >= a.first && static_cast<const char*>(p) < a.first + a.second) return true;
  return false;
}

// [p, p + n) inside one allocation
static bool in_one_alloc(const void* p, size_t n) {
  const char* c = static_cast<const char*>(p);
  for (auto& a : g_allocs)
    if (c >= a.first && c + n <= a.first + a.second) return true;
  return false;
}

// The allocation-free entry point's scratch array: one host block of its size.
static void* g_scratch = nullptr;
static bool g_check_buffers = false;   // grids: every workspace buffer and table inside one allocation

static int g_mom_launches = 0;

namespace muon {
// The walk of momentum_kernel: workgroup b takes tile b - etile_off[i] of
// the matrix i whose range holds b, row-major over the tiles of the matrix's
// padded natural shape, in the tile shape of its path (16 x 256 for
// matrices iterated untransposed; for tall ones 64 x 128 in the bf16 working
// format, 64 x 64 otherwise).  The tables must give every matrix exactly
// that many tiles with that row length, so that the walk covers each padded
// shape once; the U^T / U stores stay inside the X buffer.
hipError_t launch_momentum(const MatDev* mats, const int32_t* etile_off, int32_t count, int64_t total_tiles, float,
                           int32_t, int32_t, int32_t mode, float*, hipStream_t) {
  ++g_mom_launches;
  CHECK(etile_off[0] == 0 && etile_off[count] == total_tiles, "momentum: %lld tiles, offsets end at %d",
        (long long)total_tiles, etile_off[count]);
  for (int i = 0; i < count; ++i) {
    const MatDev& md = mats[i];
    const bool tr = md.transposed != 0;
    const int th = !tr ? RTILE_R : (md.prec == PREC_BF16 ? TBF_R : ETILE);
    const int tw = !tr ? RTILE_C : (md.prec == PREC_BF16 ? TBF_C : ETILE);
    const int rp = tr ? md.Np : md.Mp, cp = tr ? md.Mp : md.Np;
    CHECK(tr == (md.rows > md.cols) && md.rows <= rp && md.cols <= cp, "momentum: matrix %d shape", i);
    CHECK(rp % th == 0 && cp % tw == 0, "momentum: matrix %d padded %d x %d not in %d x %d tiles", i, rp, cp, th, tw);
    CHECK(md.etile_cols == cp / tw, "momentum: matrix %d has %d tiles per row, the walk needs %d", i, md.etile_cols,
          cp / tw);
    CHECK(etile_off[i + 1] - etile_off[i] == (rp / th) * (cp / tw), "momentum: matrix %d has %d tiles, the walk %d",
          i, etile_off[i + 1] - etile_off[i], (rp / th) * (cp / tw));
    if (mode != 2)   // the last X element any tile writes
      CHECK(ws_index(md.prec, md.Mp - 1, md.Np - 1, md.ldx) < int64_t(md.Mp) * md.ldx,
            "momentum: matrix %d stores beyond X", i);
  }
  return hipSuccess;
}
hipError_t launch_norm_finalize(const int32_t*, int32_t, const float*, MatScal*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_writeback_direct(const MatDev*, const int32_t*, int32_t, int64_t, const MatScal*, float, int32_t,
                                   const float2*, hipStream_t) { return hipSuccess; }
hipError_t launch_adamw(const AdamwTensor*, const int32_t*, int32_t, int64_t, const float2*, float, float,
                        const AdamwConsts&, hipStream_t) { return hipSuccess; }
hipError_t launch_mfma_probe(int64_t, int32_t, float*, double*, hipStream_t) { return hipSuccess; }
hipError_t noalloc_scratch(int, void** out) {
  if (!g_scratch && s_malloc(&g_scratch, NOALLOC_SCRATCH_BYTES) != hipSuccess) return hipErrorOutOfMemory;
  *out = g_scratch;
  return hipSuccess;
}

// The walk of ns_gemm_kernel: workgroup g on XCD g % 8 starts at slot g / 8
// of its XCD's list, steps by the XCD's workgroup count, stops at the first
// padding entry; the grid is what launch_one sizes it to.
hipError_t launch_ns_phase(int prec, int phase, const MatDev* mats, const MatScal*, const int2* tiles,
                           const PhaseArgs& pa, hipStream_t) {
  ++g_phase_launches;
  if (pa.per_xcd <= 0) return hipSuccess;
  const int T = ns_tile(prec);
  if (g_check_buffers) {
    CHECK(in_one_alloc(mats, sizeof(MatDev) * g_count), "matrix table outside an allocation");
    CHECK(in_one_alloc(tiles, sizeof(int2) * NUM_XCD * pa.per_xcd), "tile list outside an allocation");
    for (int i = 0; i < g_count; ++i) {
      const MatDev& md = mats[i];
      const int esz = is_f32(md.prec) ? 4 : 2, npl = is_split(md.prec) ? 2 : 1;
      const size_t xb = size_t(md.Mp) * md.ldx * esz * npl, ab = size_t(md.Mp) * md.lda * esz * npl;
      CHECK(in_one_alloc(md.X[0], xb) && in_one_alloc(md.X[1], xb) && in_one_alloc(md.A, ab) &&
                in_one_alloc(md.B, ab),
            "matrix %d: a workspace buffer lies outside the allocation", i);
    }
  }
  const int per_cu = (T == 256 || is_split(prec)) ? 1 : 2;
  const int B = std::min(pa.per_xcd, pa.cus_per_xcd * per_cu);
  std::set<std::tuple<int, int, int>> expect, seen;
  for (int i = 0; i < g_count; ++i) {
    if (mats[i].prec != prec) continue;
    const int tm = mats[i].Mp / T, tn = mats[i].Np / T;
    CHECK(mats[i].Mp % T == 0 && mats[i].Np % T == 0 && mats[i].Mp >= mats[i].m && mats[i].Np >= mats[i].n,
          "matrix %d: padded shape %d x %d does not cover %d x %d in %d-tiles", i, mats[i].Mp, mats[i].Np, mats[i].m,
          mats[i].n, T);
    for (int a = 0; a < tm; ++a)
      for (int b = phase == PH_COMB ? 0 : a; b < (phase == PH_COMB ? tn : tm); ++b) expect.insert({i, a, b});
  }
  double worst = 0, total = 0;
  for (int x = 0; x < NUM_XCD; ++x) {
    // a workgroup's walk ends at its first padding entry, so no tile may
    // follow one on the same walk
    for (int b = 0; b < B; ++b) {
      bool pad = false;
      for (int slot = b; slot < pa.per_xcd; slot += B) {
        const bool is_pad = tiles[int64_t(x) * pa.per_xcd + slot].x < 0;
        CHECK(!(pad && !is_pad), "XCD %d: tile after the end of workgroup %d's walk (slot %d)", x, b, slot);
        pad = pad || is_pad;
      }
    }
    double xtotal = 0, xworst = 0, xmax = 0;
    for (int b = 0; b < B; ++b) {
      double w = 0;
      for (int slot = b; slot < pa.per_xcd; slot += B) {
        const int2 t = tiles[int64_t(x) * pa.per_xcd + slot];
        if (t.x < 0) break;
        const int a = t.y >> 16, c = t.y & 0xFFFF;
        CHECK(t.x < g_count && mats[t.x].prec == prec, "tile of matrix %d in the prec %d list", t.x, prec);
        if (t.x >= g_count) continue;
        CHECK(seen.insert({t.x, a, c}).second, "phase %d: tile (%d, %d, %d) visited twice", phase, t.x, a, c);
        CHECK(expect.count({t.x, a, c}) == 1, "phase %d: tile (%d, %d, %d) is not a tile of its matrix", phase, t.x,
              a, c);
        const double cost = phase == PH_GRAM ? mats[t.x].Np : mats[t.x].Mp;
        w += cost;
        xmax = std::max(xmax, cost);
      }
      xworst = std::max(xworst, w);
      xtotal += w;
    }
    // list-scheduling bound: no workgroup gets more than the XCD's mean plus
    // its costliest tile (5 % slack: a strided walk within 5 % of the
    // longest-first layout is kept)
    CHECK(xworst <= 1.05 * (xtotal / B + xmax) + 1e-9, "phase %d XCD %d: makespan %.0f above mean %.0f + tile %.0f",
          phase, x, xworst, xtotal / B, xmax);
    worst = std::max(worst, xworst);
    total += xtotal;
  }
  CHECK(seen.size() == expect.size(), "phase %d prec %d: %zu of %zu tiles visited", phase, prec, seen.size(),
        expect.size());
  const double mean = total / (NUM_XCD * B);
  if (mean > 0) g_max_imbalance = std::max(g_max_imbalance, worst / mean);
  printf("  phase %d prec %d: %zu tiles, makespan %.0f, mean %.0f (K-units per workgroup)\n", phase, prec,
         seen.size(), worst, mean);
  return hipSuccess;
}

hipError_t launch_ns_chain(int prec, const MatDev* imats, const MatScal*, const ChainItem* items, const int32_t* xoff,
                           int32_t per_xcd_max, PhaseArgs*, int32_t*, int32_t nsync, int32_t*, const ChainArgs& a,
                           hipStream_t) {
  ++g_chain_launches;
  const int per_cu = (ns_tile(prec) == 256 || is_split(prec)) ? 1 : 2;
  const int per_xcd = std::min(per_xcd_max, a.cus_per_xcd * per_cu);
  const int nitems = xoff[NUM_XCD];
  const int ncnt = nsync - CHAIN_SYNC_HEAD;
  std::vector<int> done(ncnt, 0), signals(ncnt, 0);
  for (int i = 0; i < nitems; ++i) {
    const ChainItem& it = items[i];
    CHECK(it.signal >= 0 && it.signal < ncnt, "item %d: signal counter %d out of range", i, it.signal);
    if (it.signal >= 0 && it.signal < ncnt) signals[it.signal]++;
    CHECK(it.wait < ncnt, "item %d: wait counter %d out of range", i, it.wait);
    const MatDev& md = imats[it.desc];
    CHECK(in_alloc(md.X[0]) && in_alloc(md.A) && in_alloc(md.B), "item %d: a buffer lies outside the workspace", i);
  }
  for (int i = 0; i < nitems; ++i) {
    const ChainItem& it = items[i];
    if (it.wait >= 0 && it.wait < ncnt)
      CHECK(signals[it.wait] == it.need, "item %d waits for %d signals on counter %d, which gets %d", i, it.need,
            it.wait, signals[it.wait]);
  }
  std::vector<int> head(NUM_XCD, 0);
  struct Blk { int q, item; };
  std::vector<Blk> blocks;
  for (int b = 0; b < NUM_XCD * per_xcd; ++b) blocks.push_back({b % NUM_XCD, -2});
  int finished = 0, rounds = 0;
  while (finished < nitems) {
    bool prog = false;
    for (auto& bl : blocks) {
      if (bl.item == -1) continue;
      if (bl.item == -2) {  // take the next item of this XCD's queue
        const int i = xoff[bl.q] + head[bl.q]++;
        bl.item = i < xoff[bl.q + 1] ? i : -1;
        prog = true;
        continue;
      }
      const ChainItem& it = items[bl.item];
      if (it.wait >= 0 && done[it.wait] < it.need) continue;
      done[it.signal]++;
      ++finished;
      bl.item = -2;
      prog = true;
    }
    ++rounds;
    if (!prog) {
      CHECK(false, "chain deadlock after %d of %d items", finished, nitems);
      break;
    }
  }
  printf("  chain prec %d: %d items, %d steps, %d queues x %d workgroups, %d scheduler rounds\n", prec, nitems,
         a.steps, NUM_XCD, per_xcd, rounds);
  return hipSuccess;
}
}  // namespace muon

struct Shape { int rows, cols, prec; };

static muon_matrix_desc desc_of(const Shape& s) {
  const bool f32 = s.prec == MUON_NS_F32 || s.prec == MUON_NS_BF16X3;
  return {s.rows, s.cols, s.cols, s.cols, s.cols, f32 ? MUON_DTYPE_F32 : MUON_DTYPE_BF16, MUON_DTYPE_BF16,
          MUON_DTYPE_F32, s.prec};
}

// Per-phase grids over shapes whose data is never touched: far-apart fake
// device addresses (validation only compares them).
static void grid_case(const char* name, const std::vector<Shape>& shapes, double max_imbalance) {
  const int n = int(shapes.size());
  std::vector<muon_matrix_desc> d(n);
  std::vector<void*> P(n), G(n), M(n);
  for (int i = 0; i < n; ++i) {
    d[i] = desc_of(shapes[i]);
    P[i] = reinterpret_cast<void*>(uintptr_t(0x100000000000ull) + uintptr_t(i) * (uintptr_t(3) << 34));
    G[i] = reinterpret_cast<void*>(uintptr_t(P[i]) + (uintptr_t(1) << 34));
    M[i] = reinterpret_cast<void*>(uintptr_t(P[i]) + (uintptr_t(2) << 34));
  }
  printf("CASE grids %s (%d matrices)\n", name, n);
  g_count = n;
  g_max_imbalance = 0;
  const int before = g_phase_launches, mom_before = g_mom_launches;
  const muon_ns_coeffs co{3.4445f, -4.775f, 2.0315f};
  muon_step_options o{};
  o.launch_mode = MUON_LAUNCH_PHASE_GRIDS;
  const muon_status st = muon_step_batched_v2(P.data(), G.data(), M.data(), d.data(), n, 0.02f, 0.95f, 1, co, 1, 0,
                                              &o, nullptr, nullptr);
  CHECK(st == MUON_OK, "status %d: %s", int(st), muon_last_error());
  CHECK(g_phase_launches > before, "no phase launched");
  CHECK(g_mom_launches > mom_before, "no momentum pass launched");
  CHECK(g_max_imbalance <= max_imbalance, "makespan / mean %.3f above %.3f", g_max_imbalance, max_imbalance);
  printf("  worst makespan / mean %.3f\n", g_max_imbalance);
}

// The persistent chain over small matrices with real (host) buffers.
static void chain_case(const char* name, const std::vector<Shape>& shapes, int steps, bool schedule) {
  const int n = int(shapes.size());
  std::vector<muon_matrix_desc> d(n);
  std::vector<void*> P(n), G(n), M(n);
  for (int i = 0; i < n; ++i) {
    d[i] = desc_of(shapes[i]);
    const size_t el = size_t(shapes[i].rows) * shapes[i].cols;
    (void)s_malloc(&P[i], el * (d[i].param_dtype == MUON_DTYPE_F32 ? 4 : 2));
    (void)s_malloc(&G[i], el * 2);
    (void)s_malloc(&M[i], el * 4);
  }
  printf("CASE chain %s (%d matrices, %d steps)\n", name, n, steps);
  g_count = n;
  const int before = g_chain_launches;
  const muon_ns_coeffs co{3.4445f, -4.775f, 2.0315f}, cubic{1.5f, -0.5f, 0.f};
  std::vector<muon_ns_coeffs> sched;
  for (int k = 0; k < steps; ++k) sched.push_back(k % 2 ? cubic : co);
  muon_step_options o{};
  o.launch_mode = MUON_LAUNCH_CHAIN;
  if (schedule) o.ns_schedule = sched.data();
  const muon_status st = muon_step_batched_v2(P.data(), G.data(), M.data(), d.data(), n, 0.02f, 0.95f, 1, co, steps,
                                              0, &o, nullptr, nullptr);
  CHECK(st == MUON_OK, "status %d: %s", int(st), muon_last_error());
  CHECK(g_chain_launches > before, "no chain launched");
  for (int i = 0; i < n; ++i) {
    (void)s_free(P[i]);
    (void)s_free(G[i]);
    (void)s_free(M[i]);
  }
}

// The allocation-free entry point over small matrices with real (host)
// buffers: every workspace buffer and table inside the scratch block, and
// inputs too large for it refused.
static void noalloc_case(const char* name, const std::vector<Shape>& shapes, muon_status expect) {
  const int n = int(shapes.size());
  std::vector<muon_matrix_desc> d(n);
  std::vector<void*> P(n), G(n), M(n);
  for (int i = 0; i < n; ++i) {
    d[i] = desc_of(shapes[i]);
    const size_t el = size_t(shapes[i].rows) * shapes[i].cols;
    (void)s_malloc(&P[i], el * (d[i].param_dtype == MUON_DTYPE_F32 ? 4 : 2));
    (void)s_malloc(&G[i], el * 2);
    (void)s_malloc(&M[i], el * 4);
  }
  printf("CASE no-allocation %s (%d matrices)\n", name, n);
  g_count = n;
  g_check_buffers = true;
  const int before = g_phase_launches;
  const size_t allocs = g_allocs.size();
  const muon_ns_coeffs co{3.4445f, -4.775f, 2.0315f};
  const muon_status st = muon_step_batched_noalloc(P.data(), G.data(), M.data(), d.data(), n, 0.02f, 0.95f, 1, co, 5,
                                                   0, nullptr, nullptr);
  g_check_buffers = false;
  CHECK(st == expect, "status %d (expected %d): %s", int(st), int(expect), muon_last_error());
  if (expect == MUON_OK) CHECK(g_phase_launches > before, "no phase launched");
  else CHECK(g_phase_launches == before, "a refused call launched");
  // the scratch block may appear on the first call; nothing else is allocated
  CHECK(g_allocs.size() <= allocs + (g_scratch && allocs == g_allocs.size() ? 0 : 1), "the call allocated");
  printf("  status %d%s%s\n", int(st), st == MUON_OK ? "" : ": ", st == MUON_OK ? "" : muon_last_error());
  for (int i = 0; i < n; ++i) {
    (void)s_free(P[i]);
    (void)s_free(G[i]);
    (void)s_free(M[i]);
  }
}

// The allocation fault hook: with MUON_FAULT_ALLOC set, a call that needs a
// new plan (or workspace) fails with OUT_OF_MEMORY before any launch, and
// the next call without it succeeds.
static void fault_case() {
  const std::vector<Shape> shapes = {{333, 444, MUON_NS_BF16}, {444, 333, MUON_NS_BF16}};
  const int n = int(shapes.size());
  std::vector<muon_matrix_desc> d(n);
  std::vector<void*> P(n), G(n), M(n);
  for (int i = 0; i < n; ++i) {
    d[i] = desc_of(shapes[i]);
    P[i] = reinterpret_cast<void*>(uintptr_t(0x300000000000ull) + uintptr_t(i) * (uintptr_t(3) << 34));
    G[i] = reinterpret_cast<void*>(uintptr_t(P[i]) + (uintptr_t(1) << 34));
    M[i] = reinterpret_cast<void*>(uintptr_t(P[i]) + (uintptr_t(2) << 34));
  }
  printf("CASE allocation fault hook\n");
  g_count = n;
  const muon_ns_coeffs co{3.4445f, -4.775f, 2.0315f};
  setenv("MUON_FAULT_ALLOC", "1", 1);
  int before = g_phase_launches;
  muon_status st = muon_step_batched(P.data(), G.data(), M.data(), d.data(), n, 0.02f, 0.95f, 1, co, 5, 0, nullptr);
  CHECK(st == MUON_ERR_OUT_OF_MEMORY, "with the hook: status %d (%s)", int(st), muon_last_error());
  CHECK(g_phase_launches == before, "a call that failed to allocate launched");
  const int32_t grp[2] = {0, 1};
  muon_stream_plan sp = nullptr;
  st = muon_stream_plan_create(P.data(), G.data(), M.data(), d.data(), n, grp, 2, 0, nullptr, &sp);
  CHECK(st == MUON_ERR_OUT_OF_MEMORY && sp == nullptr, "stream plan with the hook: status %d", int(st));
  unsetenv("MUON_FAULT_ALLOC");
  st = muon_step_batched(P.data(), G.data(), M.data(), d.data(), n, 0.02f, 0.95f, 1, co, 5, 0, nullptr);
  CHECK(st == MUON_OK, "without the hook: status %d (%s)", int(st), muon_last_error());
  CHECK(g_phase_launches > before, "no launch without the hook");
  printf("  out of memory with the hook, launched without it\n");
}

int main() {
  const int BF = MUON_NS_BF16, F32 = MUON_NS_F32, X3 = MUON_NS_BF16X3;
  std::vector<Shape> share, d24, lm;
  for (int l = 0; l < 24; ++l) {
    std::vector<Shape> layer = {{1536, 1536, BF}, {1536, 1536, BF}, {1536, 1536, BF}, {1536, 1536, BF},
                                {1536, 6144, BF}, {6144, 1536, BF}};
    d24.insert(d24.end(), layer.begin(), layer.end());
    if (l < 3) share.insert(share.end(), layer.begin(), layer.end());
  }
  for (int l = 0; l < 2; ++l) {
    std::vector<Shape> layer = {{3072, 3072, BF}, {3072, 1024, BF}, {3072, 1024, BF},
                                {3072, 3072, BF}, {3072, 12288, BF}, {12288, 3072, BF}};
    lm.insert(lm.end(), layer.begin(), layer.end());
  }
  grid_case("d24 stack", d24, 1.05);
  grid_case("d24, one GPU's share (3 layers)", share, 1e9);
  grid_case("3.8B-like, 2 layers", lm, 1e9);
  grid_case("ragged, mixed formats",
            {{700, 1100, BF}, {1100, 700, BF}, {769, 769, F32}, {300, 520, X3}, {64, 64, BF}, {1, 300, F32},
             {2049, 257, BF}, {257, 2049, X3}, {5000, 3, BF}, {1, 1, BF}},
            1e9);
  grid_case("single 256 x 256, binary32 (64 x 64 tiles)", {{256, 256, F32}}, 1e9);
  grid_case("binary32 stack on 128 x 128 tiles", {{2048, 2048, F32}, {2048, 2048, F32}, {1024, 4096, F32},
                                                  {4096, 1024, F32}},
            1e9);
  grid_case("split-bf16 stack on 256 x 256 tiles", std::vector<Shape>(8, Shape{2048, 2048, X3}), 1e9);
  const std::vector<Shape> mixed = {{700, 1100, BF}, {1100, 700, BF}, {769, 769, BF},
                                    {300, 520, BF},  {64, 64, BF},    {1, 300, BF}};
  chain_case("bf16, 5 steps", mixed, 5, false);
  chain_case("bf16, 1 step", mixed, 1, false);
  chain_case("bf16, schedule with c = 0 steps", mixed, 4, true);
  chain_case("binary32 and split-bf16, 3 steps",
             {{769, 769, F32}, {300, 520, X3}, {64, 64, F32}, {129, 257, X3}}, 3, false);
  fault_case();
  noalloc_case("twelve 768 x 768 bf16", std::vector<Shape>(12, Shape{768, 768, BF}), MUON_OK);
  noalloc_case("ragged, mixed formats", {{700, 1100, BF}, {1100, 700, BF}, {300, 520, X3}, {64, 64, F32}, {1, 300, BF}},
               MUON_OK);
  noalloc_case("one d24 layer (too large)", {{1536, 1536, BF}, {1536, 1536, BF}, {1536, 1536, BF},
                                             {1536, 1536, BF}, {1536, 6144, BF}, {6144, 1536, BF}},
               MUON_ERR_UNSUPPORTED);
  printf(g_fail ? "PLAN-CHECK FAILED\n" : "PLAN-CHECK OK\n");
  return g_fail;
}
