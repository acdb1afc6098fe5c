// Host runtime and C ABI of libmuon_mi355x.so: argument validation, the
// per-device workspace, cached launch plans and the launch sequence of one
// Muon step (declared in include/muon.h).
#include "muon.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "muon_internal.h"

namespace muon {
namespace {

thread_local std::string t_last_error;

muon_status fail(muon_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return s;
}

constexpr int64_t MAX_DIM = 65536;
constexpr int32_t MAX_COUNT = 1 << 20;
constexpr int32_t MAX_NS_STEPS = 1000;
constexpr size_t MAX_PLANS = 8;

enum Mode { MODE_STEP = 0, MODE_NS = 1, MODE_NORMS = 2 };

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int dtype_size(int32_t dt) { return dt == MUON_DTYPE_BF16 ? 2 : 4; }

struct Interval {
  uintptr_t lo, hi;  // [lo, hi)
  bool written;
  int idx;
  const char* what;
};

// Bytes spanned by a rows x cols matrix with row stride ld.
uint64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int esz) {
  return uint64_t((rows - 1) * ld + cols) * uint64_t(esz);
}

struct MatGeom {
  int64_t m, n, Mp, Np;
  int64_t ldx, lda;  // workspace row strides (elements)
  bool transposed;
  int prec;
  int esz, npl;
  size_t x_bytes, a_bytes;  // one X buffer, one A buffer (all planes)
};

MatGeom geom_of(const muon_matrix_desc& d) {
  MatGeom g;
  g.transposed = d.rows > d.cols;
  g.m = std::min(d.rows, d.cols);
  g.n = std::max(d.rows, d.cols);
  g.Mp = round_up(g.m, PAD);
  g.Np = round_up(g.n, PAD);
  g.ldx = g.Np + LDPAD;
  g.lda = g.Mp + LDPAD;
  g.prec = d.precision;
  g.esz = is_f32(g.prec) ? 4 : 2;
  g.npl = is_split(g.prec) ? 2 : 1;
  g.x_bytes = align256(size_t(g.Mp) * size_t(g.ldx) * g.esz * g.npl);
  g.a_bytes = align256(size_t(g.Mp) * size_t(g.lda) * g.esz * g.npl);
  return g;
}

size_t workspace_bytes(const muon_matrix_desc* shapes, int32_t count) {
  size_t tot = 0;
  for (int32_t i = 0; i < count; ++i) {
    MatGeom g = geom_of(shapes[i]);
    tot += 2 * g.x_bytes + 2 * g.a_bytes;
  }
  return tot;
}

muon_status validate_desc(const muon_matrix_desc* shapes, int32_t count, Mode mode) {
  for (int32_t i = 0; i < count; ++i) {
    const muon_matrix_desc& d = shapes[i];
    if (d.rows < 1 || d.cols < 1)
      return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: rows and cols must be >= 1 (got %lld x %lld)", i,
                  (long long)d.rows, (long long)d.cols);
    if (d.rows > MAX_DIM || d.cols > MAX_DIM)
      return fail(MUON_ERR_UNSUPPORTED, "matrix %d: rows and cols must be <= %lld", i, (long long)MAX_DIM);
    if (d.grad_dtype != MUON_DTYPE_F32 && d.grad_dtype != MUON_DTYPE_BF16)
      return fail(MUON_ERR_UNSUPPORTED, "matrix %d: grad_dtype %d is not F32 or BF16", i, d.grad_dtype);
    if (d.ld_grad < d.cols)
      return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: ld_grad %lld < cols %lld", i, (long long)d.ld_grad,
                  (long long)d.cols);
    if (mode != MODE_NORMS && d.precision != MUON_NS_BF16 && d.precision != MUON_NS_BF16X3 &&
        d.precision != MUON_NS_F32)
      return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: unknown precision %d", i, d.precision);
    if (mode != MODE_NORMS) {
      // the products address a workspace matrix (all planes) with 32-bit
      // buffer offsets from its first element
      const MatGeom g = geom_of(d);
      if (g.x_bytes > size_t(INT32_MAX) || g.a_bytes > size_t(INT32_MAX))
        return fail(MUON_ERR_UNSUPPORTED,
                    "matrix %d: %lld x %lld needs a %.2f GiB working copy in this precision; the limit is 2 GiB", i,
                    (long long)d.rows, (long long)d.cols, double(std::max(g.x_bytes, g.a_bytes)) / double(1 << 30));
    }
    if (mode == MODE_STEP) {
      if (d.param_dtype != MUON_DTYPE_F32 && d.param_dtype != MUON_DTYPE_BF16)
        return fail(MUON_ERR_UNSUPPORTED, "matrix %d: param_dtype %d is not F32 or BF16", i, d.param_dtype);
      if (d.mom_dtype != MUON_DTYPE_F32)
        return fail(MUON_ERR_UNSUPPORTED, "matrix %d: momentum must be F32 (mom_dtype %d)", i, d.mom_dtype);
      if (d.ld_param < d.cols || d.ld_mom < d.cols)
        return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: ld_param/ld_mom < cols", i);
    }
  }
  return MUON_OK;
}

muon_status check_ptr(const void* p, int esz, int i, const char* what) {
  if (!p) return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: %s pointer is NULL", i, what);
  if (reinterpret_cast<uintptr_t>(p) % uintptr_t(esz) != 0)
    return fail(MUON_ERR_UNSUPPORTED, "matrix %d: %s pointer is not aligned to %d bytes", i, what, esz);
  return MUON_OK;
}

// Overlap check in O(k log k): sort by start; track the maximum end seen so
// far over all intervals and over written ones.
muon_status check_alias_fast(std::vector<Interval>& iv) {
  std::sort(iv.begin(), iv.end(), [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
  uintptr_t max_any = 0, max_w = 0;
  int any_i = -1, w_i = -1;
  for (size_t i = 0; i < iv.size(); ++i) {
    const Interval& c = iv[i];
    if (any_i >= 0) {
      if (c.written && max_any > c.lo)
        return fail(MUON_ERR_ALIAS, "%s of matrix %d overlaps %s of matrix %d", c.what, c.idx, iv[any_i].what,
                    iv[any_i].idx);
      if (w_i >= 0 && max_w > c.lo)
        return fail(MUON_ERR_ALIAS, "%s of matrix %d overlaps %s of matrix %d", c.what, c.idx, iv[w_i].what,
                    iv[w_i].idx);
    }
    if (any_i < 0 || c.hi > max_any) { max_any = c.hi; any_i = int(i); }
    if (c.written && (w_i < 0 || c.hi > max_w)) { max_w = c.hi; w_i = int(i); }
  }
  return MUON_OK;
}

struct Plan {
  std::vector<uint64_t> key;
  int32_t count = 0;
  int64_t total_etiles = 0;
  void* dmem = nullptr;
  MatDev* d_mats = nullptr;
  int32_t* d_etile_off = nullptr;
  MatScal* d_scal = nullptr;
  float* d_partials = nullptr;
  float2* d_wb = nullptr;        // per-matrix write-back scalars {t, d}, filled per call when used
  struct Group {
    int prec;
    int2* tiles[3];
    int32_t per_xcd[3];
  };
  std::vector<Group> groups;
  // persistent chains (one per precision group), built on first use
  struct Chain {
    int prec = 0;
    std::vector<uint64_t> key;     // steps, c == 0 pattern, chain workspace
    void* dmem = nullptr;
    MatDev* d_imats = nullptr;     // per (step, matrix) descriptors
    ChainItem* d_items = nullptr;
    int32_t* d_xcd_off = nullptr;
    PhaseArgs* d_steps = nullptr;
    int32_t* d_sync = nullptr;
    int32_t nsync = 0;
    int32_t per_xcd_max = 0;
  };
  std::vector<Chain> chains;
  std::vector<MatDev> host_mats;   // host copy of d_mats (the chain derives its descriptors from it)
  hipEvent_t last_use = nullptr;
};

// Launch plan of an AdamW call: the device table of its non-empty tensors
// and their first workgroups.
struct AdamwPlan {
  std::vector<uint64_t> key;
  int32_t count = 0;              // tensors with numel > 0
  int64_t total_chunks = 0;
  std::vector<int32_t> kept;      // caller index of each tensor in the table
  void* dmem = nullptr;
  AdamwTensor* d_tensors = nullptr;
  int32_t* d_chunk_off = nullptr;
  float2* d_rates = nullptr;      // per tensor {lr, d}, filled per call when used
  hipEvent_t last_use = nullptr;
};

// Pinned host staging of the small per-call tables (per-matrix write-back
// scalars, per-tensor AdamW rates): copies from pinned memory are DMA
// transfers that do not wait on the host for earlier work on the stream,
// which copies from pageable memory may.  A ring of regions, each held until
// the event recorded after its copy has completed.
struct PinnedRing {
  char* host = nullptr;
  size_t bytes = 0;
  size_t head = 0;
  struct Use {
    size_t off, len;
    hipEvent_t ev;
  };
  std::vector<Use> busy;
  std::vector<hipEvent_t> idle_events;
};

struct DeviceState {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* chain_ws = nullptr;            // per-step buffers of the persistent chain
  size_t chain_ws_bytes = 0;
  int32_t* fail_flag = nullptr;        // pinned host word the chain raises when a wait times out
  hipEvent_t chain_done = nullptr;     // recorded after the last persistent-chain launch
  bool chain_pending = false;          // a chain was launched since the flag was last read
  // recorded after every call's last launch on this device, one per family
  // of calls that share device memory: the Muon step (workspace, plans,
  // tables) and AdamW (its plans' rate tables)
  hipEvent_t last_call[2] = {nullptr, nullptr};
  bool last_call_recorded[2] = {false, false};
  PinnedRing ring;
  int cus_per_xcd = 0;
  std::list<Plan*> plans;              // most recently used first
  std::list<AdamwPlan*> adamw_plans;   // most recently used first
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

// ------------------------------------------------------------ timing hook
struct TimedLaunch {
  hipEvent_t beg, end;
  int kc;
};
bool g_timing = false;
std::vector<TimedLaunch> g_timed;       // recorded, not yet read
std::vector<hipEvent_t> g_event_pool;   // reusable events

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

// Runs `launch` bracketed by events when timing is on.
template <class F>
hipError_t timed(int kc, hipStream_t stream, F&& launch) {
  if (!g_timing) return launch();
  hipEvent_t b = pool_event(), e = pool_event();
  if (!b || !e) return launch();
  (void)hipEventRecord(b, stream);
  hipError_t r = launch();
  (void)hipEventRecord(e, stream);
  g_timed.push_back({b, e, kc});
  return r;
}

// timed(), or the bare launch when `plain`.
template <class F>
hipError_t timed_unless(bool plain, int kc, hipStream_t stream, F&& launch) {
  return plain ? launch() : timed(kc, stream, launch);
}

void free_plan(Plan* p) {
  if (p->last_use) {
    (void)hipEventSynchronize(p->last_use);
    (void)hipEventDestroy(p->last_use);
  }
  if (p->dmem) (void)hipFree(p->dmem);
  for (auto& ch : p->chains)
    if (ch.dmem) (void)hipFree(ch.dmem);
  delete p;
}

void free_adamw_plan(AdamwPlan* p) {
  if (p->last_use) {
    (void)hipEventSynchronize(p->last_use);
    (void)hipEventDestroy(p->last_use);
  }
  if (p->dmem) (void)hipFree(p->dmem);
  delete p;
}

void drop_plans(DeviceState& ds) {
  for (Plan* p : ds.plans) free_plan(p);
  ds.plans.clear();
  for (AdamwPlan* p : ds.adamw_plans) free_adamw_plan(p);
  ds.adamw_plans.clear();
}

void release_ring(PinnedRing& r) {
  for (auto& u : r.busy) {
    (void)hipEventSynchronize(u.ev);
    r.idle_events.push_back(u.ev);
  }
  r.busy.clear();
  for (hipEvent_t e : r.idle_events) (void)hipEventDestroy(e);
  r.idle_events.clear();
  if (r.host) (void)hipHostFree(r.host);
  r.host = nullptr;
  r.bytes = 0;
  r.head = 0;
}

// Copies `len` bytes from `src` to device memory `dst` on `stream` through
// the device's pinned ring.  Waits on the host only when the ring region it
// needs still feeds a copy that has not completed.
hipError_t staged_copy(DeviceState& ds, void* dst, const void* src, size_t len, hipStream_t stream) {
  PinnedRing& r = ds.ring;
  const size_t need = align256(std::max<size_t>(len, 1));
  if (need > r.bytes) {
    release_ring(r);
    const size_t bytes = std::max<size_t>(size_t(1) << 18, 2 * need);
    void* h = nullptr;
    if (hipHostMalloc(&h, bytes, hipHostMallocDefault) != hipSuccess) return hipErrorOutOfMemory;
    r.host = reinterpret_cast<char*>(h);
    r.bytes = bytes;
  }
  size_t off = r.head;
  if (off + need > r.bytes) off = 0;
  // retire completed copies; wait for any still in flight over [off, off + need)
  for (size_t i = 0; i < r.busy.size();) {
    PinnedRing::Use& u = r.busy[i];
    const bool overlap = u.off < off + need && off < u.off + u.len;
    bool done = hipEventQuery(u.ev) == hipSuccess;
    if (!done && overlap) done = hipEventSynchronize(u.ev) == hipSuccess;
    if (done) {
      r.idle_events.push_back(u.ev);
      r.busy[i] = r.busy.back();
      r.busy.pop_back();
    } else {
      ++i;
    }
  }
  (void)hipGetLastError();  // hipEventQuery reports hipErrorNotReady for copies in flight
  memcpy(r.host + off, src, len);
  hipError_t e = hipMemcpyAsync(dst, r.host + off, len, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  hipEvent_t ev = nullptr;
  if (!r.idle_events.empty()) {
    ev = r.idle_events.back();
    r.idle_events.pop_back();
  } else if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
    // without an event the region cannot be tracked: wait for the copy
    (void)hipGetLastError();
    return hipStreamSynchronize(stream);
  }
  if ((e = hipEventRecord(ev, stream)) != hipSuccess) {
    r.idle_events.push_back(ev);
    return e;
  }
  r.busy.push_back({off, need, ev});
  r.head = off + need;
  return hipSuccess;
}

// Every call on a device first makes its stream wait for the device's
// previous call of the same family (Muon steps share the workspace, plans and
// tables; AdamW calls their plans' rate tables), so calls issued on different
// streams run in the order they were made.  The two families share no device
// memory and may overlap.
enum CallFamily : int { FAMILY_MUON = 0, FAMILY_ADAMW = 1 };

hipError_t order_after_last_call(DeviceState& ds, hipStream_t stream, int family = FAMILY_MUON) {
  if (!ds.last_call[family]) {
    if (hipEventCreateWithFlags(&ds.last_call[family], hipEventDisableTiming) != hipSuccess) {
      ds.last_call[family] = nullptr;
      return hipGetLastError();
    }
  }
  if (!ds.last_call_recorded[family]) return hipSuccess;
  return hipStreamWaitEvent(stream, ds.last_call[family], 0);
}

void record_last_call(DeviceState& ds, hipStream_t stream, int family = FAMILY_MUON) {
  if (ds.last_call[family] && hipEventRecord(ds.last_call[family], stream) == hipSuccess)
    ds.last_call_recorded[family] = true;
}

// Device allocations of the library.  MUON_FAULT_ALLOC set to anything but
// "" or "0" makes every one fail as if the device were out of memory (a fault
// hook for testing the allocation-failure paths; read per allocation).
hipError_t device_alloc(void** p, size_t bytes) {
  const char* f = std::getenv("MUON_FAULT_ALLOC");
  if (f && *f && std::strcmp(f, "0") != 0) {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipMalloc(p, bytes);
}

struct TileSrc {
  int mat;
  int ti, tj;
  double cost;
};

// Split each matrix's tiles over the XCDs: matrices in order, tiles of one
// matrix contiguous, each XCD taking a contiguous run of about 1/8 of the
// total cost.  Returns per-XCD lists padded to a common length with -1.
// `blocks` > 0 is the number of workgroups that will walk each XCD's list
// (entry b, b + blocks, ... for workgroup b).  Where that strided walk leaves
// one workgroup far more work than the others (tiles of very different cost,
// few per workgroup: a stack's rectangular GRAM tiles beside its square
// ones), the XCD's list is laid out instead as the workgroups' longest-first
// assignments, interleaved (workgroup b's k-th tile at entry b + blocks k,
// its walk ending at its first empty entry).
std::vector<int2> xcd_lists(const std::vector<TileSrc>& src, int32_t* per_xcd, int blocks = 0) {
  double total = 0;
  for (const auto& t : src) total += t.cost;
  std::vector<std::vector<int2>> bins(NUM_XCD);
  std::vector<std::vector<double>> costs(NUM_XCD);
  const double target = total / NUM_XCD;
  double acc = 0;
  int bin = 0;
  for (const auto& t : src) {
    // move on once this XCD holds its share (the last XCD takes the rest)
    if (bin < NUM_XCD - 1 && acc + 0.5 * t.cost > target * (bin + 1)) ++bin;
    bins[bin].push_back(make_int2(t.mat, (t.ti << 16) | t.tj));
    costs[bin].push_back(t.cost);
    acc += t.cost;
  }
  std::vector<std::vector<int2>> lay(NUM_XCD);
  for (int x = 0; x < NUM_XCD; ++x) {
    lay[x] = bins[x];
    const size_t n = bins[x].size();
    if (blocks <= 0 || n <= size_t(blocks)) continue;
    double strided = 0;
    for (int b = 0; b < blocks; ++b) {
      double w = 0;
      for (size_t i = size_t(b); i < n; i += size_t(blocks)) w += costs[x][i];
      strided = std::max(strided, w);
    }
    std::vector<size_t> idx(n);
    for (size_t i = 0; i < n; ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return costs[x][a] > costs[x][b]; });
    std::vector<double> load(size_t(blocks), 0.0);
    std::vector<std::vector<int2>> per(static_cast<size_t>(blocks));
    for (size_t i : idx) {
      const size_t b = size_t(std::min_element(load.begin(), load.end()) - load.begin());
      load[b] += costs[x][i];
      per[b].push_back(bins[x][i]);
    }
    const double lpt = *std::max_element(load.begin(), load.end());
    if (lpt > 0.95 * strided) continue;
    size_t kmax = 0;
    for (auto& v : per) kmax = std::max(kmax, v.size());
    lay[x].assign(kmax * size_t(blocks), make_int2(-1, 0));
    for (int b = 0; b < blocks; ++b)
      for (size_t k = 0; k < per[size_t(b)].size(); ++k) lay[x][size_t(b) + k * size_t(blocks)] = per[size_t(b)][k];
  }
  size_t mx = 0;
  for (auto& l : lay) mx = std::max(mx, l.size());
  *per_xcd = int32_t(mx);
  std::vector<int2> out(mx * NUM_XCD, make_int2(-1, 0));
  for (int x = 0; x < NUM_XCD; ++x)
    for (size_t i = 0; i < lay[x].size(); ++i) out[x * mx + i] = lay[x][i];
  return out;
}

// Workgroups of a phase kernel per compute unit (as the launchers size their grids).
int per_cu_blocks(int prec) { return (ns_tile(prec) == 256 || is_split(prec)) ? 1 : 2; }

// Matrices by decreasing Newton-Schulz cost, so large ones start first.
std::vector<int> cost_order(const std::vector<MatDev>& hm) {
  std::vector<int> order(hm.size());
  for (size_t i = 0; i < hm.size(); ++i) order[i] = int(i);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    const double ca = double(hm[a].Mp) * hm[a].Mp * hm[a].Np;
    const double cb = double(hm[b].Mp) * hm[b].Mp * hm[b].Np;
    return ca > cb;
  });
  return order;
}

// Tile rows per raster band of a matrix with tm tile rows.  The tiles in
// flight on one XCD (32 of 256 x 256, 64 of the smaller sizes) then cover h
// row panels and about 32 / h (64 / h) column panels; h + 32 / h is least
// near h = 6, and a band height that divides tm leaves no short band.
// 256 x 256: the whole height up to 8 rows, else the divisor of tm in 4..8
// nearest 6, else 6; smaller tiles: 8.  (d24 COMBINE, tm = 6: 1 % faster
// than 4-row bands.)
int band_rows(int tm, int T) {
  if (T != 256) return 8;
  if (tm <= 8) return std::max(tm, 1);
  int best = 0;
  for (int h = 4; h <= 8; ++h)
    if (tm % h == 0 && (best == 0 || std::abs(h - 6) <= std::abs(best - 6))) best = h;
  return best ? best : 6;
}

// The tiles of one phase over the matrices of one precision, in `order`:
// a grouped raster (bands of band_rows tile rows walked column by column) so
// that tiles in flight together share row and column operand panels; GRAM
// and POLY take the tiles on or above the diagonal.  Cost = K.
std::vector<TileSrc> phase_tiles(const std::vector<MatDev>& hm, const std::vector<int>& order, int prec, int ph) {
  std::vector<TileSrc> src;
  for (int i : order) {
    const MatDev& m = hm[i];
    if (m.prec != prec) continue;
    const int T = ns_tile(prec);
    const int tm = m.Mp / T, tn = m.Np / T;
    const int GROUP_M = band_rows(tm, T);
    if (ph == PH_COMB) {
      for (int g0 = 0; g0 < tm; g0 += GROUP_M)
        for (int b = 0; b < tn; ++b)
          for (int a = g0; a < std::min(tm, g0 + GROUP_M); ++a) src.push_back({i, a, b, double(m.Mp)});
    } else {
      const double k = ph == PH_GRAM ? double(m.Np) : double(m.Mp);
      for (int g0 = 0; g0 < tm; g0 += GROUP_M)
        for (int b = g0; b < tm; ++b)
          for (int a = g0; a < std::min(tm, g0 + GROUP_M) && a <= b; ++a) src.push_back({i, a, b, k});
    }
  }
  return src;
}

// Host image of a launch plan's device tables: matrix descriptors, the
// elementwise tiles' offsets, norm scalars, norm partials, write-back
// scalars and the per-phase tile lists of each working format.
struct PlanImage {
  std::vector<char> host;
  size_t off_mats = 0, off_etile = 0, off_scal = 0, off_part = 0, off_wb = 0;
  std::vector<size_t> off_lists;
  std::vector<Plan::Group> groups;
};

void plan_image(const std::vector<MatDev>& hm, const std::vector<int32_t>& etile_off, int cus_per_xcd,
                PlanImage& im) {
  const int32_t count = int32_t(hm.size());
  const std::vector<int> order = cost_order(hm);
  std::vector<int> precs;
  for (const auto& m : hm)
    if (std::find(precs.begin(), precs.end(), m.prec) == precs.end()) precs.push_back(m.prec);
  std::sort(precs.begin(), precs.end());

  std::vector<std::vector<int2>> lists;
  im.groups.clear();
  for (int prec : precs) {
    Plan::Group g;
    g.prec = prec;
    for (int ph = 0; ph < 3; ++ph) {
      const int blocks = cus_per_xcd * per_cu_blocks(prec);
      lists.push_back(xcd_lists(phase_tiles(hm, order, prec, ph), &g.per_xcd[ph], blocks));
      g.tiles[ph] = nullptr;
    }
    im.groups.push_back(g);
  }

  size_t off = 0;
  im.off_mats = off;
  off = align256(off + sizeof(MatDev) * count);
  im.off_etile = off;
  off = align256(off + sizeof(int32_t) * (count + 1));
  im.off_scal = off;
  off = align256(off + sizeof(MatScal) * count);
  im.off_part = off;
  off = align256(off + sizeof(float) * size_t(std::max<int64_t>(etile_off[count], 1)));
  im.off_wb = off;
  off = align256(off + sizeof(float2) * count);
  im.off_lists.clear();
  for (auto& l : lists) {
    im.off_lists.push_back(off);
    off = align256(off + sizeof(int2) * std::max<size_t>(l.size(), 1));
  }
  im.host.assign(off, 0);
  memcpy(im.host.data() + im.off_mats, hm.data(), sizeof(MatDev) * count);
  memcpy(im.host.data() + im.off_etile, etile_off.data(), sizeof(int32_t) * (count + 1));
  for (size_t i = 0; i < lists.size(); ++i)
    memcpy(im.host.data() + im.off_lists[i], lists[i].data(), sizeof(int2) * lists[i].size());
}

// Points `plan` at the tables of `im` uploaded to device memory `base`.
void bind_plan(Plan* plan, const PlanImage& im, char* base, const std::vector<MatDev>& hm,
               const std::vector<int32_t>& etile_off) {
  const int32_t count = int32_t(hm.size());
  plan->count = count;
  plan->total_etiles = etile_off[count];
  plan->d_mats = reinterpret_cast<MatDev*>(base + im.off_mats);
  plan->d_etile_off = reinterpret_cast<int32_t*>(base + im.off_etile);
  plan->d_scal = reinterpret_cast<MatScal*>(base + im.off_scal);
  plan->d_partials = reinterpret_cast<float*>(base + im.off_part);
  plan->d_wb = reinterpret_cast<float2*>(base + im.off_wb);
  plan->groups = im.groups;
  size_t li = 0;
  for (auto& g : plan->groups)
    for (int ph = 0; ph < 3; ++ph) g.tiles[ph] = reinterpret_cast<int2*>(base + im.off_lists[li++]);
  plan->host_mats = hm;
  plan->chains.resize(plan->groups.size());
  for (size_t gi = 0; gi < plan->groups.size(); ++gi) plan->chains[gi].prec = plan->groups[gi].prec;
}

muon_status build_plan(Plan* plan, const std::vector<MatDev>& hm, const std::vector<int32_t>& etile_off,
                       int cus_per_xcd, hipStream_t stream) {
  PlanImage im;
  plan_image(hm, etile_off, cus_per_xcd, im);
  const size_t bytes = im.host.size();
  void* dmem = nullptr;
  if (device_alloc(&dmem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_OUT_OF_MEMORY, "plan allocation of %zu bytes failed", bytes);
  }
  if (hipMemcpyAsync(dmem, im.host.data(), bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipFree(dmem);
    return fail(MUON_ERR_HIP, "plan upload failed: %s", hipGetErrorString(hipGetLastError()));
  }
  plan->dmem = dmem;
  bind_plan(plan, im, reinterpret_cast<char*>(dmem), hm, etile_off);
  if (hipEventCreateWithFlags(&plan->last_use, hipEventDisableTiming) != hipSuccess) {
    plan->last_use = nullptr;
    return fail(MUON_ERR_HIP, "hipEventCreate failed");
  }
  return MUON_OK;
}

// ------------------------------------------------------------ chain plan
// Polls (about 1 us each) before a chain dependency wait gives up: 2^20, or
// MUON_CHAIN_SPIN_LIMIT from the environment (read per call), which tests
// set very low to drive the give-up path from the host.
int64_t chain_spin_limit() {
  const char* e = std::getenv("MUON_CHAIN_SPIN_LIMIT");
  if (e && *e) {
    char* end = nullptr;
    const long long v = std::strtoll(e, &end, 10);
    if (end && *end == '\0' && v >= 0) return int64_t(v);
  }
  return int64_t(1) << 20;
}


// GRAM tiles of a matrix in working format `prec` (the phase that fills
// the grid least in the d24-like stacks).
int64_t gram_tiles_of(const muon_matrix_desc& d, int prec) {
  const int64_t tm = geom_of(d).Mp / ns_tile(prec);
  return tm * (tm + 1) / 2;
}

// Chain workspace of one matrix for k steps: iterates X_1 .. X_{k-1} (X_0 is
// the momentum kernel's output in the main workspace) and A, B per step.
size_t chain_bytes(const MatGeom& g, int k) { return size_t(k - 1) * g.x_bytes + size_t(2 * k) * g.a_bytes; }

// Builds the persistent chain of precision group `gi` for `k` steps whose
// c == 0 pattern is `cmask` (bit it set: step it has c == 0, so POLY is
// skipped and GRAM stores B = b A).  `use` marks the matrices of the call
// that take the chain; their step buffers start at `chain_ws`.
muon_status build_chain(Plan* plan, size_t gi, int k, uint32_t cmask, char* chain_ws,
                        const std::vector<MatGeom>& geo, hipStream_t stream) {
  Plan::Chain& ch = plan->chains[gi];
  if (ch.dmem) {
    (void)hipFree(ch.dmem);
    ch.dmem = nullptr;
  }
  const int prec = ch.prec;
  const std::vector<MatDev>& hm = plan->host_mats;
  const int32_t count = int32_t(hm.size());
  // per (step, matrix) descriptors with the step's own buffers
  std::vector<MatDev> im(size_t(k) * count);
  size_t wo = 0;
  for (int32_t i = 0; i < count; ++i) {
    const bool mine = hm[i].prec == prec;
    char* base = chain_ws + wo;
    if (mine) wo += chain_bytes(geo[i], k);
    for (int it = 0; it < k; ++it) {
      MatDev m = hm[i];
      if (mine) {
        auto xbuf = [&](int j) -> void* { return j == 0 ? hm[i].X[0] : base + size_t(j - 1) * geo[i].x_bytes; };
        m.X[0] = xbuf(it);
        m.X[1] = it + 1 < k ? xbuf(it + 1) : nullptr;
        m.A = base + size_t(k - 1) * geo[i].x_bytes + size_t(2 * it) * geo[i].a_bytes;
        m.B = reinterpret_cast<char*>(m.A) + geo[i].a_bytes;
      }
      im[size_t(it) * count + i] = m;
    }
  }
  // work items: phase instances in order, each split into XCD-local runs
  const std::vector<int> order = cost_order(hm);
  // done counter of (step, phase, matrix): index into the counters that
  // follow the CHAIN_SYNC_HEAD words of queue heads and abort flag
  auto counter = [&](int it, int ph, int mat) { return (it * 3 + ph) * count + mat; };
  std::vector<std::vector<ChainItem>> q(NUM_XCD);
  std::vector<int32_t> ntiles(size_t(3) * count, 0);   // tiles per (phase, matrix)
  for (int ph = 0; ph < 3; ++ph)
    for (const TileSrc& t : phase_tiles(hm, order, prec, ph)) ++ntiles[size_t(ph) * count + t.mat];
  for (int it = 0; it < k; ++it) {
    const bool cz = (cmask >> it) & 1u;
    for (int ph = 0; ph < 3; ++ph) {
      if (ph == PH_POLY && cz) continue;
      int32_t per = 0;
      const std::vector<int2> lists = xcd_lists(phase_tiles(hm, order, prec, ph), &per);
      for (int x = 0; x < NUM_XCD; ++x)
        for (int32_t j = 0; j < per; ++j) {
          const int2 e = lists[size_t(x) * per + j];
          if (e.x < 0) continue;
          const int mat = e.x;
          ChainItem ci;
          ci.desc = it * count + mat;
          ci.mat = mat;
          ci.step = it;
          ci.tile = e.y;
          ci.signal = counter(it, ph, mat);
          if (ph == PH_GRAM) {
            ci.kind = cz ? CHAIN_GRAM_B : CHAIN_GRAM_A;
            ci.wait = it == 0 ? -1 : counter(it - 1, PH_COMB, mat);
            ci.need = it == 0 ? 0 : ntiles[size_t(PH_COMB) * count + mat];
          } else if (ph == PH_POLY) {
            ci.kind = CHAIN_POLY;
            ci.wait = counter(it, PH_GRAM, mat);
            ci.need = ntiles[size_t(PH_GRAM) * count + mat];
          } else {
            ci.kind = it == k - 1 ? CHAIN_COMB_LAST : CHAIN_COMB;
            const int prev = cz ? PH_GRAM : PH_POLY;
            ci.wait = counter(it, prev, mat);
            ci.need = ntiles[size_t(prev) * count + mat];
          }
          q[x].push_back(ci);
        }
    }
  }
  std::vector<int32_t> xoff(NUM_XCD + 1, 0);
  int32_t mx = 0;
  for (int x = 0; x < NUM_XCD; ++x) {
    xoff[x + 1] = xoff[x] + int32_t(q[x].size());
    mx = std::max(mx, int32_t(q[x].size()));
  }
  const int32_t nitems = xoff[NUM_XCD];
  const int32_t nsync = CHAIN_SYNC_HEAD + 3 * k * count;
  size_t off = 0;
  const size_t o_im = off;
  off = align256(off + sizeof(MatDev) * im.size());
  const size_t o_items = off;
  off = align256(off + sizeof(ChainItem) * std::max(nitems, 1));
  const size_t o_xoff = off;
  off = align256(off + sizeof(int32_t) * (NUM_XCD + 1));
  const size_t o_steps = off;
  off = align256(off + sizeof(PhaseArgs) * MAX_CHAIN_STEPS);
  const size_t o_sync = off;
  off = align256(off + sizeof(int32_t) * nsync);
  void* dmem = nullptr;
  if (device_alloc(&dmem, off) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_OUT_OF_MEMORY, "chain plan allocation of %zu bytes failed", off);
  }
  std::vector<char> host(off, 0);
  memcpy(host.data() + o_im, im.data(), sizeof(MatDev) * im.size());
  for (int x = 0; x < NUM_XCD; ++x)
    memcpy(host.data() + o_items + sizeof(ChainItem) * xoff[x], q[x].data(), sizeof(ChainItem) * q[x].size());
  memcpy(host.data() + o_xoff, xoff.data(), sizeof(int32_t) * (NUM_XCD + 1));
  if (hipMemcpyAsync(dmem, host.data(), off, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipFree(dmem);
    return fail(MUON_ERR_HIP, "chain plan upload failed: %s", hipGetErrorString(hipGetLastError()));
  }
  char* b = reinterpret_cast<char*>(dmem);
  ch.dmem = dmem;
  ch.d_imats = reinterpret_cast<MatDev*>(b + o_im);
  ch.d_items = reinterpret_cast<ChainItem*>(b + o_items);
  ch.d_xcd_off = reinterpret_cast<int32_t*>(b + o_xoff);
  ch.d_steps = reinterpret_cast<PhaseArgs*>(b + o_steps);
  ch.d_sync = reinterpret_cast<int32_t*>(b + o_sync);
  ch.nsync = nsync;
  ch.per_xcd_max = mx;
  return MUON_OK;
}

struct Call {
  Mode mode;
  void* const* params;
  const void* const* grads;
  void* const* momenta;
  float* const* updates;
  const muon_matrix_desc* shapes;
  int32_t count;
  float lr, beta;
  int32_t nesterov;
  muon_ns_coeffs co;
  int32_t ns_steps;
  int32_t scale_rule;
  const muon_step_options* opt;  // update variants (MODE_STEP), or null
  float* norms_out;
  hipStream_t stream;
};

// Scale s of the update from the rule, in binary64 (the device computes the
// same in update_scale).
double rule_scale(int rule, int64_t rows, int64_t cols) {
  if (rule == MUON_SCALE_SQRT_ASPECT) return std::sqrt(std::max(1.0, double(rows) / double(cols)));
  if (rule == MUON_SCALE_RMS_MATCH) return 0.2 * std::sqrt(double(std::max(rows, cols)));
  return 1.0;
}

// The products add a X and (b/c) A on the matrix cores, each scale split into
// bfloat16 hi + lo parts of its binary32 value, and B = c (A A + (b/c) A).  A
// triple is usable when a and, for c != 0, fl32(b/c) are finite and round to a
// finite bfloat16 hi part (magnitude below 0x7F7F8000 as binary32, about
// 3.3961e38): a subnormal c beside an ordinary b gives b/c = +-inf, whose
// split would fill B with NaN.
bool split_ok(float v) {
  const uint32_t lim = 0x7F7F8000u;
  float fl;
  memcpy(&fl, &lim, sizeof(fl));
  return std::isfinite(v) && std::fabs(v) < fl;
}

muon_status check_triple(const muon_ns_coeffs& co, const char* what, int k) {
  if (!std::isfinite(co.a) || !std::isfinite(co.b) || !std::isfinite(co.c))
    return fail(MUON_ERR_INVALID_ARGUMENT, "%s[%d] is not finite", what, k);
  if (!split_ok(co.a))
    return fail(MUON_ERR_UNSUPPORTED, "%s[%d]: a = %g is too large to split into bfloat16 hi + lo", what, k,
                double(co.a));
  if (co.c != 0.f) {
    const float q = co.b / co.c;
    if (!split_ok(q))
      return fail(MUON_ERR_UNSUPPORTED, "%s[%d]: b/c = %g/%g is %g in binary32, too large to split into bfloat16 "
                  "hi + lo", what, k, double(co.b), double(co.c), double(q));
  }
  return MUON_OK;
}

// Whether the write-back takes per-matrix scalars from the host.
bool per_matrix_wb(const Call& c) {
  return c.opt && (c.opt->weight_decay != 0.f || c.opt->lr_per_matrix || c.opt->scale_per_matrix);
}

muon_status validate_call(const Call& c) {
  if (c.count < 0 || c.count > MAX_COUNT)
    return fail(MUON_ERR_INVALID_ARGUMENT, "count %d out of range [0, %d]", c.count, MAX_COUNT);
  if (c.count == 0) return MUON_OK;
  if (!c.shapes) return fail(MUON_ERR_INVALID_ARGUMENT, "shapes is NULL");
  if (!c.grads) return fail(MUON_ERR_INVALID_ARGUMENT, "grads (x_in) is NULL");
  if (c.mode == MODE_STEP) {
    if (!c.params || !c.momenta) return fail(MUON_ERR_INVALID_ARGUMENT, "params or momenta is NULL");
    if (!std::isfinite(c.lr)) return fail(MUON_ERR_INVALID_ARGUMENT, "lr is not finite");
    if (!(c.beta >= 0.f && c.beta < 1.f)) return fail(MUON_ERR_INVALID_ARGUMENT, "beta must be in [0, 1)");
    if (c.nesterov != 0 && c.nesterov != 1) return fail(MUON_ERR_INVALID_ARGUMENT, "nesterov must be 0 or 1");
    if (c.scale_rule < MUON_SCALE_NONE || c.scale_rule > MUON_SCALE_RMS_MATCH)
      return fail(MUON_ERR_INVALID_ARGUMENT, "unknown scale_rule %d", c.scale_rule);
  }
  if (c.opt && c.mode == MODE_STEP) {
    const muon_step_options& o = *c.opt;
    if (!std::isfinite(o.weight_decay) || o.weight_decay < 0.f)
      return fail(MUON_ERR_INVALID_ARGUMENT, "weight_decay must be finite and >= 0");
    if (o.momentum_kind != MUON_MOMENTUM_HEAVY_BALL && o.momentum_kind != MUON_MOMENTUM_EMA)
      return fail(MUON_ERR_INVALID_ARGUMENT, "unknown momentum_kind %d", o.momentum_kind);
    if (o.launch_mode < MUON_LAUNCH_AUTO || o.launch_mode > MUON_LAUNCH_CHAIN)
      return fail(MUON_ERR_INVALID_ARGUMENT, "unknown launch_mode %d", o.launch_mode);
    if (o.tile_mode < MUON_TILES_AUTO || o.tile_mode > MUON_TILES_SMALL)
      return fail(MUON_ERR_INVALID_ARGUMENT, "unknown tile_mode %d", o.tile_mode);
    if (o.launch_mode == MUON_LAUNCH_CHAIN && c.ns_steps > MAX_CHAIN_STEPS)
      return fail(MUON_ERR_UNSUPPORTED, "the persistent chain takes at most %d Newton-Schulz steps", MAX_CHAIN_STEPS);
    if (o.ns_schedule)
      for (int32_t k = 0; k < c.ns_steps; ++k) {
        const muon_status st = check_triple(o.ns_schedule[k], "ns_schedule", k);
        if (st != MUON_OK) return st;
      }
    for (int32_t i = 0; i < c.count; ++i) {
      if (o.lr_per_matrix && !std::isfinite(o.lr_per_matrix[i]))
        return fail(MUON_ERR_INVALID_ARGUMENT, "lr_per_matrix[%d] is not finite", i);
      if (o.scale_per_matrix && !std::isfinite(o.scale_per_matrix[i]))
        return fail(MUON_ERR_INVALID_ARGUMENT, "scale_per_matrix[%d] is not finite", i);
    }
  }
  if (c.mode == MODE_NS && !c.updates) return fail(MUON_ERR_INVALID_ARGUMENT, "x_out is NULL");
  if (c.mode == MODE_NORMS && !c.norms_out) return fail(MUON_ERR_INVALID_ARGUMENT, "norms_out is NULL");
  if (c.mode != MODE_NORMS) {
    if (c.ns_steps < 0 || c.ns_steps > MAX_NS_STEPS)
      return fail(MUON_ERR_INVALID_ARGUMENT, "ns_steps %d out of range [0, %d]", c.ns_steps, MAX_NS_STEPS);
    if (!std::isfinite(c.co.a) || !std::isfinite(c.co.b) || !std::isfinite(c.co.c))
      return fail(MUON_ERR_INVALID_ARGUMENT, "ns_coeffs must be finite");
    const bool sched = c.mode == MODE_STEP && c.opt && c.opt->ns_schedule;
    if (!sched && c.ns_steps > 0) {
      const muon_status st = check_triple(c.co, "ns_coeffs", 0);
      if (st != MUON_OK) return st;
    }
  }
  muon_status st = validate_desc(c.shapes, c.count, c.mode);
  if (st != MUON_OK) return st;

  std::vector<Interval> iv;
  iv.reserve(size_t(c.count) * 4);
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_matrix_desc& d = c.shapes[i];
    const int gsz = dtype_size(d.grad_dtype);
    if ((st = check_ptr(c.grads[i], gsz, i, c.mode == MODE_STEP ? "grad" : "x_in")) != MUON_OK) return st;
    uintptr_t g = reinterpret_cast<uintptr_t>(c.grads[i]);
    iv.push_back({g, g + span_bytes(d.rows, d.cols, d.ld_grad, gsz), false, i, "grad"});
    if (c.mode == MODE_STEP) {
      const int psz = dtype_size(d.param_dtype);
      if ((st = check_ptr(c.params[i], psz, i, "param")) != MUON_OK) return st;
      if ((st = check_ptr(c.momenta[i], 4, i, "momentum")) != MUON_OK) return st;
      uintptr_t p = reinterpret_cast<uintptr_t>(c.params[i]);
      uintptr_t m = reinterpret_cast<uintptr_t>(c.momenta[i]);
      iv.push_back({p, p + span_bytes(d.rows, d.cols, d.ld_param, psz), true, i, "param"});
      iv.push_back({m, m + span_bytes(d.rows, d.cols, d.ld_mom, 4), true, i, "momentum"});
    }
    if (c.updates && c.updates[i]) {
      if ((st = check_ptr(c.updates[i], 4, i, "update")) != MUON_OK) return st;
      uintptr_t u = reinterpret_cast<uintptr_t>(c.updates[i]);
      iv.push_back({u, u + span_bytes(d.rows, d.cols, d.cols, 4), true, i, "update"});
    } else if (c.mode == MODE_NS) {
      return fail(MUON_ERR_INVALID_ARGUMENT, "matrix %d: x_out pointer is NULL", i);
    }
  }
  if (c.mode == MODE_NORMS) {
    uintptr_t n = reinterpret_cast<uintptr_t>(c.norms_out);
    if (n % 4 != 0) return fail(MUON_ERR_UNSUPPORTED, "norms_out is not 4-byte aligned");
    iv.push_back({n, n + sizeof(float) * size_t(c.count), true, -1, "norms_out"});
  }
  return check_alias_fast(iv);
}

bool vec_aligned(const void* p, int64_t ld, int esz) {
  return (reinterpret_cast<uintptr_t>(p) % uintptr_t(4 * esz) == 0) && (ld % 4 == 0);
}

// The calling thread's current device and its state (g_mu held): compute
// units per XCD, and the give-up flag of an earlier persistent chain.
muon_status acquire_device(DeviceState** out, int* dev_out = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_HIP, "hipGetDevice failed (no HIP device?)");
  }
  DeviceState& ds = g_dev[dev];
  *out = &ds;
  if (dev_out) *dev_out = dev;
  if (ds.cus_per_xcd == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return fail(MUON_ERR_HIP, "cannot query the compute-unit count of device %d", dev);
    }
    ds.cus_per_xcd = std::max(1, cus / NUM_XCD);
  }

  // a persistent chain of an earlier call whose dependency wait timed out
  if (!ds.fail_flag) {
    void* f = nullptr;
    if (hipHostMalloc(&f, sizeof(int32_t), hipHostMallocCoherent) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MUON_ERR_OUT_OF_MEMORY, "pinned failure flag allocation failed");
    }
    ds.fail_flag = reinterpret_cast<int32_t*>(f);
    *ds.fail_flag = 0;
  }
  // the flag is final once the chain that may raise it has ended
  if (ds.chain_pending) {
    if (hipEventSynchronize(ds.chain_done) != hipSuccess)
      return fail(MUON_ERR_HIP, "waiting for the earlier persistent Newton-Schulz launch failed: %s",
                  hipGetErrorString(hipGetLastError()));
    ds.chain_pending = false;
  }
  if (__atomic_load_n(ds.fail_flag, __ATOMIC_ACQUIRE) != 0) {
    __atomic_store_n(ds.fail_flag, 0, __ATOMIC_RELEASE);
    return fail(MUON_ERR_HIP, "an earlier persistent Newton-Schulz launch on this device gave up waiting for a "
                "dependency; the results of that call are invalid");
  }
  return MUON_OK;
}

// Working format of each matrix (a Prec) for a call of `mode` with tile mode
// `tmode` on a GPU with `cus` compute units.
std::vector<int> working_formats(const muon_matrix_desc* shapes, int32_t count, Mode mode, int32_t tmode,
                                 int64_t cus) {
  std::vector<int> iprec(size_t(count), PREC_BF16);
  if (mode != MODE_NORMS) {
    int64_t bf16_gram = 0, f32_gram = 0, x3_gram = 0;
    for (int32_t i = 0; i < count; ++i) {
      if (shapes[i].precision == MUON_NS_BF16) bf16_gram += gram_tiles_of(shapes[i], PREC_BF16);
      if (shapes[i].precision == MUON_NS_F32) f32_gram += gram_tiles_of(shapes[i], PREC_F32);
      if (shapes[i].precision == MUON_NS_BF16X3) x3_gram += gram_tiles_of(shapes[i], PREC_BF16X3);
    }
    const bool small_bf16 = tmode == MUON_TILES_SMALL || (tmode == MUON_TILES_AUTO && bf16_gram < cus);
    const bool small_f32 = tmode == MUON_TILES_SMALL || (tmode == MUON_TILES_AUTO && f32_gram < cus);
    const bool small_x3 = tmode == MUON_TILES_SMALL || (tmode == MUON_TILES_AUTO && x3_gram < cus);
    for (int32_t i = 0; i < count; ++i) {
      const int p = shapes[i].precision;
      iprec[size_t(i)] = (p == MUON_NS_BF16 && small_bf16) ? int(PREC_BF16S)
                         : (p == MUON_NS_F32 && small_f32) ? int(PREC_F32S)
                         : (p == MUON_NS_BF16X3 && small_x3) ? int(PREC_BF16X3S)
                                                             : p;
    }
  }
  return iprec;
}

// Device descriptors of the call's matrices with workspace buffers laid out
// from `ws`, and the elementwise tiles' offsets.
muon_status host_mats(const Call& c, const std::vector<int>& iprec, char* ws, std::vector<MatDev>& hm,
                      std::vector<int32_t>& etile_off) {
  hm.assign(size_t(c.count), MatDev{});
  etile_off.assign(size_t(c.count) + 1, 0);
  size_t wo = 0;
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_matrix_desc& d = c.shapes[i];
    MatGeom g = geom_of(d);
    MatDev& m = hm[i];
    memset(&m, 0, sizeof(m));
    m.param = c.mode == MODE_STEP ? c.params[i] : nullptr;
    m.grad = c.grads[i];
    m.mom = c.mode == MODE_STEP ? reinterpret_cast<float*>(c.momenta[i]) : nullptr;
    m.upd = c.updates ? c.updates[i] : nullptr;
    m.ld_param = d.ld_param;
    m.ld_grad = d.ld_grad;
    m.ld_mom = d.ld_mom;
    m.ld_upd = d.cols;
    m.rows = int32_t(d.rows);
    m.cols = int32_t(d.cols);
    m.m = int32_t(g.m);
    m.n = int32_t(g.n);
    m.Mp = int32_t(g.Mp);
    m.Np = int32_t(g.Np);
    m.ldx = int32_t(g.ldx);
    m.lda = int32_t(g.lda);
    m.transposed = g.transposed ? 1 : 0;
    m.param_bf16 = (c.mode == MODE_STEP && d.param_dtype == MUON_DTYPE_BF16) ? 1 : 0;
    m.grad_bf16 = d.grad_dtype == MUON_DTYPE_BF16 ? 1 : 0;
    bool vec = vec_aligned(c.grads[i], d.ld_grad, dtype_size(d.grad_dtype));
    if (c.mode == MODE_STEP) vec = vec && vec_aligned(c.momenta[i], d.ld_mom, 4);
    m.vec_ok = vec ? 1 : 0;
    if (c.mode == MODE_STEP) {
      const int psz = dtype_size(d.param_dtype);
      // rows start 16-byte aligned; columns go in groups of 8 from a multiple of 8
      m.wvec_ok = (reinterpret_cast<uintptr_t>(c.params[i]) % 16 == 0 && (d.ld_param * psz) % 16 == 0) ? 1 : 0;
    }
    if (m.upd) m.uvec_ok = (reinterpret_cast<uintptr_t>(m.upd) % 16 == 0 && d.cols % 4 == 0) ? 1 : 0;
    m.prec = c.mode == MODE_NORMS ? int(PREC_BF16) : iprec[size_t(i)];
    const int64_t rp = g.transposed ? g.Np : g.Mp;  // natural padded rows
    const int64_t cp = g.transposed ? g.Mp : g.Np;  // natural padded cols
    // elementwise tiles: TBF_R x TBF_C for tall matrices in bf16, ETILE x
    // ETILE for the other tall ones, RTILE_R x RTILE_C for the rest (all
    // divide the 256-padded shape)
    const bool tbf = g.transposed && m.prec == int(PREC_BF16);
    const int64_t th = g.transposed ? (tbf ? TBF_R : ETILE) : RTILE_R;
    const int64_t tw = g.transposed ? (tbf ? TBF_C : ETILE) : RTILE_C;
    m.etile_cols = int32_t(cp / tw);
    etile_off[i + 1] = etile_off[i] + int32_t((rp / th) * (cp / tw));
    if (c.mode != MODE_NORMS) {
      m.plane_X = g.Mp * g.ldx;
      m.plane_A = g.Mp * g.lda;
      m.X[0] = ws + wo; wo += g.x_bytes;
      m.X[1] = ws + wo; wo += g.x_bytes;
      m.A = ws + wo; wo += g.a_bytes;
      m.B = ws + wo; wo += g.a_bytes;
    }
  }
  if (int64_t(etile_off[c.count]) >= (int64_t(1) << 31) - 1)
    return fail(MUON_ERR_UNSUPPORTED, "too many elements in one call");
  return MUON_OK;
}

// Launch plan of the call's matrices with workspace buffers laid out from
// `ws` (device tables uploaded on c.stream, which is synchronised).
muon_status new_plan(const Call& c, const std::vector<int>& iprec, char* ws, int cus_per_xcd, Plan** out) {
  std::vector<MatDev> hm;
  std::vector<int32_t> etile_off;
  muon_status hs = host_mats(c, iprec, ws, hm, etile_off);
  if (hs != MUON_OK) return hs;
  Plan* plan = new Plan();
  const muon_status st = build_plan(plan, hm, etile_off, cus_per_xcd, c.stream);
  if (st != MUON_OK) {
    if (plan->dmem) (void)hipFree(plan->dmem);
    delete plan;
    return st;
  }
  *out = plan;
  return MUON_OK;
}

// Enqueues the launch sequence of one step of `c` with `plan` on c.stream:
// after the device's previous call and, when given, after `ready`.  `plain`
// (the allocation-free entry point): no ordering, timing or plan events, no
// per-matrix table (c has no options) and no persistent chain, so nothing
// here creates an event or allocates.
muon_status enqueue_step(DeviceState& ds, Plan* plan, const Call& c, const std::vector<int>& iprec,
                         std::map<int, bool>& use_chain, hipEvent_t ready, bool plain = false) {
  hipError_t e = plain ? hipSuccess : order_after_last_call(ds, c.stream);
  if (e == hipSuccess && ready) e = hipStreamWaitEvent(c.stream, ready, 0);
  muon_status st = MUON_OK;
  const int kmode = c.mode == MODE_STEP ? 0 : (c.mode == MODE_NS ? 1 : 2);
  const int32_t ema = (c.mode == MODE_STEP && c.opt && c.opt->momentum_kind == MUON_MOMENTUM_EMA) ? 1 : 0;
  // per-matrix write-back scalars t_i = fl32(lr_i * s_i), d_i = fl32(1 - fl32(lr_i * wd))
  const float2* wb = nullptr;
  if (e == hipSuccess && c.mode == MODE_STEP && per_matrix_wb(c)) {
    std::vector<float2> hwb(size_t(c.count));
    for (int32_t i = 0; i < c.count; ++i) {
      const float lr_i = c.opt->lr_per_matrix ? c.opt->lr_per_matrix[i] : c.lr;
      const double s_i = c.opt->scale_per_matrix ? double(c.opt->scale_per_matrix[i])
                                                 : rule_scale(c.scale_rule, c.shapes[i].rows, c.shapes[i].cols);
      const float decay = c.opt->weight_decay;
      const float lw = lr_i * decay;
      hwb[size_t(i)] = make_float2(float(double(lr_i) * s_i), decay != 0.f ? 1.f - lw : 1.f);
    }
    e = staged_copy(ds, plan->d_wb, hwb.data(), sizeof(float2) * size_t(c.count), c.stream);
    wb = plan->d_wb;
  }
  if (e == hipSuccess)
    e = timed_unless(plain, MUON_KC_MOMENTUM, c.stream, [&] {
      return launch_momentum(plan->d_mats, plan->d_etile_off, plan->count, plan->total_etiles, c.beta,
                             c.nesterov, ema, kmode, plan->d_partials, c.stream);
    });
  if (e == hipSuccess)
    e = timed_unless(plain, MUON_KC_NORM, c.stream, [&] {
      return launch_norm_finalize(plan->d_etile_off, plan->count, plan->d_partials, plan->d_scal,
                                  c.mode == MODE_NORMS ? c.norms_out : nullptr, c.stream);
    });
  if (e == hipSuccess && c.mode != MODE_NORMS) {
    if (c.ns_steps == 0) {
      e = timed_unless(plain, MUON_KC_WRITEBACK, c.stream, [&] {
        return launch_writeback_direct(plan->d_mats, plan->d_etile_off, plan->count, plan->total_etiles,
                                       plan->d_scal, c.lr, c.scale_rule, wb, c.stream);
      });
    } else {
      // step coefficients and the c == 0 pattern
      std::vector<muon_ns_coeffs> cos(size_t(c.ns_steps));
      uint32_t cmask = 0;
      for (int it = 0; it < c.ns_steps; ++it) {
        cos[size_t(it)] = (c.opt && c.opt->ns_schedule) ? c.opt->ns_schedule[it] : c.co;
        if (cos[size_t(it)].c == 0.f && it < 32) cmask |= 1u << it;
      }
      // precision groups that run as one persistent chain
      std::vector<MatGeom> geo;
      for (size_t gi = 0; gi < plan->groups.size() && e == hipSuccess; ++gi) {
        const int prec = plan->groups[gi].prec;
        if (!use_chain[prec]) continue;
        Plan::Chain& ch = plan->chains[gi];
        const std::vector<uint64_t> ckey = {uint64_t(c.ns_steps), uint64_t(cmask),
                                            reinterpret_cast<uint64_t>(ds.chain_ws)};
        if (ch.key != ckey || !ch.dmem) {
          if (geo.empty())
            for (int32_t i = 0; i < c.count; ++i) geo.push_back(geom_of(c.shapes[i]));
          // chain buffers of the earlier precision groups come first
          size_t base = 0;
          for (int32_t i = 0; i < c.count; ++i)
            if (iprec[size_t(i)] < prec && use_chain[iprec[size_t(i)]]) base += chain_bytes(geo[i], c.ns_steps);
          ch.key.clear();
          st = build_chain(plan, gi, c.ns_steps, cmask, reinterpret_cast<char*>(ds.chain_ws) + base, geo, c.stream);
          if (st != MUON_OK) return st;
          ch.key = ckey;
        }
        ChainArgs ca;
        memset(&ca, 0, sizeof(ca));
        for (int it = 0; it < c.ns_steps; ++it) {
          ca.a[it] = cos[size_t(it)].a;
          ca.b[it] = cos[size_t(it)].b;
          ca.c[it] = cos[size_t(it)].c;
        }
        ca.lr = c.lr;
        ca.steps = c.ns_steps;
        ca.scale_rule = c.scale_rule;
        ca.cus_per_xcd = ds.cus_per_xcd;
        ca.wb = wb;
        ca.spin_limit = chain_spin_limit();
        e = timed_unless(plain, MUON_KC_CHAIN, c.stream, [&] {
          return launch_ns_chain(prec, ch.d_imats, plan->d_scal, ch.d_items, ch.d_xcd_off, ch.per_xcd_max,
                                 ch.d_steps, ch.d_sync, ch.nsync, ds.fail_flag, ca, c.stream);
        });
        if (e == hipSuccess) {
          if (!ds.chain_done && hipEventCreateWithFlags(&ds.chain_done, hipEventDisableTiming) != hipSuccess) {
            ds.chain_done = nullptr;
            e = hipGetLastError();
          }
          if (e == hipSuccess) e = hipEventRecord(ds.chain_done, c.stream);
          if (e == hipSuccess) ds.chain_pending = true;
        }
      }
      for (int it = 0; it < c.ns_steps && e == hipSuccess; ++it) {
        const muon_ns_coeffs co = cos[size_t(it)];
        PhaseArgs pa;
        pa.a = co.a;
        pa.b = co.b;
        pa.c = co.c;
        pa.wb = wb;
        pa.lr = c.lr;
        pa.cur = it & 1;
        pa.first = it == 0;
        pa.last = it == c.ns_steps - 1;
        pa.scale_rule = c.scale_rule;
        pa.cus_per_xcd = ds.cus_per_xcd;
        for (const auto& g : plan->groups) {
          if (use_chain[g.prec]) continue;
          for (int ph = 0; ph < 3 && e == hipSuccess; ++ph) {
            if (ph == PH_POLY && co.c == 0.f) continue;  // GRAM already formed B = b A
            pa.per_xcd = g.per_xcd[ph];
            e = timed_unless(plain, MUON_KC_GRAM + ph, c.stream, [&] {
              return launch_ns_phase(g.prec, ph, plan->d_mats, plan->d_scal, g.tiles[ph], pa, c.stream);
            });
          }
        }
      }
    }
  }
  if (e != hipSuccess) return fail(MUON_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (!plain) {
    (void)hipEventRecord(plan->last_use, c.stream);
    record_last_call(ds, c.stream);
  }
  return MUON_OK;
}

muon_status run(const Call& c) {
  t_last_error.clear();
  muon_status st = validate_call(c);
  if (st != MUON_OK || c.count == 0) return st;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState* dsp = nullptr;
  if ((st = acquire_device(&dsp)) != MUON_OK) return st;
  DeviceState& ds = *dsp;

  // working format per matrix: a bf16 stack whose GRAM phase has fewer
  // 256 x 256 tiles than the GPU has compute units takes 128 x 128 tiles
  // (measured: 12 x 768^2 0.41 -> 0.34 ms per step; with three d24 layers,
  // 378 GRAM tiles, the pipelined 256 x 256 tiles stay faster), and a
  // binary32 stack with fewer 128 x 128 GRAM tiles than that takes 64 x 64
  // tiles (one 256 x 256 matrix: 3 GRAM tiles of 128, 10 of 64)
  const int32_t tmode = (c.mode == MODE_STEP && c.opt) ? c.opt->tile_mode : MUON_TILES_AUTO;
  const std::vector<int> iprec =
      working_formats(c.shapes, c.count, c.mode, tmode, int64_t(NUM_XCD) * ds.cus_per_xcd);

  // which working formats run as one persistent chain: only when asked for
  // (AUTO keeps the per-phase grids: measured on MI355X, the chain is slower
  // on every workload tried; it gives up the grids' cross-tile prefetch of
  // stage 0, pays a release per tile, and spills more)
  std::map<int, bool> use_chain;
  size_t chain_need = 0;
  if (c.mode != MODE_NORMS && c.ns_steps >= 1) {
    const int32_t lm = (c.mode == MODE_STEP && c.opt) ? c.opt->launch_mode : MUON_LAUNCH_AUTO;
    for (int32_t i = 0; i < c.count; ++i)
      use_chain[iprec[size_t(i)]] = c.ns_steps <= MAX_CHAIN_STEPS && lm == MUON_LAUNCH_CHAIN;
    for (int32_t i = 0; i < c.count; ++i)
      if (use_chain[iprec[size_t(i)]]) chain_need += chain_bytes(geom_of(c.shapes[i]), c.ns_steps);
  }

  // workspace
  const size_t need = c.mode == MODE_NORMS ? 0 : workspace_bytes(c.shapes, c.count);
  if (need > ds.ws_bytes) {
    if (hipDeviceSynchronize() != hipSuccess) {
      return fail(MUON_ERR_HIP, "hipDeviceSynchronize failed: %s", hipGetErrorString(hipGetLastError()));
    }
    drop_plans(ds);
    if (ds.ws) (void)hipFree(ds.ws);
    ds.ws = nullptr;
    ds.ws_bytes = 0;
    void* p = nullptr;
    if (device_alloc(&p, need) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MUON_ERR_OUT_OF_MEMORY, "workspace allocation of %zu bytes failed", need);
    }
    ds.ws = p;
    ds.ws_bytes = need;
  }
  if (chain_need > ds.chain_ws_bytes) {
    if (hipDeviceSynchronize() != hipSuccess) {
      return fail(MUON_ERR_HIP, "hipDeviceSynchronize failed: %s", hipGetErrorString(hipGetLastError()));
    }
    drop_plans(ds);
    if (ds.chain_ws) (void)hipFree(ds.chain_ws);
    ds.chain_ws = nullptr;
    ds.chain_ws_bytes = 0;
    void* p = nullptr;
    if (device_alloc(&p, chain_need) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MUON_ERR_OUT_OF_MEMORY, "chain workspace allocation of %zu bytes failed", chain_need);
    }
    ds.chain_ws = p;
    ds.chain_ws_bytes = chain_need;
  }

  // plan key
  std::vector<uint64_t> key;
  key.reserve(size_t(c.count) * 14 + 3);
  key.push_back(uint64_t(c.mode));
  key.push_back(uint64_t(c.count));
  key.push_back(reinterpret_cast<uint64_t>(ds.ws));
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_matrix_desc& d = c.shapes[i];
    key.push_back(reinterpret_cast<uint64_t>(c.grads[i]));
    key.push_back(c.mode == MODE_STEP ? reinterpret_cast<uint64_t>(c.params[i]) : 0);
    key.push_back(c.mode == MODE_STEP ? reinterpret_cast<uint64_t>(c.momenta[i]) : 0);
    key.push_back(c.updates ? reinterpret_cast<uint64_t>(c.updates[i]) : 0);
    key.push_back(uint64_t(d.rows));
    key.push_back(uint64_t(d.cols));
    key.push_back(uint64_t(d.ld_param));
    key.push_back(uint64_t(d.ld_grad));
    key.push_back(uint64_t(d.ld_mom));
    key.push_back((uint64_t(uint32_t(d.param_dtype)) << 32) | uint32_t(d.grad_dtype));
    key.push_back((uint64_t(uint32_t(d.mom_dtype)) << 32) | uint32_t(iprec[size_t(i)]));
  }
  Plan* plan = nullptr;
  for (auto it = ds.plans.begin(); it != ds.plans.end(); ++it) {
    if ((*it)->key == key) {
      plan = *it;
      ds.plans.erase(it);
      ds.plans.push_front(plan);
      break;
    }
  }
  if (!plan) {
    if ((st = new_plan(c, iprec, reinterpret_cast<char*>(ds.ws), ds.cus_per_xcd, &plan)) != MUON_OK) return st;
    plan->key = key;
    ds.plans.push_front(plan);
    while (ds.plans.size() > MAX_PLANS) {
      free_plan(ds.plans.back());
      ds.plans.pop_back();
    }
  }
  return enqueue_step(ds, plan, c, iprec, use_chain, nullptr);
}

// ------------------------------------------------------------ no allocation
// muon_step_batched_ex over the device's fixed scratch array: the workspace
// from its start, the launch tables after it, uploaded every call from a
// host image kept per device until the next call.  No plan cache, no events,
// no device or pinned allocation.
std::map<int, PlanImage> g_noalloc_image;

muon_status run_noalloc(const Call& c) {
  t_last_error.clear();
  muon_status st = validate_call(c);
  if (st != MUON_OK || c.count == 0) return st;
  const size_t ws_need = workspace_bytes(c.shapes, c.count);
  if (ws_need > NOALLOC_SCRATCH_BYTES)
    return fail(MUON_ERR_UNSUPPORTED,
                "the matrices need %zu bytes of Newton-Schulz workspace; the allocation-free entry point has a "
                "fixed %zu-byte scratch array per GPU (use muon_step_batched_ex)", ws_need,
                size_t(NOALLOC_SCRATCH_BYTES));
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return fail(MUON_ERR_HIP, "cannot query the current device");
  }
  void* scratch = nullptr;
  hipError_t e = noalloc_scratch(dev, &scratch);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_HIP, "cannot take the scratch array's address on device %d: %s", dev, hipGetErrorString(e));
  }
  const int cus_per_xcd = std::max(1, cus / NUM_XCD);
  const std::vector<int> iprec = working_formats(c.shapes, c.count, MODE_STEP, MUON_TILES_AUTO, int64_t(cus));
  char* base = reinterpret_cast<char*>(scratch);
  std::vector<MatDev> hm;
  std::vector<int32_t> etile_off;
  if ((st = host_mats(c, iprec, base, hm, etile_off)) != MUON_OK) return st;
  PlanImage& im = g_noalloc_image[dev];
  plan_image(hm, etile_off, cus_per_xcd, im);
  const size_t tables = align256(ws_need);
  if (tables + im.host.size() > NOALLOC_SCRATCH_BYTES)
    return fail(MUON_ERR_UNSUPPORTED,
                "the matrices need %zu bytes of workspace and %zu of launch tables; the allocation-free entry point "
                "has a fixed %zu-byte scratch array per GPU (use muon_step_batched_ex)", ws_need, im.host.size(),
                size_t(NOALLOC_SCRATCH_BYTES));
  e = hipMemcpyAsync(base + tables, im.host.data(), im.host.size(), hipMemcpyHostToDevice, c.stream);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, "launch table upload failed: %s", hipGetErrorString(e));
  Plan plan;
  bind_plan(&plan, im, base + tables, hm, etile_off);
  std::map<int, bool> use_chain;
  DeviceState& ds = g_dev[dev];
  if (ds.cus_per_xcd == 0) ds.cus_per_xcd = cus_per_xcd;   // sizes the persistent grids
  return enqueue_step(ds, &plan, c, iprec, use_chain, nullptr, true);
}

// ------------------------------------------------------------ stream plans
// One launch plan per group over a workspace of the plan's own; the working
// format of every matrix is fixed from the whole set at creation, so each
// matrix runs exactly the tile code one call over the whole set would run.
struct StreamGroup {
  std::vector<int32_t> members;          // indices in the whole set
  std::vector<muon_matrix_desc> shapes;  // argument arrays in group order
  std::vector<void*> params, moms;
  std::vector<const void*> grads;
  std::vector<float*> upd;
  std::vector<int> prec;                 // working format of each member
  Plan* plan = nullptr;
};

struct StreamPlanImpl {
  int dev = 0;
  int32_t count = 0;
  bool has_upd = false;
  std::vector<StreamGroup> groups;
  void* ws = nullptr;
};

void free_stream_plan(StreamPlanImpl* sp) {
  for (auto& g : sp->groups)
    if (g.plan) free_plan(g.plan);       // waits for the group's last use
  if (sp->ws) (void)hipFree(sp->ws);
  delete sp;
}

Call group_call(const StreamGroup& g, bool has_upd) {
  Call c{};
  c.mode = MODE_STEP;
  c.params = g.params.data();
  c.grads = g.grads.data();
  c.momenta = g.moms.data();
  c.updates = has_upd ? g.upd.data() : nullptr;
  c.shapes = g.shapes.data();
  c.count = int32_t(g.members.size());
  return c;
}

muon_status stream_plan_create(void* const* params, const void* const* grads, void* const* momenta,
                               const muon_matrix_desc* shapes, int32_t count, const int32_t* group_of,
                               int32_t ngroups, int32_t tile_mode, float* const* updates_out,
                               muon_stream_plan* plan_out) {
  t_last_error.clear();
  if (!plan_out) return fail(MUON_ERR_INVALID_ARGUMENT, "plan_out is NULL");
  *plan_out = nullptr;
  if (count < 1 || count > MAX_COUNT) return fail(MUON_ERR_INVALID_ARGUMENT, "count %d out of [1, %d]", count, MAX_COUNT);
  if (ngroups < 1 || ngroups > MAX_COUNT)
    return fail(MUON_ERR_INVALID_ARGUMENT, "ngroups %d out of [1, %d]", ngroups, MAX_COUNT);
  if (!group_of) return fail(MUON_ERR_INVALID_ARGUMENT, "group_of is NULL");
  if (tile_mode < MUON_TILES_AUTO || tile_mode > MUON_TILES_SMALL)
    return fail(MUON_ERR_INVALID_ARGUMENT, "unknown tile_mode %d", tile_mode);
  for (int32_t i = 0; i < count; ++i)
    if (group_of[i] < 0 || group_of[i] >= ngroups)
      return fail(MUON_ERR_INVALID_ARGUMENT, "group_of[%d] = %d out of [0, %d)", i, group_of[i], ngroups);
  // the matrices and pointers, checked as one step call over the whole set
  Call all{};
  all.mode = MODE_STEP;
  all.params = params;
  all.grads = grads;
  all.momenta = momenta;
  all.updates = updates_out;
  all.shapes = shapes;
  all.count = count;
  all.co = {1.f, 0.f, 0.f};
  muon_status st = validate_call(all);
  if (st != MUON_OK) return st;

  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState* ds = nullptr;
  int dev = 0;
  if ((st = acquire_device(&ds, &dev)) != MUON_OK) return st;
  const std::vector<int> iprec =
      working_formats(shapes, count, MODE_STEP, tile_mode, int64_t(NUM_XCD) * ds->cus_per_xcd);
  StreamPlanImpl* sp = new StreamPlanImpl();
  sp->dev = dev;
  sp->count = count;
  sp->has_upd = updates_out != nullptr;
  sp->groups.resize(size_t(ngroups));
  for (int32_t i = 0; i < count; ++i) {
    StreamGroup& g = sp->groups[size_t(group_of[i])];
    g.members.push_back(i);
    g.shapes.push_back(shapes[i]);
    g.params.push_back(params[i]);
    g.grads.push_back(grads[i]);
    g.moms.push_back(momenta[i]);
    g.upd.push_back(updates_out ? updates_out[i] : nullptr);
    g.prec.push_back(iprec[size_t(i)]);
  }
  size_t need = 0;
  for (const auto& g : sp->groups) need = std::max(need, workspace_bytes(g.shapes.data(), int32_t(g.shapes.size())));
  if (device_alloc(&sp->ws, std::max<size_t>(need, 256)) != hipSuccess) {
    (void)hipGetLastError();
    sp->ws = nullptr;
    free_stream_plan(sp);
    return fail(MUON_ERR_OUT_OF_MEMORY, "stream plan workspace allocation of %zu bytes failed", need);
  }
  for (auto& g : sp->groups) {
    if (g.members.empty()) continue;
    Call c = group_call(g, sp->has_upd);
    if ((st = new_plan(c, g.prec, reinterpret_cast<char*>(sp->ws), ds->cus_per_xcd, &g.plan)) != MUON_OK) {
      g.plan = nullptr;
      free_stream_plan(sp);
      return st;
    }
  }
  *plan_out = reinterpret_cast<muon_stream_plan>(sp);
  return MUON_OK;
}

muon_status stream_submit(StreamPlanImpl* sp, int32_t group, void* ready, const muon_step_hparams* hp,
                          void* stream) {
  t_last_error.clear();
  if (!sp) return fail(MUON_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!hp) return fail(MUON_ERR_INVALID_ARGUMENT, "hparams is NULL");
  if (group < 0 || group >= int32_t(sp->groups.size()))
    return fail(MUON_ERR_INVALID_ARGUMENT, "group %d out of [0, %d)", group, int32_t(sp->groups.size()));
  const StreamGroup& g = sp->groups[size_t(group)];
  // options for the group: per-matrix arrays taken in group order
  muon_step_options opt{};
  std::vector<float> lrs, scs;
  if (hp->options) {
    opt = *hp->options;
    if (opt.launch_mode == MUON_LAUNCH_CHAIN)
      return fail(MUON_ERR_UNSUPPORTED, "a stream plan runs the per-phase grids; launch_mode CHAIN is not supported");
    if (opt.launch_mode == MUON_LAUNCH_AUTO) opt.launch_mode = MUON_LAUNCH_PHASE_GRIDS;
    opt.tile_mode = MUON_TILES_AUTO;      // the plan's formats are fixed
    if (opt.lr_per_matrix) {
      for (int32_t i : g.members) lrs.push_back(opt.lr_per_matrix[i]);
      opt.lr_per_matrix = lrs.data();
    }
    if (opt.scale_per_matrix) {
      for (int32_t i : g.members) scs.push_back(opt.scale_per_matrix[i]);
      opt.scale_per_matrix = scs.data();
    }
  }
  Call c = group_call(g, sp->has_upd);
  c.lr = hp->lr;
  c.beta = hp->beta;
  c.nesterov = hp->nesterov;
  c.co = hp->ns_coeffs;
  c.ns_steps = hp->ns_steps;
  c.scale_rule = hp->scale_rule;
  c.opt = hp->options ? &opt : nullptr;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  muon_status st = validate_call(c);
  if (st != MUON_OK || g.members.empty()) return st;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState* ds = nullptr;
  int dev = 0;
  if ((st = acquire_device(&ds, &dev)) != MUON_OK) return st;
  if (dev != sp->dev)
    return fail(MUON_ERR_INVALID_ARGUMENT, "the plan belongs to device %d, the current device is %d", sp->dev, dev);
  std::map<int, bool> use_chain;          // every group runs the per-phase grids
  return enqueue_step(*ds, g.plan, c, g.prec, use_chain, reinterpret_cast<hipEvent_t>(ready));
}

// ------------------------------------------------------------------ AdamW
constexpr int64_t MAX_ADAMW_NUMEL = int64_t(1) << 40;

struct AdamwCall {
  void* const* params;
  const void* const* grads;
  float* const* m;
  float* const* v;
  const muon_adamw_desc* tensors;
  int32_t count;
  const muon_adamw_hparams* hp;
  hipStream_t stream;
};

bool finite_f(float x) { return std::isfinite(x); }

muon_status validate_adamw(const AdamwCall& c) {
  if (c.count < 0 || c.count > MAX_COUNT)
    return fail(MUON_ERR_INVALID_ARGUMENT, "count %d out of [0, %d]", c.count, MAX_COUNT);
  if (!c.hp) return fail(MUON_ERR_INVALID_ARGUMENT, "hparams is NULL");
  const muon_adamw_hparams& h = *c.hp;
  if (!finite_f(h.lr)) return fail(MUON_ERR_INVALID_ARGUMENT, "lr must be finite");
  if (!(h.beta1 >= 0.f && h.beta1 < 1.f) || !(h.beta2 >= 0.f && h.beta2 < 1.f))
    return fail(MUON_ERR_INVALID_ARGUMENT, "beta1 and beta2 must lie in [0, 1)");
  if (!finite_f(h.eps) || h.eps < 0.f) return fail(MUON_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (!finite_f(h.weight_decay) || h.weight_decay < 0.f)
    return fail(MUON_ERR_INVALID_ARGUMENT, "weight_decay must be finite and >= 0");
  if (h.step < 1) return fail(MUON_ERR_INVALID_ARGUMENT, "step must be >= 1 (got %lld)", (long long)h.step);
  if (c.count == 0) return MUON_OK;
  if (!c.params || !c.grads || !c.m || !c.v || !c.tensors)
    return fail(MUON_ERR_INVALID_ARGUMENT, "a pointer array is NULL");
  for (int32_t i = 0; i < c.count; ++i) {
    if (h.lr_per_tensor && !finite_f(h.lr_per_tensor[i]))
      return fail(MUON_ERR_INVALID_ARGUMENT, "tensor %d: lr_per_tensor is not finite", i);
    if (h.wd_per_tensor && (!finite_f(h.wd_per_tensor[i]) || h.wd_per_tensor[i] < 0.f))
      return fail(MUON_ERR_INVALID_ARGUMENT, "tensor %d: wd_per_tensor must be finite and >= 0", i);
  }
  std::vector<Interval> iv;
  iv.reserve(size_t(c.count) * 4);
  int64_t chunks = 0;
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_adamw_desc& d = c.tensors[i];
    if (d.numel < 0 || d.numel > MAX_ADAMW_NUMEL)
      return fail(d.numel < 0 ? MUON_ERR_INVALID_ARGUMENT : MUON_ERR_UNSUPPORTED,
                  "tensor %d: numel %lld out of [0, 2^40]", i, (long long)d.numel);
    if (d.param_dtype != MUON_DTYPE_F32 && d.param_dtype != MUON_DTYPE_BF16)
      return fail(MUON_ERR_UNSUPPORTED, "tensor %d: param_dtype %d is not F32 or BF16", i, d.param_dtype);
    if (d.grad_dtype != MUON_DTYPE_F32 && d.grad_dtype != MUON_DTYPE_BF16)
      return fail(MUON_ERR_UNSUPPORTED, "tensor %d: grad_dtype %d is not F32 or BF16", i, d.grad_dtype);
    if (d.numel == 0) continue;
    const int pe = dtype_size(d.param_dtype), ge = dtype_size(d.grad_dtype);
    muon_status st;
    if ((st = check_ptr(c.params[i], pe, i, "param")) != MUON_OK) return st;
    if ((st = check_ptr(c.grads[i], ge, i, "grad")) != MUON_OK) return st;
    if ((st = check_ptr(c.m[i], 4, i, "exp_avg")) != MUON_OK) return st;
    if ((st = check_ptr(c.v[i], 4, i, "exp_avg_sq")) != MUON_OK) return st;
    const uint64_t n = uint64_t(d.numel);
    auto add = [&](const void* ptr, uint64_t bytes, bool w, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      iv.push_back({lo, lo + bytes, w, int(i), what});
    };
    add(c.params[i], n * pe, true, "param");
    add(c.grads[i], n * ge, false, "grad");
    add(c.m[i], n * 4, true, "exp_avg");
    add(c.v[i], n * 4, true, "exp_avg_sq");
    chunks += (d.numel + ADAMW_CHUNK - 1) / ADAMW_CHUNK;
    if (chunks > int64_t(INT32_MAX))
      return fail(MUON_ERR_UNSUPPORTED, "more than 2^31 - 1 workgroups of %d elements", ADAMW_CHUNK);
  }
  return check_alias_fast(iv);
}

muon_status build_adamw_plan(AdamwPlan* plan, const AdamwCall& c) {
  std::vector<AdamwTensor> ht;
  std::vector<int32_t> off(1, 0);
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_adamw_desc& d = c.tensors[i];
    if (d.numel == 0) continue;
    AdamwTensor t;
    memset(&t, 0, sizeof(t));
    t.p = c.params[i];
    t.g = c.grads[i];
    t.m = c.m[i];
    t.v = c.v[i];
    t.numel = d.numel;
    t.p_bf16 = d.param_dtype == MUON_DTYPE_BF16;
    t.g_bf16 = d.grad_dtype == MUON_DTYPE_BF16;
    auto al = [](const void* p, int bytes) { return reinterpret_cast<uintptr_t>(p) % uintptr_t(bytes) == 0; };
    t.vec_ok = al(t.p, 4 * dtype_size(d.param_dtype)) && al(t.g, 4 * dtype_size(d.grad_dtype)) && al(t.m, 16) &&
               al(t.v, 16);
    ht.push_back(t);
    plan->kept.push_back(i);
    off.push_back(off.back() + int32_t((d.numel + ADAMW_CHUNK - 1) / ADAMW_CHUNK));
  }
  const int32_t n = int32_t(ht.size());
  plan->count = n;
  plan->total_chunks = off.back();
  if (n == 0) return MUON_OK;
  size_t bytes = 0;
  const size_t o_t = bytes;
  bytes = align256(bytes + sizeof(AdamwTensor) * n);
  const size_t o_off = bytes;
  bytes = align256(bytes + sizeof(int32_t) * (n + 1));
  const size_t o_rates = bytes;
  bytes = align256(bytes + sizeof(float2) * n);
  void* dmem = nullptr;
  if (device_alloc(&dmem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_OUT_OF_MEMORY, "AdamW plan allocation of %zu bytes failed", bytes);
  }
  std::vector<char> host(bytes, 0);
  memcpy(host.data() + o_t, ht.data(), sizeof(AdamwTensor) * n);
  memcpy(host.data() + o_off, off.data(), sizeof(int32_t) * (n + 1));
  if (hipMemcpyAsync(dmem, host.data(), bytes, hipMemcpyHostToDevice, c.stream) != hipSuccess ||
      hipStreamSynchronize(c.stream) != hipSuccess) {
    (void)hipFree(dmem);
    return fail(MUON_ERR_HIP, "AdamW plan upload failed: %s", hipGetErrorString(hipGetLastError()));
  }
  char* base = reinterpret_cast<char*>(dmem);
  plan->dmem = dmem;
  plan->d_tensors = reinterpret_cast<AdamwTensor*>(base + o_t);
  plan->d_chunk_off = reinterpret_cast<int32_t*>(base + o_off);
  plan->d_rates = reinterpret_cast<float2*>(base + o_rates);
  if (hipEventCreateWithFlags(&plan->last_use, hipEventDisableTiming) != hipSuccess) {
    plan->last_use = nullptr;
    return fail(MUON_ERR_HIP, "hipEventCreate failed");
  }
  return MUON_OK;
}

// d = fl32(1 - fl32(lr*wd)), each operation rounded to binary32 (this file
// is compiled without contraction).
float decay_factor(float lr, float wd) {
  const float lw = lr * wd;
  return 1.0f - lw;
}

muon_status run_adamw(const AdamwCall& c) {
  t_last_error.clear();
  muon_status st = validate_adamw(c);
  if (st != MUON_OK) return st;
  bool any = false;
  for (int32_t i = 0; i < c.count && !any; ++i) any = c.tensors[i].numel > 0;
  if (!any) return MUON_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MUON_ERR_HIP, "hipGetDevice failed (no HIP device?)");
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& ds = g_dev[dev];

  std::vector<uint64_t> key;
  key.reserve(size_t(c.count) * 6 + 1);
  key.push_back(uint64_t(c.count));
  for (int32_t i = 0; i < c.count; ++i) {
    const muon_adamw_desc& d = c.tensors[i];
    const bool live = d.numel > 0;
    key.push_back(uint64_t(d.numel));
    key.push_back((uint64_t(uint32_t(d.param_dtype)) << 32) | uint32_t(d.grad_dtype));
    key.push_back(live ? reinterpret_cast<uint64_t>(c.params[i]) : 0);
    key.push_back(live ? reinterpret_cast<uint64_t>(c.grads[i]) : 0);
    key.push_back(live ? reinterpret_cast<uint64_t>(c.m[i]) : 0);
    key.push_back(live ? reinterpret_cast<uint64_t>(c.v[i]) : 0);
  }
  AdamwPlan* plan = nullptr;
  for (auto it = ds.adamw_plans.begin(); it != ds.adamw_plans.end(); ++it) {
    if ((*it)->key == key) {
      plan = *it;
      ds.adamw_plans.erase(it);
      ds.adamw_plans.push_front(plan);
      break;
    }
  }
  if (!plan) {
    plan = new AdamwPlan;
    plan->key = key;
    st = build_adamw_plan(plan, c);
    if (st != MUON_OK) {
      free_adamw_plan(plan);
      return st;
    }
    ds.adamw_plans.push_front(plan);
    while (ds.adamw_plans.size() > MAX_PLANS) {
      free_adamw_plan(ds.adamw_plans.back());
      ds.adamw_plans.pop_back();
    }
  }
  if (plan->count == 0) return MUON_OK;

  const muon_adamw_hparams& h = *c.hp;
  AdamwConsts k;
  k.b1 = h.beta1;
  k.b2 = h.beta2;
  k.c1 = 1.0f - h.beta1;
  k.c2 = 1.0f - h.beta2;
  k.bc1 = float(1.0 - std::pow(double(h.beta1), double(h.step)));
  k.bc2 = float(1.0 - std::pow(double(h.beta2), double(h.step)));
  k.eps = h.eps;
  const float2* rates = nullptr;
  hipError_t e = order_after_last_call(ds, c.stream, FAMILY_ADAMW);
  if (e == hipSuccess && (h.lr_per_tensor || h.wd_per_tensor)) {
    std::vector<float2> hr(plan->count);
    for (int32_t j = 0; j < plan->count; ++j) {
      const int32_t i = plan->kept[j];
      const float lr = h.lr_per_tensor ? h.lr_per_tensor[i] : h.lr;
      const float wd = h.wd_per_tensor ? h.wd_per_tensor[i] : h.weight_decay;
      hr[j] = make_float2(lr, decay_factor(lr, wd));
    }
    e = staged_copy(ds, plan->d_rates, hr.data(), sizeof(float2) * hr.size(), c.stream);
    rates = plan->d_rates;
  }
  if (e == hipSuccess) {
    e = timed(MUON_KC_ADAMW, c.stream, [&] {
      return launch_adamw(plan->d_tensors, plan->d_chunk_off, plan->count, plan->total_chunks, rates, h.lr,
                          decay_factor(h.lr, h.weight_decay), k, c.stream);
    });
  }
  if (e != hipSuccess) return fail(MUON_ERR_HIP, "AdamW launch failed: %s", hipGetErrorString(e));
  (void)hipEventRecord(plan->last_use, c.stream);
  record_last_call(ds, c.stream, FAMILY_ADAMW);
  return MUON_OK;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

muon_status muon_step_batched(void* const* params, const void* const* grads, void* const* momenta,
                              const muon_matrix_desc* shapes, int32_t count, float lr, float beta,
                              int32_t nesterov, muon_ns_coeffs ns_coeffs, int32_t ns_steps, int32_t scale_rule,
                              void* stream) {
  return muon_step_batched_ex(params, grads, momenta, shapes, count, lr, beta, nesterov, ns_coeffs, ns_steps,
                              scale_rule, nullptr, stream);
}

muon_status muon_step_batched_ex(void* const* params, const void* const* grads, void* const* momenta,
                                 const muon_matrix_desc* shapes, int32_t count, float lr, float beta,
                                 int32_t nesterov, muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                 int32_t scale_rule, float* const* updates_out, void* stream) {
  Call c{};
  c.mode = MODE_STEP;
  c.params = params;
  c.grads = grads;
  c.momenta = momenta;
  c.updates = updates_out;
  c.shapes = shapes;
  c.count = count;
  c.lr = lr;
  c.beta = beta;
  c.nesterov = nesterov;
  c.co = ns_coeffs;
  c.ns_steps = ns_steps;
  c.scale_rule = scale_rule;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return run(c);
}

muon_status muon_step_batched_noalloc(void* const* params, const void* const* grads, void* const* momenta,
                                      const muon_matrix_desc* shapes, int32_t count, float lr, float beta,
                                      int32_t nesterov, muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                      int32_t scale_rule, float* const* updates_out, void* stream) {
  Call c{};
  c.mode = MODE_STEP;
  c.params = params;
  c.grads = grads;
  c.momenta = momenta;
  c.updates = updates_out;
  c.shapes = shapes;
  c.count = count;
  c.lr = lr;
  c.beta = beta;
  c.nesterov = nesterov;
  c.co = ns_coeffs;
  c.ns_steps = ns_steps;
  c.scale_rule = scale_rule;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return run_noalloc(c);
}

muon_status muon_step_batched_v2(void* const* params, const void* const* grads, void* const* momenta,
                                 const muon_matrix_desc* shapes, int32_t count, float lr, float beta,
                                 int32_t nesterov, muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                 int32_t scale_rule, const muon_step_options* options,
                                 float* const* updates_out, void* stream) {
  Call c{};
  c.mode = MODE_STEP;
  c.params = params;
  c.grads = grads;
  c.momenta = momenta;
  c.updates = updates_out;
  c.shapes = shapes;
  c.count = count;
  c.lr = lr;
  c.beta = beta;
  c.nesterov = nesterov;
  c.co = ns_coeffs;
  c.ns_steps = ns_steps;
  c.scale_rule = scale_rule;
  c.opt = options;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return run(c);
}

muon_status muon_ns_batched(const void* const* x_in, float* const* x_out, const muon_matrix_desc* shapes,
                            int32_t count, muon_ns_coeffs ns_coeffs, int32_t ns_steps, void* stream) {
  Call c{};
  c.mode = MODE_NS;
  c.grads = x_in;
  c.updates = x_out;
  c.shapes = shapes;
  c.count = count;
  c.co = ns_coeffs;
  c.ns_steps = ns_steps;
  c.lr = 0.f;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return run(c);
}

muon_status muon_frobenius_norms(const void* const* x_in, const muon_matrix_desc* shapes, int32_t count,
                                 float* norms_out, void* stream) {
  Call c{};
  c.mode = MODE_NORMS;
  c.grads = x_in;
  c.shapes = shapes;
  c.count = count;
  c.norms_out = norms_out;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return run(c);
}

muon_status muon_adamw_batched(void* const* params, const void* const* grads, float* const* exp_avg,
                               float* const* exp_avg_sq, const muon_adamw_desc* tensors, int32_t count,
                               const muon_adamw_hparams* hparams, void* stream) {
  AdamwCall c{params, grads, exp_avg, exp_avg_sq, tensors, count, hparams, reinterpret_cast<hipStream_t>(stream)};
  return run_adamw(c);
}

muon_status muon_stream_plan_create(void* const* params, const void* const* grads, void* const* momenta,
                                    const muon_matrix_desc* shapes, int32_t count, const int32_t* group_of,
                                    int32_t ngroups, int32_t tile_mode, float* const* updates_out,
                                    muon_stream_plan* plan_out) {
  return stream_plan_create(params, grads, momenta, shapes, count, group_of, ngroups, tile_mode, updates_out,
                            plan_out);
}

muon_status muon_stream_submit(muon_stream_plan plan, int32_t group, void* ready_event,
                               const muon_step_hparams* hparams, void* stream) {
  return stream_submit(reinterpret_cast<StreamPlanImpl*>(plan), group, ready_event, hparams, stream);
}

muon_status muon_stream_plan_destroy(muon_stream_plan plan) {
  t_last_error.clear();
  if (!plan) return MUON_OK;
  std::lock_guard<std::mutex> lock(g_mu);
  free_stream_plan(reinterpret_cast<StreamPlanImpl*>(plan));
  return MUON_OK;
}

muon_status muon_mfma_probe(int64_t iterations, float* sink, double* flops_out, void* stream) {
  t_last_error.clear();
  if (iterations < 1 || iterations > (int64_t(1) << 30))
    return fail(MUON_ERR_INVALID_ARGUMENT, "iterations %lld out of [1, 2^30]", (long long)iterations);
  if (!sink || !flops_out) return fail(MUON_ERR_INVALID_ARGUMENT, "sink or flops_out is NULL");
  if (reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(MUON_ERR_UNSUPPORTED, "sink is not aligned to 4 bytes");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return fail(MUON_ERR_HIP, "cannot query the current device");
  }
  const hipError_t e = launch_mfma_probe(iterations, cus, sink, flops_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MUON_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return MUON_OK;
}

muon_status muon_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  t_last_error.clear();
  if (!enable) {
    for (auto& t : g_timed) {
      (void)hipEventSynchronize(t.end);
      g_event_pool.push_back(t.beg);
      g_event_pool.push_back(t.end);
    }
    g_timed.clear();
  }
  g_timing = enable != 0;
  return MUON_OK;
}

muon_status muon_timing_read(double* ms_out, int64_t* launches_out) {
  if (!ms_out || !launches_out) return fail(MUON_ERR_INVALID_ARGUMENT, "ms_out or launches_out is NULL");
  std::lock_guard<std::mutex> lock(g_mu);
  t_last_error.clear();
  for (int k = 0; k < MUON_KC_COUNT; ++k) {
    ms_out[k] = 0.0;
    launches_out[k] = 0;
  }
  muon_status st = MUON_OK;
  for (auto& t : g_timed) {
    float ms = 0.f;
    if (hipEventSynchronize(t.end) != hipSuccess || hipEventElapsedTime(&ms, t.beg, t.end) != hipSuccess) {
      (void)hipGetLastError();
      st = fail(MUON_ERR_HIP, "reading a timing event failed");
    } else {
      ms_out[t.kc] += double(ms);
      launches_out[t.kc] += 1;
    }
    g_event_pool.push_back(t.beg);
    g_event_pool.push_back(t.end);
  }
  g_timed.clear();
  return st;
}

uint64_t muon_workspace_bytes(const muon_matrix_desc* shapes, int32_t count) {
  if (!shapes || count < 0 || count > MAX_COUNT) return 0;
  if (validate_desc(shapes, count, MODE_NS) != MUON_OK) return 0;
  return uint64_t(workspace_bytes(shapes, count));
}

muon_status muon_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  const bool have_dev = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_dev) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    drop_plans(kv.second);
    if (kv.second.ws) (void)hipFree(kv.second.ws);
    kv.second.ws = nullptr;
    kv.second.ws_bytes = 0;
    if (kv.second.chain_ws) (void)hipFree(kv.second.chain_ws);
    kv.second.chain_ws = nullptr;
    kv.second.chain_ws_bytes = 0;
    if (kv.second.fail_flag) (void)hipHostFree(kv.second.fail_flag);
    kv.second.fail_flag = nullptr;
    release_ring(kv.second.ring);
    if (kv.second.chain_done) (void)hipEventDestroy(kv.second.chain_done);
    for (hipEvent_t ev : kv.second.last_call)
      if (ev) (void)hipEventDestroy(ev);
  }
  if (have_dev) (void)hipSetDevice(cur);
  g_dev.clear();
  (void)hipGetLastError();
  return MUON_OK;
}

const char* muon_status_string(muon_status status) {
  switch (status) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARGUMENT: return "MUON_ERR_INVALID_ARGUMENT";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_ALIAS: return "MUON_ERR_ALIAS";
    case MUON_ERR_OUT_OF_MEMORY: return "MUON_ERR_OUT_OF_MEMORY";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
  }
  return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error(void) { return t_last_error.c_str(); }

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

}  // extern "C"
