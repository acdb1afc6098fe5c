// Internal types shared by the host runtime and the HIP kernels of
// libmuon_mi355x.so.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Workspace matrices are padded to a multiple of PAD in both dimensions and
// the padding holds zeros, so the Newton-Schulz products run without bounds
// checks: zero rows and columns contribute nothing and stay zero.
constexpr int PAD = 256;
// Workspace rows may hold LDPAD elements beyond the padded width (never
// read); a pad of 64 was measured to change nothing on the d24 stack.
constexpr int LDPAD = 0;
// Elementwise tiles (momentum, transposed copy, norm partials), 4096
// elements each: ETILE x ETILE for tall matrices (transposed through LDS),
// RTILE_R x RTILE_C for the others (one 256-element row run per wave and
// instruction: 1 KB of binary32 momentum).
constexpr int ETILE = 64;
constexpr int RTILE_R = 16, RTILE_C = 256;
// Tall matrices in the bf16 working format: TBF_R x TBF_C tiles (8192
// elements), staged through LDS as bf16 (two 128-element row runs per wave
// and load, 128-byte U^T runs per store; 16.5 KB of LDS, about what a
// 64 x 64 binary32 tile takes, so occupancy stays full).
constexpr int TBF_R = 64, TBF_C = 128;
// Dispatch order puts consecutive workgroups on different XCDs.
constexpr int NUM_XCD = 8;

// Working formats of the Newton-Schulz products.  PREC_BF16S is the bf16
// format on 128 x 128 tiles (a one-stage k-loop), chosen for stacks too small
// to fill the GPU with 256 x 256 tiles; it stores exactly what PREC_BF16 does.
// PREC_BF16X3S is likewise the split-bf16 format on 128 x 128 tiles, and
// PREC_F32S the binary32 format on 64 x 64 tiles, for binary32 stacks too
// small to fill the GPU with 128 x 128 tiles.
enum Prec : int { PREC_BF16 = 0, PREC_BF16X3 = 1, PREC_F32 = 2, PREC_BF16S = 3, PREC_F32S = 4, PREC_BF16X3S = 5 };

// Per-matrix device descriptor.  "natural" means the caller's orientation
// (rows x cols); the iteration runs on the wide orientation m x n (m <= n).
struct MatDev {
  // caller memory
  void* param;            // rows x cols, param dtype; null for NS-only calls
  const void* grad;       // rows x cols, grad dtype
  float* mom;             // rows x cols float; null for NS-only calls
  float* upd;             // rows x cols float export (nullable), row stride ld_upd
  int64_t ld_param, ld_grad, ld_mom, ld_upd;
  int32_t rows, cols;     // natural shape
  int32_t m, n;           // wide shape
  int32_t Mp, Np;         // padded wide shape
  int32_t ldx, lda;       // workspace row strides (elements) of X and of A, B
  int32_t transposed;     // rows > cols
  int32_t param_bf16, grad_bf16;
  int32_t vec_ok;         // grad/mom rows allow 4-element vector access
  int32_t wvec_ok;        // param rows allow 8-element vector access (16-byte aligned)
  int32_t uvec_ok;        // update-export rows allow 4-float vector access
  int32_t prec;           // Prec
  int32_t etile_cols;     // elementwise tiles along the natural columns
  // workspace: element buffers; BF16X3 keeps the lo plane `plane_*`
  // elements after the hi plane
  void* X[2];             // Mp x Np (ping-pong)
  void* A;                // Mp x Mp Gram matrix (tiles on or above the diagonal)
  void* B;                // Mp x Mp b A + c A^2 (tiles on or above the diagonal)
  int64_t plane_X, plane_A;
};

// Arguments of one Newton-Schulz phase launch.
struct PhaseArgs {
  float a, b, c;
  float lr;
  int32_t cur;            // which X buffer holds the current iterate
  int32_t first;          // apply 1/(||U||+eps) folded into this step
  int32_t last;           // combine: write back instead of storing X
  int32_t scale_rule;
  int32_t per_xcd;        // tile-list entries per XCD
  int32_t cus_per_xcd;    // compute units per XCD (persistent grid size)
  const float2* wb;       // per matrix {t = fl32(lr*s), decay d}, or null: t from lr and the rule, d = 1
};

// Per-matrix scalars written by the norm finalize kernel.
struct MatScal {
  float inv;              // 1 / (||U||_F + eps)
  float inv2;             // inv * inv
  float norm;             // ||U||_F
  float pad;
};

// One tensor of an AdamW call: numel contiguous elements.
struct AdamwTensor {
  void* p;                // param dtype, updated in place
  const void* g;          // grad dtype
  float* m;               // first moment
  float* v;               // second moment
  int64_t numel;
  int32_t p_bf16, g_bf16;
  int32_t vec_ok;         // every pointer allows 4-element vector access
  int32_t pad;
};
// Elements per AdamW workgroup.
constexpr int ADAMW_CHUNK = 4096;

// Binary32 constants of an AdamW step (formed on the host).
struct AdamwConsts {
  float b1, b2;           // beta1, beta2
  float c1, c2;           // fl32(1 - beta)
  float bc1, bc2;         // fl32(1 - beta^t)
  float eps;
};

// One work item of the persistent Newton-Schulz chain: a tile of one phase
// of one step of one matrix.
enum ChainKind : int { CHAIN_GRAM_B = 0, CHAIN_GRAM_A = 1, CHAIN_POLY = 2, CHAIN_COMB = 3, CHAIN_COMB_LAST = 4 };
struct ChainItem {
  int32_t desc;           // descriptor of (step, matrix): buffers of that step
  int32_t mat;            // matrix index (norm scalars, write-back table)
  int32_t kind;           // ChainKind
  int32_t step;           // Newton-Schulz step (index of its PhaseArgs)
  int32_t tile;           // ti << 16 | tj
  int32_t wait;           // done counter to wait for, -1 for none
  int32_t need;           // its complete value
  int32_t signal;         // done counter of this item's phase instance
};

// Launchers (defined in the .hip files).  All enqueue on `stream`.
hipError_t launch_momentum(const MatDev* mats, const int32_t* etile_off, int32_t count,
                           int64_t total_tiles, float beta, int32_t nesterov, int32_t ema, int32_t mode,
                           float* partials, hipStream_t stream);
hipError_t launch_norm_finalize(const int32_t* etile_off, int32_t count, const float* partials,
                                MatScal* scal, float* norms_out, hipStream_t stream);
hipError_t launch_writeback_direct(const MatDev* mats, const int32_t* etile_off, int32_t count,
                                   int64_t total_tiles, const MatScal* scal, float lr,
                                   int32_t scale_rule, const float2* wb, hipStream_t stream);
enum Phase : int { PH_GRAM = 0, PH_POLY = 1, PH_COMB = 2 };
hipError_t launch_adamw(const AdamwTensor* tensors, const int32_t* chunk_off, int32_t count, int64_t total_chunks,
                        const float2* rates, float lr, float d, const AdamwConsts& k, hipStream_t stream);
hipError_t launch_mfma_probe(int64_t iterations, int32_t cus, float* sink, double* flops, hipStream_t stream);
// Chain sync words: NUM_XCD queue heads, an abort word, padding, then the
// completion counters.
constexpr int CHAIN_SYNC_HEAD = 16;

// Per-call scalars of a chain launch: the step coefficients and the
// write-back parameters (PhaseArgs of each step are formed on the device
// from these, so no host copy precedes the launch).
constexpr int MAX_CHAIN_STEPS = 16;
struct ChainArgs {
  float a[MAX_CHAIN_STEPS], b[MAX_CHAIN_STEPS], c[MAX_CHAIN_STEPS];
  float lr;
  int32_t steps;
  int32_t scale_rule;
  int32_t cus_per_xcd;
  const float2* wb;
  int64_t spin_limit;     // polls before a dependency wait gives up
};

// Zeroes sync[0, nsync) (heads, abort word, completion counters) and writes
// the PhaseArgs of each step into `steps`, then runs the chain;
// per_xcd_max is the longest XCD queue.
hipError_t launch_ns_chain(int prec, const MatDev* imats, const MatScal* scal, const ChainItem* items,
                           const int32_t* xcd_off, int32_t per_xcd_max, PhaseArgs* steps, int32_t* sync,
                           int32_t nsync, int32_t* fail, const ChainArgs& args, hipStream_t stream);
hipError_t launch_ns_phase(int prec, int phase, const MatDev* mats, const MatScal* scal,
                           const int2* tiles, const PhaseArgs& args, hipStream_t stream);

// Bytes of the per-GPU device array of muon_step_batched_noalloc (its
// Newton-Schulz workspace and launch tables), and its device address on
// device `dev` (taken once per device, with `dev` current).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t noalloc_scratch(int dev, void** out);

// Tile edge of the Newton-Schulz products (square tiles) per format: 256 for
// bf16 and split-bf16 (LDS holds two stages of 256x64 bf16 per operand; the
// split-bf16 products stage one plane at a time); 128 for float32 (an operand
// takes twice the bytes) and for the small-stack bf16 and split-bf16 tiles;
// 64 for the small-stack binary32 tiles.
constexpr int ns_tile(int prec) {
  return (prec == PREC_BF16 || prec == PREC_BF16X3) ? 256 : prec == PREC_F32S ? 64 : 128;
}
constexpr bool bf16_single(int prec) { return prec == PREC_BF16 || prec == PREC_BF16S; }
constexpr bool is_f32(int prec) { return prec == PREC_F32 || prec == PREC_F32S; }
constexpr bool is_split(int prec) { return prec == PREC_BF16X3 || prec == PREC_BF16X3S; }

// Element (row, col) of a workspace matrix (X, A or B; wide orientation, row
// stride ld elements; for split-bf16, of either plane).  The 256 x 256 bf16
// and split-bf16 formats store their buffers tile by tile: tile (row / 256, col / 256) is 128 KB holding its 256 rows of 512
// bytes one after the other, and the tiles of a tile row follow each other
// (ld / 256 of them).  A product tile's output then leaves as one contiguous
// block, and a 64-k stage of an operand is 256 runs of 128 bytes 512 bytes
// apart (or, for a k-row operand, 32 KB in one piece).  The other formats
// keep rows of ld elements.
static_assert(LDPAD % PAD == 0, "tiled rows are whole tiles");
// Bytes from one tile to the next (no gap: gaps of 256 B to 8.25 KB between
// tiles were measured to change nothing).
constexpr int WS_TILE_STRIDE = 256 * 256 * 2;
__host__ __device__ inline int64_t ws_index(int prec, int64_t row, int64_t col, int64_t ld) {
  if (prec == PREC_BF16 || prec == PREC_BF16X3)
    return ((row >> 8) * (ld >> 8) + (col >> 8)) * (WS_TILE_STRIDE / 2) + ((row & 255) << 8) + (col & 255);
  return row * ld + col;
}

}  // namespace muon
