/*
 * muon.h -- C ABI of libmuon_mi355x.so: the Muon optimizer step for
 * MI355X (gfx950), run as hand-written HIP kernels.
 *
 * What the step computes, per 2-D weight matrix W (rows x cols) with
 * gradient G and momentum buffer M:
 *
 *   M <- beta*M + G                      heavy-ball momentum, binary32, unfused
 *   U <- nesterov ? G + beta*M : M       (M is the updated buffer)
 *   X <- U / (||U||_F + 1e-7)            Frobenius normalisation
 *   repeat ns_steps times:               polynomial Newton-Schulz
 *       A <- X X^T ; B <- b A + c A A ; X <- a X + B X
 *   W <- W - fl32(lr*s) * X              scaled write-back (s: scale rule)
 *
 * Matrices with rows > cols are iterated on their transpose so that the
 * Gram matrix X X^T is min(rows, cols) square; the update is transposed
 * back before the write-back.
 *
 * Sources.  The pages that motivate this library describe Muon only in
 * words: "把 GPT-2 的训练租金估算从 4.3 万美元压到 40 美元…" (magicnetworld.com),
 * table 符号与约定, row "Muon", defines it as an optimizer for matrix
 * parameters that orthogonalises the momentum; "开发者千美元训3.8B模型
 * 击败GPT-2" (aiproducthub.cn), paragraph 影响, says the orthogonalisation
 * is Newton-Schulz and that every non-matrix parameter goes to AdamW (the
 * Muon entry points take 2-D matrices; muon_adamw_batched below updates
 * the other parameters).  The polynomial form of the
 * iteration is the textbook one (N. J. Higham, Functions of Matrices,
 * ch. 8); the momentum form, eps, orientation and scale rules are readings
 * the pages leave open, stated at each declaration below.
 *
 * Conventions for every entry point:
 *   - All tensors are device memory on the current HIP device, owned by the
 *     caller.  The library never frees or keeps caller pointers after the
 *     call returns (it may cache their values as a lookup key).
 *   - Matrices are row-major with a row stride `ld_*` in elements
 *     (ld >= cols).  Pointers must be aligned to their element size.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it and the call returns without synchronising; a kernel fault
 *     surfaces at the caller's next synchronisation.
 *   - Every argument is validated on the host before anything is enqueued,
 *     so a call that returns an error has changed nothing.
 *   - The library keeps a per-device workspace (grown on demand, freed by
 *     muon_release_workspace) and a cache of launch plans keyed by the
 *     pointers and shapes.  Every Muon call (muon_step_batched*,
 *     muon_ns_batched, muon_frobenius_norms, muon_stream_submit) first makes
 *     its stream wait for the device's previous Muon call, and every AdamW
 *     call for the previous AdamW call (an event recorded after each call's
 *     last launch): calls of one family made on different streams, or from
 *     different host threads, run on the device one after another in the
 *     order they were made, never overlapping.  A Muon call and an AdamW call
 *     share no device memory and may run concurrently on two streams.
 *   - Nothing crosses the ABI as an exception; errors are status codes with
 *     a thread-local message from muon_last_error().
 *   - The persistent chain (muon_launch_mode) bounds every dependency wait;
 *     a wait that gives up (only possible when the GPU cannot hold the whole
 *     grid at once) skips its tile and raises a flag.  The next call on that
 *     device waits on the host for that launch to end, reads the flag and
 *     returns MUON_ERR_HIP saying the earlier results are invalid.
 *   - Small per-call tables (per-matrix rates, per-tensor AdamW rates) are
 *     copied to the device from pinned staging memory: the call does not
 *     wait for earlier work on its stream.
 *   - Fault hook for tests: with the environment variable MUON_FAULT_ALLOC
 *     set to anything but "" or "0", every device allocation the library
 *     attempts fails, so a call that needs one returns OUT_OF_MEMORY having
 *     changed nothing.
 *   - The optimizer's state is the caller's weights and momenta: saved and
 *     restored, they give the same next step bit for bit, whatever the
 *     library's caches hold.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 4

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad scalar     */
  MUON_ERR_UNSUPPORTED = 2,      /* dtype combination, alignment, size cap */
  MUON_ERR_ALIAS = 3,            /* written buffers overlap another buffer */
  MUON_ERR_OUT_OF_MEMORY = 4,    /* workspace or plan allocation failed    */
  MUON_ERR_HIP = 5               /* a HIP call or launch failed            */
} muon_status;

typedef enum muon_dtype { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1 } muon_dtype;

/* Arithmetic of the Newton-Schulz matrix products.
 *   BF16    operands stored in bfloat16, binary32 accumulation (MFMA).
 *   BF16X3  operands stored as hi + lo bfloat16 pairs; each product is
 *           hi*hi + hi*lo + lo*hi in binary32 (about 16 significant bits).
 *   F32     binary32 operands and binary32 MFMA.                          */
typedef enum muon_ns_precision {
  MUON_NS_BF16 = 0,
  MUON_NS_BF16X3 = 1,
  MUON_NS_F32 = 2
} muon_ns_precision;

/* Per-matrix scale s of the update (the pages give none; NONE is the
 * default reading).  SQRT_ASPECT: s = sqrt(max(1, rows/cols)).
 * RMS_MATCH: s = 0.2*sqrt(max(rows, cols)).                               */
typedef enum muon_scale_rule {
  MUON_SCALE_NONE = 0,
  MUON_SCALE_SQRT_ASPECT = 1,
  MUON_SCALE_RMS_MATCH = 2
} muon_scale_rule;

/* Newton-Schulz step X <- a X + (b A + c A^2) X, A = X X^T.               */
typedef struct muon_ns_coeffs {
  float a, b, c;
} muon_ns_coeffs;

/* Momentum forms (muon_step_options.momentum_kind).
 *   HEAVY_BALL  M <- beta*M + G; Nesterov U = G + beta*M (the default).
 *   EMA         M <- beta*M + (1-beta)*G with (1-beta) rounded to binary32;
 *               Nesterov U = (1-beta)*G + beta*M.  Every product and sum is
 *               rounded once in binary32.                                 */
typedef enum muon_momentum_kind {
  MUON_MOMENTUM_HEAVY_BALL = 0,
  MUON_MOMENTUM_EMA = 1
} muon_momentum_kind;

/* How the Newton-Schulz steps are launched (muon_step_options.launch_mode).
 *   AUTO         PHASE_GRIDS (the faster of the two on every workload
 *                measured on MI355X).
 *   PHASE_GRIDS  one persistent grid per phase and step over all matrices.
 *   CHAIN        one persistent grid for every phase of every step: per-XCD
 *                queues of (step, phase, matrix, tile) items, each waiting
 *                on per-(matrix, phase) completion counts; ns_steps <= 16.
 *                It keeps each step's A, B and iterate in buffers of their
 *                own (a second workspace, (k - 1) iterates and 2k Gram-sized
 *                matrices per matrix for k steps).
 * Every mode gives the same results bit for bit.                            */
typedef enum muon_launch_mode {
  MUON_LAUNCH_AUTO = 0,
  MUON_LAUNCH_PHASE_GRIDS = 1,
  MUON_LAUNCH_CHAIN = 2
} muon_launch_mode;

/* Tile size of the Newton-Schulz products (muon_step_options.tile_mode).
 *   AUTO   bf16 and split-bf16 (each counted on its own): 128 x 128 when the
 *          call's matrices of that precision have fewer 256 x 256 GRAM tiles
 *          than the GPU has compute units (GPT-2-small-sized stacks), else
 *          256 x 256.  fp32: 64 x 64 when its fp32 matrices have fewer
 *          128 x 128 GRAM tiles than that, else 128 x 128.
 *   LARGE  bf16 and split-bf16: 256 x 256 tiles, eight waves,
 *          software-pipelined k-loop (a split-bf16 product as three bf16
 *          products over K).  fp32: 128 x 128 tiles, four waves.
 *   SMALL  bf16 and split-bf16: 128 x 128 tiles, four waves, one-stage
 *          k-loop.  fp32: 64 x 64 tiles, two waves.
 * The working format is the same either way.  The split-bf16 results of the
 * two tile sizes differ within the format's rounding (the sums over K are
 * taken in another order).                                                  */
typedef enum muon_tile_mode {
  MUON_TILES_AUTO = 0,
  MUON_TILES_LARGE = 1,
  MUON_TILES_SMALL = 2
} muon_tile_mode;

/* Update variants of muon_step_batched_v2.  The pages describe none of
 * them; they are the forms commonly used with Muon.  A zero-initialised
 * struct (or a NULL pointer) gives muon_step_batched bit for bit.
 *
 * ns_schedule       host array of ns_steps finite triples, step k using
 *                   entry k (a step with c = 0 skips its A*A product); NULL:
 *                   ns_coeffs at every step.
 * weight_decay      decoupled weight decay wd, finite and >= 0:
 *                   W <- rnd(fl32(fl32(W*d) - fl32(t*O))), d = fl32(1 -
 *                   fl32(lr_i*wd)); 0 leaves the write-back unchanged.
 * momentum_kind     a muon_momentum_kind.
 * lr_per_matrix     host array of `count` finite learning rates replacing
 *                   lr for matrix i (in t and d), or NULL.
 * scale_per_matrix  host array of `count` finite scales s_i replacing the
 *                   scale rule for matrix i (t = fl32(lr_i*s_i), the product
 *                   in binary64), or NULL.
 * launch_mode       a muon_launch_mode.
 * tile_mode         a muon_tile_mode.
 * The arrays are read during the call and not kept.                        */
typedef struct muon_step_options {
  const muon_ns_coeffs* ns_schedule;
  float weight_decay;
  int32_t momentum_kind;
  const float* lr_per_matrix;
  const float* scale_per_matrix;
  int32_t launch_mode;
  int32_t tile_mode;
} muon_step_options;

/* One 2-D matrix.  rows, cols in [1, 65536]; ld_* >= cols.
 * param_dtype and grad_dtype: MUON_DTYPE_F32 or MUON_DTYPE_BF16;
 * mom_dtype: MUON_DTYPE_F32 only; precision: a muon_ns_precision.
 * Size cap (UNSUPPORTED): the library's working copy of the matrix, both
 * dimensions rounded up to multiples of 256, stays below 2 GiB: 2 bytes per
 * element for BF16, 4 for BF16X3 and F32 (a bf16 32512 x 32512 or an fp32
 * 23040 x 23040 matrix is accepted; 32768 x 32768 bf16 is not).           */
typedef struct muon_matrix_desc {
  int64_t rows, cols;
  int64_t ld_param, ld_grad, ld_mom;
  int32_t param_dtype, grad_dtype, mom_dtype;
  int32_t precision;
} muon_matrix_desc;

/* One Muon step on `count` matrices in one grouped launch sequence.
 * Source: the Muon optimizer of "把 GPT-2 的训练租金估算从 4.3 万美元压到 40
 * 美元…" (magicnetworld.com), table 符号与约定, row "Muon" (momentum of a
 * matrix parameter, orthogonalised), with the Newton-Schulz orthogonalisation
 * of "开发者千美元训3.8B模型 击败GPT-2" (aiproducthub.cn), paragraph 影响.
 *
 * params[i]  rows x cols weight (param_dtype), updated in place.
 * grads[i]   rows x cols gradient (grad_dtype), read only.
 * momenta[i] rows x cols binary32 momentum buffer, updated in place.
 * shapes[i]  the descriptor of matrix i.
 * lr         learning rate, finite, as a binary32 value; t = fl32(lr*s).
 * beta       momentum coefficient in [0, 1), used as its binary32 value.
 * nesterov   0 or 1.
 * ns_coeffs  finite a, b, c (c = 0 skips the A*A product).  The products
 *            add a X and (b/c) A as bfloat16 hi + lo pairs, so a and, when
 *            c != 0, fl32(b/c) must round to a finite bfloat16 (magnitude
 *            below about 3.3961e38; a subnormal c beside an ordinary b is
 *            not): UNSUPPORTED otherwise.  Checked only when ns_steps > 0.
 * ns_steps   >= 0; 0 writes back the normalised momentum direction.
 * scale_rule a muon_scale_rule.
 *
 * The momentum update is bit-exact binary32 (one rounding per operation,
 * no fused multiply-add).  The result does not depend on the order of the
 * matrices in the arrays.  count == 0 is a no-op returning MUON_OK.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, ALIAS (a written buffer overlaps
 * any other buffer), OUT_OF_MEMORY, HIP.                                  */
muon_status muon_step_batched(void* const* params, const void* const* grads,
                              void* const* momenta, const muon_matrix_desc* shapes,
                              int32_t count, float lr, float beta, int32_t nesterov,
                              muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                              int32_t scale_rule, void* stream);

/* muon_step_batched, and additionally exports the update O (the
 * orthogonalised, oriented-back Newton-Schulz output before the lr*s
 * scaling) as binary32 rows x cols, row stride cols, into updates_out[i].
 * updates_out may be NULL, and so may any entry.  The exported O is the
 * binary32 value the write-back used, so W_new = rnd(W - fl32(t*O))
 * holds bit for bit.                                                      */
muon_status muon_step_batched_ex(void* const* params, const void* const* grads,
                                 void* const* momenta, const muon_matrix_desc* shapes,
                                 int32_t count, float lr, float beta, int32_t nesterov,
                                 muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                 int32_t scale_rule, float* const* updates_out,
                                 void* stream);

/* muon_step_batched_ex with the update variants of `options` (may be NULL,
 * see muon_step_options).  Per-matrix learning rates, scales or a weight
 * decay add one small host-to-device copy (8 bytes per matrix) on `stream`,
 * from pinned staging memory.
 * Errors as muon_step_batched, and INVALID_ARGUMENT for an option out of
 * its range.                                                              */
muon_status muon_step_batched_v2(void* const* params, const void* const* grads,
                                 void* const* momenta, const muon_matrix_desc* shapes,
                                 int32_t count, float lr, float beta, int32_t nesterov,
                                 muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                 int32_t scale_rule, const muon_step_options* options,
                                 float* const* updates_out, void* stream);

/* muon_step_batched_ex for callers that cannot allocate memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, kernels and results bit for bit, with no device,
 * pinned or event allocation.  Its Newton-Schulz workspace and launch tables
 * live in a fixed 64 MiB device array that the library holds on every GPU
 * it runs on until the process ends, rewritten by every call; nothing in it
 * needs to start at zero.  Inputs whose workspace (2 bytes per element of
 * two iterates and two Gram matrices for BF16, 4 for BF16X3 and F32, each
 * dimension padded to 256) and tables exceed it are rejected with
 * UNSUPPORTED (a stack of twelve bf16 768 x 768 matrices fits; one d24
 * layer does not).  Calls on one GPU share the array: calls that overlap in
 * time on one GPU (two streams, two host threads) race, and are not ordered
 * against each other or against the other entry points.  The launch tables
 * are copied from host memory on `stream` and the call may wait on the host
 * for that copy.  Errors as muon_step_batched_ex.                          */
muon_status muon_step_batched_noalloc(void* const* params, const void* const* grads, void* const* momenta,
                                      const muon_matrix_desc* shapes, int32_t count, float lr, float beta,
                                      int32_t nesterov, muon_ns_coeffs ns_coeffs, int32_t ns_steps,
                                      int32_t scale_rule, float* const* updates_out, void* stream);

/* Newton-Schulz orthogonalisation only: x_out[i] = NS^ns_steps(x / (||x||_F
 * + 1e-7)) for x = x_in[i] (rows x cols, grad_dtype, row stride ld_grad),
 * oriented as above.  x_out[i] is binary32 rows x cols with row stride
 * cols.  param, momentum fields of the descriptors are ignored.
 * Source: the Newton-Schulz orthogonalisation named in "开发者千美元训3.8B模型
 * 击败GPT-2" (aiproducthub.cn), paragraph 影响, in its polynomial form
 * (Higham, Functions of Matrices, ch. 8).  Errors as muon_step_batched,
 * INVALID_ARGUMENT for a NULL x_out entry.                                 */
muon_status muon_ns_batched(const void* const* x_in, float* const* x_out,
                            const muon_matrix_desc* shapes, int32_t count,
                            muon_ns_coeffs ns_coeffs, int32_t ns_steps, void* stream);

/* Frobenius norms: norms_out[i] = ||x_in[i]||_F (binary32, device array of
 * `count` floats), summed as binary32 partials per tile (16 x 256, or
 * 64 x 128 for matrices with more rows than columns; the step's own
 * reduction takes 64 x 64 tiles for tall matrices in the binary32 and split
 * formats) and reduced in a fixed order (deterministic).  x_in[i] is
 * grad_dtype with row stride ld_grad.  The same reduction gives the step's
 * normalisation X = U / (||U||_F + 1e-7); the pages leave the normalisation
 * open, and dividing by the Frobenius norm bounds every singular value by
 * 1, which the iteration needs to converge (Higham, Functions of Matrices,
 * ch. 8).  Errors:
 * INVALID_ARGUMENT (NULL arrays or entries, bad sizes), UNSUPPORTED
 * (dtype, alignment), ALIAS (norms_out overlaps an input), HIP.           */
muon_status muon_frobenius_norms(const void* const* x_in, const muon_matrix_desc* shapes,
                                 int32_t count, float* norms_out, void* stream);

/* ---------------------------------------------------------------------
 * AdamW for the parameters that are not given to Muon (embeddings, the
 * output head, scalars): "开发者千美元训3.8B模型 击败GPT-2" (aiproducthub.cn),
 * paragraph 影响, pairs Muon with AdamW for every other parameter.  The
 * update is Adam's (D. P. Kingma and J. Ba, "Adam: A Method for Stochastic
 * Optimization", Algorithm 1) with decoupled weight decay (I. Loshchilov and
 * F. Hutter, "Decoupled Weight Decay Regularization", Algorithm 2).  Per
 * element, in binary32 with one rounding per operation, no fused
 * multiply-add, division and square root correctly rounded:
 *
 *   m <- beta1*m + c1*g           c1 = fl32(1 - beta1)
 *   v <- beta2*v + c2*(g*g)       c2 = fl32(1 - beta2)
 *   u  = (m / bc1) / (sqrt(v / bc2) + eps)
 *                                 bc_k = fl32(1 - beta_k^t), beta^t in binary64
 *   p <- rnd(fl32(p*d) - fl32(lr*u))
 *                                 d = fl32(1 - fl32(lr*wd)); rnd: to the
 *                                 parameter type (bfloat16 to nearest-even)
 * --------------------------------------------------------------------- */

/* One tensor: numel contiguous elements (any shape, flattened).
 * param_dtype, grad_dtype: MUON_DTYPE_F32 or MUON_DTYPE_BF16; the moment
 * buffers are binary32.  numel in [0, 2^40]; 0 skips the tensor.          */
typedef struct muon_adamw_desc {
  int64_t numel;
  int32_t param_dtype;
  int32_t grad_dtype;
} muon_adamw_desc;

/* Hyperparameters of one AdamW step.
 * lr            finite learning rate (binary32).
 * beta1, beta2  in [0, 1).
 * eps           finite, >= 0 (eps = 0 with v = 0 gives NaN, as the formula).
 * weight_decay  finite, >= 0.
 * step          t >= 1, the number of this step (bias corrections).
 * lr_per_tensor NULL, or a host array of `count` finite rates replacing lr.
 * wd_per_tensor NULL, or a host array of `count` finite decays >= 0
 *               replacing weight_decay.
 * The arrays are read during the call and not kept.                        */
typedef struct muon_adamw_hparams {
  float lr;
  float beta1, beta2;
  float eps;
  float weight_decay;
  int64_t step;
  const float* lr_per_tensor;
  const float* wd_per_tensor;
} muon_adamw_hparams;

/* One AdamW step on `count` tensors in one launch.
 *
 * params[i]      numel elements (param_dtype), updated in place.
 * grads[i]       numel elements (grad_dtype), read only.
 * exp_avg[i]     numel binary32 first moments m, updated in place.
 * exp_avg_sq[i]  numel binary32 second moments v, updated in place.
 * Pointers must be aligned to their element size; 16-byte alignment of
 * all four (8-byte for bfloat16) takes the vector path.  Every result is
 * bit-exact to the formula above.  count == 0 is a no-op returning MUON_OK.
 * Per-tensor rates add one small host-to-device copy (8 bytes per tensor)
 * on `stream`.  Errors: INVALID_ARGUMENT (null pointer, bad size or
 * hyperparameter), UNSUPPORTED (dtype, alignment, size cap), ALIAS (a
 * written buffer overlaps any other buffer), OUT_OF_MEMORY, HIP.          */
muon_status muon_adamw_batched(void* const* params, const void* const* grads,
                               float* const* exp_avg, float* const* exp_avg_sq,
                               const muon_adamw_desc* tensors, int32_t count,
                               const muon_adamw_hparams* hparams, void* stream);

/* ---------------------------------------------------------------------
 * Streaming the step into backward.  "把 GPT-2 的训练租金估算从 4.3 万美元压到
 * 40 美元…" (magicnetworld.com), section "speedrun 全流程：一条命令背后发生了什么",
 * places the Muon step inside pretraining (base_train), after every backward
 * pass.  Backward produces the last layer's gradients first; a stream plan
 * lets the step of each group of matrices (a layer, say) start on the device
 * as soon as that group's gradients are complete, on the optimizer's stream,
 * while backward goes on with the earlier layers on its own.
 * --------------------------------------------------------------------- */

typedef struct muon_stream_plan_s* muon_stream_plan;

/* The arguments of one step, as muon_step_batched_v2 takes them.           */
typedef struct muon_step_hparams {
  float lr;
  float beta;
  int32_t nesterov;
  muon_ns_coeffs ns_coeffs;
  int32_t ns_steps;
  int32_t scale_rule;
  const muon_step_options* options;   /* may be NULL */
} muon_step_hparams;

/* Builds a stream plan over `count` >= 1 matrices split into `ngroups` >= 1
 * groups.  params, grads, momenta, shapes and updates_out (may be NULL) are
 * as for muon_step_batched_ex and must stay valid until the plan is
 * destroyed; group_of is a host array of `count` group indices in
 * [0, ngroups) (groups may be empty), read during the call.  tile_mode (a
 * muon_tile_mode) fixes the working format of every matrix from the whole
 * set, as one call over all of them would choose it.  The plan owns a
 * workspace for its largest group and uploads every launch table here, so a
 * submit neither allocates nor synchronises.  *plan_out receives the plan.
 * Errors: those of muon_step_batched_ex's matrices and pointers,
 * INVALID_ARGUMENT for a bad group index, count, ngroups or tile_mode,
 * OUT_OF_MEMORY, HIP.                                                       */
muon_status muon_stream_plan_create(void* const* params, const void* const* grads, void* const* momenta,
                                    const muon_matrix_desc* shapes, int32_t count, const int32_t* group_of,
                                    int32_t ngroups, int32_t tile_mode, float* const* updates_out,
                                    muon_stream_plan* plan_out);

/* Enqueues one whole Muon step (momentum, normalisation, Newton-Schulz,
 * write-back) of the matrices of `group` on `stream`, behind `ready_event`
 * and behind the device's previous call.  ready_event is a hipEvent_t that
 * the caller recorded after the last write of those gradients (typically on
 * its backward stream) BEFORE this call, since a wait on an event never
 * recorded does not wait; NULL: no wait.  Submit every group once per step,
 * in any order.  W, M and the exported O of every matrix are then
 * bit-identical to one muon_step_batched_v2 call over the whole set with the
 * same hparams: the per-matrix arithmetic does not depend on the grouping.
 * The groups' steps share the plan's workspace and run one after another on
 * the device.  hparams->options: lr_per_matrix and scale_per_matrix are
 * indexed over the whole set; launch_mode must be AUTO or PHASE_GRIDS
 * (CHAIN: UNSUPPORTED); tile_mode is ignored (fixed by the plan).  The
 * current device must be the plan's.  An empty group is a no-op.
 * Errors: INVALID_ARGUMENT (null plan or hparams, group out of range, a bad
 * hyperparameter, another device), UNSUPPORTED, HIP.                        */
muon_status muon_stream_submit(muon_stream_plan plan, int32_t group, void* ready_event,
                               const muon_step_hparams* hparams, void* stream);

/* Waits for the plan's submitted work, then frees its workspace and tables.
 * NULL is a no-op.                                                          */
muon_status muon_stream_plan_destroy(muon_stream_plan plan);

/* Kernel classes of the launch sequence, for muon_timing_read.            */
typedef enum muon_kernel_class {
  MUON_KC_MOMENTUM = 0,  /* momentum / Nesterov + U copies + norm partials  */
  MUON_KC_NORM = 1,      /* norm finalize                                  */
  MUON_KC_GRAM = 2,      /* A = X X^T                                      */
  MUON_KC_POLY = 3,      /* B = b A + c A A                                */
  MUON_KC_COMBINE = 4,   /* X = a X + B X (last step: write-back)          */
  MUON_KC_WRITEBACK = 5, /* write-back when ns_steps == 0                  */
  MUON_KC_ADAMW = 6,     /* muon_adamw_batched                             */
  MUON_KC_CHAIN = 7,     /* the persistent chain (all steps, one launch)   */
  MUON_KC_COUNT = 8
} muon_kernel_class;

/* Measurement hook.  While enabled (enable = 1), every launch the library
 * enqueues is bracketed by two HIP events recorded on the launch stream.
 * muon_timing_read waits for the recorded events, writes the summed
 * milliseconds and the launch count of each kernel class into
 * ms_out[MUON_KC_COUNT] and launches_out[MUON_KC_COUNT] (host arrays), and
 * clears the record.  enable = 0 stops recording and drops what was held.
 * Not thread-safe against concurrent steps.                                */
muon_status muon_timing_enable(int32_t enable);
muon_status muon_timing_read(double* ms_out, int64_t* launches_out);

/* Measurement aid: enqueue on `stream` a kernel that keeps every matrix
 * core busy with four independent v_mfma_f32_32x32x16_bf16 chains per wave
 * for `iterations` rounds (1 to 2^30), two waves per SIMD, operands in
 * registers: eight fragments of random bf16 values per lane, taken in turn;
 * *flops_out receives its operation count.  Timing the launch gives the
 * dense bf16 rate the chip sustains under MFMA load on random data (the
 * clock it holds then stays well below the nominal 2.4 GHz).  `sink` is a
 * device float that the kernel never writes (it keeps the chains live).  */
muon_status muon_mfma_probe(int64_t iterations, float* sink, double* flops_out, void* stream);

/* Bytes of device workspace a step on these shapes needs (0 on error).    */
uint64_t muon_workspace_bytes(const muon_matrix_desc* shapes, int32_t count);

/* Free the workspace and cached plans of every device (synchronises each). */
muon_status muon_release_workspace(void);

/* Static string for a status code.                                         */
const char* muon_status_string(muon_status status);

/* Detail of the last error on the calling thread ("" if none).             */
const char* muon_last_error(void);

/* MUON_ABI_VERSION of the built library.                                   */
int32_t muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
