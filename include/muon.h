/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer-step library.
 *
 * One call of muon_step runs one Muon optimizer step over a group of 2-D
 * matrices on one GPU, stream-ordered, with no host synchronisation:
 *
 *   K1  momentum lerp + Nesterov blend + per-block Frobenius reduction +
 *       copy into the wide orientation (bf16 or fp32)         (HBM-bound)
 *   K2  Newton-Schulz, 'standard' or 'gram' form, as grouped MFMA GEMMs
 *       with the quintic fused into their epilogues            (MFMA-bound)
 *   K3  transpose back, shape scale, owned-slice scatter into the fp32 flat
 *       partitions, padding untouched                           (HBM-bound)
 *
 * What the step computes comes from the DeepSpeed pull-request pages it is
 * built from, cited by title and section:
 *   [8526] "Support Muon in BF16_Optimizer with FP32 gradient accumulation",
 *          description (fp32 momentum; Muon on the original matrices; only
 *          each rank's owned intersection is copied into its fp32 partition;
 *          alignment padding excluded; unsupported set-ups rejected up front).
 *   [8600] "Run Muon once per optimizer step under ZeRO-3, not once per
 *          micro-batch", "The problem" / "The change" (once per step on the
 *          accumulated gradient, after the overflow check and before the
 *          norm; Newton-Schulz once per matrix per step; full-shape gradients
 *          passed with each parameter's flat offset) and review thread (the
 *          per-matrix routine takes momentum, beta, the method 'standard' or
 *          'gram' and a per-parameter head count).
 *   [8464] "Fix Muon optimizer under ZeRO CPU offload and bound gather
 *          buffers", momentum-dtype commit (momentum in the fp32 master
 *          dtype; padded final partitions).
 * The numeric form (lerp momentum, Nesterov blend, Frobenius normalisation,
 * quintic coefficients, wide orientation, shape scale sqrt(max(1,rows/cols)))
 * is the plain reading of that prose; the library's design notes list every
 * reading.
 *
 * Conventions for every entry point:
 *  - Every function returns a muon_status; nothing crosses the ABI as an
 *    exception or abort.  All argument checks run before anything is
 *    enqueued, so a call that fails has no side effects.  Asynchronous device
 *    errors surface as MUON_ERR_HIP at a later call or at the caller's own
 *    synchronisation.  muon_last_error() gives a thread-local detail text.
 *  - Pointer tables (grads, momenta, partitions, updates, acc, grad_mb) are
 *    HOST arrays whose elements are DEVICE pointers owned by the caller.
 *    The library never allocates device memory: the caller supplies every
 *    buffer and the workspace.
 *  - Matrices are dense row-major rows x cols in their original orientation.
 *    Only element alignment is required.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is ordered on
 *    it; no call synchronises the host.  A plan is not thread-safe; distinct
 *    plans are independent.
 *  - NaN or Inf inputs are not checked; they propagate to the outputs.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* null pointer, bad size or unknown enum value   */
  MUON_ERR_UNSUPPORTED = 2, /* a configuration this library does not handle   */
  MUON_ERR_LAYOUT = 3,      /* flat ranges overlap or exceed the partitions   */
  MUON_ERR_ALIAS = 4,       /* buffers given to one call overlap              */
  MUON_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned     */
  MUON_ERR_HIP = 6          /* a HIP runtime call failed                      */
} muon_status;

typedef enum { MUON_NS_STANDARD = 0, MUON_NS_GRAM = 1 } muon_ns_method;

/* Arithmetic of Newton-Schulz.  FP32: fp32 operands and accumulation
 * throughout.  BF16: bf16 MFMA operands with fp32 accumulation; the Gram
 * form's small-side chain (R, P, Q) is fp32 for blocks with m < 256 and a
 * split-bf16 pair (hi + lo, three bf16 products per product) for m >= 256,
 * except that blocks with m >= 2048 accumulate Q with one bf16 product.
 * Blocks with 64 <= m <= 128 (either form) run their whole iteration in one
 * workgroup; there the Gram form's output product takes Q as a bf16 pair
 * (hi + lo) rather than its bf16 value. */
typedef enum { MUON_PREC_FP32 = 0, MUON_PREC_BF16 = 1 } muon_ns_precision;

/* How the Newton-Schulz products of blocks with m >= 256 (bf16) are put on
 * the device.  LAUNCHES: one launch per product of the schedule over every
 * such block of a wave.  PERSISTENT: one launch per wave runs every product
 * of every such block: a workgroup per CU takes tiles from a queue of its
 * XCD, each block's products stay on one XCD, and a tile starts once its
 * block's previous product is complete (a counter per block), so no
 * device-wide barrier separates the products.  Results are bitwise those
 * of LAUNCHES.  PERSISTENT falls back to LAUNCHES on a device that does not
 * have 8 XCDs of 32 CUs.  Neither form is fixed by the pages, which run the
 * products as framework matmuls; LAUNCHES is the faster one on MI355X for
 * the groups measured, and is the default. */
typedef enum { MUON_SCHED_LAUNCHES = 0, MUON_SCHED_PERSISTENT = 1 } muon_ns_schedule;

/* Storage type of a gradient or update buffer. */
typedef enum { MUON_DT_FP32 = 0, MUON_DT_BF16 = 1 } muon_dtype;

/* One matrix of the group.  num_heads 0 or 1 = one Newton-Schulz block;
 * h > 1 = h equal contiguous row blocks, each orthogonalised on its own
 * ([8600] review thread: the head count is the parameter's own).  flat_offset
 * = index of element (0,0) in the group's flat index space, which the
 * partitions cut into num_partitions pieces of partition_numel elements. */
typedef struct {
  int64_t rows;
  int64_t cols;
  int32_t num_heads;
  int32_t reserved; /* must be 0 */
  int64_t flat_offset;
} muon_matrix;

typedef struct {
  float beta;          /* momentum coefficient, in [0, 1)                  */
  int32_t nesterov;    /* 1: u = (1-beta) G + beta m_new;  0: u = m_new    */
  int32_t method;      /* muon_ns_method                                   */
  int32_t ns_steps;    /* >= 0                                             */
  float a, b, c;       /* quintic coefficients, the same at every step     */
  float eps;           /* X <- u / (||u||_F + eps), per block              */
  int32_t precision;   /* muon_ns_precision                                */
  int32_t grad_dtype;  /* muon_dtype of the grads given to muon_step       */
  uint64_t max_inflight_bytes; /* cap on the workspace's data; 0 = no cap  */
  int32_t schedule;    /* muon_ns_schedule                                 */
  int32_t reserved;    /* must be 0                                        */
} muon_options;

typedef struct {
  int64_t partition_numel; /* elements per partition (P), > 0          */
  int32_t num_partitions;  /* R, > 0                                   */
  int32_t reserved;        /* must be 0                                */
} muon_layout;

/* Host-side counters.  The host never reads a device skip flag, so a step
 * enqueued with one is counted in steps and ns_invocations whether or not
 * the flag later discards it on the device; flagged_steps says how many of
 * the counted steps were such conditional ones.  For a run whose flags all
 * held 0 the counts are exact: ns_invocations = matrices x steps ([8600]
 * "The problem" results table: once per matrix per optimizer step). */
typedef struct {
  uint64_t steps;          /* muon_step / muon_step_ex calls that enqueued */
  uint64_t ns_invocations; /* Newton-Schulz runs enqueued: one per matrix  */
                           /* per counted step                             */
  uint64_t accumulations;  /* muon_accumulate calls that enqueued work     */
  uint64_t waves;          /* workspace waves per step (>= 1)              */
  uint64_t flagged_steps;  /* counted steps enqueued with a skip flag      */
} muon_stats;

/* A contiguous owned intersection of one matrix with one partition:
 * elements [first, first+length) of the row-major flattened matrix go to
 * partitions[partition][offset .. offset+length). */
typedef struct {
  int32_t matrix;
  int32_t partition;
  int64_t offset;
  int64_t first;
  int64_t length;
} muon_run;

/* One Newton-Schulz problem of a plan (a whole matrix or one head block),
 * in its wide orientation m <= n. */
typedef struct {
  int32_t matrix;
  int32_t head;
  int32_t m, n;
  int32_t transposed; /* 1 if the block has more rows than columns */
  int32_t wave;
  double flops;       /* nominal Newton-Schulz flops of this problem */
} muon_problem_info;

/* The default workspace cap: groups needing more run in waves (measured on
 * MI355X: no slower for the Llama-7B and per-head groups, faster for the
 * 70B share, against one wave). */
#define MUON_DEFAULT_INFLIGHT_BYTES ((uint64_t)24 << 30)

typedef struct muon_plan muon_plan;

/* Default options: beta 0.95, Nesterov on, standard form, 5 steps,
 * (a,b,c) = (3.4445, -4.7750, 2.0315), eps 1e-7, bf16 precision, bf16
 * grads, the workspace's data capped at MUON_DEFAULT_INFLIGHT_BYTES (24 GiB:
 * a larger group runs in waves), one launch per product.  Errors: INVALID_ARG if out is NULL. */
muon_status muon_default_options(muon_options *out);

/* Build a plan for a group of n matrices (host only; no device call).
 * The layout is static and computed once ([8526] review thread: split
 * tables computed at init).  Rejected: n < 1; rows or cols < 1; rows or cols
 * beyond 2^31-1; num_heads < 0 or not dividing rows; ns_steps < 0; beta
 * outside [0,1); unknown enums; reserved != 0 (INVALID_ARG / UNSUPPORTED);
 * flat ranges that overlap or leave [0, R*P) (LAYOUT).  On success *out owns
 * host memory only, released by muon_plan_destroy. */
muon_status muon_plan_create(muon_plan **out, const muon_matrix *mats, int32_t n,
                             const muon_options *opt, const muon_layout *layout);

/* Device workspace muon_step needs, in bytes (256-byte aligned base).  The
 * caller allocates it: the library holds no device memory of its own, in
 * place of the gather-buffer cache ([8464] "Changes": cached gather buffers
 * capped at 256 MB and freed on destroy).  With opt.max_inflight_bytes set
 * (as by default) it is proportional to the matrices in flight, not to the
 * whole group
 * ([8526] description: temporary memory proportional to the largest Muon
 * group).  Errors: INVALID_ARG for NULL. */
muon_status muon_plan_workspace_bytes(const muon_plan *p, size_t *bytes);

/* Gradient accumulation into fp32 ([8526] description; [8600] "The change":
 * the partitions accumulate the raw gradient, Muon runs only at the step).
 * acc[i] (fp32, rows x cols) = grad_mb[i] if first != 0, else
 * acc[i] + grad_mb[i].  mb_dtype: muon_dtype of grad_mb.  Runs no
 * Newton-Schulz and touches no momentum.  ws/ws_bytes: the plan's workspace
 * (it holds the launch table).  Errors: INVALID_ARG (null tables or
 * entries, unknown dtype), ALIAS (any two buffers of the call overlap),
 * WORKSPACE, HIP. */
muon_status muon_accumulate(muon_plan *p, float *const *acc, const void *const *grad_mb,
                            int32_t mb_dtype, int32_t first, void *ws, size_t ws_bytes,
                            void *stream);

/* One Muon step over the whole group ([8600] "The change": once per
 * optimizer step, on the accumulated gradient; call it only for steps the
 * overflow check keeps, so a discarded step leaves momentum untouched).
 *   grads[i]      read only, rows x cols, opt.grad_dtype
 *   momenta[i]    fp32 rows x cols, updated in place
 *   partitions[r] fp32, partition_numel each; written only on the owned
 *                 intersections of the matrices, never on padding
 *   ws, ws_bytes  device workspace of at least muon_plan_workspace_bytes,
 *                 256-byte aligned; its contents need not be preserved
 *                 between calls
 * Errors: INVALID_ARG (null table or entry), ALIAS (any two buffers of the
 * call overlap, the workspace included), WORKSPACE (too small / unaligned),
 * HIP (a launch failed). */
muon_status muon_step(muon_plan *p, const void *const *grads, float *const *momenta,
                      float *const *partitions, void *ws, size_t ws_bytes, void *stream);

/* muon_step with the two inputs a mixed-precision training loop adds
 * ([8600] "The change": Muon runs after the overflow check, so a step the
 * loss scaler discards leaves the momentum untouched; [8464] commits:
 * results are checked to agree across loss scales):
 *   skip_flag   DEVICE pointer to an int32, or NULL.  The kernels read it
 *               when they run: non-zero = a discarded step, and nothing
 *               outside the workspace is written (momenta and partitions
 *               keep their contents).  The host never waits for it, so the
 *               plan's counters still count the call (see muon_stats).
 *   grad_scale  multiplies every gradient element before the momentum blend,
 *               in fp32 (1/S for gradients produced under loss scale S);
 *               1.0f gives muon_step bit for bit.  Must be finite.
 * It also leaves, in the workspace, the per-chunk sums of squares of the
 * values written to the partitions, for muon_apply_update.
 * Errors: as muon_step; INVALID_ARG for a non-finite grad_scale, ALIAS if
 * skip_flag overlaps another buffer. */
muon_status muon_step_ex(muon_plan *p, const void *const *grads, float *const *momenta,
                         float *const *partitions, const int32_t *skip_flag, float grad_scale,
                         void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (a serving loop that may
 * not call hipMalloc, a harness that forbids allocation, code that wants no
 * caller workspace at all): muon_step_ex with the same kernels, arguments
 * and results, minus the workspace.  Its workspace is a device array of
 * MUON_NOALLOC_SCRATCH_BYTES compiled into the library; each GPU the library
 * runs on holds one copy from the first call on it until the process ends.
 * The launch tables reach that array as kernel arguments (at most 96 KB of
 * tables, copied by the runtime at launch), so the call allocates nothing:
 * no hipMalloc, hipHostMalloc or hipFree, and no host heap on success.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; the step writes every byte it later reads, so nothing
 *     needs clearing between calls.  Calls that can overlap on one GPU (two
 *     streams, two host threads) race on it: the caller orders them.
 *   - The update-norm partials it leaves stay in the array, so
 *     muon_apply_update cannot follow it (it reports that no step ran on its
 *     workspace); run muon_step_ex when the parameter update follows.
 *   - It enqueues kernels only (no copy, memset or event), so it can be
 *     captured into a graph on a capturing stream: the tables travel in the
 *     captured kernel arguments and each replay uploads them again.  The
 *     plan's counters (muon_plan_stats) count the capture, not the replays.
 * Errors: WORKSPACE if the plan's workspace (muon_plan_workspace_bytes)
 * exceeds MUON_NOALLOC_SCRATCH_BYTES (max_inflight_bytes can cut it into
 * waves that fit); UNSUPPORTED if its tables exceed 96 KB; then as
 * muon_step_ex. */
#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
muon_status muon_step_noalloc(muon_plan *p, const void *const *grads, float *const *momenta,
                              float *const *partitions, const int32_t *skip_flag, float grad_scale,
                              void *stream);

/* Overflow check on the step's gradients: *flag (DEVICE int32) = 1 if any
 * element of any grads[i] (rows x cols, `dtype`) is Inf or NaN, else 0.
 * The result can be handed to muon_step_ex / muon_apply_update as their
 * skip flag without a host round trip.  ws/ws_bytes: the plan's workspace
 * (it holds the matrix table).  Errors: INVALID_ARG, ALIAS, WORKSPACE, HIP. */
muon_status muon_check_finite(muon_plan *p, const void *const *grads, int32_t dtype,
                              int32_t *flag, void *ws, size_t ws_bytes, void *stream);

/* The step after the path ([8600] "The change": the gradient norm is taken
 * over the Muon update, clipping semantics unchanged):
 *   norm = sqrt(sum of squares of every owned update element), taken from
 *          the sums the last muon_step / muon_step_ex on this plan and this
 *          workspace left there (fp64, fixed order: deterministic);
 *   clip = max_norm > 0 ? min(1, max_norm / (norm + 1e-6)) : 1;
 *   params[r][j] = params[r][j] * (1 - lr * weight_decay)
 *                  - (lr * clip) * partitions[r][j]      (fp32, one fma)
 * on the owned intersections only; padding untouched.
 *   params[r]      fp32 master partitions, the partitions' layout, updated
 *   partitions[r]  the update as muon_step wrote it, read only
 *   skip_flag      DEVICE int32 or NULL: non-zero = nothing is written
 *   norm_clip_out  DEVICE float[2] or NULL: receives {norm, clip}
 * Call it after the step, with the same workspace and skip flag, before
 * the workspace is used by another step.  Errors: INVALID_ARG (NULL
 * entries, non-finite lr / weight_decay / max_norm, no step on this
 * workspace), ALIAS, WORKSPACE, HIP. */
muon_status muon_apply_update(muon_plan *p, float *const *params, const float *const *partitions,
                              float lr, float weight_decay, float max_norm,
                              const int32_t *skip_flag, float *norm_clip_out, void *ws,
                              size_t ws_bytes, void *stream);

/* The writeback alone (the same kernel muon_step ends with; [8526]
 * description: only the intersection of each matrix's update with a rank's
 * partition is copied there, the alignment padding is not): for every
 * matrix i, partitions[r][...] = fp32(updates[i][j]) * fp32(sqrt(max(1,
 * rows/cols))) on the owned intersections, one IEEE round-to-nearest
 * multiply, padding untouched.  updates[i] is the unscaled Newton-Schulz
 * output in the original orientation, dense rows x cols of dtype `dtype`.
 * ws/ws_bytes: the plan's workspace (it holds the run table).
 * Errors: INVALID_ARG, ALIAS, WORKSPACE, HIP. */
muon_status muon_scatter(muon_plan *p, const void *const *updates, int32_t dtype,
                         float *const *partitions, void *ws, size_t ws_bytes, void *stream);

/* Counters of the plan ([8600] results table counts Newton-Schulz calls). */
muon_status muon_plan_stats(const muon_plan *p, muon_stats *out);

/* Host-side introspection of the static layout (no device call).
 * muon_plan_runs: the owned intersections of matrix `matrix`, in element
 * order; writes min(cap, total) runs and sets *count to the total.
 * muon_plan_problems: the Newton-Schulz problems in plan order, likewise. */
muon_status muon_plan_runs(const muon_plan *p, int32_t matrix, muon_run *out, int32_t cap,
                           int32_t *count);
muon_status muon_plan_problems(const muon_plan *p, muon_problem_info *out, int32_t cap,
                               int32_t *count);

/* Phase timing.  While enabled, muon_step records HIP events on its stream
 * around its three phases (K1 with the norm finalisation; all Newton-Schulz
 * launches; K3), per workspace wave.  muon_plan_phase_ms waits for the last
 * timed step's events and writes the phase times in milliseconds, summed over
 * waves: out[0] K1+norm, out[1] Newton-Schulz, out[2] K3; *ns_launches gets
 * the number of Newton-Schulz launches that step made.  Errors:
 * INVALID_ARG (NULL plan/out, or no timed step yet), HIP. */
muon_status muon_plan_set_timing(muon_plan *p, int32_t enable);
muon_status muon_plan_phase_ms(muon_plan *p, float out[3], int32_t *ns_launches);

void muon_plan_destroy(muon_plan *p);
const char *muon_status_string(muon_status s);
const char *muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
