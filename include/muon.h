/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon / AdamW optimizer-step library.
 *
 * Sources the operations follow, cited by page title and section:
 *   [OPT] "Optimizer tutorial" page on mhpq.cn (large-model training series,
 *         part 2): 2.1 momentum as an EMA of the gradient; 2.3 Adam with
 *         bias correction; 3.1 AdamW's decoupled weight decay; 3.3 fp32
 *         master weights cast back to 16 bit; 4.2 the Newton-Schulz
 *         iteration X <- (3X - X X^T X)/2, run a fixed number of times.
 *   [K2]  Zhihu answer by toothacher17 on the Kimi K2 release: 2.2 the
 *         optimizer works on all parameters flattened and concatenated,
 *         each matrix whole; 3.1 Muon's update RMS is matched to AdamW's;
 *         3.2 the max(1, sqrt(d_out/d_in)) update scale; 4 the spectral
 *         norm is bounded by the Frobenius norm.
 *   [EP]  aihot.vn news item on MoonEP, "memory contract": expert weights
 *         live in one contiguous [E, H, H'] tensor addressed by row offset.
 *   [K2]  section 4, MuonClip: the max attention logit grows in large Muon
 *         runs; since ||x W||_2 <= ||x||_2 ||W||_2 <= ||x||_2 ||W||_F, a
 *         clip of the weight's Frobenius norm bounds it; the method's author
 *         acts on the max logit itself.
 *   [OPT] 5.4 (optimizer numerical faults under mixed precision): keep
 *         gradient clipping (clip_grad_norm) as a safety net, guard the
 *         step against Inf/NaN by skipping it, and watch statistics of the
 *         optimizer state (mean and variance of m, collapse of v).
 *
 * Conventions for every call:
 *   - Returns MUON_OK (0) or a negative MUON_ERR_* code; nothing throws.
 *     muon_last_error() gives a message for the last failure on the
 *     calling thread.
 *   - Device pointers are plain HIP device addresses on the device that was
 *     current when the plan was uploaded.  All device memory is owned by
 *     the caller; the library allocates none.  The only device pointer it
 *     keeps after a call returns is a plan's table buffer (muon_plan_upload,
 *     muon_clip_plan_upload), which the caller keeps alive while the plan
 *     is used.
 *   - Work is enqueued on the caller's HIP stream; the library never
 *     synchronises.  A kernel fault surfaces at the caller's next
 *     synchronisation of that stream.
 *   - Buffers passed to one call must not alias each other.
 *   - Non-finite inputs propagate into the outputs unless the step is
 *     guarded through a clip state (grad_norm_clip below).
 *   - Muon folds the normalisation X0 = U / (||U||_F + eps) into its first
 *     products, which accumulate the unnormalised U U^T in fp32.  A matrix
 *     whose ||U||_F (finite, nonzero) lies outside [2^-40, 2^40] first has
 *     its U scaled by an exact power of two, so every step is in range for
 *     any finite fp32 U with ||U||_F below the fp32 maximum.  With eps = 0
 *     an all-zero U gives 0/0, which propagates as NaN.
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define MUON_OK 0
#define MUON_ERR_INVALID_ARG (-1)        /* null pointer, bad hyperparameter, wrong device */
#define MUON_ERR_BAD_SHAPE (-2)          /* rows/cols < 1, matrix outside the flat buffer, too large */
#define MUON_ERR_OVERLAP (-3)            /* two matrices share flat elements */
#define MUON_ERR_WORKSPACE_TOO_SMALL (-4)
#define MUON_ERR_BAD_DTYPE (-5)
#define MUON_ERR_HIP (-6)                /* a HIP runtime call failed; see muon_last_error() */
#define MUON_ERR_UNSUPPORTED (-7)

/* ---- element types ---------------------------------------------------- */
#define MUON_DTYPE_FP32 0
#define MUON_DTYPE_BF16 1
#define MUON_DTYPE_FP16 2 /* IEEE binary16: AdamW second moment only */

/* One matrix of the flat buffer ([K2] 2.2): elements
 * [offset, offset + rows*cols) of the flat params / grads / momentum
 * buffers, row-major [rows, cols].  The same offset addresses all three. */
typedef struct {
  int64_t offset;
  int32_t rows;
  int32_t cols;
} muon_matrix_t;

/* Hyperparameters of one Muon step.
 *   lr, weight_decay : W <- (1 - lr*wd) W - lr*s*O   ([OPT] 3.1 decoupled form)
 *   momentum (mu)    : M <- mu M + (1-mu) G          ([OPT] 2.1 EMA)
 *   nesterov         : nonzero: NS input U = mu M + (1-mu) G; zero: U = M
 *   ns_a, ns_b, ns_c : per NS iteration A = X X^T, B = b A + c A A,
 *                      X <- a X + B X  ([OPT] 4.2 prints (1.5, -0.5, 0))
 *   ns_steps         : number of NS iterations (>= 0; [OPT] 4.2: typically 5)
 *   eps              : X0 = U / (||U||_F + eps)      ([K2] 4)
 *   scale_mode       : s = rms_target*sqrt(max(r,c)) (0, [K2] 3.1),
 *                      sqrt(max(1, r/c)) (1, [K2] 3.2), 1 (2)
 */
/* Result of grad_norm_clip, resident in device memory ([OPT] 5.4):
 *   norm  : global L2 norm of all the gradients given (fp64 sum of squares)
 *   scale : min(1, max_norm / (norm + eps)), the factor every gradient is
 *           multiplied by before the step; 1 when clipping is off
 *   skip  : 1 when the norm is not finite (a NaN or Inf gradient): a step
 *           given this state changes no parameter and no state buffer
 * The steps read it on the device, so clipping and the guard need no host
 * synchronisation. */
typedef struct {
  float norm;
  float scale;
  int32_t skip;
  int32_t reserved;
} muon_clip_state_t;

typedef struct {
  float lr;
  float weight_decay;
  float momentum;
  int32_t nesterov;
  float ns_a;
  float ns_b;
  float ns_c;
  int32_t ns_steps;
  float eps;
  int32_t scale_mode;
  float rms_target;
  /* nullable device pointer: gradient scale and step guard from
   * grad_norm_clip; read by muon_step, muon_stage_momentum (scale, skip),
   * muon_stage_apply and muon_stage_ns_apply (skip) */
  const muon_clip_state_t* clip;
} muon_hparams_t;

/* Hyperparameters of one AdamW step ([OPT] 2.3, 3.1). */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  /* nullable device pointer: gradient scale and step guard (see above) */
  const muon_clip_state_t* clip;
} adamw_hparams_t;

/* Opaque plan: matrix descriptors validated, orientation (tall matrices
 * are iterated transposed so the Gram matrix is min(r,c) square), padding
 * to the GEMM tile, workspace layout, tile lists and waves ([K2] 2.2: the
 * flat concatenation, each matrix whole at its offset).  Creation is
 * host-only.  Its tables go to the device once, into a caller buffer, with
 * muon_plan_upload; after that the plan is read-only and steps on several
 * streams may share it. */
typedef struct muon_plan muon_plan_t;

typedef struct {
  int32_t n_mats;
  int32_t n_waves;
  int32_t tile;               /* GEMM tile edge (256 for bf16 NS, 64 for fp32 NS) */
  int32_t ns_dtype;
  int64_t k1_tiles;           /* 64x64 elementwise tiles, all waves */
  int64_t syrk_tiles;         /* X X^T tiles (one triangle), all waves */
  int64_t bx_tiles;           /* B X tiles, all waves */
  size_t workspace_bytes;
  double ns_flops_per_iter_alg;   /* algorithmic flops per NS iteration with c != 0 */
  int32_t small_mats;         /* matrices on the fused small-matrix path (below) */
  int32_t split_tile_mats;    /* tiled bf16 matrices with split tiles (below;
                                 all of them unless MUON_PLAN_WHOLE_TILES) */
  int32_t fused_apply_mats;   /* matrices whose update can be applied by the
                                 last phase 3 (muon_stage_ns_apply) */
  int32_t round_sync_phases;  /* bit p-1 set (p = 1, 2): the bf16 kernels of
                                 NS phase p hold the tile rounds of each XCD
                                 together (in at least one wave); a
                                 scheduling choice of the plan, results do
                                 not depend on it */
} muon_plan_info_t;

/* Host-only sizing: validates exactly as muon_plan_create and returns the
 * workspace size in bytes.  Makes no HIP call; usable without a GPU.
 * workspace_cap (bytes, 0 = unlimited) bounds the workspace by splitting
 * the matrices into waves that run one after another. */
int muon_workspace_size(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                        int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                        size_t workspace_cap, size_t* workspace_bytes);

/* Build a plan (host memory only; no HIP call, no device memory).  n_mats
 * may be 0 (steps are then no-ops).  On success *out owns the plan and
 * *workspace_bytes is the size of the device workspace every step needs.
 * Upload the plan (muon_plan_upload) before its first step. */
int muon_plan_create(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                     int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                     size_t workspace_cap, muon_plan_t** out, size_t* workspace_bytes);

/* muon_plan_create with flags.  By default (flags 0) a matrix with bf16 NS
 * whose padded short side m_k (min(rows, cols) rounded up to 32) is at
 * most 128 and whose m_k * n_k is at most 32768 runs each NS iteration in
 * one workgroup with X, A and B in LDS (one launch per iteration instead of
 * three single-tile launches); its iterates are bitwise those of the tiled
 * path.  MUON_PLAN_TILED_ONLY puts every matrix on the tiled path.
 *
 * X X^T and A A are symmetric: the tiled path computes the tiles on and
 * above the diagonal and mirrors them.  On a tiled bf16 matrix (split
 * tiles) a diagonal tile also computes only its upper 32x32 blocks and
 * mirrors the rest; for a matrix whose short side pads to more than 8 tiles
 * (2048) those tiles run after all off-diagonal tiles of the phase.  On a
 * matrix of at most 8 tiles per side, an edge tile whose last 128 rows or
 * columns are padding computes only the half that holds data.  The result
 * is bitwise the same either way; MUON_PLAN_WHOLE_TILES computes every tile
 * whole, in place.
 *
 * The bf16 NS kernels keep one workgroup per CU walking the tile list in
 * rounds of 32 tiles per XCD; tiles of a round share operand panels in the
 * XCD's L2.  Where the plan finds that a round's tiles cost much the same
 * (muon_plan_info_t.round_sync_phases), phases 1 and 2 hold each XCD's
 * workgroups together every few rounds: a bounded wait on a counter in the
 * workspace, a timing device only.  MUON_PLAN_FREE_ROUNDS turns it off
 * (useful when other kernels share the GPU, where the wait runs into its
 * bound); the result is bitwise the same either way. */
#define MUON_PLAN_TILED_ONLY 1u
#define MUON_PLAN_WHOLE_TILES 2u
#define MUON_PLAN_FREE_ROUNDS 4u
int muon_plan_create_ex(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                        int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                        size_t workspace_cap, uint32_t flags, muon_plan_t** out,
                        size_t* workspace_bytes);

/* Frees the plan's host memory (the caller frees its table buffer). */
void muon_plan_destroy(muon_plan_t* plan);

/* Bytes of device memory the plan's tables take (matrix descriptors, the
 * elementwise and GEMM tile lists); 0 for a plan without matrices.
 * Host-only. */
size_t muon_plan_table_bytes(const muon_plan_t* plan);

/* Copies the plan's tables into `tables` with one hipMemcpyAsync on
 * `stream` and binds the plan to the current device.
 *   tables      : device memory on the current device, owned by the caller,
 *                 >= muon_plan_table_bytes(plan) bytes, 256-byte aligned
 *                 (may be NULL when that size is 0).  The caller keeps it
 *                 alive and unmodified while the plan is used; the copy
 *                 reads the plan's host memory, so the plan must outlive it.
 *   table_bytes : size of `tables`
 * Steps on `stream` are ordered after the copy; steps on other streams must
 * be ordered after it by the caller.  Every step needs an uploaded plan
 * (MUON_ERR_INVALID_ARG otherwise) on the device it was uploaded on.
 * Uploading again (e.g. to another buffer) must not overlap running steps. */
int muon_plan_upload(muon_plan_t* plan, void* tables, size_t table_bytes, hipStream_t stream);

int muon_plan_get_info(const muon_plan_t* plan, muon_plan_info_t* info);

/* One Muon step on every matrix of the plan.
 *   params     : flat, param_dtype, updated in place (bf16 stored RNE)
 *   grads      : flat, grad_dtype, read only
 *   momentum   : flat fp32, updated in place
 *   workspace  : >= workspace_bytes of device memory, 256-byte aligned;
 *                scratch only, contents on entry are ignored
 *   out_update : nullable flat fp32; receives O (the orthogonalised update
 *                before scaling) at each matrix's elements
 * Elements of the flat buffers not covered by a matrix are never touched.
 * With hp->clip set, every gradient is multiplied by clip->scale, and if
 * clip->skip is set params, momentum and out_update are left unchanged.
 * Without out_update (and ns_steps >= 1) the last NS phase applies the
 * update itself (muon_stage_ns_apply); the result is bitwise the same.
 * Concurrent steps on one workspace race; use one workspace per stream. */
int muon_step(const muon_plan_t* plan, void* params, const void* grads, float* momentum,
              void* workspace, size_t workspace_bytes, const muon_hparams_t* hp,
              float* out_update, hipStream_t stream);

/* muon_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is the library's own static device array of
 * MUON_NOALLOC_WORKSPACE_BYTES (256 MiB), which every GPU the library runs
 * on holds until the process ends; the call allocates nothing.  The plan's
 * workspace_bytes must fit in it (create the plan with workspace_cap <=
 * MUON_NOALLOC_WORKSPACE_BYTES: larger sets of matrices then run in waves),
 * else MUON_ERR_WORKSPACE_TOO_SMALL and nothing is enqueued.  The plan must
 * have been uploaded on the current device (which also looks the array's
 * address up).  Results are bitwise those of muon_step with a workspace of
 * its own.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (as with muon_step, contents on entry are ignored):
 * calls that overlap on one GPU, on different streams or from different
 * threads, race and give wrong results; order them on one stream. */
#define MUON_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)
int muon_step_noalloc(const muon_plan_t* plan, void* params, const void* grads,
                      float* momentum, const muon_hparams_t* hp, float* out_update,
                      hipStream_t stream);

/* The stages muon_step enqueues, exposed for stepwise checks and timing.
 * muon_step(...) == for each wave w: muon_stage_momentum(w);
 *   for it in [0, ns_steps): for phase in {1, 2 (only if ns_c != 0), 3}:
 *   muon_stage_ns_phase(w, it, phase); muon_stage_apply(w); without
 *   out_update the last phase 3 and the apply are muon_stage_ns_apply(w).
 *   (muon_step runs the small matrices' iterations in one launch; the
 *   stage calls run one per phase-3 call; the results are bitwise equal.)
 * Phase 1: A = X X^T; phase 2: B = b A + c A A; phase 3: X <- a X + B X
 * (with c == 0, phase 3 uses b A for B).  The apply step is
 * W <- (1 - lr wd) W - lr s O with s the update scale of scale_mode
 * (optimizer tutorial 3.1, decoupled decay; K2 answer 3.1, 3.2). */
int muon_stage_momentum(const muon_plan_t* plan, int32_t wave, const void* grads,
                        float* momentum, void* workspace, size_t workspace_bytes,
                        const muon_hparams_t* hp, hipStream_t stream);
int muon_stage_ns_phase(const muon_plan_t* plan, int32_t wave, void* workspace,
                        size_t workspace_bytes, const muon_hparams_t* hp, int32_t iter,
                        int32_t phase, hipStream_t stream);
int muon_stage_apply(const muon_plan_t* plan, int32_t wave, void* params, void* workspace,
                     size_t workspace_bytes, const muon_hparams_t* hp, float* out_update,
                     hipStream_t stream);
/* muon_stage_ns_phase(w, ns_steps - 1, 3) followed by muon_stage_apply(w)
 * with out_update NULL, bitwise, in fewer HBM passes: with bf16 NS and
 * bf16 params in a 16-byte aligned buffer, every tiled matrix
 * (muon_plan_info_t.fused_apply_mats; any offset and cols) has its update
 * applied by the phase-3 epilogue, which reads and writes W instead of
 * writing X (X of the last iteration is then not in the workspace;
 * muon_stage_export_x must not be asked for it); the small matrices run
 * the apply kernel, and so does every matrix when the buffer is not
 * 16-byte aligned.  ns_steps must be >= 1.  With hp->clip->skip set,
 * params are left unchanged. */
int muon_stage_ns_apply(const muon_plan_t* plan, int32_t wave, void* params, void* workspace,
                        size_t workspace_bytes, const muon_hparams_t* hp, hipStream_t stream);

/* Copy the current NS iterate of every matrix of a wave into a flat fp32
 * buffer at each matrix's elements, in the caller's [rows, cols] layout
 * (after muon_stage_momentum it is U, the un-normalised NS input, or
 * U * 2^k for a matrix whose ||U||_F lies outside [2^-40, 2^40]).
 * For stepwise checks. */
int muon_stage_export_x(const muon_plan_t* plan, int32_t wave, const void* workspace,
                        size_t workspace_bytes, int32_t iter_done, float* out,
                        hipStream_t stream);
/* Copy the per-matrix Frobenius norms ||U||_F of a wave (fp32, one per
 * matrix of the wave, in plan order) after muon_stage_momentum. */
int muon_stage_export_norms(const muon_plan_t* plan, int32_t wave, const void* workspace,
                            size_t workspace_bytes, float* out, hipStream_t stream);

/* One AdamW step ([OPT] 2.3, 3.1, 3.3) over n contiguous elements:
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *   theta <- theta - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) - lr wd theta
 * master non-null: theta is the fp32 master, and params (param_dtype)
 *   receives its round-to-nearest-even cast.
 * master null: params must be fp32 and is theta itself.
 * grads: grad_dtype.  exp_avg, exp_avg_sq: fp32, updated in place.
 * step: 1-based t; the bias corrections are formed in fp64 on the host.
 * With hp->clip set, g is multiplied by clip->scale, and if clip->skip is
 * set nothing is written (the caller keeps t for the next step).
 * No alignment is required beyond the element size. */
int adamw_step(void* params, int32_t param_dtype, float* master, const void* grads,
               int32_t grad_dtype, float* exp_avg, float* exp_avg_sq, int64_t n,
               const adamw_hparams_t* hp, int64_t step, hipStream_t stream);

/* adamw_step with compressed optimizer states ([OPT] 2.4: 8-bit AdamW
 * states; 3.3: v tolerates 16-bit or 8-bit storage before m does):
 *   exp_avg_dtype    MUON_DTYPE_FP32 or MUON_DTYPE_BF16
 *   exp_avg_sq_dtype MUON_DTYPE_FP32, MUON_DTYPE_BF16 or MUON_DTYPE_FP16
 * The step reads m and v from their storage, computes in fp32 and stores
 * them rounded to nearest even.  fp16 keeps 10 fraction bits but its
 * smallest subnormal is 2^-24: (1 - beta2) g^2 below 2^-25 is stored as
 * 0, which makes later updates m_hat / eps large for small gradients;
 * bf16 keeps fp32's range with 7 fraction bits.  adamw_step(...) equals
 * adamw_step_ex(..., MUON_DTYPE_FP32, ..., MUON_DTYPE_FP32, ...). */
int adamw_step_ex(void* params, int32_t param_dtype, float* master, const void* grads,
                  int32_t grad_dtype, void* exp_avg, int32_t exp_avg_dtype, void* exp_avg_sq,
                  int32_t exp_avg_sq_dtype, int64_t n, const adamw_hparams_t* hp, int64_t step,
                  hipStream_t stream);

/* ---- gradient clipping, step guard, state statistics ([OPT] 5.4) ------ */

/* One device buffer of gradients for the global norm: n elements of dtype. */
typedef struct {
  const void* ptr;
  int64_t n;
  int32_t dtype;
  int32_t reserved;
} muon_grad_buffer_t;

/* Device workspace grad_norm_clip needs for n_bufs buffers. */
size_t grad_norm_clip_workspace_size(int32_t n_bufs);

/* Global gradient-norm clipping and the non-finite guard ([OPT] 5.4):
 * norm = sqrt(sum over every element of every buffer of g^2), accumulated
 * in fp64 in a fixed order (bitwise reproducible); scale = min(1,
 * max_norm / (norm + eps)), or 1 if max_norm <= 0; skip = norm not finite.
 * Writes *out (device memory).  Pass `out` as the `clip` field of the
 * Muon and AdamW hyperparameters of the same step.  bufs is a host array;
 * buffers with n == 0 may have a null ptr.  workspace: device memory of at
 * least grad_norm_clip_workspace_size(n_bufs) bytes, 8-byte aligned. */
int grad_norm_clip(const muon_grad_buffer_t* bufs, int32_t n_bufs, float max_norm, float eps,
                   void* workspace, size_t workspace_bytes, muon_clip_state_t* out,
                   hipStream_t stream);

/* Statistics of one fp32 optimizer-state buffer ([OPT] 5.4, the state
 * monitoring of the closing notes), over its finite elements: count, mean,
 * population variance, min, max, max |x|; plus the number of NaN and +-Inf
 * elements.  All six values are 0 over no finite element.  fp64
 * accumulation in a fixed order (bitwise reproducible). */
typedef struct {
  double mean;
  double var;
  double min;
  double max;
  double absmax;
  int64_t count;
  int64_t nonfinite;
} muon_state_stats_t;

/* Device workspace state_stats needs. */
size_t state_stats_workspace_size(void);

/* Writes *out (device memory).  x: n fp32 elements.  workspace: at least
 * state_stats_workspace_size() bytes, 8-byte aligned. */
int state_stats(const float* x, int64_t n, void* workspace, size_t workspace_bytes,
                muon_state_stats_t* out, hipStream_t stream);

/* ---- MuonClip ([K2] 4) ---------------------------------------------- */

/* One block of the flat parameter buffer to clip: rows x cols elements,
 * element (r, c) at offset + r * ld + c (ld >= cols).  A whole row-major
 * [out, in] matrix has ld = cols; one attention head's block of rows of
 * W_q or W_k is a block of that matrix's rows.  group: which entry of
 * max_logits the block follows in max-logit mode (a head, or a layer). */
typedef struct {
  int64_t offset;
  int64_t ld;
  int32_t rows;
  int32_t cols;
  int32_t group;
  int32_t reserved;
} muon_clip_target_t;

#define MUON_CLIP_FROBENIUS 0 /* gamma = min(1, tau / ||W||_F) per block */
#define MUON_CLIP_MAX_LOGIT 1 /* gamma = sqrt(tau / S_group) when S_group > tau */

typedef struct muon_clip_plan muon_clip_plan_t;

/* Validates the blocks (inside [0, flat_numel), rows and cols >= 1,
 * rows * cols < 2^31, no element in two blocks, group in [0, max(n_groups,
 * 1))) and splits them into fixed chunks, in host memory (no HIP call).
 * *workspace_bytes: device workspace muon_clip needs in Frobenius mode (0
 * in max-logit mode).  targets is a host array.  Upload the plan
 * (muon_clip_plan_upload) before its first use. */
int muon_clip_plan_create(const muon_clip_target_t* targets, int32_t n_targets,
                          int64_t flat_numel, int32_t param_dtype, int32_t n_groups,
                          muon_clip_plan_t** out, size_t* workspace_bytes);
/* Frees the plan's host memory (the caller frees its table buffer). */
void muon_clip_plan_destroy(muon_clip_plan_t* plan);
/* Bytes of device memory of the plan's block and chunk tables (0 without
 * blocks).  Host-only. */
size_t muon_clip_plan_table_bytes(const muon_clip_plan_t* plan);
/* Copies the tables into `tables` (caller-owned device memory on the
 * current device, >= muon_clip_plan_table_bytes bytes, 256-byte aligned,
 * kept alive and unmodified while the plan is used) with one
 * hipMemcpyAsync on `stream`, as muon_plan_upload does for a Muon plan. */
int muon_clip_plan_upload(muon_clip_plan_t* plan, void* tables, size_t table_bytes,
                          hipStream_t stream);

/* MuonClip on params (device, the plan's dtype, bf16 or fp32), in place,
 * after the optimizer step ([K2] 4):
 *   MUON_CLIP_FROBENIUS: per block, norm = ||W||_F (fp64 sum of squares in a
 *     fixed order), gamma = tau / norm when norm > tau, else 1; then
 *     ||W||_2 <= ||W||_F <= tau.
 *   MUON_CLIP_MAX_LOGIT: per block, S = max_logits[group] (device, n_groups
 *     floats: the largest attention logit of the forward pass), gamma =
 *     sqrt(tau / S) when S > tau, else 1; scaling a head's W_q and W_k rows
 *     by gamma scales its logits by gamma^2, so the largest becomes tau.
 * A non-finite norm or S leaves the block unchanged (gamma = 1).  Blocks
 * with gamma = 1 are not written.  New values: gamma * w in fp64, rounded
 * to fp32 and then to the storage type (round to nearest even).
 * tau: finite, > 0.  workspace: device, >= the plan's workspace_bytes,
 * 8-byte aligned (Frobenius mode; may be null in max-logit mode).
 * norms_out, scales_out: nullable device arrays of n_targets floats, the
 * block's Frobenius norm before the clip (0 in max-logit mode) and gamma. */
int muon_clip(const muon_clip_plan_t* plan, void* params, int32_t mode, float tau,
              const float* max_logits, void* workspace, size_t workspace_bytes,
              float* norms_out, float* scales_out, hipStream_t stream);

const char* muon_status_string(int32_t status);
const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
