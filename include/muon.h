/*
 * muon.h - C ABI of the Periodic Row-wise Muon optimizer step for gfx950.
 *
 * What one step computes, for every 2-D weight W (m x n, row-major) with
 * gradient G and explicitly stored momentum M:
 *
 *   M <- beta * M + G
 *   t mod K == 0 :  U = NS5(M)                 (Newton-Schulz, 5 iterations)
 *   otherwise    :  U = gamma * RowNorm_eps(M)  (slice / max(||slice||_2, eps))
 *   W <- W - lr * U
 *
 * Sources: "Scaling Muon for Diffusion Transformers", English abstract
 * (periodic full NS5 refresh, row-wise update on the current momentum,
 * momentum kept in full); PaperDaily post on that paper, section "Periodic
 * Row-wise Muon" (blog fig. 3: the update rule and refresh indicator; blog
 * fig. 4: the RowNorm formula; defaults K=3, gamma=0.15) and section
 * "distributed co-design" (paper Eq. (8): tall matrices take column
 * statistics).  The optional block-periodic variant follows "MuonBP: Faster
 * Muon via Block-Periodic Orthogonalization", English abstract.  Tensors that
 * are not 2-D weights (biases, norm scales) take an AdamW step (the post,
 * section "From 1.3B to 15B").
 *
 * Readings where the pages are silent (all are fields of muon_config):
 *   - NS5 runs on the wide orientation (m > n matrices are transposed), with
 *     X0 = M / (||M||_F + ns_eps) and coefficients (a, b, c); defaults are
 *     those of the Muon reference the post cites.
 *   - RowNorm slices are rows of the wide orientation (columns when m > n)
 *     unless rownorm_axis = 1 (stored rows always).
 *   - t is supplied by the caller and starts at 0, so t = 0 refreshes.
 *   - MuonBP: bp_blocks equal splits of the stored column axis; a full NS5
 *     with lr when t mod bp_period == 0, otherwise per-block NS5 with
 *     lr * bp_lr_ratio.
 *
 * Memory and ownership
 *   All tensor pointers are DEVICE pointers owned by the caller.  The
 *   library never allocates device memory: the caller provides one state
 *   buffer of muon_state_bytes() bytes (any device allocation, 256-byte
 *   aligned), out of which the library carves momentum, AdamW moments, the
 *   NS5 workspace and its own launch tables.  The buffer must stay alive and
 *   untouched (except through muon_state views) until muon_free.
 *
 * Asynchrony and threading
 *   muon_step only enqueues work on the stream given to muon_init and never
 *   synchronises it (no allocation, no host wait).  muon_init enqueues the
 *   zeroing of the state and the upload of its launch tables, then waits for
 *   that stream once.  Buffers must stay valid until the
 *   stream has passed the step.  One context per stream; calls on one
 *   context are not re-entrant.  Separate contexts are independent.
 *
 * Errors
 *   Every function returns a status and never throws or aborts.  Argument
 *   validation happens before anything is enqueued: a call that returns
 *   MUON_E_ARG / _SHAPE / _DTYPE / _ALIGN / _WORKSPACE has enqueued nothing.
 *   MUON_E_HIP means a HIP runtime call failed (kernel faults surface on a
 *   later call); muon_last_error() gives the text.  NaN/Inf in gradients are
 *   not checked and propagate.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
  MUON_OK = 0,
  MUON_E_ARG = 1,       /* null pointer, bad config value, negative step   */
  MUON_E_SHAPE = 2,     /* bad dims, mismatch with the plan, MuonBP split  */
  MUON_E_DTYPE = 3,     /* unsupported dtype or mismatch with the plan     */
  MUON_E_ALIGN = 4,     /* pointer not 16-byte aligned, or ld != cols      */
  MUON_E_WORKSPACE = 5, /* state buffer missing or smaller than required   */
  MUON_E_STATE = 6,     /* context unusable, index out of range            */
  MUON_E_HIP = 7        /* a HIP runtime call failed                       */
} muon_status;

typedef enum muon_dtype { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* How a parameter is updated.  MATRIX: Muon (W must be F32, 2-D).
 * ADAMW: coordinate-wise AdamW (F32 parameter of rows x cols elements). */
typedef enum muon_kind { MUON_KIND_MATRIX = 0, MUON_KIND_ADAMW = 1 } muon_kind;

/* Direction map of a step; returned by muon_branch. */
typedef enum muon_branch_id {
  MUON_BRANCH_ROWNORM = 0,   /* gamma * RowNorm_eps(M)                     */
  MUON_BRANCH_NS5 = 1,       /* NS5(M) on the whole matrix                  */
  MUON_BRANCH_BLOCK_NS5 = 2  /* MuonBP: NS5 of each column block on its own */
} muon_branch_id;

/* Arithmetic of the NS5 matrix products.  The pages fix no precision for
 * the iteration X <- a X + (b A + c A A) X; these are this library's choices. */
typedef enum muon_ns_precision {
  MUON_NS_BF16 = 0,      /* bf16 MFMA operands, fp32 accumulation          */
  MUON_NS_F32 = 1,       /* fp32 MFMA operands and accumulation            */
  MUON_NS_BF16_COMP = 2  /* as MUON_NS_BF16, and the a X term of every round
                          * also takes X's bf16 rounding remainder, kept as
                          * a second bf16 array (2 more workspace bytes per
                          * element, 4 more bytes moved per element and
                          * round).  It keeps singular directions far below
                          * the largest from being lost to X's rounding:
                          * on spectra spread over decades the bf16 form
                          * deviates from the exact iteration by 2-7e-2,
                          * this one by under 1e-2.                       */
} muon_ns_precision;

/* A dense row-major device tensor.  rows, cols >= 1 and ld == cols.
 * AdamW tensors of any rank are passed flattened (rows = 1 is fine). */
typedef struct muon_tensor {
  void* ptr;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  int32_t dtype;     /* muon_dtype */
  int32_t reserved;  /* must be 0 */
} muon_tensor;

typedef struct muon_config {
  float lr;              /* Muon learning rate (0.02)                       */
  float beta;            /* momentum (0.95)                                 */
  float gamma;           /* RowNorm multiplier (0.15)                       */
  float eps_row;         /* RowNorm floor on the slice norm (1e-8)          */
  int32_t K;             /* refresh period, >= 1 (3); K = 1 is vanilla Muon */
  int32_t ns_iters;      /* Newton-Schulz iterations, >= 1 (5)              */
  float ns_a, ns_b, ns_c;/* quintic coefficients (3.4445, -4.7750, 2.0315)  */
  float ns_eps;          /* Frobenius pre-normalisation floor (1e-7)        */
  int32_t ns_precision;  /* muon_ns_precision (MUON_NS_BF16)                */
  int32_t rownorm_axis;  /* 0: long axis (default); 1: stored rows          */
  int32_t bp_blocks;     /* MuonBP column blocks; 0 = off                   */
  int32_t bp_period;     /* MuonBP full-orthogonalisation period (3)        */
  float bp_lr_ratio;     /* block-step lr / full-step lr (0.5)              */
  float muon_wd;         /* decoupled weight decay on Muon weights (0)      */
  float adam_lr, adam_b1, adam_b2, adam_eps, adam_wd;
                         /* (1e-3, 0.9, 0.999, 1e-8, 0)                     */
  uint64_t ns_workspace_max; /* cap on NS5 workspace bytes; 0 = no cap     */
  int32_t tall_single_pass; /* 1 (default): long-axis RowNorm of a tall
                          * matrix (m > n, n even, m <= 32768) runs as
                          * one pass over its tensors, with the column norms
                          * formed across workgroups (the post's section
                          * "distributed co-design", paper Eq. (8): column
                          * sums of squares over row shards added up);
                          * 0: two passes, momentum and column sums first,
                          * then the weight update (M read twice).  Same
                          * values up to the order of the sums.             */
  int32_t reserved0;     /* must be 0                                       */
} muon_config;

typedef struct muon_ctx muon_ctx;

/* Fill *out with the defaults listed above.  Pure host function. */
muon_status muon_config_default(muon_config* out);

/* Bytes of state buffer that muon_init needs for this parameter list.
 * params[i] / kinds[i] (muon_kind) for i < n; n == 0 is a valid empty set.
 * MUON_E_SHAPE also when a matrix's Newton-Schulz working copy (short side
 * by long side, padded to the GEMM tile, 2 bytes per value in bf16, 4 in
 * fp32) reaches 4 GiB: the GEMM kernels address it with 32-bit offsets.
 * Pure host function: touches no device. */
muon_status muon_state_bytes(const muon_config* cfg, const muon_tensor* params,
                             const int32_t* kinds, int32_t n, size_t* bytes);

/* Build the launch plan, zero all optimizer state and upload the launch
 * tables into the state buffer; waits for hip_stream once before returning.
 * Source: "Scaling Muon for Diffusion Transformers", English abstract (the
 * momentum of every 2-D weight is materialised in full, so each matrix gets
 * an fp32 momentum of its own shape here, zero at init); PaperDaily post,
 * section "From 1.3B to 15B" (biases and normalisation parameters take
 * AdamW: kinds[i] = MUON_KIND_ADAMW); section "distributed co-design"
 * (same-shape matrices are gathered in buckets with a bounded number
 * materialised at once: here the NS5 problems are grouped into chunks under
 * ns_workspace_max).
 * params/grads: descriptors of the tensors later steps will pass; their
 *   shapes and dtypes are fixed here, their pointers may change per step.
 *   Matrix params must be F32; grads may be F32 or BF16.
 * state_buf/state_bytes: caller-owned device buffer on the current device,
 *   256-byte aligned, >= muon_state_bytes() (may be NULL when that is 0).
 * hip_stream: a hipStream_t (NULL = the null stream) on the current device.
 * On success *out receives a context to pass to muon_step / muon_free. */
muon_status muon_init(muon_ctx** out, const muon_config* cfg,
                      const muon_tensor* params, const muon_tensor* grads,
                      const int32_t* kinds, int32_t n,
                      void* state_buf, size_t state_bytes, void* hip_stream);

/* Enqueue one optimizer step t >= 0 on the context's stream: updates every
 * param in place and the state in the buffer.  params/grads must match the
 * init-time shapes and dtypes (pointers may differ).  Does not synchronise.
 * Source: PaperDaily post, section "Periodic Row-wise Muon", blog fig. 3
 * (M <- beta M + G; t mod K == 0 takes NS5(M), the other steps
 * gamma * RowNorm_eps(M) of the current momentum; W <- W - lr * U), blog
 * fig. 4 (RowNorm divides each slice by max(||slice||_2, eps)) and section
 * "distributed co-design", paper Eq. (8) (tall matrices normalise columns);
 * "MuonBP: Faster Muon via Block-Periodic Orthogonalization", English
 * abstract (bp_blocks > 0: per-block NS5 with lr * bp_lr_ratio between full
 * orthogonalisations). */
muon_status muon_step(muon_ctx* ctx, const muon_tensor* params,
                      const muon_tensor* grads, int64_t step);

/* For callers that cannot allocate device memory (serving loops, harnesses
 * that forbid hipMalloc): one optimizer step of n Muon matrices, like
 * muon_step, with no context and no state buffer.  The caller passes each
 * matrix's weight (params[i], F32), gradient (grads[i], F32 or BF16) and
 * momentum (moms[i], F32, same shape; read and written, zero before the
 * first step).  Everything else the step needs - launch tables, the
 * Newton-Schulz workspace, RowNorm column partials and counters - lives in
 * one static device array of 128 MiB per GPU (held from the library's first
 * use on that GPU until the process ends).  The call allocates nothing: it
 * clears the array's counters with a kernel, copies the launch tables into
 * it, waits for hip_stream once (so it cannot be captured into a graph),
 * then enqueues the step.  Matrices are planned in chunks whose workspace
 * fits the array; a step whose largest matrix does not fit (bf16
 * workspace about 2 (2 r c + 2 r^2) bytes, r x c the padded short x long
 * side: e.g. 2048 x 12288 fits, 3072 x 18432 does not) returns
 * MUON_E_WORKSPACE with the size it needed, having enqueued nothing.  Every
 * call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other host threads, or other
 * streams not yet past an earlier call) race and give wrong results.
 * Other errors as muon_step; muon_last_error(NULL) gives the text. */
muon_status muon_step_noalloc(const muon_config* cfg, const muon_tensor* params,
                              const muon_tensor* grads, const muon_tensor* moms, int32_t n,
                              int64_t step, void* hip_stream);

/* A view into the state buffer, for checkpointing and inspection.  Source:
 * "Scaling Muon for Diffusion Transformers", English abstract (the momentum
 * is stored explicitly and in full, so it can be read back and restored).
 * which = 0: momentum of a matrix, or AdamW first moment;
 * which = 1: AdamW second moment.  The view is F32, same shape as param i;
 * writing through it (after the stream is idle) restores a checkpoint. */
muon_status muon_state(const muon_ctx* ctx, int32_t i, int32_t which,
                       muon_tensor* view);

/* muon_branch_id that step t takes under cfg, or -1 if cfg or t is invalid.
 * Pure host integer function (PaperDaily post, blog fig. 3: t multiple of K
 * refreshes; MuonBP abstract for the block variant). */
int32_t muon_branch(const muon_config* cfg, int64_t step);

/* Wait for the context's stream.  MUON_E_HIP if the wait failed (a kernel
 * fault or an earlier HIP error).  The library never waits on the host
 * otherwise; call this where a check is wanted. */
muon_status muon_sync(muon_ctx* ctx);

/* The single-pass tall RowNorm forms each column strip's norms across
 * workgroups (the post's section "distributed co-design", paper Eq. (8):
 * column sums of squares over row shards, added up).  A workgroup waits for
 * its strip's sum; after `polls` polls (default 262144, about half a
 * second) it stops waiting, leaves its tile of W alone and lists it, and a
 * repair launch that muon_step enqueues right after writes the listed tiles
 * with the same arithmetic, bit for bit.  A wait can only reach the limit
 * when other work holds most of the device's compute units.  polls = 0
 * makes every wait give up at once (for testing the repair path).  Host
 * only; applies to steps enqueued after the call. */
muon_status muon_tall_poll_limit(muon_ctx* ctx, uint32_t polls);

/* Waits for the context's stream, then writes to *count how many waits of
 * the single-pass tall RowNorm have given up (and been repaired) since
 * muon_init.  MUON_E_HIP if the wait or the read failed. */
muon_status muon_tall_giveups(muon_ctx* ctx, uint64_t* count);

/* Release host-side plan memory.  Does not touch the state buffer or the
 * stream; the caller must not free the state buffer while the stream still
 * runs the context's work.  NULL is ignored. */
void muon_free(muon_ctx* ctx);

/* Static text of a status code. */
const char* muon_status_str(int32_t status);

/* Text of the last error on ctx (or of the last failed muon_init /
 * muon_state_bytes on this thread when ctx is NULL).  Never NULL. */
const char* muon_last_error(const muon_ctx* ctx);

/* ---- Measurement --------------------------------------------------------
 * Kernel classes whose launches muon_step can time (see muon_timing_*). */
typedef enum muon_kernel_class {
  MUON_K_ROWNORM_ROWS = 0,   /* RowNorm step, row-normalised matrices        */
  MUON_K_ROWNORM_COLS1 = 1,  /* RowNorm step, tall: momentum + column sums   */
  MUON_K_ROWNORM_COLS2 = 2,  /* RowNorm step, tall: scale + weight update    */
  MUON_K_NS_PREP = 3,        /* refresh: momentum, Frobenius partials, X0    */
  MUON_K_NS_SCALE = 4,       /* refresh: 1 / (||M||_F + eps)                 */
  MUON_K_NS_GRAM = 5,        /* refresh: A = X X^T                           */
  MUON_K_NS_POLY = 6,        /* refresh: B = b A + c A A                     */
  MUON_K_NS_PRODUCT = 7,     /* refresh: X = a X + B X, rounds 1 .. n-1      */
  MUON_K_NS_PRODUCT_LAST = 8,/* refresh: last round, fused W update          */
  MUON_K_ADAMW = 9,          /* AdamW on the non-matrix tensors              */
  MUON_K_ROWNORM_COEF = 10,  /* RowNorm step, tall: column coefficients      */
  MUON_K_ROWNORM_TALL = 11,  /* RowNorm step, tall, single pass              */
  MUON_K_ROWNORM_REPAIR = 12,/* RowNorm step, tall: tiles whose wait gave up */
  MUON_K_COUNT = 13
} muon_kernel_class;

/* While enabled (enable != 0), muon_step records a HIP event before and
 * after every kernel launch, on the context's stream, so that launch
 * durations can be read back per kernel class.  Adds two event records per
 * launch; allocates no device memory.  Disabled by default. */
muon_status muon_timing_enable(muon_ctx* ctx, int32_t enable);

/* Waits for every event recorded since the last read, then writes, per
 * kernel class k < MUON_K_COUNT, the summed launch durations in ms[k]
 * (milliseconds) and the number of launches in launches[k], and clears the
 * record.  Either array may be NULL. */
muon_status muon_timing_read(muon_ctx* ctx, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
