/*
 * libmuon -- the Muon optimizer step for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ or framework types cross it.
 * All device memory (parameters, gradients, momentum buffers, outputs and the
 * workspace) is owned by the caller.  The library launches work on the
 * caller's HIP stream and never waits for it, except where a function below
 * says so.  A step whose matrices fall both into the fused class and into a
 * tiled class (muon_step) also uses one stream of the library's own per
 * device (a plan: its own), forked from the caller's stream with an event
 * after the normalisation pass and joined back before the update pass: work
 * queued on the caller's stream before the call still runs first, work queued
 * after it still sees the finished step.
 *
 * What one step computes, for every 2-D matrix in the list (pages cited by
 * title and section):
 *   1. momentum, EMA form:        M <- mu*M + (1-mu)*G
 *        ("Muon optimizer: matrix-aware LLM", airosetta.com, Muon.step loop;
 *         "Muon meets Mamba", wmrh.cn, section 4.2 _step_muon)
 *   2. Frobenius normalisation:   X0 = bf16(M / (||M||_F + eps))
 *        (airosetta.com, newtonschulz5; "AdamW vs Muon", adg.csdn.net,
 *         section "1. Preprocessing")
 *   3. short side: when rows > cols the iteration works on the transpose
 *        (airosetta.com, newtonschulz5).  Done by logical layout, never by a
 *        copy.
 *   4. ns_steps Newton-Schulz iterations, step k with (a_k, b_k, c_k):
 *        A = X X^T ; B = b_k A + c_k A A ; X <- a_k X + B X
 *        (airosetta.com newtonschulz5 loop; adg.csdn.net section
 *         "2. Newton-Schulz iteration"; the hybrid schedule of section
 *         "3. DeepSeek-V4 hybrid schedule" is a per-step coefficient list)
 *      X and A are held in bf16 (the pages cast to bf16); every product is
 *      accumulated in fp32 and rounded to bf16 once, to nearest-even.  The
 *      a_k X term is folded into the stored matrix, C = a_k I + b_k A +
 *      c_k A A, so X <- C X; C is rounded to bf16 once, and for matrices
 *      whose short side is <= 128 it is kept as a bf16 pair (C_hi + C_lo,
 *      two MFMA passes) to stay well inside the bf16 error budget.
 *   5. decayed, scaled update:    p <- p*(1 - lr*wd) - lr*s*O
 *        (wmrh.cn section 4.2; adg.csdn.net section "3. Scaling and update")
 *      s = 1, or sqrt(max(1, rows/cols)) under MUON_SCALE_SQRT_MAX1 (the
 *      csdn page asks for an RMS rescale by matrix size without a formula;
 *      this is the reading taken), or the per-matrix `scale` when > 0.
 *
 * Error behaviour: every function returns MUON_OK (0) or a negative status.
 * Argument errors are found on the host before anything is launched; nothing
 * is modified then.  Kernel faults are asynchronous and surface at the
 * caller's next synchronisation.  muon_status_string() describes a status;
 * after MUON_EHIP it includes the HIP error text of the calling thread's last
 * failure, after MUON_ENONFINITE the matrix that failed the check.
 *
 * Device: a call works on the calling thread's current HIP device.  Its
 * stream must belong to that device (else MUON_EINVAL, before anything is
 * launched), and so must every buffer it is given (not checkable here: a
 * pointer into another device's memory is the caller's error).
 *
 * Thread safety: calls may come from several host threads; two calls that
 * run concurrently must use different workspaces.
 *
 * Debugging: with MUON_DEBUG set in the environment (any value but "0"),
 * every call keeps all its launches on the caller's stream, synchronises and
 * checks for an error after each launch (MUON_EHIP names the phase), and
 * fills the workspace's iteration buffers with bf16 NaN before a step, so a
 * kernel that read a value no kernel of the step wrote would leave NaN in the
 * result.  The variable is read at every call.  Not for production: it
 * serialises the host with the device.
 *
 * Non-finite check: with MUON_CHECK_FINITE set in the environment (any value
 * but "0"), muon_step, muon_step_ex and an eager muon_plan_step wait for the
 * stream at the end of the step and read back the squared Frobenius norms of
 * the new momenta that the momentum pass already computed (one double per
 * matrix, in the workspace; the gradient's own under MUON_OPT_NS_FIRST).
 * When one is NaN or infinite (a NaN or infinite gradient or momentum entry,
 * or a sum of squares beyond the fp32 range) the call returns MUON_ENONFINITE
 * and muon_status_string() names the first such matrix (its index in the
 * call's list).  Detection only: the step has run, and that matrix's
 * parameter and momentum hold the non-finite values the arithmetic gave
 * ("Muon meets Mamba", section 6.1, lists NaN among the troubles to watch
 * for).  Ignored by muon_step_noalloc, and by a muon_plan_step on a
 * capturing stream (neither may wait or read back).
 *
 * Graph capture: every call stages its descriptor table through a small ring
 * of pinned host buffers that later calls reuse, so a captured copy would
 * replay stale tables.  A call on a stream that is capturing returns
 * MUON_ECAPTURE before anything is launched; muon_plan_step (below) is the
 * capturable form of a step.
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MUON_OK          0
#define MUON_EINVAL     -1   /* bad argument (shape, pointer, count, value)   */
#define MUON_EWORKSPACE -2   /* workspace missing, too small or misaligned    */
#define MUON_EHIP       -3   /* a HIP runtime call or kernel launch failed    */
#define MUON_EALIAS     -4   /* param / grad / momentum ranges overlap        */
#define MUON_ECAPTURE   -5   /* the stream is capturing a graph (see below)    */
#define MUON_ENONFINITE -6   /* MUON_CHECK_FINITE: a momentum norm is NaN/inf  */

/* ---- element types ----------------------------------------------------- */
#define MUON_F32  0
#define MUON_BF16 1

/* ---- RMS scale modes (call level) -------------------------------------- */
#define MUON_SCALE_NONE        0   /* s = 1                                  */
#define MUON_SCALE_SQRT_MAX1   1   /* s = sqrt(max(1, rows / cols))          */

/* One matrix of a muon_step call.
 *   param     fp32, rows x cols, row-major, contiguous; updated in place.
 *   grad      rows x cols, row-major, contiguous, element type grad_dtype
 *             (MUON_F32 or MUON_BF16).  NULL: the matrix is skipped entirely
 *             (no momentum update, no decay), as the pages' optimizer skips
 *             parameters without a gradient.
 *   momentum  fp32, rows x cols, row-major, contiguous; updated in place.
 *             The caller zero-initialises it before the first step.
 *   rows, cols  >= 1 and <= MUON_MAX_DIM.  Only 2-D matrices are accepted;
 *             routing 1-D parameters, embeddings and heads elsewhere is the
 *             caller's job.
 *   scale     per-matrix update scale s when > 0; otherwise the call's
 *             rms_scale_mode decides.
 * param, grad and momentum must be 4-byte aligned (16-byte alignment and
 * cols % 8 == 0 select the vectorised path) and must not overlap each other
 * or any other matrix's param / momentum. */
typedef struct {
  float*       param;
  const void*  grad;
  float*       momentum;
  int64_t      rows;
  int64_t      cols;
  int32_t      grad_dtype;
  float        scale;
} muon_matrix_t;

/* Coefficients of one Newton-Schulz iteration X <- a X + (b A + c A^2) X. */
typedef struct { float a, b, c; } muon_ns_coeff_t;

#define MUON_MAX_DIM      (1 << 20)
#define MUON_MAX_NS_STEPS 64

/* Bytes of device workspace a muon_step (or muon_orthogonalize) call over
 * these shapes needs.  Depends only on the shapes (grad == NULL entries are
 * counted too, so one workspace serves every call over the same list).
 * Returns 0 when the list is invalid or empty. */
size_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t n_mats);

/* One Muon step over a list of matrices, as grouped launches: one launch per
 * phase covers every matrix, whatever their number and shapes.  Matrices
 * whose whole iteration fits one workgroup's LDS (short side <= 128 and, with
 * both sides padded to 32, m x n + 2 m x m bf16 within 160 KB) run every
 * Newton-Schulz step in one fused launch; the others take three launches per
 * step (Gram, C, X update) by tile class.  In all at most 4 + 3 * ns_steps
 * launches (one more with zero-centering).
 *   lr, mu, wd   learning rate, momentum, decoupled weight decay (finite).
 *   ns_steps     0 .. MUON_MAX_NS_STEPS Newton-Schulz iterations.
 *   coeffs       n_coeffs triples: 1 (used for every step) or ns_steps (one
 *                per step).  May be NULL only when ns_steps == 0.
 *   rms_scale_mode  MUON_SCALE_NONE or MUON_SCALE_SQRT_MAX1.
 *   eps          >= 0, added to ||M||_F before dividing.
 *   workspace    device memory of at least muon_workspace_bytes(mats,
 *                n_mats) bytes, 256-byte aligned.  Its contents on entry do
 *                not matter; on return (once the stream reaches that point)
 *                it holds every intermediate, see muon_workspace_view().
 *   stream       HIP stream all work is queued on (0: the null stream).
 * The matrix list itself is read during the call only. */
int muon_step(const muon_matrix_t* mats, int64_t n_mats,
              float lr, float mu, float wd, int ns_steps,
              const muon_ns_coeff_t* coeffs, int n_coeffs,
              int rms_scale_mode, float eps,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step variants, as flags of muon_options_t (any combination except
 * NESTEROV | NS_FIRST).
 *   MUON_OPT_ZERO_CENTER  G <- G minus its column means (the mean over rows of
 *       each column of the stored rows x cols gradient), before anything else
 *       uses G ("Muon meets Mamba", wmrh.cn, section 2.1 zerocenter, applied by
 *       _step_muon in section 4.2).  Costs one extra read of G (a column-sum
 *       pass with fp64 accumulation) and sizeof(double) * cols of workspace,
 *       which muon_workspace_bytes() always reserves.
 *   MUON_OPT_NESTEROV     the iteration runs on mu*M_new + (1-mu)*G instead
 *       of M_new.  The pages carry a nesterov switch but never say what it
 *       computes (airosetta.com, Muon constructor; wmrh.cn section 4.1); this
 *       look-ahead form is the reading taken.  M itself is still the EMA.
 *   MUON_OPT_NS_FIRST     the other order that wmrh.cn section 4.2 discusses:
 *       O = NS(G / (||G||_F + eps)), then M <- mu*M + (1-mu)*O and
 *       p <- p*(1 - lr*wd) - lr*s*M.  The norm slot of the workspace then
 *       holds ||G||_F^2. */
#define MUON_OPT_ZERO_CENTER 1u
#define MUON_OPT_NESTEROV    2u
#define MUON_OPT_NS_FIRST    4u
typedef struct {
  uint32_t flags;     /* MUON_OPT_* */
  uint32_t reserved;  /* must be 0 */
} muon_options_t;

/* muon_step with step variants.  options == NULL (or flags == 0) is exactly
 * muon_step.  Unknown flags, reserved != 0 or NESTEROV together with
 * NS_FIRST give MUON_EINVAL before anything is launched; everything else is
 * as muon_step. */
int muon_step_ex(const muon_matrix_t* mats, int64_t n_mats,
                 float lr, float mu, float wd, int ns_steps,
                 const muon_ns_coeff_t* coeffs, int n_coeffs,
                 int rms_scale_mode, float eps, const muon_options_t* options,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- a step that allocates nothing ---------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step as muon_step, with the workspace replaced by a fixed scratch array of
 * MUON_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on, for the life of the process.  The caller still passes every parameter,
 * gradient and momentum buffer.  The call allocates no device or pinned host
 * memory and creates no stream or event: the descriptor table reaches the
 * device in kernel arguments, and every launch stays on `stream` (no side
 * stream; phase timing and MUON_DEBUG do not apply).
 *   Arguments and errors as muon_step, plus MUON_EWORKSPACE when
 *   muon_workspace_bytes(mats, n_mats) exceeds MUON_NOALLOC_SCRATCH_BYTES
 *   (found before anything is launched; nothing is modified then).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (each call rewrites what it reads before reading it): two
 * calls whose work overlaps on one device race, so order them on one stream
 * or with events.  The intermediates of the last call are readable through
 * muon_noalloc_scratch() at the offsets muon_workspace_view() gives. */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)
int muon_step_noalloc(const muon_matrix_t* mats, int64_t n_mats, float lr, float mu, float wd,
                      int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs,
                      int rms_scale_mode, float eps, hipStream_t stream);
/* Device address of the current device's scratch array (for reading the last
 * muon_step_noalloc call's intermediates); NULL if it cannot be resolved. */
void* muon_noalloc_scratch(void);

/* ---- a step prepared once over fixed buffers ----------------------------
 * The pages' optimizer steps the same parameters every iteration (the
 * Muon.step loop of airosetta.com; _step_muon of wmrh.cn section 4.2).  A plan
 * fixes that list once: validation, the workspace plan and the descriptor
 * table (with the coefficients) happen in muon_plan_create, which uploads the
 * table into the workspace and waits for that copy.  muon_plan_step then only
 * launches kernels: no host staging, no allocation, no synchronisation, so it
 * may be captured into a HIP graph and replayed.
 *   muon_plan_create  arguments as muon_step_ex (same errors, found before
 *       anything is launched; MUON_EHIP also when the host object cannot be
 *       allocated); *plan receives a host object the caller frees
 *       with muon_plan_destroy.  The param, grad and momentum pointers and the
 *       workspace are recorded: they must stay valid, and the workspace must
 *       not be used by other calls, while the plan lives.  New gradients are
 *       written into the same grad buffers.
 *   muon_plan_step    one step of the plan on `stream`, on the device the plan
 *       was created on (else MUON_EINVAL).  `hyper` points to three floats in
 *       device memory, {lr, mu, wd}, read by the kernels when they run, so a
 *       schedule updates them between replays.
 * Each step clears the workspace's norm slots with a fill kernel (no
 * memset), so replays do not depend on the previous step's workspace.  Phase
 * timing (muon_timing_enable) is skipped while the stream is capturing.  A
 * plan over both fused and tiled matrices owns a stream and two events
 * (created here, released by muon_plan_destroy, which first waits for the
 * work its steps queued there); a captured step forks onto that stream and
 * joins back, so the graph holds two parallel branches. */
typedef struct muon_plan muon_plan_t;
int muon_plan_create(const muon_matrix_t* mats, int64_t n_mats, int ns_steps,
                     const muon_ns_coeff_t* coeffs, int n_coeffs, int rms_scale_mode, float eps,
                     const muon_options_t* options, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, muon_plan_t** plan);
int muon_plan_step(const muon_plan_t* plan, const float* hyper, hipStream_t stream);
void muon_plan_destroy(muon_plan_t* plan);

/* Orthogonalisation alone: out = NS(in) with the same normalisation,
 * short-side rule and bf16 iteration as muon_step, for a list of matrices.
 * The Newton-Schulz routine of the airosetta.com article (newtonschulz5) as a
 * standalone call.
 *   in       rows x cols, row-major, contiguous, type in_dtype (MUON_F32 or
 *            MUON_BF16); read only.
 *   out      bf16 (raw 16-bit patterns), rows x cols, row-major, contiguous;
 *            written.  Must not overlap `in`.
 * The workspace is sized by muon_workspace_bytes() over the same shapes
 * (build the muon_matrix_t list with any grad pointer). */
typedef struct {
  const void*  in;
  void*        out;
  int64_t      rows;
  int64_t      cols;
  int32_t      in_dtype;
} muon_ortho_t;

int muon_orthogonalize(const muon_ortho_t* mats, int64_t n_mats, int ns_steps,
                       const muon_ns_coeff_t* coeffs, int n_coeffs, float eps,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Where matrix `index`'s intermediates live in the workspace after a call
 * over the same shapes (byte offsets from the workspace base).  Each bf16
 * buffer is zero-padded: X buffers are rows_pad x cols_pad in the stored
 * (rows x cols) orientation, A and C are m_pad x m_pad with m the short side.
 *   x_off[0]  X0 and every even iterate; x_off[1] the odd iterates.
 *   a_off     A = X X^T of the last iteration.
 *   c_off     C = a I + b A + c A A of the last iteration (bf16 high part).
 *   c_lo_off  its low part C - bf16(C) (short side <= 128), else 0.
 *   o_off     the final iterate O for `ns_steps` iterations.
 *   nrm2_off  one double: sum of squares of M (of `in` for orthogonalize).
 * Host-only; launches nothing.  For tests and diagnostics. */
typedef struct {
  size_t  x_off[2];
  size_t  a_off;
  size_t  c_off;
  size_t  c_lo_off;
  size_t  o_off;
  size_t  nrm2_off;
  int64_t rows_pad;
  int64_t cols_pad;
  int64_t m_pad;
  int32_t transposed;   /* 1 when rows > cols: the iteration runs on X^T */
  int32_t tile;         /* padding granule: 256 or 128 (tiled kernels) or
                           32 (the fused small-matrix iteration)           */
} muon_workspace_view_t;

int muon_workspace_view(const muon_matrix_t* mats, int64_t n_mats, int64_t index,
                        int ns_steps, muon_workspace_view_t* view);

/* ------------------------------------------------------------------------
 * AdamW branch: the update the pages pair with Muon for the parameters Muon
 * does not take (1-D biases and norm weights, embeddings, output heads).
 * "Muon meets Mamba" (wmrh.cn), section 4.2, method _step_adamw; defaults in
 * section 4.1 (lr 1e-3, betas (0.9, 0.95), eps 1e-8, weight decay 0.01 shared
 * with the Muon group).  Per tensor with a gradient, elementwise in fp32:
 *
 *   p <- p (1 - lr wd)
 *   m <- beta1 m + (1 - beta1) g,        v <- beta2 v + (1 - beta2) g^2
 *   p <- p - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 *
 * with t the tensor's own step count (the page keeps one per parameter).
 * ------------------------------------------------------------------------ */
typedef struct {
  float*      param;       /* fp32 [numel], updated in place                        */
  const void* grad;        /* [numel] of grad_dtype; NULL: the tensor is skipped     */
                           /* (no decay, no moment update)                           */
  float*      exp_avg;     /* fp32 [numel] first moment m, in place; caller zero-inits */
  float*      exp_avg_sq;  /* fp32 [numel] second moment v, in place; caller zero-inits */
  int64_t     numel;       /* >= 1 elements (any tensor shape, flattened)            */
  int64_t     step;        /* t of this update, >= 1: the caller keeps the per-tensor */
                           /* count and increments it before the call                */
  int32_t     grad_dtype;  /* MUON_F32 or MUON_BF16                                  */
  int32_t     reserved;    /* must be 0                                              */
} muon_adamw_tensor_t;

/* Workspace for n_tensors tensors (descriptor table); 0 if n_tensors <= 0. */
size_t muon_adamw_workspace_bytes(int64_t n_tensors);

/* One AdamW update of every tensor with a gradient, one grouped launch on
 * `stream`.  Arguments: 0 <= beta1, beta2 < 1, eps >= 0, lr and wd finite.
 * Same ownership, aliasing and error rules as muon_step: MUON_EINVAL for a
 * bad argument (numel < 1, step < 1, unknown dtype, missing buffer, reserved
 * != 0), MUON_EALIAS when any two buffers of the call overlap,
 * MUON_EWORKSPACE for a missing, small or unaligned workspace, all found
 * before anything is launched; MUON_EHIP when a launch fails. */
int muon_adamw_step(const muon_adamw_tensor_t* tensors, int64_t n_tensors, float lr, float beta1,
                    float beta2, float eps, float wd, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Phase timing with HIP events, for benchmarks.  When enabled, every launch
 * is bracketed by a pair of events on the call's stream, and a step keeps
 * all its launches on that stream (no side-stream overlap, so that each
 * phase's events bracket its own kernels only).  muon_timing_read()
 * waits for the recorded events, returns the summed milliseconds and launch
 * counts per phase (MUON_PHASES entries each; either pointer may be NULL) and
 * clears the record.  Phases: momentum+norm, normalise+cast, Gram X X^T,
 * Gram A A with the b A + c A^2 epilogue, X update, apply (or export),
 * AdamW, and the fused iteration of small matrices (every Newton-Schulz
 * step of each matrix whose whole iteration fits one workgroup's LDS). */
#define MUON_PHASES 8
int muon_timing_enable(int on);
int muon_timing_read(double* ms, int64_t* launches);

/* Static text for a status code (with HIP detail after MUON_EHIP). */
const char* muon_status_string(int status);

/* Library version, e.g. "libmuon 0.1 gfx950". */
const char* muon_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMUON_MUON_H */
