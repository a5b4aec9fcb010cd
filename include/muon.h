/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step library.
 *
 * The operations follow "Muon is Scalable for LLM Training" (Moonshot AI /
 * UCLA, 2025), as given on the Traditional-Chinese translation page of the
 * technical report:
 *   - section 2.1, Eq. 1: momentum M_t = mu M_{t-1} + G_t, M_0 = 0;
 *   - section 2.1, paragraph after Eq. 1: Nesterov-style input mu M_t + G_t;
 *   - section 2.1, Eq. 2: X_0 = M / ||M||_F, then N quintic Newton-Schulz
 *     iterations X <- a X + b (X X^T) X + c (X X^T)^2 X with
 *     (a, b, c) = (3.4445, -4.7750, 2.0315);
 *   - section 2.2, Eq. 3 and Eq. 4 (= section 3.1, Eq. 7): decoupled weight
 *     decay and the shape scale 0.2 * sqrt(max(A, B));
 *   - section 2.2 (matching AdamW's update RMS): RMSNorm, embedding and LM
 *     head parameters use AdamW with the same learning rate and decay;
 *   - section 2.3, Algorithm 1: the per-matrix update RMS is reported;
 *   - section 3.1, Eq. 5 and Eq. 6: the alternative update scalings
 *     0.2 * sqrt(H) and 0.2 / RMS(O) (mo_muon_plan_set_scaling);
 *   - section 3.4 and appendix F: the SVD entropy and the sorted singular
 *     values of weight matrices (mo_svd_entropy, a diagnostic).
 *
 * General rules for every entry point
 *   Memory   All tensor pointers are DEVICE pointers on the current HIP
 *            device, row-major and contiguous (leading dimension = cols),
 *            16-byte aligned.  The caller owns every buffer, including the
 *            workspace.  The library never allocates device or pinned host
 *            memory inside a step; only mo_muon_plan_create allocates (its
 *            descriptor table).  Descriptor arrays (mo_tensor) are HOST
 *            memory, read during the call only: one-shot calls copy them to
 *            the workspace with small kernels that carry the table in their
 *            launch arguments, so no call waits for an earlier one.
 *   Streams  `stream` is a hipStream_t passed as void* (NULL = the null
 *            stream).  Work is enqueued on it in order, and calls return
 *            without waiting for the GPU.  Calls on different streams with
 *            disjoint buffers and workspaces are independent; calls that
 *            share a workspace must be ordered by the caller.
 *   Errors   Every call returns an mo_status.  Arguments are validated in
 *            full before anything is enqueued, so a non-OK status from
 *            validation means no device state was touched.  A thread-local
 *            message for the last failure is available from mo_last_error().
 *            Faults during execution surface at the caller's next
 *            synchronisation as a HIP error (set MO_DEBUG_SYNC=1 in the
 *            environment to synchronise after every launch and map them to
 *            MO_EHIP).  NaN and Inf propagate per IEEE arithmetic: a
 *            NaN or Inf in a matrix's gradient or momentum reaches its
 *            Frobenius norm, so that matrix's whole update -- and its
 *            parameter -- becomes NaN, and its update_rms entry is NaN
 *            (the per-matrix non-finite flag); the momentum is non-finite
 *            only where its inputs were; every other matrix of the call is
 *            unaffected.
 *   Threads  Entry points are thread-safe except that a plan must not be
 *            stepped from two threads at once.
 *   Tuning   Environment switches for tests and measurement only (MO_TILE
 *            is read when matrices are binned, i.e. at plan creation or per
 *            one-shot call; the others at launch); results stay within the
 *            same tolerances:
 *              MO_TILE=64|128|256  force the output tile of every shape
 *                                  group (256: bf16 only);
 *              MO_WAVES=4|8        waves per 256-tile workgroup (default 8);
 *              MO_NO_SMALL=1       run groups of small matrices (m <= 128)
 *                                  through the per-product kernels instead
 *                                  of the fused one.
 *            Groups of at least 32 bf16 matrices with m <= 128 take a fused
 *            kernel that iterates on the m x m Gram matrix at about fp32
 *            precision (ns_steps <= 5; longer iterations take the
 *            per-product kernels): its results are more accurate than the
 *            bf16 iterates of the per-product kernels, not bitwise equal.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MO_ABI_VERSION 4

/* Status codes. */
typedef enum mo_status {
    MO_OK = 0,
    MO_EINVAL = -1,        /* bad argument (null, misaligned, range, alias) */
    MO_EUNSUPPORTED = -2,  /* valid request the library does not implement  */
    MO_EWORKSPACE = -3,    /* workspace missing, misaligned or too small    */
    MO_EHIP = -4           /* the HIP runtime reported an error             */
} mo_status;

/* Element types. */
typedef enum mo_dtype {
    MO_F32 = 0,
    MO_BF16 = 1
} mo_dtype;

/* One parameter tensor and its optimizer state (all device pointers).
 *   param   fp32 [rows, cols], updated in place.
 *   grad    [rows, cols] in the call's grad dtype, read only.
 *   state0  Muon: momentum buffer [rows, cols] in the momentum dtype,
 *           updated in place (zero before the first step).
 *           AdamW: first moment m, fp32 [rows * cols], updated in place.
 *   state1  AdamW: second moment v, fp32 [rows * cols], updated in place.
 *           Muon: must be NULL.
 *   rows, cols >= 1.  AdamW treats the tensor as rows * cols elements. */
typedef struct mo_tensor {
    void*       param;
    const void* grad;
    void*       state0;
    void*       state1;
    int64_t     rows;
    int64_t     cols;
} mo_tensor;

/* Library ABI version (MO_ABI_VERSION of the build). */
int mo_abi_version(void);

/* Message describing the last non-OK status returned on this thread. */
const char* mo_last_error(void);

/* Workspace needed by mo_muon_step for `tensors` with Newton-Schulz dtype
 * `ns_dtype`.  *full_bytes: every matrix of every shape group resident at
 * once, so that each Newton-Schulz product is one launch over all groups
 * (fastest).  *min_bytes (may be NULL): the smallest workspace accepted
 * (one matrix at a time); between the two, shape groups are processed one
 * after another, each in as few passes as fit.  Results do not depend on
 * the workspace size.  Host-only; touches no device state. */
int mo_muon_workspace_size(const mo_tensor* tensors, int64_t count,
                           int ns_dtype, size_t* full_bytes, size_t* min_bytes);

/* One Muon step (section 2.1 Eq. 1-2, section 2.2 Eq. 4) for `count` matrix
 * parameters, as one batch of launches on `stream`:
 *   M <- mu M + G;  N = mu M + G (nesterov != 0) or N = M;
 *   X_0 = N / (||N||_F + eps);  ns_steps iterations of Eq. 2 with abc;
 *   W <- W - lr * (rms_scale * sqrt(max(rows, cols)) * X_N + wd * W_old).
 * Matrices with rows > cols are processed as their transpose (exact for
 * the odd polynomial of Eq. 2) so the Gram matrix is min x min.
 *   grad_dtype, mom_dtype: MO_F32 or MO_BF16.  The momentum update is done
 *       in fp32 and stored rounded to nearest-even in mom_dtype; N is formed
 *       from the unrounded fp32 momentum.
 *   ns_dtype: MO_BF16 -- Newton-Schulz operands stored in bf16, products
 *       accumulated in fp32 (the pages run Newton-Schulz in bf16, section
 *       2.3); MO_F32 -- fp32 throughout.
 *   ns_steps in [0, 16] (0: X_N = X_0).  abc: 3 floats or NULL for
 *   (3.4445, -4.7750, 2.0315).  rms_scale: 0.2 in the pages.  eps >= 0.
 *   update_rms: NULL, or a device fp32 array [count] that receives
 *       sqrt(mean(X_N^2)) of each matrix (unscaled, section 2.3).
 *   workspace: device buffer, 256-byte aligned, >= min_bytes of
 *       mo_muon_workspace_size; its contents need no initialisation and are
 *       garbage afterwards.
 * No two tensors' param, grad or state0 ranges may overlap.
 * Returns MO_OK, MO_EINVAL, MO_EWORKSPACE or MO_EHIP. */
int mo_muon_step(const mo_tensor* tensors, int64_t count,
                 int grad_dtype, int mom_dtype, int ns_dtype,
                 float lr, float wd, float mu, int nesterov, int ns_steps,
                 const float* abc, float rms_scale, float eps,
                 float* update_rms, void* workspace, size_t workspace_bytes,
                 void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step of
 * mo_muon_step, same arguments and results, with the library's own scratch
 * memory in place of the caller's workspace.  The call allocates nothing
 * (no hipMalloc, hipFree, pinned or library allocation).
 *   Scratch: one static device array of MO_NOALLOC_SCRATCH_MIB MiB per GPU
 *       the library runs on, held until the process ends; its address is
 *       looked up on the first call on each device.  Matrices whose
 *       minimum workspace (min_bytes of mo_muon_workspace_size) exceeds it
 *       are rejected with MO_EWORKSPACE before anything is enqueued; below
 *       the full size, shape groups are processed in chunks that fit, with
 *       results identical to mo_muon_step's.
 *   Sharing: every call on one GPU uses that GPU's scratch, so calls that
 *       overlap on one GPU (different streams, or threads without ordering)
 *       race; calls on one stream are ordered and safe.  Nothing in the
 *       scratch needs clearing between calls (each kernel writes what it
 *       later reads).
 * Returns MO_OK, MO_EINVAL, MO_EWORKSPACE, MO_EUNSUPPORTED or MO_EHIP. */
#define MO_NOALLOC_SCRATCH_MIB 256
int mo_muon_step_noalloc(const mo_tensor* tensors, int64_t count,
                         int grad_dtype, int mom_dtype, int ns_dtype,
                         float lr, float wd, float mu, int nesterov,
                         int ns_steps, const float* abc, float rms_scale,
                         float eps, float* update_rms, void* stream);

/* A plan binds one list of tensors (pointers, shapes, dtypes) so that
 * repeated steps skip validation, grouping and the descriptor upload of
 * mo_muon_step.  mo_muon_plan_create validates like mo_muon_step, allocates
 * and fills a small device descriptor table (synchronously), and owns it
 * until mo_muon_plan_destroy.  The tensors must stay allocated at the same
 * addresses while the plan is used. */
typedef struct mo_muon_plan mo_muon_plan;

int mo_muon_plan_create(const mo_tensor* tensors, int64_t count,
                        int grad_dtype, int mom_dtype, int ns_dtype,
                        mo_muon_plan** plan);

/* Workspace sizes of a plan (same meaning as mo_muon_workspace_size). */
int mo_muon_plan_workspace_size(const mo_muon_plan* plan, size_t* full_bytes,
                                size_t* min_bytes);

/* The step of mo_muon_step on a plan's tensors.  It only enqueues kernels
 * (no allocation, memset, host copy or synchronisation), so it can be
 * captured into a HIP graph; replays reuse the captured hyper-parameters,
 * scaling, workspace and update_rms pointer, and read the tensors' current
 * contents. */
int mo_muon_plan_step(mo_muon_plan* plan, float lr, float wd, float mu,
                      int nesterov, int ns_steps, const float* abc,
                      float rms_scale, float eps, float* update_rms,
                      void* workspace, size_t workspace_bytes, void* stream);

/* How X_N (= O_t) is scaled in the update (section 3.1):
 *   MO_SCALE_SHAPE        Eq. 4 / Eq. 7: rms_scale * sqrt(max(rows, cols)),
 *                         the default of every step entry point;
 *   MO_SCALE_HIDDEN       Eq. 5: rms_scale * sqrt(H) for one model-wide H
 *                         (the hidden size), whatever the matrix shape;
 *   MO_SCALE_UPDATE_NORM  Eq. 6: rms_scale / RMS(X_N), RMS over the
 *                         rows * cols elements, so the update term has RMS
 *                         exactly rms_scale; a matrix whose X_N is zero gets
 *                         a decay-only update.  X_N's RMS is computed on the
 *                         device from the fp32 values before the apply (one
 *                         extra pass of the last Newton-Schulz product). */
typedef enum mo_scaling {
    MO_SCALE_SHAPE = 0,
    MO_SCALE_HIDDEN = 1,
    MO_SCALE_UPDATE_NORM = 2
} mo_scaling;

/* Sets the scaling used by the plan's later mo_muon_plan_step calls
 * (initially MO_SCALE_SHAPE).  hidden: H for MO_SCALE_HIDDEN (finite,
 * >= 1), ignored otherwise.  Host-only.  With MO_SCALE_UPDATE_NORM,
 * update_rms receives RMS(X_N) as with the other scalings.
 * Returns MO_OK or MO_EINVAL (plan unchanged). */
int mo_muon_plan_set_scaling(mo_muon_plan* plan, int scaling, float hidden);

/* Rebinds the plan's gradients (section 2.1, Eq. 1's G_t) to new buffers
 * without recreating it, for callers whose gradient tensors move between
 * steps (a framework that frees gradients after each step).  grads[i] is the
 * gradient of the plan's tensor i (the order given to mo_muon_plan_create),
 * same shape and dtype as before, 16-byte aligned, not overlapping any
 * param, momentum or other gradient of the plan.  When every pointer is
 * unchanged nothing is enqueued; otherwise the descriptor table is updated
 * on `stream` by one small kernel per 96 tensors (no host synchronisation),
 * so later plan steps on the same stream use the new gradients.  Steps of
 * the plan queued on other streams must be ordered by the caller.
 * Validation is complete before anything changes: MO_EINVAL leaves the plan
 * as it was.  Returns MO_OK, MO_EINVAL or MO_EHIP. */
int mo_muon_plan_set_grads(mo_muon_plan* plan, const void* const* grads,
                           int64_t count, void* stream);

/* Frees the plan's descriptor table (synchronises the device first). */
int mo_muon_plan_destroy(mo_muon_plan* plan);

/* AdamW for non-matrix parameters (section 2.2: RMSNorm, embedding and LM
 * head keep AdamW with the shared learning rate and weight decay):
 *   m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2;
 *   W <- W - lr * ( (m / (1 - beta1^step)) /
 *                   (sqrt(v / (1 - beta2^step)) + eps)  + wd * W_old ).
 * param, state0 (m) and state1 (v) are fp32; grad is grad_dtype.  Each
 * tensor is rows * cols elements.  step >= 1 is the 1-based step count
 * used for bias correction.  beta1 and beta2 are doubles so that 1 - beta
 * is formed exactly (0.999 rounded to fp32 would shift 1 - beta2 by
 * 1.3e-5 relative); the elementwise arithmetic is fp32.  Decay applies to every tensor (the pages keep
 * it on RMSNorm gains too).  Needs no workspace. */
int mo_adamw_step(const mo_tensor* tensors, int64_t count, int grad_dtype,
                  float lr, float wd, double beta1, double beta2, float eps,
                  int64_t step, void* stream);

/* Workspace for mo_newton_schulz on `batch` matrices [rows, cols]. */
int mo_newton_schulz_workspace_size(int64_t batch, int64_t rows, int64_t cols,
                                    int dtype, size_t* bytes);

/* Diagnostic: Frobenius normalisation and ns_steps iterations of Eq. 2 only
 * (section 2.1), on `batch` contiguous matrices [rows, cols]:
 *   output[b] = NS(input[b] / (||input[b]||_F + eps)).
 * input and output are device arrays of `dtype` (MO_F32 or MO_BF16; the
 * arithmetic is that of ns_dtype = dtype in mo_muon_step), may not overlap;
 * the final iterate is rounded once to `dtype`. */
int mo_newton_schulz(const void* input, void* output, int64_t batch,
                     int64_t rows, int64_t cols, int dtype, int ns_steps,
                     const float* abc, float eps, void* workspace,
                     size_t workspace_bytes, void* stream);

/* One matrix for the SVD-entropy diagnostic. */
typedef struct mo_matrix {
    const void* data;      /* device [rows, cols], row-major, 16-byte aligned */
    int64_t     rows;
    int64_t     cols;
} mo_matrix;

/* Workspace for mo_svd_entropy (full/min as in mo_muon_workspace_size): per
 * matrix about 8 m (m + m / 64 + 37) bytes, m = min(rows, cols).  The
 * matrices are checked as for mo_svd_entropy (dtype aside).  Host-only. */
int mo_svd_entropy_workspace_size(const mo_matrix* mats, int64_t count,
                                  size_t* full_bytes, size_t* min_bytes);

/* SVD entropy (section 3.4) and singular values (appendix F) of `count`
 * matrices, on `stream`:
 *   entropy[i] = -(1 / log n) sum_j p_j log p_j,
 *       p_j = sigma_j^2 / sum_l sigma_l^2, n = min(rows_i, cols_i)
 *   (0 log 0 = 0; entropy 0 when n = 1 or the matrix is zero).
 *   dtype: MO_F32 or MO_BF16, the element type of every matrix.
 *   entropy: device double [count].
 *   sigma: NULL, or device double [sum_i min(rows_i, cols_i)] that receives
 *       each matrix's singular values, largest first, packed in the
 *       caller's order (appendix F divides them by the first).
 *   1 <= min(rows, cols) <= 8192, max(rows, cols) < 2^31 and
 *   rows * cols <= 2^31.
 * The singular values are the square roots of the eigenvalues of the fp64
 * Gram matrix of the short side (exact products, fp64 sums), found by a
 * Householder reduction to tridiagonal form and bisection, all in fp64:
 * sigma_j^2 carries an absolute error of a small multiple of
 * (rows + cols) * 2^-52 * sigma_1^2.  Results do not depend on the
 * workspace size or on the other matrices of the call.  Outputs may not
 * overlap each other, an input or the workspace.
 * Returns MO_OK, MO_EINVAL, MO_EWORKSPACE or MO_EHIP. */
int mo_svd_entropy(const mo_matrix* mats, int64_t count, int dtype,
                   double* entropy, double* sigma, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Kernel classes for the timing counters below. */
typedef enum mo_kernel_class {
    MO_K_MOMENTUM = 0,     /* momentum + Nesterov + norm partials + X_0 copy */
    MO_K_NORM = 1,         /* per-matrix norm finalisation                   */
    MO_K_GRAM = 2,         /* S = X X^T (lower tiles, mirrored)              */
    MO_K_POLY = 3,         /* P = b S + c S S (lower tiles, mirrored)        */
    MO_K_UPDATE = 4,       /* X <- P' X = a X + P X (P' = a I + b S + c S S)  */
    MO_K_APPLY = 5,        /* last update fused with scale, decay and apply  */
    MO_K_APPLY_X0 = 6,     /* apply for ns_steps = 0                         */
    MO_K_RMS = 7,          /* update-RMS finalisation                        */
    MO_K_ADAMW = 8,        /* AdamW elementwise                              */
    MO_K_SVD_GRAM = 9,     /* SVD entropy: fp64 Gram (block-lower tiles)     */
    MO_K_SVD_REDUCE = 10,  /* SVD entropy: matrix-vector products of a step  */
    MO_K_SVD_COLUMN = 11,  /* SVD entropy: per-step reflector (one WG/matrix) */
    MO_K_SVD_EIG = 12,     /* SVD entropy: bisection, entropy and sigma      */
    MO_K_SVD_PANEL = 13,   /* SVD entropy: deferred rank-2 updates of a panel */
    MO_K_COUNT = 14
} mo_kernel_class;

/* Timing counters.  mo_profile_enable(mask): for every class k with bit k
 * set, each later launch of that class is bracketed by HIP events recorded
 * on the launch stream.  mo_profile_read synchronises on the recorded
 * events and returns, for class k since the last reset: the number of
 * launches, their summed GPU time in ms, and the summed algorithmic work
 * (flops for the GEMM classes, bytes for the others; see the design
 * notes).  mo_profile_reset clears the counters and releases the events.
 * Not thread-safe; a diagnostic for benchmarks. */
int mo_profile_enable(unsigned int class_mask);
int mo_profile_read(int kernel_class, int64_t* launches, double* total_ms,
                    double* total_work);
int mo_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
