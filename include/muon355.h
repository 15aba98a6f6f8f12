/*
 * muon355.h - C ABI of libmuon355, the Muon optimizer step on AMD Instinct
 * MI355X (gfx950).
 *
 * One Muon step for a hidden 2-D weight W (m x n) with gradient G is three
 * calls, in this order, all asynchronous on one HIP stream:
 *
 *   muon_momentum       M <- beta*M + (1-beta)*G, the Nesterov blend N, and
 *                       the sum of squares of N.
 *   muon_orthogonalize  O = K Newton-Schulz steps on N / (||N||_F + eps),
 *                       run on the smaller side (transposed when m > n).
 *   muon_apply          W <- (1 - lr*wd)*W - lr*s*O with the shape factor s.
 *
 * Sources ("the pages") cited below:
 *   [NOTES]  "Reading notes on SOAP, Muon and higher-order optimizers",
 *            section 1 "AdamW vs. SOAP vs. Muon" (moving-average momentum).
 *   [GUIDE]  "LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
 *            Training", sections 11.3 (momentum, Nesterov), 11.4
 *            (Newton-Schulz equations, epsilon, tall transpose) and 11.5
 *            (shape factors, decoupled weight decay).
 *   [LESSON] "Matrix optimizers: K-FAC, Shampoo and Muon" (Lesson 12),
 *            subsection "Newton-Schulz: UV^T with matrix products only"
 *            (Lemma 3 and the three-step algorithm) and subsection "Muon"
 *            (steps 1-4, update size).
 *   [PREPRINT] "SOAP, Muon, and Beyond: Pushing LLM Pretraining Scales"
 *            (epsilon 1e-7 for Muon).
 *   [ZH]     "初探优化器（一）：从SGD到SOAP-Muon", section 6.2 (the SOAP
 *            step; one power-iteration step plus QR for the bases).
 *
 * Beside the Muon step, muon_adamw updates the parameters Muon leaves to
 * AdamW ([GUIDE] sections 5 and 6), and the soap_* calls run SOAP, Adam in
 * the eigenbasis of Shampoo's statistics ([GUIDE] 11.1-11.2).
 *
 * Conventions shared by every entry point:
 *   - All matrix memory and all workspaces are caller-owned DEVICE memory.
 *     The library never allocates, frees or synchronizes; every call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns.  Debugging aid: with MUON355_DEBUG_SYNC=1 in
 *     the environment every call waits for the work it enqueued and reports
 *     a failed kernel as MUON_ERR_LAUNCH naming the call.
 *   - Matrices are row-major with a leading dimension `ld` (elements between
 *     consecutive rows, ld >= cols).  A batch holds `count` matrices of one
 *     shape and dtype: matrix i lives at ptrs[i] when `ptrs` is non-NULL (a
 *     DEVICE array of count pointers) and at base + i*stride elements
 *     otherwise.  All pointers must be 16-byte aligned.
 *   - Arguments are validated before anything is enqueued.  A non-OK status
 *     means nothing was enqueued (except MUON_ERR_LAUNCH, which reports a
 *     failed launch); muon_last_error() then gives a thread-local message.
 *     No C++ exception crosses this boundary.
 *   - Non-finite values in G or M propagate to sumsq and to the outputs; the
 *     caller may test sumsq and skip muon_apply (the library never skips).
 *   - Calls on one stream are ordered; calls that share a workspace must not
 *     run concurrently on different streams.
 */
#ifndef MUON355_H
#define MUON355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON355_ABI_VERSION 1

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_VALUE = 1, /* a NULL required pointer, a bad size or a bad hyperparameter */
  MUON_ERR_UNSUPPORTED = 2,   /* a dtype or mode combination that is not built */
  MUON_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace() query */
  MUON_ERR_LAUNCH = 4         /* a kernel launch failed (hipGetLastError) */
} muon_status_t;

typedef enum muon_dtype {
  MUON_F32 = 0,  /* IEEE binary32 */
  MUON_BF16 = 1  /* bfloat16 (upper half of binary32), round-to-nearest-even on store */
} muon_dtype_t;

typedef enum muon_scale {
  MUON_SCALE_MATCH_RMS = 0, /* s = coeff * sqrt(max(m, n)); coeff = 0.2 matches AdamW's update RMS
                               ([GUIDE] 11.5, [LESSON] "Muon" step 4 and "Update size") */
  MUON_SCALE_ORIGINAL = 1,  /* s = sqrt(max(1, m / n)) ([GUIDE] 11.5, [LESSON] "Muon" step 4) */
  MUON_SCALE_NONE = 2       /* s = 1 */
} muon_scale_t;

typedef struct muon_batch {
  void* const* ptrs; /* device array of `count` matrix pointers, or NULL to use base/stride */
  void* base;        /* matrix i at base + i*stride elements when ptrs == NULL */
  int64_t stride;    /* elements between consecutive matrices (strided batch) */
  int64_t count;     /* number of matrices, 1 .. 65535 (split larger batches) */
  int64_t rows;      /* m >= 1; rows * cols <= 2^31 - 1 */
  int64_t cols;      /* n >= 1 */
  int64_t ld;        /* leading dimension in elements, >= cols */
  int32_t dtype;     /* muon_dtype_t */
  int32_t reserved;  /* must be 0 */
} muon_batch_t;

/* Bytes of device workspace muon_momentum needs for `count` matrices of
 * rows x cols (per-block partial sums of the Frobenius reduction). */
size_t muon_momentum_workspace(int64_t count, int64_t rows, int64_t cols);

/*
 * Momentum, Nesterov blend and the sum of squares of the Newton-Schulz input.
 *
 *   M <- beta*M + (1-beta)*G                          ([NOTES] section 1)
 *   N  = (1-beta)*G + beta*M   if nesterov, else N = M
 *   sumsq[i] = sum of N_i^2 over all entries          ([GUIDE] 11.4, X_0)
 *
 * The pages write the accumulating form B <- beta*B + G, N = G + beta*B
 * ([GUIDE] 11.3, [LESSON] "Muon" steps 1-2); the moving average here is
 * (1-beta) times it, which Newton-Schulz's normalization removes.
 *
 * grad : G, BF16 or F32, read only.
 * mom  : M, F32, read and written in place.
 * nout : N, BF16 or F32, written; may be NULL only when nesterov == 0, in
 *        which case M itself is the Newton-Schulz input.
 * sumsq: device float[count], written (sum of squares of N as computed in
 *        fp32, before any bf16 rounding of N; partials are added in fp64).
 * beta : in [0, 1).  nesterov: 0 or 1.
 * Arithmetic is fp32.  Shapes of grad, mom and nout must match.
 */
muon_status_t muon_momentum(const muon_batch_t* grad, const muon_batch_t* mom,
                            const muon_batch_t* nout, float* sumsq, float beta,
                            int nesterov, void* workspace, size_t ws_bytes,
                            void* stream);

/* Bytes of device workspace muon_momentum_grouped needs: the sum of
 * muon_momentum_workspace over the groups; 0 for invalid arguments. */
size_t muon_momentum_grouped_workspace(int ngroups, const int64_t* counts,
                                       const int64_t* rows, const int64_t* cols);

/*
 * muon_momentum for several shape classes in one launch (plus one launch of
 * the sum-of-squares finalization): group g is the batch grads[g], moms[g],
 * nouts[g] with its own device float[count] sumsqs[g], all with the meaning,
 * layout and rules of muon_momentum; beta and nesterov are shared.  The
 * pages' per-layer and per-expert matrices come in a few shape classes
 * ([NOTES] section 1 and 3), so one step's momentum is one grid here.
 *
 * ngroups: 1..8.  grads, moms: host arrays of ngroups descriptors.  nouts:
 * host array of ngroups descriptors, or NULL (only without Nesterov: M is
 * then the Newton-Schulz input of every group).  sumsqs: host array of
 * ngroups device pointers.  workspace: at least
 * muon_momentum_grouped_workspace bytes, 16-byte aligned.  Every group is
 * validated before anything is enqueued; muon_last_error() names the
 * failing group.  Results equal separate muon_momentum calls bit for bit.
 */
muon_status_t muon_momentum_grouped(int ngroups, const muon_batch_t* grads,
                                    const muon_batch_t* moms,
                                    const muon_batch_t* nouts,
                                    float* const* sumsqs, float beta,
                                    int nesterov, void* workspace,
                                    size_t ws_bytes, void* stream);

/*
 * Allocation-free form of muon_momentum_grouped, for callers that cannot
 * allocate device memory or hand the library a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, meaning, validation and results (bit for bit) as
 * muon_momentum_grouped, without `workspace` and `ws_bytes`: the per-block
 * partial sums go to a static device array of MUON_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends (its
 * address is looked up on the first call on a device).  The call allocates
 * and frees nothing.
 *
 * Limit: muon_momentum_grouped_workspace(...) of the call must not exceed
 * MUON_NOALLOC_SCRATCH_BYTES (8 MiB: about two million partial sums, i.e.
 * up to about 1.7e10 matrix elements per call); larger calls return
 * MUON_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU uses that GPU's one array: calls that may overlap
 * on a GPU (unordered streams, several host threads) race on it and must be
 * serialized by the caller.  Nothing in the array needs to start at zero:
 * each call writes every partial it reads.
 */
#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

muon_status_t muon_momentum_grouped_noalloc(int ngroups, const muon_batch_t* grads,
                                            const muon_batch_t* moms,
                                            const muon_batch_t* nouts,
                                            float* const* sumsqs, float beta,
                                            int nesterov, void* stream);

/* Bytes of device workspace muon_orthogonalize needs for `count` matrices
 * of stored shape rows x cols computed in `compute` (MUON_BF16 or MUON_F32).
 * Returns 0 for invalid arguments. */
size_t muon_orthogonalize_workspace(int64_t count, int64_t rows, int64_t cols,
                                    int32_t compute);

/*
 * Newton-Schulz orthogonalization ([GUIDE] 11.4; [LESSON] Lemma 3 and the
 * algorithm after it):
 *   X_0 = N / (sqrt(sumsq) + eps), transposed when rows > cols;
 *   K times: A = X X^T;  B = b*A + c*A*A;  X <- a*X + B*X;
 *   O = X_K in the stored orientation.
 *
 * in     : N, BF16 or F32 (the momentum output), read only.
 * sumsq  : device float[count] from muon_momentum, or NULL to have it
 *          computed here from `in`.
 * out    : O, BF16 or F32, same rows/cols as `in`, written.  May alias
 *          `in` (the iteration runs in the workspace).
 * steps  : K >= 0 (5 in Muon).  a, b, c: finite coefficients, the same at
 *          every step ((3.4445, -4.7750, 2.0315) in Muon).
 * eps    : finite, >= 0 (1e-7 in Muon, [PREPRINT]); added to the norm.
 * compute: MUON_BF16 = bf16 MFMA operands with fp32 accumulation; X is
 *          carried between steps as a bf16 high part (the MFMA operand)
 *          plus its rounding residual as 8-bit codes with an exponent shared
 *          by 16 values, about 16 significant bits together, for the a*X
 *          term (the fast path);
 *          MUON_F32   = fp32 MFMA throughout (the parity path).
 *          With MUON_BF16 an F32 `in` is preferred: the high/low copy of X
 *          starts from it, while a BF16 `in` starts the iteration from
 *          bf16-rounded values, an error the iteration amplifies on
 *          ill-conditioned inputs (about 10x larger output error at
 *          condition number 1e4).
 * The Gram and polynomial GEMMs compute only upper-triangle tiles and
 * mirror them.  The Newton-Schulz shape padded to the tile size (128 or
 * 256) may hold at most 2^30 elements; larger shapes return
 * MUON_ERR_UNSUPPORTED.
 */
muon_status_t muon_orthogonalize(const muon_batch_t* in, const float* sumsq,
                                 const muon_batch_t* out, int steps, float a,
                                 float b, float c, float eps, int32_t compute,
                                 void* workspace, size_t ws_bytes,
                                 void* stream);

/* Grouped form: `ngroups` batches of different shapes orthogonalized with
 * one kernel launch per stage (every group's tiles packed into one grid).
 * ins[g], outs[g] and sumsqs[g] are as in muon_orthogonalize (sumsqs may be
 * NULL, or hold NULL entries, to compute them here).  1 <= ngroups <= 8.
 * The workspace query takes the same per-group arrays. */
size_t muon_orthogonalize_grouped_workspace(int ngroups, const int64_t* counts,
                                            const int64_t* rows,
                                            const int64_t* cols,
                                            int32_t compute);
muon_status_t muon_orthogonalize_grouped(int ngroups, const muon_batch_t* ins,
                                         const float* const* sumsqs,
                                         const muon_batch_t* outs, int steps,
                                         float a, float b, float c, float eps,
                                         int32_t compute, void* workspace,
                                         size_t ws_bytes, void* stream);

/*
 * The momentum and the Newton-Schulz input in one pass ("packed" pair).
 *
 * muon_momentum_packed_grouped does what muon_momentum_grouped does for M and
 * the sums of squares (same arithmetic: M is bit-identical; the sums of
 * squares are added per 64 x 64 tile instead of per block, then in fp64 in
 * a fixed order), but instead of writing the Nesterov blend N to a caller
 * buffer it writes N straight into `workspace` in the layout the
 * Newton-Schulz kernels read (bf16 high part and 8-bit residual with
 * MUON_BF16; fp32 with MUON_F32; padded, and transposed when rows > cols).
 * muon_orthogonalize_packed_grouped then runs the iteration of
 * muon_orthogonalize_grouped from that workspace, dividing by
 * sqrt(sumsq) + eps inside its first step ([GUIDE] 11.4, X_0 equation: the
 * Gram of step 0 is scaled by 1/(||N||+eps)^2 and its update by
 * 1/(||N||+eps)), so N never makes a round trip through memory.
 *
 * Contract: both calls take the same groups (the shapes of grads[g] in the
 * first are the shapes of outs[g] in the second), the same compute and the
 * same workspace of at least muon_packed_grouped_workspace bytes (16-byte
 * aligned), in this order on one stream; the workspace carries the packed
 * input from the first call to the second.  sumsqs[g]: device float[count]
 * written by the first call, read by the second.  steps >= 1 (steps == 0
 * takes the separate calls).  Arguments, hyperparameters, outputs and
 * errors otherwise as muon_momentum_grouped and muon_orthogonalize_grouped.
 * The result differs from the separate calls only by rounding (the input is
 * scaled after its bf16 rounding instead of before).
 */
size_t muon_packed_grouped_workspace(int ngroups, const int64_t* counts,
                                     const int64_t* rows, const int64_t* cols,
                                     int32_t compute);
muon_status_t muon_momentum_packed_grouped(int ngroups, const muon_batch_t* grads,
                                           const muon_batch_t* moms,
                                           float* const* sumsqs, float beta,
                                           int nesterov, int32_t compute,
                                           void* workspace, size_t ws_bytes,
                                           void* stream);
muon_status_t muon_orthogonalize_packed_grouped(int ngroups, const float* const* sumsqs,
                                                const muon_batch_t* outs, int steps,
                                                float a, float b, float c, float eps,
                                                int32_t compute, void* workspace,
                                                size_t ws_bytes, void* stream);

/*
 * The second call of the packed pair with the parameter update folded into
 * its last step ([GUIDE] 11.5 update equation; [LESSON] "Muon" step 4):
 * instead of writing O it updates each weight in place,
 *   W <- (1 - lr*weight_decay) * W - lr * s * O,
 * s from `mode` and `coeff` and (m, n) = (rows, cols) of W, as
 * muon_apply_grouped does for an O of the same shape.  O is never stored:
 * each value goes from the last GEMM's fp32 accumulator into the update, so
 * the result differs from muon_orthogonalize_packed_grouped followed by
 * muon_apply_grouped only by O's rounding to the dtype of a caller buffer
 * (none for fp32 O).  weights[g] takes the place of outs[g] (same shapes,
 * bf16 or fp32, read and written in place); every other argument, the
 * workspace and the errors are those of muon_orthogonalize_packed_grouped,
 * and lr, weight_decay, mode and coeff are checked as in muon_apply.
 */
muon_status_t muon_orthogonalize_apply_packed_grouped(int ngroups, const float* const* sumsqs,
                                                      const muon_batch_t* weights, int steps,
                                                      float a, float b, float c, float eps,
                                                      float lr, float weight_decay, int32_t mode,
                                                      float coeff, int32_t compute,
                                                      void* workspace, size_t ws_bytes,
                                                      void* stream);

/*
 * Parameter update ([GUIDE] 11.5 update equation; [LESSON] "Muon" step 4):
 *   W <- (1 - lr*weight_decay) * W - lr * s * O
 * with s from `mode` and `coeff` (see muon_scale_t) and (m, n) = (rows,
 * cols) of W.  Both terms read the old W.  Arithmetic is fp32; a BF16 W is
 * rounded once to nearest even.
 *
 * weight: W, BF16 or F32, in place.  ortho: O, BF16 or F32, same shape.
 * lr, weight_decay, coeff: finite.
 */
muon_status_t muon_apply(const muon_batch_t* weight, const muon_batch_t* ortho,
                         float lr, float weight_decay, int32_t mode,
                         float coeff, void* stream);

/*
 * muon_apply for several shape classes in one launch: group g updates
 * weights[g] from orthos[g] with the meaning and rules of muon_apply, its
 * scale s taken from its own (rows, cols); lr, weight_decay, mode and coeff
 * are shared.  ngroups: 1..8; weights, orthos: host arrays of ngroups
 * descriptors.  Every group is validated before the launch; results equal
 * separate muon_apply calls bit for bit.
 */
muon_status_t muon_apply_grouped(int ngroups, const muon_batch_t* weights,
                                 const muon_batch_t* orthos, float lr,
                                 float weight_decay, int32_t mode, float coeff,
                                 void* stream);

/*
 * AdamW for the parameters Muon does not take (embeddings, output head, norms,
 * biases), many tensors in one launch ([GUIDE] section 5 "Adam, line by
 * line" and section 6, decoupled weight decay):
 *   m <- beta1*m + (1-beta1)*g;   v <- beta2*v + (1-beta2)*g^2
 *   m_hat = m / (1 - beta1^t);    v_hat = v / (1 - beta2^t)
 *   theta <- (1 - lr*weight_decay)*theta - lr * m_hat / (sqrt(v_hat) + eps)
 * Epsilon is added outside the square root.  Arithmetic is fp32 (bias
 * corrections in double on the host); a BF16 theta is rounded once to
 * nearest even.
 *
 * Every tensor is a contiguous run of numels[i] elements (any shape),
 * 16-byte aligned.  The tensor list lives in DEVICE memory and is only
 * read by the kernel: params[i] (theta, in/out, param_dtype), grads[i]
 * (read, grad_dtype), exp_avg[i] and exp_avg_sq[i] (F32 state, in/out,
 * zero before step 1), numels[i], and chunk_offsets[0..count] = prefix sums
 * of ceil(numels[i] / MUON_ADAMW_CHUNK) with chunk_offsets[0] = 0;
 * total_chunks = chunk_offsets[count] is passed by value (the library does
 * not read device memory on the host).  Each kernel access is bounded by
 * its tensor's numel, so an inconsistent chunk table leaves elements
 * un-updated but never reads or writes outside a tensor.
 *
 * step : t >= 1, the number of this update for every tensor in the list
 *        (one list per parameter group; a tensor whose gradient is absent
 *        is left out of the call, [GUIDE] 6.2).
 * beta1, beta2 in [0, 1); eps finite >= 0; lr, weight_decay finite.
 */
#define MUON_ADAMW_CHUNK 4096

typedef struct muon_tensor_list {
  int64_t count;                 /* tensors, >= 1 */
  int64_t total_chunks;          /* chunk_offsets[count]; 1 .. 2^31-1 */
  void* const* params;           /* device array [count] */
  const void* const* grads;      /* device array [count] */
  float* const* exp_avg;         /* device array [count] */
  float* const* exp_avg_sq;      /* device array [count] */
  const int64_t* numels;         /* device array [count] */
  const int64_t* chunk_offsets;  /* device array [count + 1] */
  int32_t param_dtype;           /* muon_dtype_t of every theta */
  int32_t grad_dtype;            /* muon_dtype_t of every gradient */
} muon_tensor_list_t;

muon_status_t muon_adamw(const muon_tensor_list_t* tensors, int64_t step, float lr, float beta1,
                         float beta2, float eps, float weight_decay, void* stream);

/*
 * SOAP: Adam run in the eigenbasis of Shampoo's row and column statistics
 * ([GUIDE] section 11.1 "SOAP: Adam in Shampoo's eigenbasis" and 11.2;
 * [ZH] section 6.2), for `count` same-shape
 * m x n matrices.  All SOAP state is caller-owned F32 device memory, one
 * muon_batch_t each, with the gradient's count:
 *   L (m x m), R (n x n)   row and column statistics, zero before step 1;
 *   QL (m x m), QR (n x n) their bases, the identity before step 1;
 *   mbar, vbar (m x n)     Adam's moments in the rotated basis, zero before
 *                          step 1.
 * A side passed as NULL (statistic and basis together) keeps the identity
 * basis: an axis too long to precondition ([GUIDE] 11.2).  One update at
 * step t = 1, 2, ... with refresh interval f:
 *   soap_statistics(G, L, R, beta_s);
 *   if ((t - 1) % f == 0) soap_refresh(L, R, QL, QR, mbar, ...);
 *   soap_precondition(G, QL, QR, mbar, vbar, D, t, beta1, beta2, eps, ...);
 *   muon_apply(W, D, lr, weight_decay, MUON_SCALE_NONE, 1, stream);
 * the last line being W <- (1 - lr*wd) W - lr D.  All arithmetic is fp32
 * (the products on the fp32 matrix cores).  The calls enqueue on `stream`
 * and never allocate or synchronize; a workspace (16-byte aligned, of the
 * size its query returns, 0 for arguments out of range) holds temporaries
 * and is free again when the stream reaches the end of the call.
 * Errors: as for the Muon calls (NULL or mismatched descriptors, BF16 where
 * F32 is required, betas outside [0, 1), step < 1, eps not finite or < 0,
 * a short workspace), checked before anything is enqueued.
 */

/* L <- beta_s L + (1-beta_s) G G^T and R <- beta_s R + (1-beta_s) G^T G
 * ([GUIDE] 11.1 first display).  grad: F32 or BF16, m x n.  L or R may be
 * NULL.  Only the upper triangle of the old statistic is read and both
 * triangles are written, so a statistic stays exactly symmetric. */
muon_status_t soap_statistics(const muon_batch_t* grad, const muon_batch_t* L, const muon_batch_t* R,
                              float beta_s, void* stream);

/* soap_statistics for up to 8 groups (shape classes) at once: grads[g] is
 * group g's gradient descriptor and Ls[g], Rs[g] point to its statistics or
 * are NULL.  The products
 * of all groups share launches (one per operand layout, longest reduction
 * first), so small groups fill the chip beside large ones; every statistic
 * is bit-identical to soap_statistics on its group.  The three arrays are
 * host arrays of ngroups entries.  Errors name the group; nothing is
 * enqueued unless every group is valid. */
muon_status_t soap_statistics_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* Ls,
                                      const muon_batch_t* const* Rs, float beta_s, void* stream);

/* Q factor of a QR factorization, the triangular factor's diagonal made
 * non-negative (unique for a full-rank input): Householder reflections
 * in 16-column panels with blocked trailing updates.  a (read only) and q:
 * F32, n x n, n <= 32768. */
size_t soap_qr_workspace(int64_t count, int64_t n);
muon_status_t soap_qr(const muon_batch_t* a, const muon_batch_t* q, void* workspace, size_t ws_bytes,
                      void* stream);

/* Basis refresh by one power-iteration step plus QR ([GUIDE] 11.2, [ZH]
 * 6.2 step 2): QL <- qr(L QL), QR <- qr(R QR) as soap_qr, and the first
 * moment carried exactly into the new bases ([GUIDE] 11.1 third display):
 * mbar <- QL_new^T QL_old mbar QR_old^T QR_new.  mbar (m x n) gives the
 * shape; a NULL side is left out. */
size_t soap_refresh_workspace(int64_t count, int64_t rows, int64_t cols, int with_l, int with_r);
muon_status_t soap_refresh(const muon_batch_t* L, const muon_batch_t* R, const muon_batch_t* QL,
                           const muon_batch_t* QR, const muon_batch_t* mbar, void* workspace, size_t ws_bytes,
                           void* stream);

/* soap_refresh for up to 8 groups (shape classes) at once: Ls[g], Rs[g],
 * QLs[g], QRs[g] point to group g's descriptors or are NULL for a side
 * without statistic; mbars[g] is group g's first moment.  All QRs of one
 * order, over every group and side, run as one batched factorization. */
size_t soap_refresh_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows,
                                      const int64_t* cols, const int* with_l, const int* with_r);
muon_status_t soap_refresh_grouped(int ngroups, const muon_batch_t* const* Ls, const muon_batch_t* const* Rs,
                                   const muon_batch_t* const* QLs, const muon_batch_t* const* QRs,
                                   const muon_batch_t* mbars, void* workspace, size_t ws_bytes, void* stream);

/* [GUIDE] 11.1 between refreshes:
 *   Gbar = QL^T G QR;  mbar <- beta1 mbar + (1-beta1) Gbar;
 *   vbar <- beta2 vbar + (1-beta2) Gbar^2;
 *   D = QL [ (mbar / (1-beta1^t)) / (sqrt(vbar / (1-beta2^t)) + eps) ] QR^T
 * with epsilon after the square root.  grad: F32 or BF16, m x n; QL, QR
 * as above or NULL (identity); mbar, vbar in/out; dir (D, out): F32 m x n,
 * not aliasing the others. */
size_t soap_precondition_workspace(int64_t count, int64_t rows, int64_t cols);
muon_status_t soap_precondition(const muon_batch_t* grad, const muon_batch_t* QL, const muon_batch_t* QR,
                                const muon_batch_t* mbar, const muon_batch_t* vbar, const muon_batch_t* dir,
                                int64_t step, float beta1, float beta2, float eps, void* workspace,
                                size_t ws_bytes, void* stream);

/* soap_precondition for up to 8 groups (shape classes) at once, with one
 * step count and one set of hyperparameters: grads, mbars, vbars and dirs
 * are host arrays of ngroups descriptors, QLs and QRs host arrays of
 * ngroups pointers (NULL: identity).  Each rotation stage launches the
 * products of all groups together; every direction is bit-identical to
 * soap_precondition on its group.  The workspace holds two m x n
 * temporaries per group (the sum of the groups' soap_precondition
 * workspaces).  Errors name the group; nothing is enqueued unless every
 * group is valid. */
size_t soap_precondition_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows,
                                           const int64_t* cols);
muon_status_t soap_precondition_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* QLs,
                                        const muon_batch_t* const* QRs, const muon_batch_t* mbars,
                                        const muon_batch_t* vbars, const muon_batch_t* dirs, int64_t step,
                                        float beta1, float beta2, float eps, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Static text for a status code. */
const char* muon_status_string(muon_status_t status);
/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* muon_last_error(void);
/* MUON355_ABI_VERSION of the loaded library. */
int muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON355_H */
