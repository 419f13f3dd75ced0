/*
 * lrc.h -- C ABI of liblrc, activation-aware low-rank compression on MI355X (gfx950).
 *
 * The method (Swift-SVD page, "Swift-SVD: Theoretical Optimality Meets Practical
 * Efficiency in Low-Rank LLM Compression", section 2-ga): calibration activations X
 * stream through Y = X W; the output covariance C = sum_t y_t^T y_t is accumulated; one
 * symmetric eigendecomposition C = V diag(lambda) V^T gives the right singular vectors
 * and squared singular values of Y; the closed-form optimum of rank k is
 * W_k = (W V_k) V_k^T and its error eps_k = sum_{i>k} lambda_i.  Ranks are spread over
 * many matrices by a greedy allocation under a parameter budget (LASER page, "LASER:
 * Loss-Aware Singular-value Decomposition and Rank Allocation", method 2) weighted by the
 * Fisher importance alpha = sum (G (.) W)^2 (FLRC page, "FLRC: Fine-grained Low-Rank
 * Compressor for Efficient LLM Inference", method 1).
 *
 * Orientation: Y = X W with X n_tok x d_in (tokens x input features), W d_in x d_out,
 * C d_out x d_out.  A PyTorch nn.Linear weight is the transpose of this W.
 *
 * Conventions shared by every entry point:
 *  - All matrices are row-major with an explicit leading dimension (elements).
 *  - All array pointers are DEVICE pointers unless marked (host).  Buffers are owned by
 *    the caller; the library keeps no state between calls except per-device kernel
 *    modules.
 *  - `stream` is a hipStream_t (NULL = the default stream).  A call only enqueues work
 *    on that stream and returns; buffers must stay alive until the stream reaches it.
 *  - Argument errors are reported synchronously as an lrc_status and then nothing is
 *    launched.  lrc_last_error() gives a thread-local message for the last failure.
 *  - Numerical outcomes found on the device are written to a caller-provided int32
 *    `info` array in device memory (one entry per matrix unless stated), readable after
 *    the stream has been synchronised:  0 ok, 1 non-finite input, 2 no convergence,
 *    3 not positive definite, 4 mandatory ranks exceed the budget, 5 negative or NaN
 *    score.  Entry points that write info set it on every call (0 when all is well).
 *  - Workspace (`ws`, `ws_bytes`) is caller-allocated device memory of at least the size
 *    returned by the matching *_workspace() query, 256-byte aligned; it may be NULL when
 *    that size is 0.  Its contents are scratch and need no initialisation.
 *  - Results are deterministic: identical inputs and launch give bit-identical outputs
 *    (fixed-order reductions, no floating-point atomics).
 */
#ifndef LRC_H
#define LRC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRC_ABI_VERSION 1

typedef enum {
    LRC_OK = 0,
    LRC_ERR_ARG = 1,           /* bad size, stride, pointer or flag */
    LRC_ERR_DTYPE = 2,         /* dtype not supported by this entry point */
    LRC_ERR_WORKSPACE = 3,     /* ws NULL or smaller than the query says */
    LRC_ERR_HIP = 4,           /* a HIP runtime call failed (message in lrc_last_error) */
    LRC_ERR_UNIMPLEMENTED = 5  /* valid request the library does not implement */
} lrc_status;

typedef enum { LRC_BF16 = 0, LRC_F32 = 1, LRC_F64 = 2 } lrc_dtype;

enum {
    LRC_INFO_OK = 0,
    LRC_INFO_NONFINITE = 1,
    LRC_INFO_NO_CONVERGENCE = 2,
    LRC_INFO_NOT_PD = 3,
    LRC_INFO_BUDGET = 4,
    LRC_INFO_BAD_SCORE = 5
};

/* ------------------------------------------------------------------------------------
 * Kernel timing (instrumentation, not part of the method).  lrc_timing_enable(stride) with
 * stride >= 1 makes the library record a HIP event pair on the launch stream around every
 * stride-th launch of each of the named kernels ("k_cov_syrk", "k_cov_gemm_y", "k_trd_symv",
 * "k_dgemm"; a uniform sample, counted per kernel from the enable call) and remember each
 * recorded launch's algorithmic work: flops for the contractions, bytes for k_trd_symv (the
 * upper triangle of the trailing matrix, read once).  stride 0 disables.  lrc_timing_read
 * synchronises on the recorded events and returns, for one kernel name, the number of recorded
 * launches, their summed duration in milliseconds and their summed algorithmic work since the
 * last reset; reset != 0 then discards the records of every kernel.  lrc_timing_set_stride
 * gives one kernel its own stride (>= 1), overriding the one of lrc_timing_enable.  Sampled
 * launches go through hipExtLaunchKernel with a start and a stop event that the dispatch itself
 * records, so the durations are the kernels' own, without queueing.  Not thread-safe with
 * respect to concurrent lrc_timing_read calls.
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_timing_enable(int stride);
lrc_status lrc_timing_set_stride(const char *kernel, int stride);
lrc_status lrc_timing_read(const char *kernel, int64_t *launches, double *total_ms, double *total_work,
                           int reset);

/* LRC_ABI_VERSION of the built library. */
int lrc_abi_version(void);
/* Static text for a status code. */
const char *lrc_status_string(lrc_status s);
/* Thread-local description of the last non-OK status returned on this thread. */
const char *lrc_last_error(void);

/* ------------------------------------------------------------------------------------
 * Covariance accumulation (Swift-SVD page, section 2-ga: the covariance of Y = XW is
 * aggregated incrementally over calibration tokens).
 *
 *   C[upper] += (X W)^T (X W)   over the n_tok rows of X.
 *
 * X: n_tok x d_in, leading dim ldx >= d_in, dtype x_t (LRC_BF16 or LRC_F32).
 * W: d_in x d_out, leading dim ldw >= d_out, dtype w_t (must equal x_t); W == NULL means
 *    the identity (then d_out must equal d_in and C += X^T X).
 * n_blocks == 1: C is d_out x d_out fp32 (ldc >= d_out); the upper triangle including the
 *    diagonal is accumulated, the strict lower triangle is never read or written.
 * n_blocks > 1 (per-head, WSVD page "WSVD: Weighted Low-Rank Approximation for Fast and
 *    Efficient Execution of Low-Precision Vision-Language Models", methodology 1): only
 *    the n_blocks diagonal blocks of width hd = d_out / n_blocks are formed; block h is
 *    Y[:, h hd:(h+1) hd]^T Y[:, h hd:(h+1) hd], stored at C + h*hd*ldc as an hd x hd
 *    matrix with leading dim ldc >= hd (upper triangle accumulated).
 * Accumulates: the caller zeroes C before the first chunk.  Any chunking of the tokens
 *    gives the same C up to fp32 rounding of the running sum.
 * Arithmetic: bf16 inputs use bf16 MFMA with fp32 accumulation for Y.  Output i is then
 *    scaled by an exact power of two 2^e_i, chosen per call from max_t ||x_t|| ||W[:, i]||
 *    so that |y 2^e_i| < 2^14, and split into fp16 hi + lo (22 bits of y).  C gains
 *    2^-(e_i + e_j) (hi hi^T + hi lo^T + lo hi^T) from three fp16 MFMA products (fp32
 *    accumulation), plus sum_t lo_i(t)^2 on the diagonal; the off-diagonal lo lo^T terms
 *    (about 2^-24 of hi hi^T) are left out.  W == NULL: X^T X from one bf16 product (exact
 *    products, fp32 sums).
 *    fp32 inputs use fp32 arithmetic throughout.
 *    A non-finite x or W entry reaches C as before (the scale is then 1).
 *    Per-head blocks of 128 with the environment variable LRC_HEAD_FUSED=1: the same arithmetic
 *    with each head's Y tile kept in LDS (one kernel), the token ranges' partial sums added in
 *    order; results agree with the default path to fp32 rounding (not bit for bit).
 * info: one int32; set to 1 when the updated C has a non-finite diagonal entry.
 * Errors: LRC_ERR_ARG for non-positive sizes, small leading dims, d_out % n_blocks != 0,
 *    NULL X or C; LRC_ERR_DTYPE for other dtypes or x_t != w_t; LRC_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t lrc_cov_accumulate_workspace(lrc_dtype x_t, int64_t n_tok, int64_t d_in, int has_w,
                                    int64_t d_out, int32_t n_blocks);
lrc_status lrc_cov_accumulate(const void *X, lrc_dtype x_t, int64_t n_tok, int64_t d_in, int64_t ldx,
                              const void *W, lrc_dtype w_t, int64_t d_out, int64_t ldw, int32_t n_blocks,
                              float *C, int64_t ldc, void *ws, size_t ws_bytes, int32_t *info,
                              void *stream);

/* ------------------------------------------------------------------------------------
 * Range-projected covariance (Swift-SVD page, section 2-ga: only Y^T Y's eigenpairs enter
 * the closed form; for a layer that widens, d_in < d_out, C = Y^T Y has rank at most d_in).
 *
 * lrc_range_factor: L (d_in x d_in, fp64, lower; its strict upper triangle set to 0) with
 *    W W^T = L L^T, W: d_in x n (ldw >= n, n >= d_in) of dtype LRC_BF16,
 *    LRC_F32 or LRC_F64, widened exactly to fp64; W W^T and its Cholesky factorisation in
 *    fp64 (the kernels of lrc_cholesky).  info (one int32): 0; 3 when W W^T is not
 *    positive definite or L's diagonal spans more than a factor 1e5 (W not of full row rank
 *    or too ill-conditioned for Q = W^T L^{-T} to be orthonormal in fp64).
 * lrc_cov_accumulate_range: B[upper] += (X L)^T (X L) over the n_tok rows of X (bf16,
 *    n_tok x d_in, ldx >= d_in, 16-byte aligned, ldx a multiple of 8); B d_in x d_in fp32
 *    (ldb >= d_in), the caller zeroes it before the first chunk.  With Q = W^T L^{-T}, an
 *    orthonormal basis of range(W^T), X L = X W Q, so B = Q^T C Q for C = (X W)^T (X W):
 *    C's covariance of Y = X W in the coordinates of the basis, C = Q B Q^T, and the
 *    eigenpairs of C are those of B (V = Q U) plus n - d_in zeros.  lrc_eigh_multi takes B
 *    with projected = 1.  Arithmetic: L^T is rounded to three bf16 pieces (hi, mid, lo, their
 *    sum within about 2^-26 of L), X L is their three bf16 MFMA products with one fp32
 *    accumulator (block rows of the triangular L^T start at their diagonal), then the
 *    scaled fp16 hi/lo split and the three-product SYRK of lrc_cov_accumulate.
 * info: one int32; 1 when the updated B has a non-finite diagonal entry.
 * Errors: LRC_ERR_ARG for sizes (d_in a multiple of 32), leading dims, NULL pointers or an
 *    unaligned X; LRC_ERR_DTYPE for x_t other than LRC_BF16; LRC_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t lrc_range_factor_workspace(int64_t d_in, int64_t n);
lrc_status lrc_range_factor(const void *W, lrc_dtype w_t, int64_t d_in, int64_t n, int64_t ldw, double *L,
                            int64_t ldl, void *ws, size_t ws_bytes, int32_t *info, void *stream);
size_t lrc_cov_accumulate_range_workspace(int64_t n_tok, int64_t d_in);
lrc_status lrc_cov_accumulate_range(const void *X, lrc_dtype x_t, int64_t n_tok, int64_t d_in, int64_t ldx,
                                    const double *L, int64_t ldl, float *B, int64_t ldb, void *ws,
                                    size_t ws_bytes, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Symmetric eigendecomposition (Swift-SVD page, section 2-ga: one eigendecomposition of
 * Y^T Y gives V and Sigma^2 of Y).
 *
 * C: batch matrices n x n fp32, matrix b at C + b*stride_c, leading dim ldc >= n; only the
 *    upper triangle (incl. diagonal) is read.  Not modified.
 * lambda: batch x n fp64 (matrix b at lambda + b*n), all eigenvalues, descending.
 * V: batch x n x n_vec fp32 (matrix b at V + b*stride_v, leading dim ldv >= n_vec): column
 *    j is the unit eigenvector of lambda[j], j < n_vec, with its entry of largest
 *    magnitude positive (first index on ties).  V may be NULL when n_vec == 0.
 * prec: working precision, LRC_F32 or LRC_F64.
 *    n <= 128: one-sided Jacobi, one matrix per workgroup held in LDS, always in fp64
 *    (prec has no effect there).
 *    n > 128: Householder tridiagonalisation and back-transformation in prec; the
 *    tridiagonal eigenproblem (bisection, inverse iteration) always in fp64.
 * Batches with n > 128: up to eight members are decomposed at once, each on a helper
 *    stream of the library's (default priority, created per device on first use and kept
 *    until the process ends) with a workspace of its own, fed by a host thread of its
 *    own; the call returns once every launch is enqueued (without waiting for the GPU)
 *    and the caller's stream waits for every member, so results are ordered on `stream`
 *    as for any other call.  Each member's result does not depend on the batch it is in.
 *    Calls may run at once from several host threads (each with its own workspace and
 *    stream): each call takes its helper streams from a rotating base, so calls that
 *    together hold at most eight members do not queue behind one another.
 *    With the environment variable LRC_EIGH_HOST_THREADS=0 the calling thread enqueues
 *    all members itself, on one helper stream (for tools that cannot follow launches
 *    from several host threads); results are the same.
 * info: batch int32: 2 when the Jacobi sweeps did not converge, 1 for non-finite input.
 * Errors: LRC_ERR_ARG (sizes, strides, n_vec > n), LRC_ERR_DTYPE (prec), LRC_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t lrc_eigh_workspace(int64_t n, int64_t batch, int64_t n_vec, lrc_dtype prec);
lrc_status lrc_eigh(const float *C, int64_t n, int64_t ldc, int64_t batch, int64_t stride_c,
                    lrc_dtype prec, double *lambda, float *V, int64_t ldv, int64_t n_vec,
                    int64_t stride_v, void *ws, size_t ws_bytes, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Several eigendecompositions in one call (the operation of lrc_eigh, on each group).
 *
 * A block of a network has matrices of several widths (4096 and 11008 wide covariances in
 * a LLaMA-7B block); one call over all of them lets the library run the matrices of
 * different widths at the same time, which separate calls cannot (each call returns only
 * after it has handed all of its launches to the GPU).
 * groups[i]: the arguments of one lrc_eigh call (same meaning, layout and checks); all
 *    groups use the working precision prec.  Groups must not overlap in lambda, V, info.
 * Groups with n <= 128 run first, one Jacobi launch each, on `stream`; every member of
 *    the groups with n > 128 is then decomposed on the helper streams described under
 *    lrc_eigh, up to eight at once, largest n first.  `stream` waits for all of them.
 *    When there are 2 to 8 such members and all have one tridiagonal order (n, or d_in
 *    for a member decomposed through its range basis), their tridiagonalisations run in
 *    lockstep on `stream`, one launch per column for all of them, before the rest of each
 *    decomposition moves to the helper streams (environment LRC_EIGH_LOCKSTEP=0: off).
 *    Each member's result equals that of a call on the member alone, bit for bit.
 * Range basis (optional, per group; Swift-SVD page, section 2-ga: C = Y^T Y with Y = X W):
 *    W != NULL states that each member's C is (X W)^T (X W) for some X, with W (d_in x n,
 *    row-major, ldw >= n, dtype w_t: LRC_BF16, LRC_F32 or LRC_F64; member b at W +
 *    b * stride_w elements) of full row rank.  C's rank is then at most d_in, its range
 *    lies in that of W^T, and when 128 < d_in < n and n_vec <= d_in the member is
 *    decomposed through B = Q^T C Q, Q (n x d_in) an orthonormal basis of range(W^T)
 *    (Q^T = L^{-1} W with W W^T = L L^T, in fp64): lambda = the d_in eigenvalues of B and
 *    n - d_in zeros, in descending order, V = Q U.  The part of the computed C outside
 *    range(W^T) is rounding error, which the full decomposition would report as
 *    eigenvalues of about 1e-7 of the largest; here they are exact zeros.  info 3: W W^T
 *    is not positive definite, or the diagonal of L spans more than a factor 1e5 (W not
 *    of full row rank, or so ill-conditioned that Q loses orthogonality: use the full
 *    decomposition); 6: fewer than n_vec eigenvalues of B are non-negative.  Other d_in,
 *    or n_vec > d_in: W is ignored.
 * projected = 1 (needs W with 128 < d_in < n and n_vec <= d_in, else LRC_ERR_ARG): C points
 *    at B itself, d_in x d_in fp32 (upper triangle read, ldc >= d_in, stride_c between
 *    members), as lrc_cov_accumulate_range forms it from the L of lrc_range_factor; the
 *    library forms Q from W with the same kernels (the same L bit for bit) and proceeds as
 *    above from B.  lambda (n values) and V (n x n_vec) keep their meaning.  0: C is n x n.
 * L (optional, with W): the lower factor of W W^T = L L^T that lrc_range_factor gave (info 0),
 *    d_in x d_in fp64, ldl >= d_in, member b at L + b * stride_l; the library then uses it
 *    instead of forming its own (the same values when it came from lrc_range_factor on the
 *    same W).  For a projected member V = W^T (L^{-T} U), the same Q U.  NULL: formed here.
 * A (optional, projected groups only): also the factor A = W V[:, :n_vec] of lrc_factorize
 *    (d_in x n_vec fp32, lda >= n_vec, member b at A + b * stride_a), formed as L U with U's
 *    columns signed as V's (W V = W W^T L^{-T} U = L U exactly), in fp64, rounded once; the
 *    caller then needs lrc_factorize only for B.  NULL: not formed.
 * ws: lrc_eigh_multi_workspace(groups, count, prec) bytes, 256-byte aligned (one region
 *    per concurrent member, each sized for the largest n and n_vec among the groups, or
 *    for the largest member with a range basis if that needs more).
 * Errors: those of lrc_eigh, for the first group that fails a check; LRC_ERR_ARG for a
 *    NULL groups or count <= 0.  The workspace query returns 0 for invalid sizes.
 * ------------------------------------------------------------------------------------ */
typedef struct lrc_eigh_group {
    const float *C;
    int64_t n, ldc, batch, stride_c;
    double *lambda;
    float *V;
    int64_t ldv, n_vec, stride_v;
    int32_t *info;
    const void *W;      /* optional range basis, d_in x n; NULL for none */
    lrc_dtype w_t;
    int64_t d_in, ldw, stride_w;
    int32_t projected;  /* 1: C holds B = Q^T C Q (d_in x d_in) from lrc_cov_accumulate_range */
    const double *L;    /* optional factor of W W^T from lrc_range_factor (info 0); NULL: formed here */
    int64_t ldl, stride_l;
    float *A;           /* optional, projected groups: the factor W V[:, :n_vec], d_in x n_vec */
    int64_t lda, stride_a;
} lrc_eigh_group;
size_t lrc_eigh_multi_workspace(const lrc_eigh_group *groups, int32_t count, lrc_dtype prec);
lrc_status lrc_eigh_multi(const lrc_eigh_group *groups, int32_t count, lrc_dtype prec, void *ws,
                          size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------------------
 * Error curve (Swift-SVD page, section 2-ga: the closed-form minimal error eps*_k).
 *
 *   eps[b][k] = sum_{i >= k} lambda[b][i]  (0-based lambda; = sum of the eigenvalues
 *   beyond the first k), k = 0..n, eps[b][n] = 0, summed from the smallest term.
 * lambda: batch x n fp64; eps: batch x (n+1) fp64.
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_error_curve(const double *lambda, int64_t n, int64_t batch, double *eps, void *stream);

/* ------------------------------------------------------------------------------------
 * Factor projection (Swift-SVD page, section 2-ga: W_k = (W V_k) V_k^T).
 *
 * trans_w == 0:  A = W V[:, :k]   (A: d_in x k),  W d_in x d_out, V d_out x (>= k).
 * trans_w == 1:  A = W^T V[:, :k] (A: d_out x k), W d_in x d_out, V d_in x (>= k).
 * B = V[:, :k]^T (k x rows(V)) when B != NULL.  A may be NULL when B is not (only B is formed:
 *    a projected decomposition of lrc_eigh_multi can return A itself).
 * W: dtype w_t (LRC_BF16, LRC_F32 or LRC_F64), leading dim ldw >= d_out; V fp32 with
 *    leading dim ldv >= k; A fp32 (lda >= k); B fp32 (ldb >= rows of V).
 * Batched: matrix b uses W + b*stride_w, V + b*stride_v, A + b*stride_a, B + b*stride_b
 *    (element offsets; a per-head W_h is a column slice: stride_w = head width).
 * Arithmetic: products and sums in fp64 (fp64 MFMA), A rounded once to fp32.
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_factorize(const void *W, lrc_dtype w_t, int32_t trans_w, int64_t d_in, int64_t d_out,
                         int64_t ldw, const float *V, int64_t ldv, int64_t k, int64_t batch,
                         int64_t stride_w, int64_t stride_v, float *A, int64_t lda, int64_t stride_a,
                         float *B, int64_t ldb, int64_t stride_b, void *stream);

/* ------------------------------------------------------------------------------------
 * Fisher importance (FLRC page, method 1: alpha_{l,p} = sum_i (G_{l,p}[i] W_{l,p}[i])^2).
 *
 * G, W, numel: (host) arrays of n_mats device pointers / element counts; G[m] and W[m]
 *    hold numel[m] contiguous elements of dtype t (LRC_BF16 or LRC_F32).
 * alpha: n_mats fp64 (device).  Products are exact in fp32 for bf16 inputs; squares and
 *    sums in fp64 with a fixed-order reduction.
 * info: n_mats int32, 1 when alpha[m] is not finite.
 * ------------------------------------------------------------------------------------ */
size_t lrc_fisher_scores_workspace(int32_t n_mats, const int64_t *numel /* host */);
lrc_status lrc_fisher_scores(int32_t n_mats, const void *const *G /* host */, const void *const *W /* host */,
                             const int64_t *numel /* host */, lrc_dtype t, double *alpha, void *ws,
                             size_t ws_bytes, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * lrc_fisher_scores without workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, result and info as lrc_fisher_scores minus ws / ws_bytes.  The per-block partial
 * sums go to a scratch array that the library holds in device memory, 4 MiB (2^19 fp64
 * partials) per GPU, allocated when the library is loaded and kept until the process ends.  No
 * hipMalloc, hipFree or other allocating call is made.  Limit: the total number of 32768-element
 * blocks over all matrices (sum of ceil(numel[m] / 32768)) must not exceed 2^19, about 1.7e10
 * elements in one call; larger inputs return LRC_ERR_ARG and nothing is launched.  Every call on
 * one GPU shares that GPU's scratch array: calls that overlap on one GPU (several streams or host
 * threads at once) race and must be serialised by the caller.
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_fisher_scores_noalloc(int32_t n_mats, const void *const *G /* host */,
                                     const void *const *W /* host */, const int64_t *numel /* host */,
                                     lrc_dtype t, double *alpha, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Greedy global rank allocation under a parameter budget (LASER page, method 2: take the
 * singular components of highest importance per parameter cost until the budget is
 * reached; FLRC page, method 1: Fisher importance per projection; Swift-SVD page, section
 * 2-na: a guaranteed minimum rank per layer).
 *
 * For matrix m (0 <= m < n_mats), candidates are ranks k = k_min[m]+1 .. K_m with
 * K_m = offsets[m+1] - offsets[m]; candidate k has cost cost[m] parameters (d_in + d_out)
 * and priority p = w_m * max(lambda_m[k-1], 0), w_m = alpha[m] / (eps0[m] * cost[m])
 * (w_m = 0 when eps0[m] == 0), each step one IEEE fp64 multiply or divide.  Candidates are
 * ordered by p descending, then m ascending, then k ascending; the mandatory
 * sum_m k_min[m] cost[m] is charged first; candidates are taken in order while they fit
 * in the budget, stopping at the first that does not.  k_out[m] = k_min[m] + number taken.
 *
 * alpha, eps0: n_mats fp64; lambda_packed: fp64, matrix m's lambda at offsets[m];
 * offsets: n_mats+1 int64 (device); cost: n_mats int64 (> 0); k_min: n_mats int32 or NULL
 * (all 0); n_items = offsets[n_mats] (host copy, for launch sizing); k_out: n_mats int32.
 * info: one int32: 4 mandatory ranks exceed the budget, 5 an alpha/eps0 negative or NaN.
 * Bit-exact: the result depends only on the fp64 priorities, computed as stated.
 * ------------------------------------------------------------------------------------ */
size_t lrc_allocate_ranks_workspace(int32_t n_mats, int64_t n_items);
lrc_status lrc_allocate_ranks(int32_t n_mats, const double *alpha, const double *lambda_packed,
                              const int64_t *offsets, int64_t n_items, const double *eps0,
                              const int64_t *cost, const int32_t *k_min, int64_t budget_params,
                              int32_t *k_out, void *ws, size_t ws_bytes, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Proportional rank allocation (FLRC page, method 1: each projection's rank in proportion to
 * its Fisher importance, r_m = round(alpha_m / S * R) with S = sum of alpha; method 2: the same
 * rule for each budget R(t) of a non-increasing per-token schedule).
 *
 * alpha: n_mats fp64 (1 <= n_mats <= 1024), e.g. lrc_fisher_scores' output.
 * budgets: n_budgets int64 total rank budgets R (one row of output each).
 * r_out: n_budgets x n_mats int64 ranks, row t for budgets[t].
 * Rounding (the page leaves it open): half away from zero, then the row is brought to sum to
 *    exactly R by largest remainders (short by d: the d matrices with the largest alpha_m R / S
 *    - r_m gain one, ties to the smaller m; over by d: the d matrices with r_m > 0 and the
 *    smallest remainders lose one, ties to the smaller m).  q_m = (alpha_m R) / S in fp64 with S
 *    summed in index order, so the result is bit-exact against a sequential evaluation.
 *    Along a falling schedule R(t) a matrix's rank can rise by one from one budget to the next
 *    (largest-remainder rounding is subject to the Alabama paradox), never by more.
 * info: one int32: 0, or 5 when an alpha is negative or NaN, S is not positive and finite, or a
 *    budget is negative (every rank is then 0).
 * Errors: LRC_ERR_ARG (NULL pointers, n_mats outside 1 .. 1024, n_budgets <= 0).
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_allocate_proportional(int32_t n_mats, const double *alpha, int32_t n_budgets,
                                     const int64_t *budgets, int64_t *r_out, int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Swift-SVD allocation candidates (Swift-SVD page, section 2-na, dynamic rank allocation: step 1
 * scores each matrix by s_i = beta_i^alpha * log(e + eps_{kbar,i})^(1 - alpha), combining its
 * importance beta_i with its closed-form error at the uniform rank; step 2 keeps a minimum rank
 * kbar * delta per matrix; step 3 compares candidates over a grid of alpha -- that selection, by
 * validation loss, is the caller's).
 *
 * beta: n_mats fp64 importances (e.g. lrc_fisher_scores' alpha).  eps_kbar: n_mats fp64, matrix
 *    i's error eps_i[kbar_i] from lrc_error_curve (a negative rounding residue counts as 0).
 * kbar: n_mats int64 uniform ranks, 0 <= kbar_i <= k_cap_i; cost: n_mats int64 parameters per
 *    rank (d_in + d_out, > 0); k_cap: n_mats int64 largest ranks.  delta in [0, 1].
 * alpha_grid: n_alpha fp64 values in [0, 1] (device), one candidate allocation each.
 * scores: n_alpha x n_mats fp64 (row a for alpha_grid[a]); k_out: n_alpha x n_mats int32 ranks.
 * Ranks (a reading, the page does not print the rule): k_i = floor(kbar_i delta) + extra_i, where
 *    the parameters left after the minima, E = budget - sum floor(kbar_i delta) cost_i, are split
 *    in proportion to the scores: with S the index-order sum of the scores of the matrices still
 *    open and R the parameters not yet committed, extra_i = floor(((s_i R) / S) / cost_i) (fp64,
 *    one operation at a time); a matrix whose rank would reach k_cap_i is set to k_cap_i and
 *    closed, and the split is redone among the others until none reaches its cap.  If rounding
 *    ever made the total exceed the budget, the open matrices of highest index give ranks back.
 *    pow and log are the device's fp64 functions; the ranks are bit-exact against a sequential
 *    evaluation given the same scores.
 * info: n_alpha int32: 0; 4 when the minima exceed the budget (k = minima); 5 when a score is
 *    negative, NaN or infinite, a kbar lies outside [0, k_cap], a cost is <= 0, or alpha or delta
 *    lies outside [0, 1] (k = 0).
 * Errors: LRC_ERR_ARG (NULL pointers, n_mats outside 1 .. 1024, n_alpha outside 1 .. 65535,
 *    negative budget).
 * ------------------------------------------------------------------------------------ */
lrc_status lrc_allocate_swift(int32_t n_mats, const double *beta, const double *eps_kbar, const int64_t *kbar,
                              const int64_t *cost, const int64_t *k_cap, double delta, int32_t n_alpha,
                              const double *alpha_grid, int64_t budget_params, double *scores, int32_t *k_out,
                              int32_t *info, void *stream);

/* ------------------------------------------------------------------------------------
 * Per-component empirical-Fisher importance (LASER page, method 2: each singular component is
 * scored by its contribution to the empirical-Fisher quadratic loss, from the component's
 * magnitude and its alignment with the calibration gradient).
 *
 *   score[b][i] = ((W v_i) . (G v_i))^2 = <G, W v_i v_i^T>^2,  i < k,
 *
 * the squared first-order loss change of removing component i (W v_i v_i^T) of the truncation
 * W_k = (W V_k) V_k^T (a reading: the page does not print the score).
 * W, G: d_in x d_out of dtype t (LRC_BF16 or LRC_F32; G the calibration gradient of W), leading
 *    dims ldw, ldg >= d_out.  V: d_out x (>= k) fp32 (lrc_eigh's V), leading dim ldv >= k.
 * Batched: matrix b uses W + b stride_w, G + b stride_g, V + b stride_v, score + b stride_s.
 * score: fp64.  Arithmetic: W V_k and G V_k in fp64 (inputs widened exactly, fp64 MFMA), the dot
 *    products in fp64 with a fixed-order reduction.
 * ws: lrc_component_fisher_workspace(d_in, k, batch) bytes, 256-byte aligned (fp64 partial dot
 *    products per 64-row tile).
 * Errors: LRC_ERR_ARG, LRC_ERR_DTYPE, LRC_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t lrc_component_fisher_workspace(int64_t d_in, int64_t k, int64_t batch);
lrc_status lrc_component_fisher(const void *W, const void *G, lrc_dtype t, int64_t d_in, int64_t d_out, int64_t ldw,
                                int64_t ldg, const float *V, int64_t ldv, int64_t k, int64_t batch, int64_t stride_w,
                                int64_t stride_g, int64_t stride_v, double *score, int64_t stride_s, void *ws,
                                size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------------------
 * Greedy selection of single components (LASER page, method 2: the components of highest
 * importance score per parameter cost are taken until the parameter budget is reached).
 *
 * score_packed: fp64 per-component scores, matrix m's K_m = offsets[m+1] - offsets[m] scores at
 *    offsets[m] in component order (e.g. lrc_component_fisher's output).  cost: n_mats int64 (> 0)
 *    parameters per component (d_in + d_out).  k_min: n_mats int32 or NULL: the first k_min[m]
 *    components of m are kept and charged first.
 * Candidates are the other components, priority p = score / cost_m (one IEEE fp64 division),
 *    ordered by p descending, then m ascending, then component ascending, taken while they fit in
 *    the budget; the first that does not fit ends the scan.  The kept components of a matrix need
 *    not be its leading ones.
 * k_out: n_mats int32 numbers of kept components; selected: n_items bytes (device) or NULL, 1 for
 *    a kept component.
 * info: one int32: 4 mandatory components exceed the budget (k = k_min), 5 a score negative or
 *    NaN, a cost <= 0 or a k_min outside [0, K_m].
 * ws: lrc_allocate_components_workspace(n_mats, n_items) bytes, 256-byte aligned.
 * Bit-exact: the result depends only on the fp64 priorities, computed as stated.
 * ------------------------------------------------------------------------------------ */
size_t lrc_allocate_components_workspace(int32_t n_mats, int64_t n_items);
lrc_status lrc_allocate_components(int32_t n_mats, const double *score_packed, const int64_t *offsets,
                                   int64_t n_items, const int64_t *cost, const int32_t *k_min, int64_t budget_params,
                                   int32_t *k_out, uint8_t *selected, void *ws, size_t ws_bytes, int32_t *info,
                                   void *stream);

/* ------------------------------------------------------------------------------------
 * Curvature-weighted variant (LASER page, method 1: the loss increase of a perturbation dW
 * is approximated by 1/2 vec(dW)^T (G (x) X) vec(dW) with X, G the activation and gradient
 * covariances; W is moved to W~ = S_x W S_g with Cholesky factors S_x, S_g, truncated there
 * by SVD, and the factors are mapped back).  With lower factors Sigma = L L^T the transform
 * is W~ = L_x^T W L_g, so ||L_x^T dW L_g||_F^2 = vec(dW)^T (Sigma_g (x) Sigma_x) vec(dW) for
 * Y = X W.  All matrices fp64, row-major, in place where stated.
 *
 * lrc_cholesky: A <- L, the lower Cholesky factor of the n x n SPD matrix A (lower triangle
 *   read; strict upper triangle set to 0).  info (one entry): 3 when a pivot is <= 0, 1 when
 *   a pivot is not finite (the first failure is kept; the factor is then not usable).
 * lrc_trmm: B <- op(L) B (side 0; B m x n, L m x m) or B <- B op(L) (side 1; L n x n), with
 *   op(L) = L (trans 0) or L^T (trans 1), L lower triangular (upper part not read).  Needs
 *   workspace of lrc_trmm_workspace(m, n) bytes (the product is formed out of place).
 * lrc_trsm: B <- op(L)^{-1} B (side 0) or B <- B op(L)^{-1} (side 1), same conventions, in
 *   place; workspace of lrc_trsm_workspace(side, m, n) bytes holds the inverted 64x64
 *   diagonal blocks of L and, when one 64-wide block of B spans at least 8192 columns
 *   (side 0) or rows (side 1), up to 8 partial products of a block update.  A zero or
 *   non-finite diagonal of L gives non-finite results.
 * lrc_sym_to_f64: A (n x n, both triangles) = scale * C, C fp32 with its upper triangle read
 *   (the layout lrc_cov_accumulate writes).
 * lrc_to_f64: Y (rows x cols) = scale * X, X of dtype t (LRC_BF16, LRC_F32 or LRC_F64).
 * lrc_gram_f64: G[upper] = B B^T for B m x n fp64, fp64 sums, G m x m fp32 (upper triangle
 *   incl. diagonal written, strict lower never touched) -- the Gram matrix of W~ whose
 *   eigendecomposition gives its left singular vectors and squared singular values.
 * ------------------------------------------------------------------------------------ */
size_t lrc_cholesky_workspace(int64_t n);
lrc_status lrc_cholesky(double *A, int64_t n, int64_t lda, void *ws, size_t ws_bytes, int32_t *info,
                        void *stream);
size_t lrc_trmm_workspace(int64_t m, int64_t n);
lrc_status lrc_trmm(int32_t side, int32_t trans, int64_t m, int64_t n, const double *L, int64_t ldl,
                    double *B, int64_t ldb, void *ws, size_t ws_bytes, void *stream);
size_t lrc_trsm_workspace(int32_t side, int64_t m, int64_t n);
lrc_status lrc_trsm(int32_t side, int32_t trans, int64_t m, int64_t n, const double *L, int64_t ldl,
                    double *B, int64_t ldb, void *ws, size_t ws_bytes, void *stream);
lrc_status lrc_sym_to_f64(const float *C, int64_t n, int64_t ldc, double scale, double *A, int64_t lda,
                          void *stream);
lrc_status lrc_to_f64(const void *X, lrc_dtype t, int64_t rows, int64_t cols, int64_t ldx, double scale,
                      double *Y, int64_t ldy, void *stream);
lrc_status lrc_gram_f64(const double *B, int64_t m, int64_t n, int64_t ldb, float *G, int64_t ldg,
                        void *stream);

/* ------------------------------------------------------------------------------------
 * Covariance from the input covariance (SAES-SVD page "SAES-SVD", section 1 of the method
 * (CEALC): the closed form works from a layer's input covariance H).  For Y = X W,
 * Y^T Y = W^T (X^T X) W, so one H = X^T X (lrc_cov_accumulate with W == NULL) serves every
 * matrix that reads the same X.
 *
 *   C[upper] = W^T H W
 *
 * H: d_in x d_in fp32, leading dim ldh >= d_in, upper triangle incl. diagonal read (the layout
 *    lrc_cov_accumulate writes).
 * W: d_in x d_out, leading dim ldw >= d_out, dtype w_t (LRC_BF16, LRC_F32 or LRC_F64).
 * C: d_out x d_out fp32, ldc >= d_out: the upper triangle incl. diagonal is overwritten (not
 *    accumulated), the strict lower triangle is never written.
 * Arithmetic: H and W widened exactly to fp64, T = H W and W^T T on fp64 MFMA with fp64 sums,
 *    rounded once to fp32.
 * ws: lrc_cov_from_input_workspace(d_in, d_out) bytes, 256-byte aligned (fp64 copies of H and
 *    W and the product T: 8 (d_in^2 + 2 d_in d_out) bytes); caller-owned, used on `stream`.
 * Errors: LRC_ERR_ARG (NULL pointers, sizes, leading dims), LRC_ERR_DTYPE, LRC_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t lrc_cov_from_input_workspace(int64_t d_in, int64_t d_out);
lrc_status lrc_cov_from_input(const float *H, int64_t d_in, int64_t ldh, const void *W, lrc_dtype w_t,
                              int64_t d_out, int64_t ldw, float *C, int64_t ldc, void *ws, size_t ws_bytes,
                              void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LRC_H */
