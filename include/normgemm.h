/*
 * libnormgemm -- normalization fused into bf16 GEMM on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every matrix is a dense row-major array of raw bfloat16 bit patterns
 * (uint16_t) in device memory; statistics are float32 in device memory.  All
 * device pointers are owned by the caller.  The library never allocates or
 * frees memory and never synchronizes on the compute calls: each call checks
 * its arguments on the host (before any HIP call), enqueues its kernel(s) on
 * `stream` (a hipStream_t; NULL means the null stream) and returns.  Device
 * faults surface at the caller's next synchronization, as in HIP.
 *
 * Common argument rules (violations return NG_ERR_INVALID_ARG unless noted):
 *   - M >= 0 (M == 0 is a no-op that returns NG_OK), N >= 1, K >= 1 and each
 *     at most 2^24;
 *   - N and K must be multiples of 8 (16-byte rows) -> else NG_ERR_UNSUPPORTED;
 *   - K at most 2^22 -> else NG_ERR_UNSUPPORTED (a tile reads up to 256 rows
 *     of A [M, K], or of B stored [N, K], through 32-bit offsets from one
 *     base, which must stay below 2 GiB); the weight-gradient products
 *     (ng_gemm_at, ng_rmsnorm_gemm_lazy_backward_weight), which read no rows
 *     of length K, take K up to 2^24;
 *   - no matrix with 2^34 or more elements -> else NG_ERR_UNSUPPORTED;
 *   - eps finite and >= 0;
 *   - every matrix pointer non-NULL (A and C, or X and Y, may be NULL when
 *     M, or rows, is 0) and 16-byte aligned; gamma/beta (when given) 16-byte
 *     aligned; the float32 statistic outputs 4-byte aligned;
 *   - b_layout is NG_B_KN (B stored [K, N], N contiguous) or NG_B_NK (B stored
 *     [N, K], K contiguous: a Linear layer's weight).
 * Outputs must not overlap inputs (the residual forms below name the
 * exceptions).
 *
 * Accuracy: bf16 inputs, fp32 accumulation and fp32 row statistics, outputs
 * rounded to bf16 (nearest, ties to even).  Against a float64 evaluation of
 * the plain definition every output element satisfies
 * |out - exact| <= 1e-2 * (1 + |exact|).
 */
#ifndef NORMGEMM_H
#define NORMGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t ng_bf16; /* raw bfloat16 bits */

/* Every entry point that returns a status returns one of these values. */
typedef enum {
  NG_OK = 0,
  NG_ERR_INVALID_ARG = 1, /* NULL/misaligned pointer, bad size, bad eps or enum */
  NG_ERR_UNSUPPORTED = 2, /* a valid request the library does not tile (see the limits) */
  NG_ERR_WORKSPACE = 3,   /* workspace NULL, too small or misaligned */
  NG_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  NG_ERR_TIMEOUT = 5      /* a cross-workgroup wait gave up (reported by ng_workspace_status) */
} ng_status;

enum { NG_NORM_RMS = 0, NG_NORM_LAYER = 1 };
enum { NG_B_KN = 0, NG_B_NK = 1 };
enum {
  NG_OP_RMSNORM_GEMM_LAZY = 0,
  NG_OP_GEMM_RMSNORM = 1,
  NG_OP_GEMM_LAYERNORM = 2,
  NG_OP_GEMM = 3,
  NG_OP_NORM = 4,
  NG_OP_GEMM_ADD_RMSNORM = 5,
  NG_OP_GEMM_ADD_LAYERNORM = 6,
  NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT = 7
};

/*
 * Lazy Pre-Norm: C = rmsnorm(A) @ B for RMSNorm without affine parameters.
 * ("Free normalization fusion", aixai.ru, section "Lazy Pre-Norm": the
 * per-row scale rstd commutes with the product, so C = (A @ B) * rstd(A); the
 * sum of squares of each row of A accumulates inside the GEMM k-loop and the
 * scaling runs in the epilogue.)
 *   rstd[m] = 1 / sqrt((1/K) * sum_k A[m,k]^2 + eps)
 *   C[m,n]  = rstd[m] * sum_k A[m,k] * B[k,n]
 * A: [M, K]; B: see b_layout; C: [M, N] bf16 out.
 * rstd_out: float32 [M] or NULL.  Needs no workspace.
 */
ng_status ng_rmsnorm_gemm_lazy(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N,
                               int64_t K, int b_layout, float eps, float* rstd_out, void* stream);

/*
 * Lazy Pre-Norm with a per-column affine on the normalized A (gamma, beta of
 * length K):  C = (rmsnorm(A) * gamma + beta) @ B.
 * ("Free normalization fusion", section "Lazy Pre-Norm": the affine scales
 * columns of A, so the row-scale identity does not cover it directly; "RMSNorm
 * fusion on Ascend", section 6.4: at inference gamma is fixed and can be
 * merged into the next matmul's weights ahead of time.)  Two steps:
 *
 * ng_lazy_fold_affine, once per weight: B_folded = diag(gamma) B (row k of B,
 * as [K, N], scaled by gamma[k], rounded to bf16) in B's layout, and
 * bias[n] = sum_k beta[k] B[k,n] in fp32.  gamma NULL means 1; beta NULL means
 * 0 (bias is then all zero); bias NULL skips it.  B_folded may equal B (the
 * bias is computed from B first, on the same stream).  B, B_folded, gamma,
 * beta 16-byte aligned; bias 4-byte aligned.  K and N multiples of 8.
 *
 * ng_rmsnorm_gemm_lazy_affine, per call: C = rstd(A) * (A @ B_folded) + bias,
 * which equals the definition above (rstd from the row of A as in
 * ng_rmsnorm_gemm_lazy).  bias: fp32 [N], 16-byte aligned, or NULL (no bias).
 * rstd_out: float32 [M] or NULL.  Needs no workspace.
 */
ng_status ng_lazy_fold_affine(const ng_bf16* B, const ng_bf16* gamma, const ng_bf16* beta,
                              ng_bf16* B_folded, float* bias, int64_t K, int64_t N, int b_layout,
                              void* stream);

ng_status ng_rmsnorm_gemm_lazy_affine(const ng_bf16* A, const ng_bf16* B_folded, const float* bias,
                                      ng_bf16* C, int64_t M, int64_t N, int64_t K, int b_layout,
                                      float eps, float* rstd_out, void* stream);

/*
 * Input gradient of Lazy Pre-Norm (C = rmsnorm(A) @ B, RMSNorm without
 * affine) for an upstream gradient dC, with the norm's backward fused into
 * the epilogue of dA_hat = dC @ B^T ("Free normalization fusion", section
 * "Lazy Pre-Norm": backward rebuilds the normalized A from A and the saved
 * rstd, and the norm's backward fuses into a different matmul than in the
 * forward pass):
 *   dA_hat = dC @ B^T;  s[m] = sum_k dA_hat[m,k] * A[m,k];
 *   dA[m,k] = rstd[m] * dA_hat[m,k] - rstd[m]^3 * s[m] / K * A[m,k]
 * (= rstd * (dA_hat - A_hat * mean_k(dA_hat * A_hat)) with A_hat = rstd * A).
 * M, N, K and b_layout are the forward product's: dC [M, N], B as in the
 * forward call, A [M, K] the forward input, rstd float32 [M] the forward's
 * rstd_out, dA [M, K] bf16 output.  Rows with K <= 256 are reduced inside a
 * workgroup; longer rows exchange per-row partial sums through `workspace`
 * (ng_workspace_bytes(NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, M, N, K) bytes; the
 * same rules as for ng_gemm_rmsnorm).  dA must not overlap the inputs.
 */
ng_status ng_rmsnorm_gemm_lazy_backward_input(const ng_bf16* dC, const ng_bf16* B, const ng_bf16* A,
                                              const float* rstd, ng_bf16* dA, int64_t M, int64_t N,
                                              int64_t K, int b_layout, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * Pre-LayerNorm fused with the following product: C = LayerNorm(A) @ B with
 * the norm over each row of A (H = K; "RMSNorm fusion on Ascend", section 1.1)
 * and per-column gamma/beta of length K.  Two stages ("RMSNorm fusion on
 * Ascend", section 2.2: row statistics first, then the product of the
 * normalized tiles): a pre-pass writes mean[m] and rstd[m] of every row of A,
 * then the product applies the norm through its linearity,
 *   C = rstd * (A @ B' - mean * colsum) + bias,
 * so A is read as stored and never rewritten.  ("Free normalization fusion",
 * section "Lazy Pre-Norm", notes that the plain row-scale form does not cover
 * LayerNorm; the mean term above is what it lacks.)
 *
 * ng_layernorm_gemm_fold (one-off weight transform): B_folded = bf16(diag(gamma)
 * B) in B's layout (may be B itself), colsum[n] = sum_k B_folded[k][n] (fp32,
 * over the rounded folded weights), bias[n] = sum_k beta[k] B[k][n] (fp32).
 * gamma, beta: bf16 [K] or NULL (1 and 0); colsum required; bias may be NULL
 * only when beta is NULL.  colsum/bias 16-byte aligned.
 *
 * ng_layernorm_gemm_prenorm: A [M, K] bf16, B_folded/colsum/bias from the
 * fold (bias may be NULL), C [M, N] bf16; mean, rstd: float32 [M] outputs,
 * required (the pre-pass writes them, the product reads them).  K at most
 * 65536 (else NG_ERR_UNSUPPORTED).  Needs no workspace.
 */
ng_status ng_layernorm_gemm_fold(const ng_bf16* B, const ng_bf16* gamma, const ng_bf16* beta,
                                 ng_bf16* B_folded, float* colsum, float* bias, int64_t K,
                                 int64_t N, int b_layout, void* stream);

ng_status ng_layernorm_gemm_prenorm(const ng_bf16* A, const ng_bf16* B_folded, const float* colsum,
                                    const float* bias, ng_bf16* C, int64_t M, int64_t N, int64_t K,
                                    int b_layout, float eps, float* mean, float* rstd,
                                    void* stream);

/*
 * GEMM with an RMSNorm epilogue over each full output row (H = N):
 *   X = A @ B;  rstd[m] = 1 / sqrt((1/N) sum_n X[m,n]^2 + eps);
 *   C[m,n] = X[m,n] * rstd[m] * gamma[n]        (gamma NULL means 1)
 * ("RMSNorm fusion on Ascend", gsyq.cn, section 1.2 for the norm; "Free
 * normalization fusion", section "Multi-CTA Norm Fusion" for reducing a row
 * that several workgroups share, then applying.)  Rows with N <= 256 are
 * normalized inside one workgroup; wider rows merge per-row fp32 partials
 * across workgroups through `workspace`, which must hold
 * ng_workspace_bytes(NG_OP_GEMM_RMSNORM, M, N, K) bytes (0 means none needed;
 * at most ~6.3 MB: it holds one round of row blocks and stops growing with M),
 * be 256-byte aligned and be zero-filled before its first use (see
 * ng_workspace_reset); calls leave it ready for the next call.  One workspace
 * must not be used by two calls that may run concurrently.  Wide rows run a
 * grid of at most as many workgroups as the device holds at once, whose
 * workgroups wait for each other: two such calls must not run concurrently
 * on one device (e.g. on two streams).  If they do, a wait may give up after
 * about a second (2^20 polls of ~1 us; see ng_set_debug_option);
 * ng_workspace_status then reports NG_ERR_TIMEOUT, and every output element
 * and statistic of a row whose exchange failed is NaN.  A row may span at
 * most as many 256-column tiles as the device holds such workgroups at once
 * (N <= 65536 on a 256-CU device); wider rows return NG_ERR_UNSUPPORTED.
 * gamma: bf16 [N] or NULL.  rstd_out: float32 [M] or NULL.
 */
ng_status ng_gemm_rmsnorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma, ng_bf16* C,
                          int64_t M, int64_t N, int64_t K, int b_layout, float eps, float* rstd_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * GEMM with a LayerNorm epilogue over each full output row (H = N):
 *   X = A @ B;  mean[m] = (1/N) sum_n X[m,n];
 *   var[m] = (1/N) sum_n (X[m,n] - mean[m])^2   (biased);
 *   rstd[m] = 1 / sqrt(var[m] + eps);
 *   C[m,n] = (X[m,n] - mean[m]) * rstd[m] * gamma[n] + beta[n]
 * (gamma NULL means 1, beta NULL means 0).  ("RMSNorm fusion on Ascend",
 * section 1.1; "Free normalization fusion", section "Multi-CTA Norm Fusion".)
 * Workspace rules as for ng_gemm_rmsnorm with NG_OP_GEMM_LAYERNORM.
 * mean_out, rstd_out: float32 [M] or NULL.
 */
ng_status ng_gemm_layernorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma,
                            const ng_bf16* beta, ng_bf16* C, int64_t M, int64_t N, int64_t K,
                            int b_layout, float eps, float* mean_out, float* rstd_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ng_gemm_layernorm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation, arguments and results, with no workspace
 * argument.  Rows wider than one workgroup tile exchange their statistics
 * through a scratch array of NG_NOALLOC_SCRATCH_BYTES (16 MiB) that the
 * library keeps in static device memory, one per device, until the process
 * ends.  The call allocates nothing.  The array holds the exchange of every
 * shape the other entry points accept (ng_workspace_bytes(
 * NG_OP_GEMM_LAYERNORM, M, N, K) <= 16 MiB for any M); a shape that would
 * need more returns NG_ERR_UNSUPPORTED.  The first
 * call on a device takes the array's address there and, unless the stream is
 * being captured, zero-fills it on `stream`.  Every call on one device shares
 * that device's array: calls that may overlap on one device (e.g. on two
 * streams without an ordering) race and must not be made; calls on one
 * stream are ordered and fine.  A wait that gives up leaves NaN in the rows
 * it affects (no status word is exposed for this variant).
 */
#define NG_NOALLOC_SCRATCH_BYTES (16u << 20)
ng_status ng_gemm_layernorm_noalloc(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma,
                                    const ng_bf16* beta, ng_bf16* C, int64_t M, int64_t N,
                                    int64_t K, int b_layout, float eps, float* mean_out,
                                    float* rstd_out, void* stream);

/*
 * Residual connection followed by a post-norm ("Free normalization fusion",
 * section "FlashNormAttention": residual add, then the post-norm, the residual
 * added to the product's accumulator; norm formulas as above):
 *   S = A @ B + R          (fp32: the product's accumulators plus R)
 *   C = RMSNorm(S) * gamma                     (ng_gemm_add_rmsnorm)
 *   C = LayerNorm(S) * gamma + beta            (ng_gemm_add_layernorm)
 *   S_out = bf16(S)        (when S_out is non-NULL: the new residual stream)
 * with the statistics taken over each full row of S (H = N in the formulas
 * above).  R: [M, N] bf16, required; S_out: [M, N] bf16 or NULL.  R may be
 * the very buffer of C or of S_out (an in-place update: every element of R
 * is read before the same element of C or S_out is written); S_out and C
 * must differ, and no other overlap is allowed.  mean_out/rstd_out describe
 * S.  Strategies and workspace rules as for ng_gemm_rmsnorm /
 * ng_gemm_layernorm, with
 * ng_workspace_bytes(NG_OP_GEMM_ADD_RMSNORM / NG_OP_GEMM_ADD_LAYERNORM, ...).
 */
ng_status ng_gemm_add_rmsnorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* R,
                              const ng_bf16* gamma, ng_bf16* C, ng_bf16* S_out, int64_t M,
                              int64_t N, int64_t K, int b_layout, float eps, float* rstd_out,
                              void* workspace, size_t workspace_bytes, void* stream);

ng_status ng_gemm_add_layernorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* R,
                                const ng_bf16* gamma, const ng_bf16* beta, ng_bf16* C,
                                ng_bf16* S_out, int64_t M, int64_t N, int64_t K, int b_layout,
                                float eps, float* mean_out, float* rstd_out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Plain GEMM, the matrix half of the unfused baseline that the fused forms
 * are measured against ("Free normalization fusion", section "why
 * normalization is a performance problem": a GEMM tiles both dimensions, so
 * no tile sees a whole row and the norm, a reduction over the row, runs as a
 * kernel of its own without the matrix units):  C = A @ B (bf16 out, fp32
 * accumulation).  A: [M, K]; B: see b_layout; C: [M, N] bf16 out.
 */
ng_status ng_gemm(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N, int64_t K,
                  int b_layout, void* stream);

/*
 * Standalone row norm, the other half of the unfused baseline.  X, Y: [rows,
 * cols] bf16 (Y may equal X for an in-place norm).  kind NG_NORM_RMS or
 * NG_NORM_LAYER with the formulas above (H = cols); for RMS a beta, when
 * given, is added after gamma (y = x * rstd * gamma + beta, the unfused form
 * of a pre-norm with a full affine).  cols must be a multiple of 8 and at
 * most 65536 (else NG_ERR_UNSUPPORTED).  mean_out (LayerNorm only) and
 * rstd_out: float32 [rows] or NULL.
 */
ng_status ng_norm(const ng_bf16* X, const ng_bf16* gamma, const ng_bf16* beta, ng_bf16* Y,
                  int64_t rows, int64_t cols, int kind, float eps, float* mean_out, float* rstd_out,
                  void* stream);

/*
 * Standalone residual add and row norm, the norm half of the unfused
 * baseline of the residual forms: S = X + R, rounded to bf16 as it is formed
 * (the residual stream's storage type); Y = norm(S) with kind, gamma, beta,
 * eps and the statistic outputs as for ng_norm; S_out (bf16 [rows, cols] or
 * NULL) receives S.  R: [rows, cols] bf16, required.  Y may equal X, and S_out
 * may equal X or R (in-place updates: each element is read before the same
 * element is written); S_out and Y must differ.  Limits as for ng_norm.
 */
ng_status ng_add_norm(const ng_bf16* X, const ng_bf16* R, const ng_bf16* gamma, const ng_bf16* beta,
                      ng_bf16* Y, ng_bf16* S_out, int64_t rows, int64_t cols, int kind, float eps,
                      float* mean_out, float* rstd_out, void* stream);

/*
 * Weight gradient of Lazy Pre-Norm: dB = A_hat^T @ dC with A_hat = rstd * A
 * rebuilt on the fly from A and the forward's saved rstd ("Free
 * normalization fusion", section "Lazy Pre-Norm": the normalized A is never
 * stored, so backward rebuilds it).  The product runs over the forward rows:
 * each k-tile of A is read on chip, its elements scaled by their row's rstd
 * and rounded to bf16 (the rounding of a stored A_hat), then multiplied.
 * M, N, K and b_layout are the forward product's: A [M, K], dC [M, N], rstd
 * float32 [M]; dB is written in B's layout ([K, N] for NG_B_KN, [N, K] for
 * NG_B_NK), bf16.  M may be any size (M == 0 writes zeros).  dB must not
 * overlap the inputs.
 */
ng_status ng_rmsnorm_gemm_lazy_backward_weight(const ng_bf16* A, const ng_bf16* dC,
                                               const float* rstd, ng_bf16* dB, int64_t M, int64_t N,
                                               int64_t K, int b_layout, void* stream);

/*
 * Both gradients of Lazy Pre-Norm (C = rmsnorm(A) @ B, RMSNorm without
 * affine), with the weight gradient regrouped ("Towards Free Normalization"
 * summary page, its abstract: backward passes get epilogue fusion by fusing
 * the norm with a different matmul than in the forward pass).  Since
 * dB = A_hat^T @ dC = A^T @ (rstd * dC), the row scale moves from the forward
 * input onto the upstream gradient: the input-gradient kernel (as in
 * ng_rmsnorm_gemm_lazy_backward_input, same arguments, workspace and rules)
 * also writes dC_scaled = rstd * dC, rounded to bf16, while it runs, and dB
 * is then the plain product over the forward rows (as ng_gemm_at):
 *   dA as in ng_rmsnorm_gemm_lazy_backward_input;
 *   dC_scaled[m, n] = bf16(rstd[m] * dC[m, n])        (bf16 [M, N], written);
 *   dB = A^T @ dC_scaled                               (bf16, B's layout).
 * dB is written in B's layout ([K, N] for NG_B_KN, [N, K] for NG_B_NK);
 * M == 0 writes dB = 0.  dC_scaled is caller-owned scratch of M * N * 2
 * bytes that must not overlap any other argument (NG_ERR_INVALID_ARG); dA
 * and dB must not overlap the inputs.  Against
 * ng_rmsnorm_gemm_lazy_backward_weight, which keeps no intermediate, this
 * trades M * N * 2 bytes of scratch for a weight gradient at the speed of the
 * plain product.
 */
ng_status ng_rmsnorm_gemm_lazy_backward(const ng_bf16* dC, const ng_bf16* B, const ng_bf16* A,
                                        const float* rstd, ng_bf16* dA, ng_bf16* dB,
                                        ng_bf16* dC_scaled, int64_t M, int64_t N, int64_t K,
                                        int b_layout, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Plain GEMM with the first operand stored transposed, the product half of
 * the weight gradient's unfused baseline: C [M, N] = A^T @ B with A stored
 * [K, M] and B stored [K, N] (the reduction runs over both matrices' rows),
 * bf16 out, fp32 accumulation.  M and N multiples of 8 (else
 * NG_ERR_UNSUPPORTED); K any size >= 1.
 */
ng_status ng_gemm_at(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N,
                     int64_t K, void* stream);

/*
 * Standalone RMSNorm backward (no affine), the norm half of the unfused
 * baseline of ng_rmsnorm_gemm_lazy_backward_input: for each row x of X
 * [rows, cols] with saved rstd (float32 [rows]) and upstream gradient dY,
 *   dX = rstd * dY - rstd^3 * (sum_k dY_k x_k) / cols * x
 * (the chain rule of y = x * rstd).  bf16 in and out; cols a multiple of 8
 * and at most 65536 (else NG_ERR_UNSUPPORTED).  dX may equal dY.
 */
ng_status ng_rmsnorm_backward(const ng_bf16* dY, const ng_bf16* X, const float* rstd, ng_bf16* dX,
                              int64_t rows, int64_t cols, void* stream);

/* Workspace bytes `op` needs for this shape (0 when it needs none). */
size_t ng_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* Zero-fill a workspace on `stream` with a fill kernel (graph-capture safe). */
ng_status ng_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronizes `stream`, then reads the workspace's error word: NG_OK, or
 * NG_ERR_TIMEOUT if a cross-workgroup wait in an earlier call gave up (its
 * output is then undefined and the workspace must be reset).
 */
ng_status ng_workspace_status(const void* workspace, void* stream);

/* Static description of a status code. */
const char* ng_status_string(ng_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char* ng_last_error(void);

/*
 * Diagnostics, process-wide, for tests and experiments (no effect on results
 * unless stated):
 *   NG_DEBUG_WAIT_SPINS     bound of each cross-workgroup wait, in polls of
 *                           ~1 us: 0 .. 2^30, or -1 for the default 2^20.
 *                           A bound of 0 makes every wait that does not find
 *                           its entry at once give up (NG_ERR_TIMEOUT, NaN
 *                           output), with no wave left waiting.
 *   NG_DEBUG_ROW_LOCAL_MAX  widest row reduced inside one workgroup: 0 .. 256,
 *                           or -1 for the default 256.  Lower values send
 *                           narrow rows through the cross-workgroup exchange
 *                           (so both strategies can be compared on one
 *                           shape); ng_workspace_bytes follows it.
 *   NG_DEBUG_TILE_ORDER     order in which the grids take their output tiles:
 *                           NG_TILE_ORDER_NATURAL (default), _REVERSED or
 *                           _SHUFFLED (a fixed permutation).  Outputs are
 *                           bit-identical in every order.
 *   NG_DEBUG_K_WALK         k-tile walk of the persistent grids of ng_gemm
 *                           and of the cross-workgroup RMSNorm/LayerNorm
 *                           epilogues (without residual): NG_K_WALK_AUTO
 *                           (default: every second round of tiles walks K
 *                           downwards when one round's operands and output
 *                           exceed 192 MiB), _UPWARD (always upwards) or
 *                           _ALTERNATE (every second round downwards whenever
 *                           there is more than one round).  The fp32 sums
 *                           over K then run in another order: outputs agree
 *                           within rounding, not bit for bit.
 * Returns NG_ERR_INVALID_ARG for an unknown option or value.  Calls already
 * enqueued keep the values they were launched with.
 */
enum {
  NG_DEBUG_WAIT_SPINS = 0,
  NG_DEBUG_ROW_LOCAL_MAX = 1,
  NG_DEBUG_TILE_ORDER = 2,
  NG_DEBUG_K_WALK = 3
};
enum { NG_TILE_ORDER_NATURAL = 0, NG_TILE_ORDER_REVERSED = 1, NG_TILE_ORDER_SHUFFLED = 2 };
enum { NG_K_WALK_AUTO = 0, NG_K_WALK_UPWARD = 1, NG_K_WALK_ALTERNATE = 2 };
ng_status ng_set_debug_option(int option, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* NORMGEMM_H */
