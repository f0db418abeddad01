/*
 * ptq.h — C ABI of libptq.so: GPTQ / AWQ layer quantization on MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  [OBJ]  "GPTQ versus AWQ objectives" (inferenceinterviews.com):
 *         "A strong answer" (objective ||X W^T - X What^T||^2, proxy Hessian
 *         X^T X, 1% mean-diagonal damping, upper Cholesky factor of H^-1, the
 *         column loop, lazy batching over column blocks, Hessian sizing, AWQ's
 *         s_j = mean|x_j|^alpha with a per-layer grid search over alpha);
 *         "What interviewers probe next" (act-order, group index per column,
 *         damping).
 *  [PTQ]  "A Comprehensive Analysis of Post-Training Quantization Strategies
 *         for Large Language Models: GPTQ, AWQ and GGUF" (uplatz.com),
 *         sections 2.1-2.2 (layer-wise objective, group size, act-order) and
 *         3.2 (AWQ's equivalent per-channel scaling).
 *
 * Conventions shared by every entry point:
 *  - W is [out, in] row-major with row stride ldw (elements); X is [rows, in]
 *    row-major with row stride ldx; H and U are [in, in] row-major, dense.
 *  - Every array argument is a DEVICE pointer owned by the caller, unless
 *    marked "host". The library allocates nothing: scratch memory comes from
 *    the caller's workspace, whose size the matching *_workspace_bytes query
 *    returns (256-byte aligned; NULL with size 0 is allowed where the query
 *    returns 0).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    Entry points that return host values (stats, alpha) synchronise that
 *    stream before returning; the others are asynchronous.
 *  - Arguments are validated before any HIP call; a bad argument returns
 *    PTQ_EINVAL and touches no memory. ptq_last_error() then holds a
 *    thread-local message naming the argument.
 *  - Device pointers must be 16-byte aligned; ldw/ldx must keep every row
 *    16-byte aligned.
 *  - Integer codes are unpacked int8 in [-qmax-1, qmax], qmax = 2^(bits-1)-1.
 *    Scales are fp32, one per (row, group); group k is the k-th run of g
 *    columns in processing order, so scales[r][g_idx[c]] dequantizes column c.
 */
#ifndef PTQ_H
#define PTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    PTQ_OK = 0,
    PTQ_EINVAL = 1,       /* bad argument (nothing was launched)                  */
    PTQ_ENOTPD = 2,       /* H + lambda I is not positive definite (a pivot <= 0) */
    PTQ_ENONFINITE = 3,   /* NaN/Inf met in the inputs or a derived quantity       */
    PTQ_EWORKSPACE = 4,   /* workspace NULL or smaller than the query's answer     */
    PTQ_EHIP = 5          /* a HIP runtime call failed                             */
};

/* Element types of W and X. */
enum { PTQ_BF16 = 0, PTQ_F32 = 1 };

/* Thread-local message for the last non-OK status of this thread. */
const char* ptq_last_error(void);
/* Static name of a status code. */
const char* ptq_status_string(int status);
/* ABI version (incremented on any signature change). */
int ptq_abi_version(void);

/* ------------------------------------------------------------------------
 * Kernel timing. With bit k of kernel_mask set, every later launch of kernel
 * class k is bracketed by two hipEvents recorded on its launch stream:
 *   0 X^T X bf16 MFMA tiles        1 fp32 GEMMs of the U recursion
 *   2 diagonal-block factor/inverse 3 GPTQ in-block column loop
 *   4 GPTQ trailing GEMM            5 AWQ error GEMM
 *   6 GPTQ fp32 update inside a super-block of columns
 *   7 fp32 GEMMs run as bf16 MFMAs on three-term bf16 splits (the large
 *     ones inside 1 and 4; main loop only)
 * Enabling (any mask, 0 included) discards earlier records. ptq_profile_read
 * waits for the recorded events of class `kernel` and returns the sum of
 * their elapsed times (ms) and the number of launches. ptq_profile_flops
 * returns the MFMA flops those launches execute, counted on the host at
 * launch time over whole output tiles (edge padding, diagonal tiles and, for
 * the split-operand GEMMs, all six bf16 term products included; 0 for the
 * classes that are not counted: 1, 2, 3, 4 and 6 as wrappers or fp32 work).
 * Process-wide; calls that overlap from several threads share the records.
 * Errors: EINVAL (kernel out of range, NULL output), EHIP (profile_read).
 * ---------------------------------------------------------------------- */
int ptq_profile_enable(unsigned kernel_mask);
int ptq_profile_read(int kernel, double* total_ms, int64_t* launches);
int ptq_profile_flops(int kernel, double* mfma_flops);

/* ------------------------------------------------------------------------
 * Stage 1 — proxy Hessian.  [OBJ] "A strong answer": H = X^T X over the
 * calibration inputs (the page's 2 X^T X differs by a constant that the
 * relative damping makes irrelevant).
 *
 * H[in, in] fp32 (+)= X^T X, accumulated on MFMA from bf16 (or fp32) X with
 * fp32 accumulation; the result is written as a full symmetric matrix
 * (H[i][j] and H[j][i] receive the same value). d[in] fp64 (+)= column sums
 * of squares sum_i x_ij^2 (the act-order key and the damping base), which may
 * be NULL. The call is additive: zero H and d before the first chunk, then
 * call once per chunk of calibration rows (large chunks are faster: each call
 * re-reads and re-writes H once). rows may be 0 (no-op).
 * Workspace: hessian_workspace_bytes(in, rows) bytes: bf16 X needs it (a
 * transposed copy of up to 65536 rows, split-K partial sums for small `in`,
 * partial sums of squares); fp32 X runs with none (NULL, 0).
 * Errors: EINVAL (in < 1, rows < 0, ldx < in, bad dtype, NULL H or X with
 * rows > 0, misalignment), EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t hessian_workspace_bytes(int64_t in, int64_t rows);
int hessian_accumulate(float* H, double* d, int64_t in,
                       const void* X, int x_dtype, int64_t rows, int64_t ldx,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hessian_accumulate without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight calibration or serving
 * loops, harnesses that forbid hipMalloc.
 *
 * Same arguments (minus the workspace) and the same results as
 * hessian_accumulate, up to the order of the fp32 sums across row chunks.
 * The scratch (the transposed copy of a chunk of bf16 rows and that chunk's
 * fp64 column sums) is a fixed array of PTQ_NOALLOC_SCRATCH_BYTES of device
 * memory that the library holds on every GPU it runs on until the process
 * ends; rows go in chunks that fit it, without splitting a launch over depth,
 * so a large `in` runs slower than with a workspace (about 1100 rows a chunk
 * at in = 28672). fp32 X needs no scratch. The call allocates nothing
 * (no hipMalloc, no library allocation). Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams or two threads)
 * race and must be serialized by the caller. Asynchronous on `stream`.
 * Errors: as hessian_accumulate, plus EINVAL when a 64-row chunk does not fit
 * the scratch (bf16 X with in > 253952).
 * ---------------------------------------------------------------------- */
#define PTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int hessian_accumulate_noalloc(float* H, double* d, int64_t in, const void* X, int x_dtype, int64_t rows,
                               int64_t ldx, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2 — damping, act-order and the upper factor of the inverse.
 * [OBJ] "A strong answer": H += damp * mean(diag H) * I; U upper triangular
 * with U^T U = H^-1. [OBJ] "What interviewers probe next": act-order
 * processes columns in decreasing Hessian diagonal.
 *
 * lambda = damp * mean(d) (d from hessian_accumulate; NULL: diag(H) in fp32
 * is used instead). With act_order, perm = stable sort of columns by
 * decreasing d (ties: lower index first); otherwise perm = identity.
 * U[in, in] (output, dense; strictly lower part set to 0) is the upper factor
 * of (P (H + lambda I) P^T)^-1 in the PROCESSING basis, computed as H = R R^T
 * (R upper, reversed-order Cholesky) and U = R^-1. perm (int32[in], may be
 * NULL when act_order == 0) receives perm[k] = original column processed
 * k-th. lambda_out (host, may be NULL). Synchronous (reads the pivot flag).
 * Errors: EINVAL (damp < 0 or not finite, in < 1), ENOTPD, ENONFINITE,
 * EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t gptq_factor_workspace_bytes(int64_t in);
int gptq_inverse_factor(const float* H, const double* d, int64_t in, double damp, int act_order,
                        float* U, int32_t* perm, double* lambda_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3 — the column loop in lazy blocks.  [OBJ] "A strong answer": per
 * group start j (j % g == 0, processing order) scale = max |W_cur| over the
 * group's columns / qmax, from the error-updated weights; code =
 * clip(round_half_even(w / scale), -qmax-1, qmax) (scale 0 gives code 0);
 * err = (w - code*scale) / U_jj is subtracted from the later columns through
 * row j of U. Updates are batched over blocks of `block_size` columns (the
 * page's lazy batch) and again over 2048-column super-blocks: in-block
 * updates in registers, then W_cur[:, b1:s1] -= E U[b0:b1, b1:s1] for the
 * rest of the block's super-block [s0, s1) (fp32 MFMA), and after each
 * super-block one GEMM W_cur[:, s1:] -= E U[s0:s1, s1:] with K = s1 - s0
 * (bf16 MFMAs on three-term bf16 splits of E and U at fp32 accuracy when
 * large, else fp32 MFMA); the arithmetic is the same up to the order of the
 * fp32 sums.
 *
 * W (not modified) in ORIGINAL column order; U from gptq_inverse_factor (in
 * the processing basis); perm as returned there (NULL = identity).
 * Outputs: codes int8[out, in] in ORIGINAL column order (row stride in);
 * scales fp32[out, ceil(in/g)] (row stride ceil(in/g)); g_idx int32[in]
 * (g_idx[c] = position of column c in processing order / g; may be NULL).
 * stats (host, may be NULL) double[4]: [0] sum of err^2 (= tr(dW H dW^T) for
 * the damped H), [1] untouched, [2] ||W - What||_F^2, [3] untouched.
 * Requires block_size % g == 0 or g % block_size == 0; block_size in
 * {32, 64, 128}; bits in [2, 8]; g >= 1. Synchronous when stats != NULL.
 * Errors: EINVAL, ENONFINITE (a non-finite error term), EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t gptq_columns_workspace_bytes(int64_t out, int64_t in, int block_size);
int gptq_quantize_columns(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                          const float* U, const int32_t* perm,
                          int bits, int group_size, int block_size,
                          int8_t* codes, float* scales, int32_t* g_idx, double* stats,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stages 2 + 3 in one call: gptq_inverse_factor then gptq_quantize_columns.
 * H is the UNDAMPED X^T X from hessian_accumulate (not modified), d its fp64
 * column sums of squares (may be NULL). perm may be NULL when act_order == 0.
 * stats (host, may be NULL) double[4]: [0] sum err^2, [1] lambda,
 * [2] ||dW||_F^2, [3] calibration objective ||X dW^T||^2 =
 * stats[0] - lambda * stats[2] (for any rounding, sum err^2 = tr(dW (H0 +
 * lambda I) dW^T), so the undamped objective follows by subtraction).
 * Synchronous. Errors: union of the two stages.
 * ---------------------------------------------------------------------- */
size_t gptq_workspace_bytes(int64_t out, int64_t in, int block_size);
int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                        const float* H, const double* d,
                        int bits, int group_size, double damp, int act_order, int block_size,
                        int8_t* codes, float* scales, int32_t* g_idx, int32_t* perm, double* stats,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stages 2 + 3 with zero-point groups.  [PTQ] 2.2: each group has its own
 * quantization parameters, a scale and a zero-point; [PTQ] 2: GPTQ also
 * serves 3- and 2-bit. The loop is gptq_quantize_layer's; only the grid
 * differs: per (row, group), at the group's first column, lo = min(0, min w)
 * and hi = max(0, max w) over the group's current weights, scale =
 * (hi - lo) / maxq with maxq = 2^bits - 1, zero = round(-lo / scale) and
 * code = clip(round(w / scale) + zero, 0, maxq) (round half to even; a group
 * of zeros gets scale 0, zero 0, code 0). What = (code - zero) * scale.
 *
 * bits in [2, 7]; codes int8[out, in] in [0, maxq] (original column order);
 * scales fp32 and zeros int8 [out, ceil(in / g)] (processing-order groups);
 * other arguments, the workspace (gptq_workspace_bytes) and stats as for
 * gptq_quantize_layer. Synchronous.
 * Errors: EINVAL, ENOTPD, ENONFINITE, EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
int gptq_quantize_layer_zp(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                           const float* H, const double* d,
                           int bits, int group_size, double damp, int act_order, int block_size,
                           int8_t* codes, float* scales, int8_t* zeros, int32_t* g_idx, int32_t* perm,
                           double* stats, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 4 — AWQ's per-layer alpha grid search.  [OBJ] "A strong answer",
 * AWQ: s_j = mean|x_j|^alpha; scale W's column j by s_j, round to nearest
 * (symmetric groups of g), and pick the alpha with the least calibration
 * output error ||X (W - What)^T||^2, What = Q(W diag s) diag(s)^-1.
 * [PTQ] 3.2: the scaled weights are quantized uniformly; 1/s is folded into
 * the previous operator by the caller.
 *
 * mean|x_j| is floored at 1e-12 * max_j mean|x_j|. alphas (host, n_alpha
 * values, n_alpha in [1, 64]). Outputs: alpha_best (host), err_per_alpha
 * (host, n_alpha doubles, may be NULL), s fp32[in] at alpha_best (device),
 * codes int8[out, in] and scales fp32[out, ceil(in/g)] of W diag(s) (device).
 * Ties go to the first alpha of the grid. Synchronous.
 * Errors: EINVAL, EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t awq_workspace_bytes(int64_t out, int64_t in, int64_t rows, int n_alpha);
int awq_search_alpha(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                     const void* X, int x_dtype, int64_t rows, int64_t ldx,
                     const float* alphas, int n_alpha, int bits, int group_size,
                     float* alpha_best, double* err_per_alpha, float* s,
                     int8_t* codes, float* scales,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * AWQ's scaling first, GPTQ's rounding after.  [OBJ] "A strong answer" (the
 * decision list: for 3-bit or aggressive targets the two compose).
 *
 * s fp32[in] (device, positive and finite; e.g. awq_search_alpha's output)
 * defines W' = W diag(s) and X' = X diag(s)^-1, which leave the layer output
 * unchanged. GPTQ then runs on the scaled layer exactly as
 * gptq_quantize_layer does on a layer: H0' = diag(s)^-1 H diag(s)^-1 (H the
 * UNDAMPED X^T X), d' = d / s^2 (may be NULL), damping on H0'. codes /
 * scales / g_idx / perm quantize W' (the caller folds 1/s into the previous
 * operator, as for AWQ: What = code * scale[g_idx] / s). stats as for
 * gptq_quantize_layer, for the scaled layer; stats[3] = ||X' dW'^T||^2 equals
 * the calibration error ||X (W - What)^T||^2 in the original basis.
 * A zero or non-finite s gives ENONFINITE or ENOTPD. Synchronous.
 * Errors: EINVAL, ENOTPD, ENONFINITE, EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t awq_gptq_quantize_layer_workspace_bytes(int64_t out, int64_t in, int block_size);
int awq_gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                            const float* H, const double* d, const float* s,
                            int bits, int group_size, double damp, int act_order, int block_size,
                            int8_t* codes, float* scales, int32_t* g_idx, int32_t* perm, double* stats,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * INT4 storage — the step after the path.  [OBJ] opening question and "A
 * strong answer": INT4 weights with group scales; "What interviewers probe
 * next" and "Common mistakes": with act-order each column carries its group
 * index, and a dequantizer that ignores it applies wrong scales.
 *
 * pack_int4: codes int8[out, in] (row stride in; bits in [2, 4]: a
 * symmetric grid's codes in [-8, 7], or a zero-point grid's in [0, 15]) ->
 * packed uint32[out, in/8]: word w of row r holds codes[r][8w .. 8w+7], code
 * 8w+k in bits 4k..4k+3 as its low nibble (two's complement for the
 * symmetric grid). Requires in % 8 == 0. Codes outside both ranges are a
 * precondition violation (only their low nibble is kept).
 * Asynchronous. Errors: EINVAL, EHIP.
 *
 * dequantize_int4: What[r][c] = code(r, c) * scales[r][gi(c)] with
 * gi(c) = g_idx[c] (g_idx may be NULL: gi(c) = c / group_size), nibbles read
 * as signed; with zeros (int8[out, ceil(in / group_size)], may be NULL)
 * nibbles are unsigned and What = (code - zeros[r][gi(c)]) * scales[r][gi(c)].
 * scales is fp32[out, ceil(in / group_size)] (row stride ceil(in /
 * group_size)); a group index outside that range gives NaN in that column.
 * What is fp32 or bf16 (out_dtype; the fp32 product rounded to nearest even)
 * [out, in] with row stride ldo (>= in, multiple of 8). Asynchronous.
 * Errors: EINVAL, EHIP.
 * ---------------------------------------------------------------------- */
int pack_int4(const int8_t* codes, int64_t out, int64_t in, int bits, uint32_t* packed, void* stream);
int dequantize_int4(const uint32_t* packed, const float* scales, const int32_t* g_idx, const int8_t* zeros,
                    int64_t out, int64_t in, int group_size, int out_dtype, void* What, int64_t ldo, void* stream);

/* ------------------------------------------------------------------------
 * Calibration output error of a quantized layer (evaluation; not part of
 * producing the codes).  [OBJ] "A strong answer": the objective
 * ||X W^T - X What^T||^2 (the quantity GPTQ's loop and AWQ's grid search
 * minimise) and its normaliser ||X W^T||^2; the page's table reports the
 * former per element as output MSE.
 *
 * What[r][c] = (codes[r][c] - z) * scales[r][gi] / s[c] with
 * gi = g_idx[c] (g_idx may be NULL: gi = c / group_size), z =
 * zeros[r][gi] (zeros may be NULL: z = 0, the symmetric grid), s fp32[in]
 * AWQ's channel scales (may be NULL: s = 1). codes int8[out, in] (row stride
 * in), scales fp32 and zeros int8 [out, ceil(in / group_size)]; a group
 * index outside that range makes the result NaN. X [rows, in] and W [out, in]
 * bf16 or fp32. out2 (host, 2 doubles) receives ||X (W - What)^T||_F^2 and
 * ||X W^T||_F^2. What is formed in fp64; with bf16 X the products run on the
 * bf16 MFMA with W and W - What split into a bf16 high part plus a bf16
 * residual (~16 significant bits), with fp32 X on the fp32 MFMA GEMM; the sums
 * of squares are fp64. The workspace depends on x_dtype. Synchronous.
 * Errors: EINVAL, EWORKSPACE, EHIP.
 * ---------------------------------------------------------------------- */
size_t layer_output_error_workspace_bytes(int64_t out, int64_t in, int64_t rows, int x_dtype);
int layer_output_error(const void* X, int x_dtype, int64_t rows, int64_t ldx,
                       const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                       const int8_t* codes, const float* scales, const int32_t* g_idx, const int8_t* zeros,
                       const float* s, int group_size, double* out2,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PTQ_H */
