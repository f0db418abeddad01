/*
 * ptq_testing.h — test hook of libptq.so (not part of the product API).
 *
 * Exposes the fp32 MFMA GEMM used inside stages 2 and 3 so its operand
 * layouts and triangle modes can be checked against a reference on their own:
 *
 *   C = alpha * op(A) op(B) + beta * C,   beta = beta_one ? 1 : 0
 *
 * layout_a: 0 = A row-major [M, K] (row stride lda), 1 = A stored [K, M].
 * layout_b: 0 = B row-major [K, N] (row stride ldb), 1 = B stored [N, K].
 * tri: 0 none; 1 A upper triangular (A[i][k] = 0 for k < i: those k are
 * skipped per row tile); 2 B upper (layout 0, B[k][j] = 0 for k > j);
 * 3 B upper stored [N][K] (entries with k < j are zero). upper_only: only
 * output tiles on or above the diagonal are written (128 x 128 tiles, or
 * 64 x 64 when the product has fewer than 1024 of 128 x 128): every entry
 * on or above the diagonal is, entries below it only inside diagonal tiles.
 * Device pointers; lda, ldb multiples of 4; asynchronous on `stream`.
 * Returns PTQ_OK, PTQ_EINVAL or PTQ_EHIP.
 */
#ifndef PTQ_TESTING_H
#define PTQ_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int ptq_test_gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int layout_a, const float* B,
                      int64_t ldb, int layout_b, float* C, int64_t ldc, float alpha, int beta_one, int tri,
                      int upper_only, void* stream);

/* The same product on the bf16 MFMA from three-term bf16 splits of A and B
 * (x = hi + mid + lo, six term products kept: fp32 GEMM accuracy), as used
 * for the large GEMMs of the U recursion. Output tiles are 256 x 256
 * (upper_only: tiles on or above the diagonal). The workspace (16-byte
 * aligned, size from the query) holds the split planes. Asynchronous.
 * Returns PTQ_OK, PTQ_EINVAL, PTQ_EWORKSPACE or PTQ_EHIP. */
size_t ptq_test_gemm_f32_split3_workspace_bytes(int64_t M, int64_t N, int64_t K);
int ptq_test_gemm_f32_split3(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int layout_a,
                             const float* B, int64_t ldb, int layout_b, float* C, int64_t ldc, float alpha,
                             int beta_one, int tri, int upper_only, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Two independent products of the fp32 GEMM in one launch, as the U
 * recursion runs H11 -= R12 R12^T and T = R12 U22 at its small levels:
 * product 0 with B stored [N][K] (layout_b 1), product 1 with B row-major
 * [K][N] (layout_b 0), A row-major [M, K] for both, each with its own C,
 * alpha, beta, tri and upper_only as in ptq_test_gemm_f32. The results are
 * those of two ptq_test_gemm_f32 calls, bit for bit (when the two cannot
 * share a launch, two launches are made). Device pointers; K, lda, ldb
 * multiples of 4. Asynchronous. Returns PTQ_OK, PTQ_EINVAL or PTQ_EHIP. */
int ptq_test_gemm_f32_pair(int64_t M0, int64_t N0, int64_t K0, const float* A0, int64_t lda0, const float* B0,
                           int64_t ldb0, float* C0, int64_t ldc0, float alpha0, int beta_one0, int tri0,
                           int upper_only0, int64_t M1, int64_t N1, int64_t K1, const float* A1, int64_t lda1,
                           const float* B1, int64_t ldb1, float* C1, int64_t ldc1, float alpha1, int beta_one1,
                           int tri1, int upper_only1, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PTQ_TESTING_H */
