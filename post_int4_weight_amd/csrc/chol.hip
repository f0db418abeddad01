// Stage 2: damping, act-order permutation and U, the upper factor of H^-1.
//
// "GPTQ versus AWQ objectives", "A strong answer": H += damp * mean(diag H) I,
// then U upper triangular with U^T U = H^-1 (the page forms it as the
// Cholesky factor of inv(H), transposed). "What interviewers probe next":
// act-order processes columns in decreasing Hessian diagonal.
//
// U is unique (positive diagonal), so it is computed here by a cheaper route
// that never forms H^-1: the reversed-order Cholesky H = R R^T with R upper
// triangular, then U = R^-1 (U^T U = R^-T R^-1 = (R R^T)^-1). Both factors are
// produced together by one recursion on the 2 x 2 block split
//
//   H = [H11 H12; H12^T H22]:  (R22, U22) from H22 (recursively),
//                              R12 = H12 U22^T,
//                              H11 <- H11 - R12 R12^T,
//                              (R11, U11) from H11 (recursively),
//                              U12 = -U11 R12 U22,
//
// so 2n^3/3 flops run as large GEMMs (the big ones on the bf16 MFMA from
// three-term bf16 splits, at fp32 accuracy; the rest on the fp32 MFMA) and only
// BASE x BASE (128 x 128) diagonal blocks are factored and inverted inside one workgroup's
// LDS. A non-positive (or NaN) pivot raises a device flag read once at the end.
#include "common.hpp"

#include <algorithm>
#include <cmath>

namespace ptq {
namespace {

constexpr int BASE = 128;                 // diagonal blocks factored by one workgroup
constexpr int BASE_THREADS = (BASE / 4) * (BASE / 4);

// lambda = damp * mean(key); key = d (fp64) or diag(H). One workgroup, fixed order.
__global__ void damping_kernel(const float* H, const double* d, int64_t n, double damp, double* lam) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += d ? d[i] : (double)H[i * n + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *lam = damp * (red[0] / (double)n);
}

// Act-order key of column j; a NaN key sorts last (so the ranks stay a
// permutation; the NaN itself is reported by the factorization).
__device__ __forceinline__ double order_key(const float* H, const double* d, int64_t n, int64_t j) {
    const double v = d ? d[j] : (double)H[j * n + j];
    return (v != v) ? -HUGE_VAL : v;
}

// perm[rank(j)] = j with rank(j) = #{k : key_k > key_j or (key_k == key_j and k < j)}:
// the stable sort of columns by decreasing key.
__global__ void act_order_rank_kernel(const float* H, const double* d, int64_t n, int32_t* perm) {
    __shared__ double tile[256];
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const double kj = (j < n) ? order_key(H, d, n, j) : 0.0;
    int64_t rank = 0;
    for (int64_t b = 0; b < n; b += 256) {
        const int64_t k = b + threadIdx.x;
        tile[threadIdx.x] = (k < n) ? order_key(H, d, n, k) : 0.0;
        __syncthreads();
        const int lim = (int)std::min<int64_t>(256, n - b);
        for (int q = 0; q < lim; ++q) {
            const double kk = tile[q];
            rank += (kk > kj || (kk == kj && b + q < j)) ? 1 : 0;
        }
        __syncthreads();
    }
    if (j < n) perm[rank] = (int32_t)j;
}

__global__ void identity_perm_kernel(int32_t* perm, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) perm[j] = (int32_t)j;
}

// A[i][j] = H[p_i][p_j] + lambda [i == j]  (p = perm or identity)
__global__ void build_damped_kernel(const float* __restrict__ H, const int32_t* __restrict__ perm, int64_t n,
                                    const double* lam, float* __restrict__ A) {
    const int64_t i = blockIdx.y;
    const int64_t pi = perm ? perm[i] : i;
    const float l = (float)*lam;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pj = perm ? perm[j] : j;
        float v = H[pi * n + pj];
        if (i == j) v = (float)((double)v + (double)l);
        A[i * n + j] = v;
    }
}

// The same without a permutation, 16 bytes per thread (n % 4 == 0).
__global__ void build_damped_vec_kernel(const float4* __restrict__ H, int64_t n4, const double* lam,
                                        float4* __restrict__ A) {
    const int64_t i = blockIdx.y;
    const float l = (float)*lam;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += (int64_t)gridDim.x * blockDim.x) {
        float4 v = H[i * n4 + q];
        const int64_t d = i - 4 * q;   // position of the diagonal inside this float4, if any
        if (d == 0) v.x = (float)((double)v.x + (double)l);
        if (d == 1) v.y = (float)((double)v.y + (double)l);
        if (d == 2) v.z = (float)((double)v.z + (double)l);
        if (d == 3) v.w = (float)((double)v.w + (double)l);
        A[i * n4 + q] = v;
    }
}

__global__ void fill_zero_kernel(float* p, int64_t count) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count;
         e += (int64_t)gridDim.x * blockDim.x)
        p[e] = 0.f;
}

__global__ void fill_int_kernel(int* p, int v) { *p = v; }

// Base case on an m x m diagonal block (m <= BASE, m % 4 == 0): the
// reversed-order Cholesky A = R R^T (R upper) and U = R^-1 in one right-looking
// sweep over j = m-1 .. 0, with the (symmetric) trailing matrix A and
// S = I - R[:, >j] U[>j, :]:
//
//   R[i][j] = A[i][j] / sqrt(A[j][j])       (i < j)
//   U[j][c] = S[j][c] / sqrt(A[j][j])       (row j of R U = I, final now)
//   A[i][k] -= R[i][j] R[k][j],  S[i][c] -= R[i][j] U[j][c]    (i, k < j)
//
// Column k of A is last needed at step k + 1 (it holds column k of R), and
// column c of S stays the identity's until step c (U[j][c] = 0 for c < j), so
// one 4 x 4 register tile per thread holds M[i][k] = A[i][k] for k < j and
// S[i][k] for k >= j: at step j column j turns into the identity's column,
// and the step's update is the single M[i][k] -= R[i][j] V[k] with
// V[k] = R[k][j] (k < j) or U[j][k] (k >= j). Only column j of A and row j of
// S go through LDS, so a step is one barrier, three 16-byte LDS reads and 16
// FMAs per thread (rows already final skip the update). Outside m the block
// is padded with the identity. U is written to the block (zeros below its
// diagonal). Bit 0 of *flag: non-positive pivot; bit 1: NaN.
__global__ __launch_bounds__(BASE_THREADS) void chol_inv_base_kernel(const float* __restrict__ A,
                                                                      float* __restrict__ U, int m, int64_t ld,
                                                                      int* flag) {
    constexpr int TB = BASE / 4;               // 4 x 4 tiles per block row
    __shared__ __attribute__((aligned(16))) float colb[BASE][BASE];   // colb[j][i] = A[i][j] at step j
    __shared__ __attribute__((aligned(16))) float rowb[BASE][BASE];   // rowb[j][c] = S[j][c] at step j
    const int t = threadIdx.x;
    const int ib = t / TB, kb = t % TB;        // this thread's tile: rows 4*ib.., columns 4*kb..
    const int i0 = 4 * ib, k0 = 4 * kb;
    float a[4][4];                             // M: A left of the current column, S from it on
#pragma unroll
    for (int di = 0; di < 4; ++di)
#pragma unroll
        for (int dk = 0; dk < 4; ++dk) {
            const int i = i0 + di, k = k0 + dk;
            const int r = min(min(i, k), m - 1), c = min(max(i, k), m - 1);   // upper triangle only
            a[di][dk] = A[(int64_t)r * ld + c];
            if (i >= m || k >= m) a[di][dk] = (i == k) ? 1.f : 0.f;
        }
    // row BASE - 1 of S is the identity's
    if (kb == TB - 1) *(float4*)&colb[BASE - 1][i0] = make_float4(a[0][3], a[1][3], a[2][3], a[3][3]);
    if (ib == TB - 1)
        *(float4*)&rowb[BASE - 1][k0] = make_float4(0.f, 0.f, 0.f, (kb == TB - 1) ? 1.f : 0.f);
    for (int jb = TB - 1; jb >= 0; --jb) {
#pragma unroll
        for (int dj = 3; dj >= 0; --dj) {
            const int j = 4 * jb + dj;
            __syncthreads();
            float piv = colb[j][j];
            const float4 ci = *(const float4*)&colb[j][i0];
            const float4 ck = *(const float4*)&colb[j][k0];
            const float4 rj = *(const float4*)&rowb[j][k0];
            if (!(piv > 0.f)) {
                if (t == 0) atomicOr(flag, (piv != piv) ? 2 : 1);
                piv = 1.f;
            }
            // 1 / sqrt(piv): the hardware reciprocal square root and one Newton
            // step (within about an ulp, as IEEE sqrt then divide; their dozens
            // of dependent instructions sat on every step's critical path)
            const float r0 = __builtin_amdgcn_rsqf(piv);
            const float r = r0 * fmaf(-0.5f * piv, r0 * r0, 1.5f);
            const float civ[4] = {ci.x, ci.y, ci.z, ci.w};
            const float ckv[4] = {ck.x, ck.y, ck.z, ck.w};
            const float rjv[4] = {rj.x, rj.y, rj.z, rj.w};
            float Ri[4], V[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                Ri[q] = (i0 + q < j) ? civ[q] * r : 0.f;
                V[q] = (k0 + q < j) ? ckv[q] * r : rjv[q] * r;
            }
            if (kb == jb) {   // column j of A is spent: it becomes column j of S (the identity's)
#pragma unroll
                for (int di = 0; di < 4; ++di) a[di][dj] = (i0 + di == j) ? 1.f : 0.f;
            }
            if (ib == jb) {   // row j of S is final: U[j][k] for k >= j
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q >= j) a[dj][q] = V[q];
            }
            if (i0 < j) {   // rows >= j are final (Ri = 0): whole waves skip the update as j falls
#pragma unroll
                for (int di = 0; di < 4; ++di)
#pragma unroll
                    for (int q = 0; q < 4; ++q) a[di][q] -= Ri[di] * V[q];
            }
            if (j > 0) {   // publish column j-1 of A and row j-1 of S (final after this update)
                const int djn = (dj + 3) & 3;
                const int jn = j - 1, jbn = jn >> 2;
                if (kb == jbn)
                    *(float4*)&colb[jn][i0] = make_float4(a[0][djn], a[1][djn], a[2][djn], a[3][djn]);
                if (ib == jbn) {
                    // S[jn][k]: the identity's left of column j, M from column j on
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = (k0 + q < j) ? ((k0 + q == jn) ? 1.f : 0.f) : a[djn][q];
                    *(float4*)&rowb[jn][k0] = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    }
#pragma unroll
    for (int di = 0; di < 4; ++di)
#pragma unroll
        for (int dk = 0; dk < 4; ++dk) {
            const int i = i0 + di, k = k0 + dk;
            if (i < m && k < m) U[(int64_t)i * ld + k] = a[di][dk];
        }
}

// GEMMs with all of M, N, K at least this large run on the bf16 MFMA from
// three-term splits of their operands (fp32 accuracy, gemm_bf16.hip); the
// smaller ones, deep in the recursion, on the fp32 MFMA GEMM (at n = 8192 its
// 2048-sized products are faster there: factor 11.3 ms at a threshold of
// 2048, 10.3 at 3072).
constexpr int64_t SPLIT3_MIN = 3072;

struct Ctx {
    float* A;      // damped (permuted) H, destroyed
    float* U;      // output
    float* T;      // scratch, >= (n/2)^2 + slack
    uint16_t* Pa;  // split planes of the GEMM operands (NULL: fp32 GEMMs only)
    uint16_t* Pb;
    int64_t n;
    int* flag;
    hipStream_t st;
};

int gemm(Ctx& c, int64_t M, int64_t N, int64_t K, const float* A, int la, int64_t lda, const float* B, int lb,
         int64_t ldb, float* C, int64_t ldc, float alpha, int beta_one, int tri, int upper_only) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layout_a = la;
    g.B = B; g.ldb = ldb; g.layout_b = lb;
    g.C = C; g.ldc = ldc;
    g.alpha = alpha; g.beta_one = beta_one; g.tri = tri; g.upper_only = upper_only;
    prof_begin(PROF_FACTOR_GEMM, c.st);
    const bool split = c.Pa && M >= SPLIT3_MIN && N >= SPLIT3_MIN && K >= SPLIT3_MIN;
    const int s = split ? launch_gemm_f32_split3(g, c.Pa, c.Pb, c.st) : launch_gemm_f32(g, c.st);
    prof_end(PROF_FACTOR_GEMM, c.st);
    return s;
}

// Factor the diagonal block [o, o+m) of A into U (see the recursion above).
int recurse(Ctx& c, int64_t o, int64_t m) {
    const int64_t n = c.n;
    if (m <= BASE) {
        prof_begin(PROF_FACTOR_BASE, c.st);
        hipLaunchKernelGGL(chol_inv_base_kernel, dim3(1), dim3(BASE_THREADS), 0, c.st, c.A + o * n + o, c.U + o * n + o,
                           (int)m, n, c.flag);
        prof_end(PROF_FACTOR_BASE, c.st);
        PTQ_LAUNCH_CHECK();
        return PTQ_OK;
    }
    // split so the trailing part is a multiple of BASE (keeps blocks aligned)
    const int64_t n2 = cdiv(m / 2, BASE) * BASE;
    const int64_t n1 = m - n2;
    float* A12 = c.A + o * n + (o + n1);
    float* A11 = c.A + o * n + o;
    float* U11 = c.U + o * n + o;
    float* U12 = c.U + o * n + (o + n1);   // holds R12 until U12 replaces it
    float* U22 = c.U + (o + n1) * n + (o + n1);
    PTQ_TRY(recurse(c, o + n1, n2));
    // R12 = H12 U22^T  (U22 stored [N][K], upper: entries with k < j are zero)
    PTQ_TRY(gemm(c, n1, n2, n2, A12, A_MK, n, U22, B_NK, n, U12, n, 1.f, 0, TRI_B_UPPER_NK, 0));
    // H11 -= R12 R12^T (upper tiles only)
    PTQ_TRY(gemm(c, n1, n1, n2, U12, A_MK, n, U12, B_NK, n, A11, n, -1.f, 1, TRI_NONE, 1));
    PTQ_TRY(recurse(c, o, n1));
    // T = R12 U22 (U22 upper: B[k][j] = 0 for k > j), T is [n1, n2] with row stride n2
    PTQ_TRY(gemm(c, n1, n2, n2, U12, A_MK, n, U22, B_KN, n, c.T, n2, 1.f, 0, TRI_B_UPPER_KN, 0));
    // U12 = -U11 T (U11 upper: A[i][k] = 0 for k < i)
    PTQ_TRY(gemm(c, n1, n2, n1, U11, A_MK, n, c.T, B_KN, n2, U12, n, -1.f, 0, TRI_A_UPPER, 0));
    return PTQ_OK;
}

}  // namespace

// Largest GEMM operand of the recursion: rows and depth at most the top
// split's trailing size.
int64_t split_half(int64_t n) { return cdiv(n / 2, BASE) * BASE; }

size_t factor_workspace_bytes(int64_t n) {
    Sizer z;
    z.take<float>((size_t)n * n);                          // A
    const int64_t half = split_half(n);
    z.take<float>((size_t)half * half + 1024);             // T
    z.take<double>(1);                                     // lambda
    z.take<int>(1);                                        // flag
    z.take<int32_t>((size_t)n);                            // perm (when the caller passes none)
    if (half >= SPLIT3_MIN) {                              // split planes of both operands
        z.take<uint16_t>(gemm_f32_split3_elems(half, half));
        z.take<uint16_t>(gemm_f32_split3_elems(half, half));
    }
    return z.bytes();
}

int run_inverse_factor(const float* H, const double* d, int64_t n, double damp, int act_order, float* U,
                       int32_t* perm, double* lambda_host, void* ws, size_t ws_bytes, hipStream_t st) {
    Arena ar(ws, ws_bytes);
    Ctx c{};
    c.n = n;
    c.st = st;
    c.A = ar.take<float>((size_t)n * n);
    const int64_t half = split_half(n);
    c.T = ar.take<float>((size_t)half * half + 1024);
    double* lam = ar.take<double>(1);
    c.flag = ar.take<int>(1);
    int32_t* ptmp = ar.take<int32_t>((size_t)n);
    const bool split = half >= SPLIT3_MIN;
    c.Pa = split ? ar.take<uint16_t>(gemm_f32_split3_elems(half, half)) : nullptr;
    c.Pb = split ? ar.take<uint16_t>(gemm_f32_split3_elems(half, half)) : nullptr;
    if (!c.A || !c.T || !lam || !c.flag || !ptmp || (split && (!c.Pa || !c.Pb))) {
        set_error("gptq_inverse_factor: workspace of %zu bytes, %zu needed", ws_bytes, factor_workspace_bytes(n));
        return PTQ_EWORKSPACE;
    }
    c.U = U;
    int32_t* p = perm ? perm : ptmp;

    hipLaunchKernelGGL(fill_int_kernel, dim3(1), dim3(1), 0, st, c.flag, 0);
    PTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(damping_kernel, dim3(1), dim3(256), 0, st, H, d, n, damp, lam);
    PTQ_LAUNCH_CHECK();
    if (act_order) {
        hipLaunchKernelGGL(act_order_rank_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, H, d, n, p);
    } else {
        hipLaunchKernelGGL(identity_perm_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, p, n);
    }
    PTQ_LAUNCH_CHECK();
    if (!act_order && n % 4 == 0 && ((uintptr_t)H & 15u) == 0)
        hipLaunchKernelGGL(build_damped_vec_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n / 4, 256), 64), (unsigned)n),
                           dim3(256), 0, st, (const float4*)H, n / 4, lam, (float4*)c.A);
    else
        hipLaunchKernelGGL(build_damped_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)n),
                           dim3(256), 0, st, H, act_order ? p : nullptr, n, lam, c.A);
    PTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(fill_zero_kernel, dim3(2048), dim3(256), 0, st, U, n * n);
    PTQ_LAUNCH_CHECK();
    PTQ_TRY(recurse(c, 0, n));

    int flag = 0;
    double lh = 0.0;
    PTQ_HIP(hipMemcpyAsync(&flag, c.flag, sizeof(int), hipMemcpyDeviceToHost, st));
    PTQ_HIP(hipMemcpyAsync(&lh, lam, sizeof(double), hipMemcpyDeviceToHost, st));
    PTQ_HIP(hipStreamSynchronize(st));
    if (lambda_host) *lambda_host = lh;
    if (flag & 2) {
        set_error("gptq_inverse_factor: NaN pivot (non-finite H or d)");
        return PTQ_ENONFINITE;
    }
    if (flag & 1) {
        set_error("gptq_inverse_factor: H + lambda I is not positive definite (lambda = %g)", lh);
        return PTQ_ENOTPD;
    }
    return PTQ_OK;
}

}  // namespace ptq
