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

// A[i][j] = H[p_i][p_j] + lambda [i == j]  (p = perm or identity), for
// j >= A_ROW_START(i): the recursion reads A on and above the diagonal only,
// and its GEMMs' output tiles (at most 256 wide, aligned) inside the diagonal
// 256 x 256 blocks, so the copy starts each row at its diagonal block
constexpr int64_t A_DIAG_TILE = 256;
__host__ __device__ inline int64_t a_row_start(int64_t i) { return (i / A_DIAG_TILE) * A_DIAG_TILE; }
__global__ void build_damped_kernel(const float* __restrict__ H, const int32_t* __restrict__ perm, int64_t n,
                                    const double* lam, float* __restrict__ A) {
    const int64_t i = blockIdx.y;
    const int64_t pi = perm ? perm[i] : i;
    const float l = (float)*lam;
    for (int64_t j = a_row_start(i) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * blockDim.x) {
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
    for (int64_t q = a_row_start(i) / 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4;
         q += (int64_t)gridDim.x * blockDim.x) {
        float4 v = H[i * n4 + q];
        const int64_t d = i - 4 * q;   // position of the diagonal inside this float4, if any
        if (d == 0) v.x = (float)((double)v.x + (double)l);
        if (d == 1) v.y = (float)((double)v.y + (double)l);
        if (d == 2) v.z = (float)((double)v.z + (double)l);
        if (d == 3) v.w = (float)((double)v.w + (double)l);
        A[i * n4 + q] = v;
    }
}

// U[i][j] = 0 for j < i: the recursion writes every entry on and above the
// diagonal (grid y = rows)
__global__ void zero_lower_kernel(float* U, int64_t n) {
    const int64_t i = blockIdx.y;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < i; j += (int64_t)gridDim.x * blockDim.x)
        U[i * n + j] = 0.f;
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
// one TS x TS register tile per thread holds M[i][k] = A[i][k] for k < j and
// S[i][k] for k >= j: at step j column j turns into the identity's column,
// and the step's update is the single M[i][k] -= Ri[i] V[k] with
// Ri[i] = R[i][j] (0 for i >= j) and V[k] = R[k][j] (k < j) or U[j][k]
// (k >= j). A is symmetric and S is upper triangular, and every value the
// steps need comes from a tile on or above the diagonal, so only those tiles
// have a thread: TB (TB + 1) / 2 threads (the ones past that count only join
// the barriers).
//
// The sweep goes one tile column (TS = 4 steps) at a time, in two phases
// between barriers. The tiles holding the block's 4 columns of A and 4 rows
// of S publish them as they stand before the block. Phase 1: thread x < BASE
// derives, for row x, Ri of each of the 4 steps and, for column x, V of each
// step, by taking the block's steps on those few values in the order and
// with the operations the tiles themselves would apply (so U is the same,
// bit for bit, as with one step and one barrier per column). Phase 2: every
// tile takes the 4 steps on its registers from the published Ri and V. Two
// barriers per 4 columns instead of one per column: the sweep is bound by
// each step's latency chain (barrier, LDS read, pivot, update, publish).
// Outside m the block is padded with the identity. U is written on and
// above the diagonal of the block (the caller zeroes the rest).
// Bit 0 of *flag: non-positive pivot; bit 1: NaN.
template <int TS>
constexpr int base_threads() {
    return ((BASE / TS) * (BASE / TS + 1) / 2 + 63) / 64 * 64;
}
template <int TS, int CB>
__global__ __launch_bounds__(base_threads<TS>()) void chol_inv_base_kernel(const float* __restrict__ A,
                                                                          float* __restrict__ U, int m, int64_t ld,
                                                                          int* flag) {
    static_assert(TS == 4 && CB % TS == 0 && BASE % CB == 0, "rounds of whole tile columns, float4 pieces in LDS");
    constexpr int TB = BASE / TS;              // TS x TS tiles per block row
    constexpr int NB = BASE / CB;              // rounds
    constexpr int TPR = CB / TS;               // tile columns per round
    // per round jb (columns / rows CB jb .. CB jb + CB - 1), index [x][t]
    // for column or row CB jb + t:
    __shared__ __attribute__((aligned(16))) float colb[BASE][CB];   // A[x][CBjb+t] before the round
    __shared__ __attribute__((aligned(16))) float rowb[BASE][CB];   // tile value at row CBjb+t, column x, before it
    __shared__ __attribute__((aligned(16))) float Rb[BASE][CB];     // Ri[x] of step CBjb+t
    __shared__ __attribute__((aligned(16))) float Vb[BASE][CB];     // V[x] of step CBjb+t
    const int t = threadIdx.x;
    // this thread's tile (rows TS*ib.., columns TS*kb.., ib <= kb): the t-th
    // of the upper triangle's tiles in row-major order
    int ib = 0, rem = t;
    while (ib < TB && rem >= TB - ib) {
        rem -= TB - ib;
        ++ib;
    }
    const bool live = ib < TB;
    const int kb = live ? ib + rem : 0;
    if (!live) ib = 0;
    const int i0 = TS * ib, k0 = TS * kb;
    float a[TS][TS];                           // M: A left of the current column, S from it on
#pragma unroll
    for (int di = 0; di < TS; ++di)
#pragma unroll
        for (int dk = 0; dk < TS; ++dk) {
            const int i = i0 + di, k = k0 + dk;
            const int r = min(min(i, k), m - 1), c = min(max(i, k), m - 1);   // upper triangle only
            a[di][dk] = A[(int64_t)r * ld + c];
            if (i >= m || k >= m) a[di][dk] = (i == k) ? 1.f : 0.f;
        }
    // the tiles in tile column jbn publish its 4 columns of A, the tiles in
    // tile row jbn its 4 rows (as they stand: left of the block they are S's
    // identity part, which phase 1 takes from the rule, not from here)
    auto publish = [&](int jbn) {
        if (!live) return;
        if (kb / TPR == jbn) {
            const int o = TS * (kb % TPR);
#pragma unroll
            for (int q = 0; q < TS; ++q) *(float4*)&colb[i0 + q][o] = make_float4(a[q][0], a[q][1], a[q][2], a[q][3]);
        }
        if (ib / TPR == jbn) {
            const int o = TS * (ib % TPR);
#pragma unroll
            for (int q = 0; q < TS; ++q) *(float4*)&rowb[k0 + q][o] = make_float4(a[0][q], a[1][q], a[2][q], a[3][q]);
        }
    };
    int bad = 0;   // thread 0: non-positive (1) or NaN (2) pivots seen
    publish(NB - 1);
    for (int jb = NB - 1; jb >= 0; --jb) {
        const int jb0 = CB * jb;
        __syncthreads();
        if (t < BASE) {
            // Phase 1, x = t. c[u] = A[x][jb0+u] (row x of the block's
            // columns), s[u] = row jb0+u of the tile at column x, d[u][v] =
            // A[jb0+v][jb0+u] (the diagonal tile, column u, row v), each taken
            // through the block's steps as the tile holding it would.
            const int x = t;
            float c[CB], s[CB], d[CB][CB];
#pragma unroll
            for (int h = 0; h < CB; h += 4) {
                const float4 cv = *(const float4*)&colb[x][h];
                const float4 sv = *(const float4*)&rowb[x][h];
                c[h] = cv.x; c[h + 1] = cv.y; c[h + 2] = cv.z; c[h + 3] = cv.w;
                s[h] = sv.x; s[h + 1] = sv.y; s[h + 2] = sv.z; s[h + 3] = sv.w;
#pragma unroll
                for (int v = 0; v < CB; ++v) {
                    const float4 dv = *(const float4*)&colb[jb0 + v][h];
                    d[h][v] = dv.x; d[h + 1][v] = dv.y; d[h + 2][v] = dv.z; d[h + 3][v] = dv.w;
                }
            }
            float Rx[CB], Vx[CB];
#pragma unroll
            for (int tt = CB - 1; tt >= 0; --tt) {
                const int j = jb0 + tt;
                float piv = d[tt][tt];
                bad |= (piv != piv) ? 2 : (piv > 0.f ? 0 : 1);
                piv = (piv > 0.f) ? piv : 1.f;
                // 1 / sqrt(piv): the hardware reciprocal square root and one
                // Newton step (within about an ulp, as IEEE sqrt then divide;
                // their dozens of dependent instructions sat on every step's
                // critical path)
                const float r0 = __builtin_amdgcn_rsqf(piv);
                const float r = r0 * fmaf(-0.5f * piv, r0 * r0, 1.5f);
                // row x's Ri and column x's V of step j: the S row is the
                // identity's up to column j (its columns turn at their own step)
                Rx[tt] = (x < j) ? c[tt] * r : 0.f;
                Vx[tt] = (x < j) ? c[tt] * r : ((x == j) ? 1.f : s[tt]) * r;
#pragma unroll
                for (int u = 0; u < tt; ++u) {
                    // column jb0+u < j of A and row jb0+u of S under step j;
                    // R[jb0+u][j] = d[tt][u] r is that column's V and that
                    // row's Ri
                    const float Rdu = d[tt][u] * r;
                    if (TS * (x / TS) < j) c[u] -= Rx[tt] * Rdu;   // the tile holding (x, jb0+u) updates iff its first row is above j
#pragma unroll
                    for (int v = 0; v < tt; ++v) {
                        const float Rdv = d[tt][v] * r;
                        d[u][v] -= Rdv * Rdu;
                    }
                    if (x == j) s[u] = 0.f;                        // column j turns into the identity's
                    s[u] -= Rdu * Vx[tt];
                }
            }
#pragma unroll
            for (int h = 0; h < CB; h += 4) {
                *(float4*)&Rb[x][h] = make_float4(Rx[h], Rx[h + 1], Rx[h + 2], Rx[h + 3]);
                *(float4*)&Vb[x][h] = make_float4(Vx[h], Vx[h + 1], Vx[h + 2], Vx[h + 3]);
            }
        }
        __syncthreads();
        if (live && i0 < jb0 + CB) {
            // Phase 2: the round's steps on this tile (tiles whose rows are
            // all at or below the round only wait: nothing of them changes)
            float Ri[TS][CB], V[TS][CB];   // [q][tt]: rows i0+q / columns k0+q at step jb0+tt
#pragma unroll
            for (int q = 0; q < TS; ++q)
#pragma unroll
                for (int h = 0; h < CB; h += 4) {
                    const float4 rv = *(const float4*)&Rb[i0 + q][h];
                    const float4 vv = *(const float4*)&Vb[k0 + q][h];
                    Ri[q][h] = rv.x; Ri[q][h + 1] = rv.y; Ri[q][h + 2] = rv.z; Ri[q][h + 3] = rv.w;
                    V[q][h] = vv.x; V[q][h + 1] = vv.y; V[q][h + 2] = vv.z; V[q][h + 3] = vv.w;
                }
#pragma unroll
            for (int tt = CB - 1; tt >= 0; --tt) {
                const int j = jb0 + tt, dj = tt % TS;
                if (kb == j / TS) {   // column j of A is spent: it becomes column j of S (the identity's)
#pragma unroll
                    for (int di = 0; di < TS; ++di) a[di][dj] = (i0 + di == j) ? 1.f : 0.f;
                }
                if (ib == j / TS) {   // row j of S is final: U[j][k] for k >= j
#pragma unroll
                    for (int q = 0; q < TS; ++q)
                        if (k0 + q >= j) a[dj][q] = V[q][tt];
                }
                if (i0 < j) {   // rows >= j are final (Ri = 0): whole waves skip the update as j falls
#pragma unroll
                    for (int di = 0; di < TS; ++di)
#pragma unroll
                        for (int q = 0; q < TS; ++q) a[di][q] -= Ri[di][tt] * V[q][tt];
                }
            }
        }
        if (jb > 0) publish(jb - 1);
    }
    if (t == 0 && bad) atomicOr(flag, bad);
    if (!live) return;
#pragma unroll
    for (int di = 0; di < TS; ++di)
#pragma unroll
        for (int dk = 0; dk < TS; ++dk) {
            const int i = i0 + di, k = k0 + dk;
            if (i < m && k < m && i <= k) U[(int64_t)i * ld + k] = a[di][dk];
        }
}

// 4 x 4 tiles: 528 threads (nine waves) for the 128 x 128 block. With 8 x 8
// tiles (136 threads, one wave per SIMD and no other wave to hide the step's
// latency behind) a block took 82 us against 63 for the full 4 x 4 grid of
// 1024 threads; leaving out the tiles below the diagonal took it to 55 us.
constexpr int BASE_TS = 4;
constexpr int BASE_THREADS = base_threads<BASE_TS>();
constexpr int BASE_CB = 4;   // steps per round of the sweep (8: 54 us per block, phase 1 grows as CB^2)

// GEMMs with all of M, N, K at least this large run on the bf16 MFMA from
// three-term splits of their operands (fp32 accuracy, gemm_bf16.hip); the
// smaller ones, deep in the recursion, on the fp32 MFMA GEMM (at n = 8192 its
// 2048-sized products are faster there: factor 11.3 ms at a threshold of
// 2048, 10.3 at 3072).
constexpr int64_t SPLIT3_MIN = 3072;

struct Ctx {
    float* A;      // damped (permuted) H, destroyed
    float* U;      // output
    uint16_t* Pa;  // split planes of the GEMM operands (NULL: fp32 GEMMs only)
    uint16_t* Pb;
    int64_t n;
    int* flag;
    hipStream_t st;
};

GemmArgs gemm_args(int64_t M, int64_t N, int64_t K, const float* A, int la, int64_t lda, const float* B, int lb,
                   int64_t ldb, float* C, int64_t ldc, float alpha, int beta_one, int tri, int upper_only) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layout_a = la;
    g.B = B; g.ldb = ldb; g.layout_b = lb;
    g.C = C; g.ldc = ldc;
    g.alpha = alpha; g.beta_one = beta_one; g.tri = tri; g.upper_only = upper_only;
    return g;
}

bool split_size(const Ctx& c, const GemmArgs& g) {
    return c.Pa && g.M >= SPLIT3_MIN && g.N >= SPLIT3_MIN && g.K >= SPLIT3_MIN;
}

int gemm(Ctx& c, const GemmArgs& g) {
    prof_begin(PROF_FACTOR_GEMM, c.st);
    const int s = split_size(c, g) ? launch_gemm_f32_split3(g, c.Pa, c.Pb, c.st) : launch_gemm_f32(g, c.st);
    prof_end(PROF_FACTOR_GEMM, c.st);
    return s;
}

// Factor the diagonal block [o, o+m) of A into U (see the recursion above).
int recurse(Ctx& c, int64_t o, int64_t m) {
    const int64_t n = c.n;
    if (m <= BASE) {
        prof_begin(PROF_FACTOR_BASE, c.st);
        hipLaunchKernelGGL((chol_inv_base_kernel<BASE_TS, BASE_CB>), dim3(1), dim3(BASE_THREADS), 0, c.st, c.A + o * n + o, c.U + o * n + o,
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
    PTQ_TRY(gemm(c, gemm_args(n1, n2, n2, A12, A_MK, n, U22, B_NK, n, U12, n, 1.f, 0, TRI_B_UPPER_NK, 0)));
    // H11 -= R12 R12^T (upper tiles only), and T = R12 U22 (U22 upper:
    // B[k][j] = 0 for k > j) into A12, whose H12 is spent: T is [n1, n2] at
    // row stride n, outside everything the recursion on H11 touches. Both
    // read R12 and neither depends on the other, so on the split-operand path
    // they are one launch with R12 split once.
    const GemmArgs syrk = gemm_args(n1, n1, n2, U12, A_MK, n, U12, B_NK, n, A11, n, -1.f, 1, TRI_NONE, 1);
    const GemmArgs tprod = gemm_args(n1, n2, n2, U12, A_MK, n, U22, B_KN, n, A12, n, 1.f, 0, TRI_B_UPPER_KN, 0);
    if (split_size(c, syrk) && split_size(c, tprod)) {
        prof_begin(PROF_FACTOR_GEMM, c.st);
        const int s = launch_gemm_f32_split3_pair(syrk, tprod, c.Pa, c.Pb, c.st);
        prof_end(PROF_FACTOR_GEMM, c.st);
        PTQ_TRY(s);
    } else if (!split_size(c, syrk) && !split_size(c, tprod)) {
        // the small levels: both on the fp32 kernel, in one launch
        prof_begin(PROF_FACTOR_GEMM, c.st);
        const int s = launch_gemm_f32_pair(syrk, tprod, c.st);
        prof_end(PROF_FACTOR_GEMM, c.st);
        PTQ_TRY(s);
    } else {
        PTQ_TRY(gemm(c, syrk));
        PTQ_TRY(gemm(c, tprod));
    }
    PTQ_TRY(recurse(c, o, n1));
    // U12 = -U11 T (U11 upper: A[i][k] = 0 for k < i)
    PTQ_TRY(gemm(c, gemm_args(n1, n2, n1, U11, A_MK, n, A12, B_KN, n, U12, n, -1.f, 0, TRI_A_UPPER, 0)));
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
    double* lam = ar.take<double>(1);
    c.flag = ar.take<int>(1);
    int32_t* ptmp = ar.take<int32_t>((size_t)n);
    const bool split = half >= SPLIT3_MIN;
    c.Pa = split ? ar.take<uint16_t>(gemm_f32_split3_elems(half, half)) : nullptr;
    c.Pb = split ? ar.take<uint16_t>(gemm_f32_split3_elems(half, half)) : nullptr;
    if (!c.A || !lam || !c.flag || !ptmp || (split && (!c.Pa || !c.Pb))) {
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
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)n), dim3(256), 0,
                       st, U, n);
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
