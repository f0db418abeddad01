// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
//   C = alpha * op(A) op(B) + beta * C        (alpha = +-1, beta in {0, 1})
//
// Used for every dense fp32 contraction on the GPTQ path: the trailing
// lazy-batch update W[:, b1:] -= E U[b0:b1, b1:] ("GPTQ versus AWQ
// objectives", "A strong answer": batching the updates over column blocks so
// the work runs as GEMMs) and the blocked products of the recursive
// Cholesky / triangular inverse that produce U.
//
// Tile: 128 x 128 per workgroup of 256 threads (4 wave64s in 2 x 2), each
// wave 64 x 64 = 2 x 2 MFMA 32x32 blocks; K staged through LDS 32 at a time,
// double buffered through registers. LDS tiles are k-major (As[k][m],
// Bs[k][n]) so an MFMA operand fetch is one conflict-free ds_read_b32 per
// lane whatever the global layout; K-contiguous global layouts are
// transposed while staging. Within a 32-deep K tile, each MFMA step (k = 2
// per step) takes one k-row from lanes 0-31 and the row 8 further from lanes
// 32-63 (the contraction is order-free); with a 132-float LDS row the two
// half-waves read disjoint banks. Operand layouts are template parameters and interior
// tiles take an unguarded load path, so the main loop has no divergent
// branches; every operand read of a stage is issued before its MFMAs.
#include "common.hpp"

namespace ptq {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_ROW = 132;  // floats per k-row of a staged tile
constexpr int NT = 256;
constexpr int PER = BK * BM / 4 / NT;   // float4 per thread per operand per stage (4)

struct Stage {
    float a[BK * LDS_ROW];
    float b[BK * LDS_ROW];
};

// element (r, c..c+3) of a row-major [R, Cn] matrix, zero outside
__device__ __forceinline__ float4 load4_guarded(const float* base, int64_t ld, int64_t r, int64_t c, int64_t R,
                                                int64_t Cn) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < R) {
        const float* p = base + r * ld + c;
        if (c + 3 < Cn) {
            v = *(const float4*)p;
        } else {
            if (c + 0 < Cn) v.x = p[0];
            if (c + 1 < Cn) v.y = p[1];
            if (c + 2 < Cn) v.z = p[2];
        }
    }
    return v;
}

// Stage an operand tile [BK x 128] (k-major in LDS) from global memory.
// KMAJOR: the global matrix is stored [K][X] (X = the M or N index).
template <bool KMAJOR, bool GUARD>
__device__ __forceinline__ void gload(float4 (&v)[PER], const float* P, int64_t ld, int64_t k0, int64_t x0,
                                      int64_t K, int64_t X, int t) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int idx = t + NT * r;
        if (KMAJOR) {
            const int k = idx >> 5, x4 = idx & 31;           // BK rows x 32 float4
            v[r] = GUARD ? load4_guarded(P, ld, k0 + k, x0 + 4 * x4, K, X)
                         : *(const float4*)(P + (k0 + k) * ld + x0 + 4 * x4);
        } else {
            const int x = idx >> 3, kq = idx & 7;            // 128 rows x 8 float4 along k
            v[r] = GUARD ? load4_guarded(P, ld, x0 + x, k0 + 4 * kq, X, K)
                         : *(const float4*)(P + (x0 + x) * ld + k0 + 4 * kq);
        }
    }
}

template <bool KMAJOR>
__device__ __forceinline__ void sstore(float* S, const float4 (&v)[PER], int t) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int idx = t + NT * r;
        if (KMAJOR) {
            const int k = idx >> 5, x4 = idx & 31;
            *(float4*)(S + k * LDS_ROW + 4 * x4) = v[r];
        } else {
            const int x = idx >> 3, kq = idx & 7;
            S[(4 * kq + 0) * LDS_ROW + x] = v[r].x;
            S[(4 * kq + 1) * LDS_ROW + x] = v[r].y;
            S[(4 * kq + 2) * LDS_ROW + x] = v[r].z;
            S[(4 * kq + 3) * LDS_ROW + x] = v[r].w;
        }
    }
}

template <bool A_KMAJOR, bool B_KMAJOR, bool GUARD>
__device__ __forceinline__ void main_loop(const GemmArgs& g, Stage (&st)[2], f32x16 (&acc)[2][2], int64_t kb,
                                          int64_t nk, int64_t m0, int64_t n0) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int li = lane & 31, lh = lane >> 5;
    float4 ra[PER], rb[PER];
    gload<A_KMAJOR, GUARD>(ra, g.A, g.lda, kb, m0, g.K, g.M, t);
    gload<B_KMAJOR, GUARD>(rb, g.B, g.ldb, kb, n0, g.K, g.N, t);
    sstore<A_KMAJOR>(st[0].a, ra, t);
    sstore<B_KMAJOR>(st[0].b, rb, t);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k1 = kb + (kt + 1) * BK;
            gload<A_KMAJOR, GUARD>(ra, g.A, g.lda, k1, m0, g.K, g.M, t);
            gload<B_KMAJOR, GUARD>(rb, g.B, g.ldb, k1, n0, g.K, g.N, t);
        }
        const float* As = st[cur].a;
        const float* Bs = st[cur].b;
        float av[BK / 2][2], bv[BK / 2][2];
#pragma unroll
        for (int s = 0; s < BK / 2; ++s) {
            const int kr = (s & 7) + 16 * (s >> 3) + 8 * lh;   // half-waves 8 rows apart: disjoint banks
            av[s][0] = As[kr * LDS_ROW + wm + li];
            av[s][1] = As[kr * LDS_ROW + wm + 32 + li];
            bv[s][0] = Bs[kr * LDS_ROW + wn + li];
            bv[s][1] = Bs[kr * LDS_ROW + wn + 32 + li];
        }
#pragma unroll
        for (int s = 0; s < BK / 2; ++s) {
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s][0], bv[s][0], acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s][0], bv[s][1], acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s][1], bv[s][0], acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s][1], bv[s][1], acc[1][1], 0, 0, 0);
        }
        // operand reads first, then the MFMAs (latency exposed once per stage)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * BK, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * BK, 0);
        if (more) {
            sstore<A_KMAJOR>(st[cur ^ 1].a, ra, t);
            sstore<B_KMAJOR>(st[cur ^ 1].b, rb, t);
        }
        __syncthreads();
    }
}

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(NT, 2) void gemm_f32_kernel(GemmArgs g) {
    const int64_t tiles_n = cdiv(g.N, BN);
    const int64_t tile = blockIdx.x;
    const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
    if (g.upper_only && tm > tn) return;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    // K range this tile needs (structural zeros of a triangular operand skipped)
    int64_t kb = 0, ke = g.K;
    if (g.tri == TRI_A_UPPER) kb = m0;                        // A[i][k] = 0 for k < i
    else if (g.tri == TRI_B_UPPER_NK) kb = n0;                // B[j][k] = 0 for k < j
    else if (g.tri == TRI_B_UPPER_KN) ke = min(g.K, n0 + BN); // B[k][j] = 0 for k > j
    kb = (kb / BK) * BK;

    __shared__ Stage st[2];
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t nk = (ke > kb) ? cdiv(ke - kb, BK) : 0;
    if (nk > 0) {
        const bool interior = (m0 + BM <= g.M) && (n0 + BN <= g.N) && (kb + nk * BK <= g.K) &&
                              (g.lda % 4 == 0) && (g.ldb % 4 == 0);
        if (interior)
            main_loop<A_KMAJOR, B_KMAJOR, false>(g, st, acc, kb, nk, m0, n0);
        else
            main_loop<A_KMAJOR, B_KMAJOR, true>(g, st, acc, kb, nk, m0, n0);
    }

    // Epilogue. 32x32 accumulator layout: lane l, register r holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int li = lane & 31, lh = lane >> 5;
    const int mi = (int)min((int64_t)BM, g.M - m0), nj = (int)min((int64_t)BN, g.N - n0);
    float* Ct = g.C + m0 * g.ldc + n0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int jj = wn + 32 * j + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ii = wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (ii < mi && jj < nj) {
                    float* c = Ct + (int64_t)ii * g.ldc + jj;
                    const float v = g.alpha * acc[i][j][r];
                    *c = g.beta_one ? (*c + v) : v;
                }
            }
        }
}

}  // namespace

int launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return PTQ_OK;
    if (a.K <= 0 && a.beta_one) return PTQ_OK;  // C += 0
    const unsigned tiles = (unsigned)(cdiv(a.M, BM) * cdiv(a.N, BN));
    const bool akm = a.layout_a == A_KM, bkn = a.layout_b == B_KN;
    if (akm && bkn) hipLaunchKernelGGL((gemm_f32_kernel<true, true>), dim3(tiles), dim3(NT), 0, st, a);
    else if (akm) hipLaunchKernelGGL((gemm_f32_kernel<true, false>), dim3(tiles), dim3(NT), 0, st, a);
    else if (bkn) hipLaunchKernelGGL((gemm_f32_kernel<false, true>), dim3(tiles), dim3(NT), 0, st, a);
    else hipLaunchKernelGGL((gemm_f32_kernel<false, false>), dim3(tiles), dim3(NT), 0, st, a);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

}  // namespace ptq
