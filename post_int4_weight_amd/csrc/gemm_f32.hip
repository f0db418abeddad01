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
// wave 64 x 64 = 2 x 2 MFMA 32x32 blocks; K staged through LDS 16 at a time,
// double buffered. LDS tiles are k-major (As[k][m], Bs[k][n]) so an MFMA
// operand fetch is one conflict-free ds_read_b32 per lane whatever the
// global layout; K-contiguous global layouts are transposed while staging.
// Within a 16-deep K tile, MFMA step s (k = 2 per step) takes k = s from
// lanes 0-31 and k = s + 8 from lanes 32-63 (the contraction is order-free);
// with a 132-float LDS row this puts the two half-waves on disjoint banks.
#include "common.hpp"

namespace ptq {
namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LDS_ROW = 132;  // floats per k-row of a staged tile
constexpr int NT = 256;

struct Stage {
    float a[BK * LDS_ROW];
    float b[BK * LDS_ROW];
};

// Per-thread staging registers: 2 float4 of A and 2 of B per K tile.
struct Regs {
    float4 a[2];
    float4 b[2];
};

__device__ __forceinline__ float4 load4_guarded(const float* base, int64_t ld, int64_t r, int64_t c,
                                                int64_t R, int64_t Cn) {
    // element (r, c..c+3) of a row-major [R, Cn] matrix, zero outside
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
// kmajor_global: the global matrix is stored [K][X] (X = the M or N index).
__device__ __forceinline__ void gload(float4 (&v)[2], const float* P, int64_t ld, bool kmajor_global,
                                      int64_t k0, int64_t x0, int64_t K, int64_t X, int t) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        int idx = t + NT * r;
        if (kmajor_global) {
            int k = idx >> 5, x4 = idx & 31;           // 16 rows x 32 float4
            v[r] = load4_guarded(P, ld, k0 + k, x0 + 4 * x4, K, X);
        } else {
            int x = idx >> 2, kq = idx & 3;            // 128 rows x 4 float4 along k
            v[r] = load4_guarded(P, ld, x0 + x, k0 + 4 * kq, X, K);
        }
    }
}

__device__ __forceinline__ void sstore(float* S, const float4 (&v)[2], bool kmajor_global, int t) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        int idx = t + NT * r;
        if (kmajor_global) {
            int k = idx >> 5, x4 = idx & 31;
            *(float4*)(S + k * LDS_ROW + 4 * x4) = v[r];
        } else {
            int x = idx >> 2, kq = idx & 3;
            S[(4 * kq + 0) * LDS_ROW + x] = v[r].x;
            S[(4 * kq + 1) * LDS_ROW + x] = v[r].y;
            S[(4 * kq + 2) * LDS_ROW + x] = v[r].z;
            S[(4 * kq + 3) * LDS_ROW + x] = v[r].w;
        }
    }
}

__global__ __launch_bounds__(NT, 2) void gemm_f32_kernel(GemmArgs g) {
    const int64_t tiles_n = cdiv(g.N, BN);
    const int64_t tile = blockIdx.x;
    const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
    if (g.upper_only && tm > tn) return;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    // K range this tile needs (structural zeros of a triangular operand skipped)
    int64_t kb = 0, ke = g.K;
    if (g.tri == TRI_A_UPPER) kb = m0;                       // A[i][k] = 0 for k < i
    else if (g.tri == TRI_B_UPPER_NK) kb = n0;               // B[j][k] = 0 for k < j
    else if (g.tri == TRI_B_UPPER_KN) ke = min(g.K, n0 + BN); // B[k][j] = 0 for k > j
    kb = (kb / BK) * BK;

    __shared__ Stage st[2];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int li = lane & 31, lh = lane >> 5;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const bool a_km = g.layout_a == A_KM;
    const bool b_kn = g.layout_b == B_KN;
    const int64_t nk = (ke > kb) ? cdiv(ke - kb, BK) : 0;

    Regs rg;
    if (nk > 0) {
        gload(rg.a, g.A, g.lda, a_km, kb, m0, g.K, g.M, t);
        gload(rg.b, g.B, g.ldb, b_kn, kb, n0, g.K, g.N, t);
        sstore(st[0].a, rg.a, a_km, t);
        sstore(st[0].b, rg.b, b_kn, t);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            int64_t k1 = kb + (kt + 1) * BK;
            gload(rg.a, g.A, g.lda, a_km, k1, m0, g.K, g.M, t);
            gload(rg.b, g.B, g.ldb, b_kn, k1, n0, g.K, g.N, t);
        }
        const float* As = st[cur].a;
        const float* Bs = st[cur].b;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int kr = s + 8 * lh;
            float av0 = As[kr * LDS_ROW + wm + li];
            float av1 = As[kr * LDS_ROW + wm + 32 + li];
            float bv0 = Bs[kr * LDS_ROW + wn + li];
            float bv1 = Bs[kr * LDS_ROW + wn + 32 + li];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av0, bv0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av0, bv1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av1, bv0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av1, bv1, acc[1][1], 0, 0, 0);
        }
        if (more) {
            sstore(st[cur ^ 1].a, rg.a, a_km, t);
            sstore(st[cur ^ 1].b, rg.b, b_kn, t);
        }
        __syncthreads();
    }

    // Epilogue. 32x32 accumulator layout: lane l, register r holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                int64_t col = n0 + wn + 32 * j + li;
                if (row < g.M && col < g.N) {
                    float* c = g.C + row * g.ldc + col;
                    float v = g.alpha * acc[i][j][r];
                    *c = g.beta_one ? (*c + v) : v;
                }
            }
}

}  // namespace

int launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return PTQ_OK;
    if (a.K <= 0) {
        if (a.beta_one) return PTQ_OK;  // C += 0
    }
    int64_t tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)tiles), dim3(NT), 0, st, a);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

}  // namespace ptq
