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
// Two kernels share the 128 x 128 workgroup tile (256 threads, 4 wave64s in
// 2 x 2, each wave 64 x 64 = 2 x 2 MFMA 32x32 blocks):
//
//  * gemm_f32_direct_kernel (below) for A K-contiguous and K, leading
//    dimensions a multiple of 4: every product on the hot path. Products
//    with fewer than 1024 such tiles run it on 64 x 64 tiles instead (each
//    wave one 32 x 32 block), so they spread over four times as many CUs;
//  * gemm_f32_kernel, the general fallback (any layout, any K): K staged
//    through LDS 32 at a time, double buffered through registers, k-major LDS
//    tiles (K-contiguous operands transposed while staging) read with one
//    ds_read_b32 per lane and MFMA step; each step takes one k-row from
//    lanes 0-31 and the row 8 further from lanes 32-63, and the 132-float
//    LDS row puts the two half-waves in disjoint banks. Interior tiles take
//    an unguarded load path.
#include "common.hpp"
#include "tile_order.hpp"

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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for A K-contiguous (A_MK) and B either K-contiguous
// (B_NK) or N-contiguous (B_KN): the forms every hot product of the path has.
// global_load_lds_dwordx4 moves each lane's 16 bytes straight into LDS at
// base + 16 * lane, so there is no register staging and no ds_write; the
// layouts below are chosen on the global side (which chunk a lane fetches).
//
//   K-contiguous operand: LDS row = one m (or n) index, the stage's 16
//     floats of k in four 16-byte chunks, chunk c stored at
//     c ^ ((row >> 2) & 3). An MFMA operand fetch is one ds_read_b128 (4
//     consecutive k) per lane, free of bank conflicts for each 16-lane group.
//   N-contiguous operand: LDS row = one k, 128 floats of n in 32 chunks,
//     chunk c stored at c ^ (8 * ((k >> 2) & 1)): the two half-waves of a
//     ds_read_b32 (rows k and k + 4) fall in opposite halves of the banks.
//
// The contraction order inside an 8-deep step j is fixed by the ds_read_b128
// fragments: MFMA e of the step takes k = 8j + e from lanes 0-31 and
// k = 8j + 4 + e from lanes 32-63, for both operands.
//
// A ring of four 16-deep stages (64 KB, two workgroups per CU; three stages
// and three workgroups for K <= 1024) keeps the next stages' loads in
// flight; one barrier per stage (no memory fence: waits count only this
// wave's own loads, which retire in order) publishes every wave's copies. Fragment reads of the next step ride under the MFMAs of the
// current one. Rows (columns) past M (N) and k past K read clamped, valid
// addresses; k past K is zeroed in the fragments of the last stage and the
// other rows are discarded by the epilogue. Requires K, lda, ldb (and N for
// B_KN) multiples of 4 and 16-byte aligned A and B.
constexpr int DBK = 16;                 // k per stage
constexpr int DNST_LONG = 4;            // ring stages for long contractions
constexpr int DNST_SHORT = 3;           // K <= 1024: a smaller ring fits three workgroups per CU
constexpr int SHORT_K = 1024;
constexpr int DWG = 2;                  // workgroups per CU the kernel is built for
template <int BT>
constexpr int DSTAGE_BYTES = 2 * BT * DBK * 4;   // A and B tiles of one stage (BT x BT tiles)
constexpr int DJ = DBK / 8;                      // 8-deep MFMA steps per stage
constexpr int DCH = DBK / 4;                     // 16-byte chunks per K-contiguous LDS row
constexpr int XCDS = 8;                          // accelerator complex dies, one L2 each
static_assert(DJ % 2 == 0, "fragment slots alternate");

typedef __attribute__((address_space(3))) void* lds_ptr_f32_t;

// chunk swizzle of a K-contiguous LDS row r: the 16 rows one ds_read_b128
// pass serves land on distinct 4-bank groups
__device__ __forceinline__ int kswz(int r) {
    static_assert(DCH == 8 || DCH == 4, "swizzle for 8 or 4 chunks per row");
    return DCH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void f32_wait_vmcnt() {
    // s_waitcnt vmcnt(N) (bits 3:0 and 15:14), expcnt and lgkmcnt at their maxima
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// workgroups of a direct launch over tm x tn tiles (tile_order::gemm_tile
// without sub-blocks)
inline unsigned direct_grid(const GemmArgs& g, int64_t tm, int64_t tn) {
    return (unsigned)tile_order::gemm_grid(tm, tn, g.tri, g.upper_only, false);
}

// BT = 128 (4 waves of 64 x 64 = 2 x 2 MFMA blocks) or 64 (4 waves of one
// 32 x 32 block each): the small tile quadruples the workgroups of the small
// products deep in the U recursion, which otherwise run on a few CUs.
template <bool B_KMAJOR, int DNST, int BT>
__device__ __forceinline__ void direct_tile(const GemmArgs& g, int64_t tiles_m, int64_t tiles_n, unsigned bid) {
    static_assert(DNST >= 3, "the ring needs three stages");
    static_assert(BT == 128 || BT == 64, "tile");
    constexpr int WB = BT / 64;                          // 32 x 32 blocks per wave and dimension
    constexpr int DQ = BT * DBK * 4 / 1024 / 4;         // 1 KB copies per wave per operand per stage
    constexpr int SB = DSTAGE_BYTES<BT>;
    // Tile order (tile_order::gemm_tile, no sub-blocks). blockIdx b runs on
    // XCD b % 8. With at least 8 tile rows, XCD x takes whole rows, its k-th
    // being row 8k + x for even k and 8k + 7 - x for odd k: the tiles one
    // XCD runs side by side share A panels (and B panels across its rows) in
    // its own L2, and the zigzag keeps the triangular products (A upper,
    // upper_only), whose work falls with the row, balanced over the XCDs.
    // Products with a triangular B take whole columns the same way, deepest
    // first. Fewer rows: plain row-major order over all XCDs.
    int64_t tm, tn;
    if (!tile_order::gemm_tile(bid, tiles_m, tiles_n, g.tri, g.upper_only, false, tm, tn)) return;
    const int64_t m0 = tm * BT, n0 = tn * BT;

    int64_t kb = 0, ke = g.K;
    if (g.tri == TRI_A_UPPER) kb = m0;
    else if (g.tri == TRI_B_UPPER_NK) kb = n0;
    else if (g.tri == TRI_B_UPPER_KN) ke = min(g.K, n0 + BT);
    kb = (kb / DBK) * DBK;
    const int64_t nst = (ke > kb) ? cdiv(ke - kb, DBK) : 0;

    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * (BT / 2), wn = (wave & 1) * (BT / 2);
    const int li = lane & 31, lh = lane >> 5;

    // per-lane global offsets (elements) of the chunks this lane moves, at k = 0
    int64_t offA[DQ], offB[DQ];
    int kcA[DQ], kcB[DQ];        // k offset of the chunk (K-contiguous) or k row (N-contiguous)
#pragma unroll
    for (int q = 0; q < DQ; ++q) {
        const int p = (wave * DQ + q) * 64 + lane;     // 16-byte position in the stage's tile
        {
            const int r = p / DCH, pc = p % DCH;
            const int c = pc ^ kswz(r);
            const int64_t row = min(m0 + r, g.M - 1);
            offA[q] = row * g.lda;
            kcA[q] = 4 * c;
        }
        if (!B_KMAJOR) {
            const int r = p / DCH, pc = p % DCH;
            const int c = pc ^ kswz(r);
            const int64_t row = min(n0 + r, g.N - 1);
            offB[q] = row * g.ldb;
            kcB[q] = 4 * c;
        } else {
            const int kr = p / (BT / 4), pc = p % (BT / 4);
            const int c = pc ^ (8 * ((kr >> 2) & 1));
            const int64_t col = min(n0 + 4 * c, g.N - 4);
            offB[q] = col;
            kcB[q] = kr;
        }
    }

    auto issue = [&](int64_t s, int buf) {
        const int64_t k0 = kb + s * DBK;
        unsigned char* sa = dsm + buf * SB;
        unsigned char* sb = sa + BT * DBK * 4;
#pragma unroll
        for (int q = 0; q < DQ; ++q) {
            const int64_t k = min(k0 + kcA[q], g.K - 4);
            __builtin_amdgcn_global_load_lds((const void*)(g.A + offA[q] + k),
                                             (lds_ptr_f32_t)(sa + (wave * DQ + q) * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < DQ; ++q) {
            const float* src;
            if (!B_KMAJOR) {
                const int64_t k = min(k0 + kcB[q], g.K - 4);
                src = g.B + offB[q] + k;
            } else {
                const int64_t k = min(k0 + kcB[q], g.K - 1);
                src = g.B + k * g.ldb + offB[q];
            }
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_f32_t)(sb + (wave * DQ + q) * 1024), 16, 0,
                                             0);
        }
    };

    f32x16 acc[WB][WB];
#pragma unroll
    for (int a = 0; a < WB; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // fragments of one 8-deep step j: fa[a] = A[row][8j + 4lh .. +3], fb likewise
    f32x4 fa[2][WB], fb[2][WB];
    const int aswz = kswz(li);
    auto frags = [&](int64_t s, int j, int slot, bool mask) {
        const unsigned char* As = dsm + (s % DNST) * SB;
        const unsigned char* Bs = As + BT * DBK * 4;
        const int c = (2 * j + lh) ^ aswz;
#pragma unroll
        for (int a = 0; a < WB; ++a) fa[slot][a] = *(const f32x4*)(As + (wm + 32 * a + li) * (DBK * 4) + 16 * c);
        if (!B_KMAJOR) {
#pragma unroll
            for (int b = 0; b < WB; ++b) fb[slot][b] = *(const f32x4*)(Bs + (wn + 32 * b + li) * (DBK * 4) + 16 * c);
        } else {
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                const int n = wn + 32 * b + li;
                const int pc = (n >> 2) ^ (8 * lh);     // ((k >> 2) & 1) == lh for k = 8j + 4lh + e
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 8 * j + 4 * lh + e;
                    fb[slot][b][e] = *(const float*)(Bs + k * (BT * 4) + 16 * pc + 4 * (n & 3));
                }
            }
        }
        if (mask) {
            const int64_t kbase = kb + s * DBK + 8 * j + 4 * lh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = kbase + e < g.K;
#pragma unroll
                for (int a = 0; a < WB; ++a) fa[slot][a][e] = ok ? fa[slot][a][e] : 0.f;
#pragma unroll
                for (int b = 0; b < WB; ++b) fb[slot][b][e] = ok ? fb[slot][b][e] : 0.f;
            }
        }
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int a = 0; a < WB; ++a)
#pragma unroll
                for (int b = 0; b < WB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[slot][a][e], fb[slot][b][e], acc[a][b], 0, 0,
                                                                    0);
    };
    constexpr int NREAD = WB * (B_KMAJOR ? 5 : 2);   // LDS reads per fragment set
    constexpr int NMF = 4 * WB * WB;                  // MFMAs per step
    constexpr int NPAIR = NREAD < NMF ? NREAD : NMF;
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NPAIR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (NMF > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NPAIR, 0);
        if constexpr (NREAD > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NPAIR, 0);
    };

    if (nst > 0) {
        const bool tail = (kb + nst * DBK > g.K);     // last stage reaches past K
#pragma unroll
        for (int s = 0; s < DNST - 1; ++s) issue(min((int64_t)s, nst - 1), s);
        f32_wait_vmcnt<2 * DQ * (DNST - 2)>();
        __builtin_amdgcn_s_barrier();
        frags(0, 0, 0, tail && nst == 1);
        for (int64_t s = 0; s + 1 < nst; ++s) {
#pragma unroll
            for (int j = 0; j < DJ - 1; ++j) {
                frags(s, j + 1, (j + 1) & 1, false);
                mfmas(j & 1);
                interleave();
            }
            f32_wait_vmcnt<2 * DQ * (DNST - 3)>();
            __builtin_amdgcn_s_barrier();
            issue(min(s + DNST - 1, nst - 1), (int)((s + DNST - 1) % DNST));
            frags(s + 1, 0, 0, tail && s + 2 == nst);
            mfmas((DJ - 1) & 1);
            interleave();
        }
#pragma unroll
        for (int j = 0; j < DJ - 1; ++j) {
            frags(nst - 1, j + 1, (j + 1) & 1, tail);
            mfmas(j & 1);
            interleave();
        }
        mfmas((DJ - 1) & 1);
        // the ring's last (duplicate) copies must land before the workgroup's
        // LDS is released
        f32_wait_vmcnt<0>();
    }

    // epilogue (same accumulator layout as above)
    const int mi = (int)min((int64_t)BT, g.M - m0), nj = (int)min((int64_t)BT, g.N - n0);
    float* Ct = g.C + m0 * g.ldc + n0;
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) {
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

template <bool B_KMAJOR, int DNST, int BT>
__global__ __launch_bounds__(NT, DWG) void gemm_f32_direct_kernel(GemmArgs g, int64_t tiles_m, int64_t tiles_n) {
    direct_tile<B_KMAJOR, DNST, BT>(g, tiles_m, tiles_n, blockIdx.x);
}

// Two independent products in one launch: workgroups below grid0 (a
// multiple of 8, so both keep their XCD order) compute g0 with B stored
// [N][K], the rest g1 with B stored [K][N]; each tile is computed exactly as
// in a launch of its own. The factor's H11 -= R12 R12^T and T = R12 U22 at
// the recursion's small levels, where each launch runs on a few CUs and its
// fixed cost dominates.
template <int DNST, int BT>
__global__ __launch_bounds__(NT, DWG) void gemm_f32_direct_pair_kernel(GemmArgs g0, int64_t tm0, int64_t tn0,
                                                                       unsigned grid0, GemmArgs g1, int64_t tm1,
                                                                       int64_t tn1) {
    if (blockIdx.x < grid0) direct_tile<false, DNST, BT>(g0, tm0, tn0, blockIdx.x);
    else direct_tile<true, DNST, BT>(g1, tm1, tn1, blockIdx.x - grid0);
}

template <bool B_KMAJOR, int DNST, int BT>
int launch_direct_ring(const GemmArgs& a, hipStream_t st) {
    static bool ready = false;
    if (!ready) {
        PTQ_HIP(hipFuncSetAttribute((const void*)gemm_f32_direct_kernel<B_KMAJOR, DNST, BT>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, DNST * DSTAGE_BYTES<BT>));
        ready = true;
    }
    const int64_t tm = cdiv(a.M, BT), tn = cdiv(a.N, BT);
    const unsigned grid = direct_grid(a, tm, tn);
    hipLaunchKernelGGL((gemm_f32_direct_kernel<B_KMAJOR, DNST, BT>), dim3(grid), dim3(NT), DNST * DSTAGE_BYTES<BT>,
                       st, a, tm, tn);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

// Short contractions (the trailing updates) are dominated by the tile's
// prologue and C read-modify-write: a 3-stage ring (48 KB) lets a third
// workgroup per CU cover them; long ones keep the deeper ring. Products
// with fewer than SMALL_TILES 128 x 128 tiles run on 64 x 64 tiles: the U
// recursion's fp32 products (n = 28672: 121.9 ms at a threshold of 128 tiles,
// 120.7 at 512 or more) and the in-super-block updates of the column stage
// (60.3 -> 56.5 ms); the larger ones keep the denser tile.
constexpr int64_t SMALL_TILES = 1024;
template <bool B_KMAJOR>
int launch_direct(const GemmArgs& a, hipStream_t st) {
    if (cdiv(a.M, BM) * cdiv(a.N, BN) < SMALL_TILES)
        return a.K <= SHORT_K ? launch_direct_ring<B_KMAJOR, DNST_SHORT, 64>(a, st)
                              : launch_direct_ring<B_KMAJOR, DNST_LONG, 64>(a, st);
    return a.K <= SHORT_K ? launch_direct_ring<B_KMAJOR, DNST_SHORT, 128>(a, st)
                          : launch_direct_ring<B_KMAJOR, DNST_LONG, 128>(a, st);
}

bool direct_ok(const GemmArgs& a) {
    if (a.layout_a != A_MK) return false;
    if (a.K < 4 || a.K % 4 || a.lda % 4 || a.ldb % 4) return false;
    if (((uintptr_t)a.A | (uintptr_t)a.B) & 15) return false;
    if (a.layout_b == B_KN && (a.N % 4 || a.N < 4)) return false;
    return true;
}

// the launch shape launch_direct picks: tile side and ring depth
int direct_shape(const GemmArgs& a) {
    const bool small = cdiv(a.M, BM) * cdiv(a.N, BN) < SMALL_TILES;
    return (small ? 64 : 128) + (a.K <= SHORT_K ? 0 : 1);
}

template <int DNST, int BT>
int launch_direct_pair(const GemmArgs& a0, const GemmArgs& a1, hipStream_t st) {
    static bool ready = false;
    if (!ready) {
        PTQ_HIP(hipFuncSetAttribute((const void*)gemm_f32_direct_pair_kernel<DNST, BT>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, DNST * DSTAGE_BYTES<BT>));
        ready = true;
    }
    const int64_t tm0 = cdiv(a0.M, BT), tn0 = cdiv(a0.N, BT), tm1 = cdiv(a1.M, BT), tn1 = cdiv(a1.N, BT);
    const unsigned grid0 = (unsigned)cdiv(direct_grid(a0, tm0, tn0), XCDS) * XCDS, grid1 = direct_grid(a1, tm1, tn1);
    hipLaunchKernelGGL((gemm_f32_direct_pair_kernel<DNST, BT>), dim3(grid0 + grid1), dim3(NT),
                       DNST * DSTAGE_BYTES<BT>, st, a0, tm0, tn0, grid0, a1, tm1, tn1);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

}  // namespace

int launch_gemm_f32_pair(const GemmArgs& a0, const GemmArgs& a1, hipStream_t st) {
    const bool pairable = a0.M > 0 && a0.N > 0 && a1.M > 0 && a1.N > 0 && direct_ok(a0) && direct_ok(a1) &&
                          a0.layout_b == B_NK && a1.layout_b == B_KN && direct_shape(a0) == direct_shape(a1);
    if (!pairable) {
        PTQ_TRY(launch_gemm_f32(a0, st));
        return launch_gemm_f32(a1, st);
    }
    switch (direct_shape(a0)) {
        case 64: return launch_direct_pair<DNST_SHORT, 64>(a0, a1, st);
        case 65: return launch_direct_pair<DNST_LONG, 64>(a0, a1, st);
        case 128: return launch_direct_pair<DNST_SHORT, 128>(a0, a1, st);
        default: return launch_direct_pair<DNST_LONG, 128>(a0, a1, st);
    }
}

int launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return PTQ_OK;
    if (a.K <= 0 && a.beta_one) return PTQ_OK;  // C += 0
    if (direct_ok(a)) return a.layout_b == B_KN ? launch_direct<true>(a, st) : launch_direct<false>(a, st);
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
