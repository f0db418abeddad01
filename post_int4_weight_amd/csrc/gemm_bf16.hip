// bf16 "NT" GEMM on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16 or
// v_mfma_f32_32x32x16_bf16):
//
//   C[i][j] = sum_k A[i][k] B[j][k]      A [M, K], B [N, K], both K-contiguous
//
// Three uses, selected by the epilogue:
//  * the proxy Hessian H (+)= X^T X ("GPTQ versus AWQ objectives", "A strong
//    answer"), run on a transposed, panel-blocked chunk of the calibration
//    rows (xt_offset) with A = B = Xt: only tiles on or above the diagonal
//    are computed; the tile is added into H (fp32) or, when a chunk is split
//    over depth (grid.y), stored into the split's own partial H; the lower
//    triangle is mirrored by a separate pass at the end of each call;
//  * AWQ's calibration output error ||X dW^T||^2 (same page, AWQ paragraph),
//    with A = X [rows, in] and B = dW [out, in] split into a bf16 high part and
//    a bf16 residual (dW = hi + lo to ~16 significant bits): the K loop runs
//    over both halves with the same A, and the epilogue reduces the tile's
//    sum of squares to one fp64 partial per workgroup (E is never written);
//  * fp32 GEMMs C = alpha A B (+ C) whose operands arrive as three-term bf16
//    splits (the large products of the U recursion and the GPTQ trailing
//    updates; see launch_gemm_f32_split3 below).
//
// Tile 256 x 256 (or 128 x 128) per workgroup of NW wave64s in NW/2 x 2
// (WaveTile), each wave a block of MF x MF MFMA accumulators (MfmaShape):
// 256-wide tiles use 8 waves of 16x16x32, 128-wide ones 4 waves of 32x32x16.
// Two main loops: the direct-to-LDS one (K segments multiples of 64, or of
// 32, which covers every call on the path) described further down, and a
// register-staged one for any K (4 waves of 32x32x16): 16-byte chunks go
// through registers into 128-byte LDS rows whose chunk index is XOR-swizzled
// by (row >> 1) & 7, so the staging writes and the ds_read_b128 operand
// fetches are free of bank conflicts.
//
// Workgroup order is XCD-aware (blockIdx b runs on XCD b % 8): Hessian tiles
// go in rounds of 16 x 16 super-blocks dealt evenly over the XCDs (see
// hessian_tile); GEMM tile rows go to the XCDs in a zigzag; AWQ tiles in
// contiguous runs per XCD.
#include "common.hpp"
#include "tile_order.hpp"

#include <algorithm>
#include <type_traits>

namespace ptq {
namespace {

constexpr int KT = 64;              // contraction depth per LDS stage
constexpr int ROWB = KT * 2;        // bytes per staged row
constexpr int CPR = ROWB / 16;      // 16-byte chunks per staged row
constexpr int NTH = 256;
constexpr int NXCD = 8;

enum { EPI_HESSIAN = 0, EPI_SUMSQ = 1, EPI_GEMM = 2 };

__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + 16 * (c ^ ((r >> 1) & 7)); }

template <int BMX>
constexpr int smem_bytes() { return 4 * BMX * ROWB; }   // A and B, two stages each

using tile_order::SB;
using tile_order::hessian_rounds;
using tile_order::hessian_round_tiles;
using tile_order::hessian_tile;

struct Bf16GemmArgs {
    // operand segments: k in [0, K1) uses (A1, B1); k in [K1, K1 + K2) uses (A2, B2) at k - K1
    const uint16_t* A1; const uint16_t* B1;
    const uint16_t* A2; const uint16_t* B2;
    int64_t K1, K2;
    int64_t lda, ldb;
    int64_t M, N;
    int64_t b_batch_stride;    // EPI_SUMSQ / EPI_HESSIAN: B offset per blockIdx.y
    // EPI_HESSIAN split over depth: blockIdx.y takes depth [y K1, min(ktot, (y+1) K1)) of A1/B1 (A1 and B1
    // advance by a_batch_stride / b_batch_stride) and writes its own partial H at H + y * h_batch_stride
    int64_t a_batch_stride, h_batch_stride, ktot;
    // EPI_HESSIAN operands are panel-blocked (xt_offset): pstride elements per panel of BMX rows
    int64_t pstride;
    // EPI_HESSIAN
    float* H; int64_t ldh; int T; int store_not_add;
    // EPI_SUMSQ
    double* partial;           // [gridDim.y][tiles]
    int64_t tiles_n, ntiles;
    // EPI_GEMM (fp32 GEMM from three-term bf16 splits): A and B are three
    // planes each (hi, mid, lo; plane strides a_plane, b_plane elements),
    // panel-blocked like the X^T X operands (split3_offset, pstride), K1 the
    // padded depth; C = alpha * sum of the six significant plane products
    // (+ C when beta_one), with GemmArgs' tri / upper_only meaning.
    const uint16_t* Ap; const uint16_t* Bp;
    int64_t a_plane, b_plane;
    float* C; int64_t ldc;
    float alpha; int beta_one; int tri; int upper_only;
    int64_t tiles_m;
    // EPI_GEMM pair: two products with one A operand (same rows and depth) in
    // one launch; workgroups from grid0 on (a multiple of 8, so both keep the
    // XCD order) compute the second, whose B, N and output differ (grid0 = 0:
    // one product)
    int64_t grid0;
    const uint16_t* Bp2; int64_t b_plane2, N2, tiles_n2;
    float* C2; int64_t ldc2;
    float alpha2; int beta_one2; int tri2; int upper_only2;
};

// EPI_GEMM tile order (tile_order::gemm_tile with sub-blocks allowed): 4 x 8
// sub-blocks per XCD for dense products of at least 8 x 8 tiles (the GPTQ
// trailing updates: column stage -0.7 ms); the triangular ones take whole
// tile rows (A upper, upper_only) or columns (B upper) in a zigzag over the
// XCDs, which balances their uneven tile depths (sub-blocks made the factor
// 10 ms slower)
static_assert(tile_order::TRI_NONE_ == TRI_NONE && tile_order::TRI_A_UP == TRI_A_UPPER &&
                  tile_order::TRI_B_UP_KN == TRI_B_UPPER_KN && tile_order::TRI_B_UP_NK == TRI_B_UPPER_NK,
              "triangle codes");

// AWQ error tiles: 4 x 8 sub-blocks of the tile grid dealt round-robin to
// the XCDs, so the 32 tiles an XCD runs side by side read 12 panels through
// its L2 (a contiguous run of whole tile rows: 33). Returns the tile's
// row-major index tm * tiles_n + tn, or -1 for a slot past the grid.
__host__ __device__ inline int64_t sumsq_tile(uint32_t b, int64_t tiles_m, int64_t tiles_n) {
    // 32-bit arithmetic (tile counts are small): with 64-bit the AWQ kernel
    // spilled 5 registers
    const uint32_t x = b % NXCD, i = b / NXCD, sbc = (uint32_t)(tiles_n + 7) / 8;
    const uint32_t sbi = NXCD * (i / 32) + x, w = i % 32;
    const uint32_t tm = 4 * (sbi / sbc) + w / 8, tn = 8 * (sbi % sbc) + w % 8;
    return (tm < tiles_m && tn < tiles_n) ? (int64_t)tm * tiles_n + tn : -1;
}
inline int64_t sumsq_grid(int64_t tiles_m, int64_t tiles_n) {
    return ((((tiles_m + 3) / 4) * ((tiles_n + 7) / 8) + NXCD - 1) / NXCD) * NXCD * 32;
}

template <int BMX>
struct Stg {
    uint4 a[BMX * CPR / NTH];
    uint4 b[BMX * CPR / NTH];
};

// Load this thread's share of a K-slab of one operand panel (rows x0.., k0..k0+KT-1).
// GUARD = false: the whole slab is inside the matrix (no bounds checks).
template <int BMX, bool GUARD>
__device__ __forceinline__ void load_panel(uint4 (&v)[BMX * CPR / NTH], const uint16_t* P, int64_t ld,
                                           int64_t x0, int64_t X, int64_t k0, int64_t K, int t) {
    if (!GUARD) {
        const uint16_t* base = P + x0 * ld + k0;
#pragma unroll
        for (int q = 0; q < BMX * CPR / NTH; ++q) {
            const int idx = t + NTH * q;
            const int r = idx / CPR, c = idx % CPR;
            v[q] = *(const uint4*)(base + (int64_t)r * ld + 8 * c);
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < BMX * CPR / NTH; ++q) {
        const int idx = t + NTH * q;          // BMX rows x CPR chunks
        const int r = idx / CPR, c = idx % CPR;
        const int64_t row = x0 + r, k = k0 + 8 * c;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (row < X) {
            const uint16_t* p = P + row * ld + k;
            if (k + 8 <= K) {
                val = *(const uint4*)p;
            } else if (k < K) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8; ++e)
                    if (k + e < K) w[e >> 1] |= ((uint32_t)p[e]) << (16 * (e & 1));
                val = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        v[q] = val;
    }
}

template <int BMX>
__device__ __forceinline__ void store_panel(unsigned char* S, const uint4 (&v)[BMX * CPR / NTH], int t) {
#pragma unroll
    for (int q = 0; q < BMX * CPR / NTH; ++q) {
        const int idx = t + NTH * q;
        const int r = idx / CPR, c = idx % CPR;
        *(uint4*)(S + swz(r, c)) = v[q];
    }
}

// Depth of the first operand segment for this workgroup's blockIdx.y (split
// over depth when ktot > 0, else K1).
__device__ __forceinline__ int64_t split_depth(const Bf16GemmArgs& g) {
    if (g.ktot <= 0) return g.K1;
    return std::max<int64_t>(0, std::min<int64_t>(g.K1, g.ktot - (int64_t)blockIdx.y * g.K1));
}

// The two bf16 MFMA shapes. Operands: lane l supplies row l % MF of its
// block and the 8 consecutive k at 8 * (l / MF) of the k-step (KDEP deep).
// Accumulator register r of lane l holds row row(l, r), column col(l).
template <int MF>
struct MfmaShape;
template <>
struct MfmaShape<32> {   // v_mfma_f32_32x32x16_bf16
    using acc_t = f32x16;
    static constexpr int NACC = 16, KDEP = 16;
    __device__ static __forceinline__ int row(int l, int r) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }
    __device__ static __forceinline__ int col(int l) { return l & 31; }
    __device__ static __forceinline__ acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<16> {   // v_mfma_f32_16x16x32_bf16
    using acc_t = f32x4;
    static constexpr int NACC = 4, KDEP = 32;
    __device__ static __forceinline__ int row(int l, int r) { return 4 * (l >> 4) + r; }
    __device__ static __forceinline__ int col(int l) { return l & 15; }
    __device__ static __forceinline__ acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// Wave layout of a BMX x BMX tile over NW waves: NW / 2 rows x 2 columns of
// waves, each a (WA x MF) x (WB x MF) block of MF x MF MFMA accumulators.
template <int BMX, int NW, int MF = 32>
struct WaveTile {
    static constexpr int TM = BMX / (NW / 2), TN = BMX / 2;
    static constexpr int WA = TM / MF, WB = TN / MF;
    using acc_t = typename MfmaShape<MF>::acc_t;
};

template <int BMX, int EPI, int NW = 4, int MF = 32>
__device__ __forceinline__ void store_tile(
    const Bf16GemmArgs& g,
    typename WaveTile<BMX, NW, MF>::acc_t (&acc)[WaveTile<BMX, NW, MF>::WA][WaveTile<BMX, NW, MF>::WB], int64_t i0,
    int64_t j0, int64_t L, unsigned char* smem);

// Register-staged variant: any shape (bounds-checked loads, zero fill).
template <int BMX, int EPI>
__global__ __launch_bounds__(NTH, 1) void gemm_bf16_nt_kernel(Bf16GemmArgs g, int64_t nwork) {
    constexpr int WT = BMX / 64;
    int64_t i0, j0, L = 0;
    if (EPI == EPI_HESSIAN) {
        int ti, tj;
        if (!hessian_tile(blockIdx.x, g.T, ti, tj)) return;
        i0 = (int64_t)ti * BMX;
        j0 = (int64_t)tj * BMX;
    } else {
        L = sumsq_tile(blockIdx.x, nwork / g.tiles_n, g.tiles_n);
        if (L < 0) return;
        i0 = (L / g.tiles_n) * BMX;
        j0 = (L % g.tiles_n) * BMX;
    }
    const uint16_t* A1 = g.A1 + (int64_t)blockIdx.y * g.a_batch_stride;
    const uint16_t* B1 = g.B1 + (int64_t)blockIdx.y * g.b_batch_stride;
    const uint16_t* B2 = g.B2 ? g.B2 + (int64_t)blockIdx.y * g.b_batch_stride : nullptr;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto smA = [&](int buf) { return smem + buf * (BMX * ROWB); };
    auto smB = [&](int buf) { return smem + (2 + buf) * (BMX * ROWB); };
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * (BMX / 2), wn = (wave & 1) * (BMX / 2);
    const int li = lane & 31, lh = lane >> 5;

    f32x16 acc[WT][WT];
#pragma unroll
    for (int a = 0; a < WT; ++a)
#pragma unroll
        for (int b = 0; b < WT; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int64_t K1 = split_depth(g);
    const int64_t n1 = cdiv(K1, KT), n2 = cdiv(g.K2, KT);
    const int64_t nst = n1 + n2;
    Stg<BMX> rg;
    const bool rows_full = (i0 + BMX <= g.M) && (j0 + BMX <= g.N);
    auto gload = [&](int64_t s) {
        const bool seg1 = s < n1;
        const uint16_t* A = seg1 ? A1 : g.A2;
        const uint16_t* B = seg1 ? B1 : B2;
        const int64_t K = seg1 ? K1 : g.K2;
        const int64_t k0 = (seg1 ? s : s - n1) * KT;
        if (rows_full && k0 + KT <= K) {
            load_panel<BMX, false>(rg.a, A, g.lda, i0, g.M, k0, K, t);
            load_panel<BMX, false>(rg.b, B, g.ldb, j0, g.N, k0, K, t);
        } else {
            load_panel<BMX, true>(rg.a, A, g.lda, i0, g.M, k0, K, t);
            load_panel<BMX, true>(rg.b, B, g.ldb, j0, g.N, k0, K, t);
        }
    };

    if (nst > 0) {
        gload(0);
        store_panel<BMX>(smA(0), rg.a, t);
        store_panel<BMX>(smB(0), rg.b, t);
    }
    __syncthreads();
    for (int64_t s = 0; s < nst; ++s) {
        const int cur = (int)(s & 1);
        const bool more = s + 1 < nst;
        if (more) gload(s + 1);
        const unsigned char* As = smA(cur);
        const unsigned char* Bs = smB(cur);
        // operand fragments double-buffered in registers: the LDS reads for
        // sub-step kk+1 are in flight while the MFMAs of sub-step kk run
        bf16x8 av[2][WT], bv[2][WT];
        auto frags = [&](int kk, int slot) {
#pragma unroll
            for (int a = 0; a < WT; ++a) av[slot][a] = *(const bf16x8*)(As + swz(wm + 32 * a + li, 2 * kk + lh));
#pragma unroll
            for (int b = 0; b < WT; ++b) bv[slot][b] = *(const bf16x8*)(Bs + swz(wn + 32 * b + li, 2 * kk + lh));
        };
        frags(0, 0);
#pragma unroll
        for (int kk = 0; kk < KT / 16; ++kk) {
            const int slot = kk & 1;
            if (kk + 1 < KT / 16) frags(kk + 1, slot ^ 1);
#pragma unroll
            for (int a = 0; a < WT; ++a)
#pragma unroll
                for (int b = 0; b < WT; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[slot][a], bv[slot][b], acc[a][b], 0, 0, 0);
        }
        if (more) {
            store_panel<BMX>(smA(cur ^ 1), rg.a, t);
            store_panel<BMX>(smB(cur ^ 1), rg.b, t);
        }
        __syncthreads();
    }

    store_tile<BMX, EPI>(g, acc, i0, j0, L, smem);
}

// Tile epilogue (accumulator layout in MfmaShape). `smem` is free scratch by now.
template <int BMX, int EPI, int NW, int MF>
__device__ __forceinline__ void store_tile(
    const Bf16GemmArgs& g,
    typename WaveTile<BMX, NW, MF>::acc_t (&acc)[WaveTile<BMX, NW, MF>::WA][WaveTile<BMX, NW, MF>::WB], int64_t i0,
    int64_t j0, int64_t L, unsigned char* smem) {
    using WTL = WaveTile<BMX, NW, MF>;
    using Sh = MfmaShape<MF>;
    constexpr int WA = WTL::WA, WB = WTL::WB, NACC = Sh::NACC;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * WTL::TM, wn = (wave & 1) * WTL::TN;
    const int mi = (int)std::min<int64_t>(BMX, g.M - i0);   // valid rows / columns of this tile
    const int nj = (int)std::min<int64_t>(BMX, g.N - j0);
    // A full tile that adds into C (or H) reads the current values of each
    // row block of the wave together, one block ahead of the block it adds
    // and stores: a few waits per tile instead of one memory round trip per
    // element. With one wait per element the read-modify-write took about
    // 90 us per 256 x 256 tile (an X^T X launch of the down_proj shape runs
    // 25 tiles per CU); batched, about 45 us, most of it the burst of H
    // traffic when a round's tiles end together.
    auto add_store_full = [&](float* Ct, int64_t ld, float alpha) {
        float old[2][WB][NACC];
        auto load_block = [&](int a, int slot) {
#pragma unroll
            for (int b = 0; b < WB; ++b)
#pragma unroll
                for (int r = 0; r < NACC; ++r)
                    old[slot][b][r] = Ct[(int64_t)(wm + MF * a + Sh::row(lane, r)) * ld + wn + MF * b + Sh::col(lane)];
        };
        load_block(0, 0);
#pragma unroll
        for (int a = 0; a < WA; ++a) {
            if (a + 1 < WA) load_block(a + 1, (a + 1) & 1);
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                const int jj = wn + MF * b + Sh::col(lane);
#pragma unroll
                for (int r = 0; r < NACC; ++r) {
                    const int ii = wm + MF * a + Sh::row(lane, r);
                    const float v = old[a & 1][b][r] + alpha * acc[a][b][r];
                    Ct[(int64_t)ii * ld + jj] = v;
                }
            }
        }
    };
    if (EPI == EPI_HESSIAN) {
        float* Hy = g.H + (int64_t)blockIdx.y * g.h_batch_stride;
        float* Ht = Hy + i0 * g.ldh + j0;                       // tile origin
        const int ld = (int)g.ldh;
        if (mi == BMX && nj == BMX && !g.store_not_add) {
            add_store_full(Ht, ld, 1.f);
            return;
        }
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                const int jj = wn + MF * b + Sh::col(lane);
#pragma unroll
                for (int r = 0; r < NACC; ++r) {
                    const int ii = wm + MF * a + Sh::row(lane, r);
                    if (ii < mi && jj < nj) {
                        float* p = Ht + (int64_t)ii * ld + jj;
                        const float v = g.store_not_add ? acc[a][b][r] : (*p + acc[a][b][r]);
                        *p = v;
                    }
                }
            }
    } else if (EPI == EPI_GEMM) {
        float* Ct = g.C + i0 * g.ldc + j0;
        if (mi == BMX && nj == BMX && g.beta_one) {
            add_store_full(Ct, g.ldc, g.alpha);
            return;
        }
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                const int jj = wn + MF * b + Sh::col(lane);
#pragma unroll
                for (int r = 0; r < NACC; ++r) {
                    const int ii = wm + MF * a + Sh::row(lane, r);
                    if (ii < mi && jj < nj) {
                        float* p = Ct + (int64_t)ii * g.ldc + jj;
                        const float v = g.alpha * acc[a][b][r];
                        *p = g.beta_one ? *p + v : v;
                    }
                }
            }
    } else {
        double s = 0.0;
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                float part = 0.f;
                const int jj = wn + MF * b + Sh::col(lane);
#pragma unroll
                for (int r = 0; r < NACC; ++r) {
                    const int ii = wm + MF * a + Sh::row(lane, r);
                    const float v = (ii < mi && jj < nj) ? acc[a][b][r] : 0.f;
                    part = fmaf(v, v, part);
                }
                s += (double)part;
            }
        // wave reduction (fixed order), then across the waves through LDS
        // (the staging buffers are free after the last barrier)
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        double* red = (double*)smem;
        if (lane == 0) red[wave] = s;
        __syncthreads();
        if (t == 0) {
            double tot = 0.0;
#pragma unroll
            for (int w = 0; w < NW; ++w) tot += red[w];
            g.partial[(int64_t)blockIdx.y * g.ntiles + L] = tot;
        }
    }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K1 and K2 multiples of DKT). global_load_lds_dwordx4
// moves each lane's 16 bytes straight into LDS at base + 16 * lane, so no
// staging registers and no ds_write are spent; the XOR swizzle is applied on
// the global side by choosing which chunk each lane fetches. A ring of NST
// stages, each DKT deep, keeps the next stages' loads in flight behind the
// MFMAs. With DKT = 64 one load instruction covers eight whole 128-byte rows
// of a panel slice (a 32-deep stage moves half rows, so every cache line is
// requested twice, one stage apart) and there is one barrier per 64 of depth.
// Rows past M (or N) read a clamped valid row: they only feed output rows
// (columns) that the epilogue discards.
template <int DKT>
struct DStage {
    static constexpr int ROWB = DKT * 2;            // bytes per staged row
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per staged row
    static constexpr int KSUB = DKT / 16;           // MFMA k-steps per stage
    // Slot of chunk c in row r: the 16 lanes of one ds_read_b128 phase read 16
    // consecutive rows at one chunk, and these swizzles put them on 64
    // distinct banks (rows sharing a 256-byte bank window get distinct slots).
    __device__ static __forceinline__ int sw(int r) { return DKT == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
};

// ring depth per stage depth: 4 x 32 or 2 x 64 (128 KB of LDS at BMX = 256)
template <int DKT>
constexpr int DNST = DKT == 32 ? 4 : 2;

template <int BMX, int DKT, int NST>
constexpr int dsmem_bytes() { return NST * 2 * BMX * DStage<DKT>::ROWB; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int N, bool LGKM0>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt at its maximum,
    // lgkmcnt at 0 (LGKM0) or at its maximum
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8));
}

template <int BMX, int EPI, int DKT, int NST, int NW, int MF>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_nt_direct_kernel(Bf16GemmArgs g_in, int64_t nwork) {
    using S = DStage<DKT>;
    using WTL = WaveTile<BMX, NW, MF>;
    using Sh = MfmaShape<MF>;
    constexpr int ROWB = S::ROWB, KSUB = DKT / Sh::KDEP;
    constexpr int WA = WTL::WA, WB = WTL::WB;          // accumulator blocks per wave (rows, columns)
    constexpr int NM = WA * WB, NR = WA + WB;          // MFMAs and fragment reads per k-step
    // X^T X: only the first wave of each SIMD (waves 0 .. NW/2 - 1) issues
    // the copies, so a copy that stalls at issue holds one of the SIMD's two
    // waves while the other keeps the MFMA pipe busy (2% on the down_proj
    // shape against copies from every wave).
    constexpr bool BLK = EPI == EPI_HESSIAN || EPI == EPI_GEMM;   // panel-blocked operands
    // waves that issue copies: half of them for X^T X; all of them for the
    // split planes (there half measured 9% slower: 124 vs 114 ms for the U
    // of n = 28672, against 110.5 ms with all eight)
    constexpr int CWV = (EPI == EPI_HESSIAN) ? NW / 2 : NW;
    constexpr int PER = BMX * S::CH / (64 * CWV);      // copies per copying wave per panel per stage
    constexpr int PANEL = BMX * ROWB;                  // bytes of one operand panel per stage
    static_assert(NST >= 2 && KSUB % 2 == 0 && NM >= NR && PER >= 1, "pipeline shape");
    static_assert(!BLK || (DKT == 64 && PER % 2 == 0), "panel-blocked copy layout");
    Bf16GemmArgs g = g_in;
    unsigned bid = blockIdx.x;
    if constexpr (EPI == EPI_GEMM) {
        if (g.grid0 > 0 && bid >= (unsigned)g.grid0) {
            bid -= (unsigned)g.grid0;
            g.Bp = g.Bp2; g.b_plane = g.b_plane2; g.N = g.N2; g.tiles_n = g.tiles_n2;
            g.C = g.C2; g.ldc = g.ldc2;
            g.alpha = g.alpha2; g.beta_one = g.beta_one2; g.tri = g.tri2; g.upper_only = g.upper_only2;
        }
    }
    int64_t i0, j0, L = 0;
    if (EPI == EPI_HESSIAN) {
        int ti, tj;
        if (!hessian_tile(blockIdx.x, g.T, ti, tj)) return;
        i0 = (int64_t)ti * BMX;
        j0 = (int64_t)tj * BMX;
    } else if (EPI == EPI_GEMM) {
        int64_t tm, tn;
        if (!tile_order::gemm_tile(bid, g.tiles_m, g.tiles_n, g.tri, g.upper_only, true, tm, tn)) return;
        i0 = tm * BMX;
        j0 = tn * BMX;
    } else {
        L = sumsq_tile(blockIdx.x, nwork / g.tiles_n, g.tiles_n);
        if (L < 0) return;
        i0 = (L / g.tiles_n) * BMX;
        j0 = (L % g.tiles_n) * BMX;
    }
    const uint16_t* A1 = g.A1 + (int64_t)blockIdx.y * g.a_batch_stride;
    const uint16_t* B1 = g.B1 + (int64_t)blockIdx.y * g.b_batch_stride;
    const uint16_t* B2 = g.B2 ? g.B2 + (int64_t)blockIdx.y * g.b_batch_stride : nullptr;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int t = threadIdx.x;
    // panel-blocked operands keep the wave index in an SGPR (scalar copy addressing and branch)
    const int lane = t & 63, wave = BLK ? __builtin_amdgcn_readfirstlane(t >> 6) : t >> 6;
    const int wm = (wave >> 1) * WTL::TM, wn = (wave & 1) * WTL::TN;
    const int cw = wave % CWV;                           // copy slot of this wave
    const bool copier = CWV == NW || wave < CWV;
    const int li = lane & 31, lh = lane >> 5;

    // Copy q of a wave moves the 16-byte granules p = 64 (cw PER + q) + lane
    // of a panel's stage: row r = p / CH, chunk (p % CH) ^ sw(r).
    // X^T X (panel-blocked Xt, xt_offset; a stage of a panel is a contiguous
    // BMX x 64 block): with q' = cw PER + q, r = 8 q' + lane / 8 and
    // sw(r) = (4 (q' & 1) + lane / 16) & 7, so the element offset within the
    // block is 512 q' plus one of two lane terms by the parity of q'. These
    // copies go through buffer resources (no per-copy 64-bit address
    // arithmetic: 41.7 -> 41.1 ms per 65536-row chunk of the down_proj shape).
    const int64_t hA = (i0 / BMX) * g.pstride, hB = (j0 / BMX) * g.pstride;
    const int lo0 = (lane >> 3) * 64 + 8 * ((lane & 7) ^ (lane >> 4));
    const int lo1 = (lane >> 3) * 64 + 8 * ((lane & 7) ^ (4 + (lane >> 4)));
    // X^T X copies through buffer resources of the tile's two panels (this
    // split's part of them), byte offsets of the lane by parity and half
    const int left = (EPI == EPI_HESSIAN) ? (int)(2 * (g.pstride - (int64_t)blockIdx.y * g.a_batch_stride)) : 0;
    __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.A1 + (int64_t)blockIdx.y * g.a_batch_stride + (EPI == EPI_HESSIAN ? hA : 0)), (short)0, left, 0x00020000);
    __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.B1 + (int64_t)blockIdx.y * g.b_batch_stride + (EPI == EPI_HESSIAN ? hB : 0)), (short)0, left, 0x00020000);
    unsigned vo00 = 0, vo01 = 0, vo10 = 0, vo11 = 0;
    if constexpr (BLK) {
        const unsigned cb = (unsigned)(cw * PER) * 1024u;
        vo00 = 2u * lo0 + cb;
        vo10 = 2u * lo1 + cb;
        vo01 = vo00 + 4096u;
        vo11 = vo10 + 4096u;
    }
    // other products: element offsets from the operand base, rows clamped to the operand
    int64_t offA[PER], offB[PER];
    if constexpr (!BLK) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int p = (cw * PER + q) * 64 + lane;
            const int r = p / S::CH;
            const int c = (p % S::CH) ^ S::sw(r);
            const int64_t ra = std::min<int64_t>(i0 + r, g.M - 1);
            const int64_t rb = std::min<int64_t>(j0 + r, g.N - 1);
            offA[q] = ra * g.lda + 8 * c;
            offB[q] = rb * g.ldb + 8 * c;
        }
    }
    int64_t n1 = split_depth(g) / DKT, nst = n1 + g.K2 / DKT;
    int64_t kb = 0;
    if (EPI == EPI_GEMM) {
        // depth range of the tile (triangular operands skip their zero
        // blocks); stage s covers depth kb + (s / 6) * DKT in plane pair s % 6
        int64_t ke = g.K1;
        if (g.tri == TRI_A_UPPER) kb = i0;
        else if (g.tri == TRI_B_UPPER_NK) kb = j0;
        else if (g.tri == TRI_B_UPPER_KN) ke = std::min<int64_t>(g.K1, j0 + BMX);
        nst = (ke > kb) ? 6 * ((ke - kb) / DKT) : 0;
    }
    // EPI_GEMM: stage s of the tile's A (or B) panel, one contiguous
    // BMX x DKT block of a plane; plane pairs (A, B) by s % 6: hi.hi,
    // hi.mid, mid.hi, hi.lo, lo.hi, mid.mid
    auto gemm_block = [&](int64_t s, bool isa) -> const uint16_t* {
        const int si = (int)s, kc = si / 6, pq = si - 6 * kc;
        const int pl = isa ? ((0x120100 >> (4 * pq)) & 15) : ((0x102010 >> (4 * pq)) & 15);
        return (isa ? g.Ap + pl * g.a_plane + hA : g.Bp + pl * g.b_plane + hB) +
               (kb / DKT + kc) * (int64_t)(BMX * DKT);
    };
    // operand bases of stage s
    auto stage_a = [&](int64_t s) -> const uint16_t* {
        if constexpr (EPI == EPI_HESSIAN || EPI == EPI_GEMM) {
            return A1 + s * (BMX * DKT);
        } else {
            return s < n1 ? A1 + s * DKT : g.A2 + (s - n1) * DKT;
        }
    };
    auto stage_b = [&](int64_t s) -> const uint16_t* {
        if constexpr (EPI == EPI_HESSIAN || EPI == EPI_GEMM) {
            return B1 + s * (BMX * DKT);
        } else {
            return s < n1 ? B1 + s * DKT : B2 + (s - n1) * DKT;
        }
    };

    // one 16-byte-per-lane copy: q < PER moves A's granules, else B's
    auto load_one = [&](int64_t s, int buf, auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr bool isa = q < PER;
        constexpr int qq = isa ? q : q - PER;
        if constexpr (BLK) {
            // Buffer copies: the panel's resource in SGPRs, the stage's byte
            // offset in soffset (X^T X; the split planes take a resource per
            // stage block), the lane's 32-bit offset (one of four: parity x
            // half) in voffset, and k KB in the immediate, which applies to
            // the global and the LDS address alike, so copies qq = 4 h + k of
            // a half h share one M0 (PER is even: q' and qq have one parity)
            constexpr int h = qq >> 2, k = qq & 3;
            unsigned char* lb = smem + buf * (2 * PANEL) + (isa ? 0 : PANEL) + (cw * PER + 4 * h) * 1024;
            const unsigned vo = (qq & 1) ? (h ? vo11 : vo10) : (h ? vo01 : vo00);
            if constexpr (EPI == EPI_HESSIAN)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? rsa : rsb, (lds_ptr_t)lb, 16, vo,
                                                         (unsigned)(s * (BMX * DKT * 2)), k * 1024, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    __builtin_amdgcn_make_buffer_rsrc((void*)gemm_block(s, isa), (short)0, BMX * DKT * 2, 0x00020000),
                    (lds_ptr_t)lb, 16, vo, 0u, k * 1024, 0);
        } else {
            const uint16_t* P = isa ? stage_a(s) + offA[qq] : stage_b(s) + offB[qq];
            unsigned char* dst = smem + buf * (2 * PANEL) + (isa ? 0 : PANEL) + (cw * PER + qq) * 1024;
            __builtin_amdgcn_global_load_lds((const void*)P, (lds_ptr_t)dst, 16, 0, 0);
        }
    };
    auto issue = [&](int64_t s, int buf) { static_for<0, 2 * PER>([&](auto qc) { load_one(s, buf, qc); }); };

    typename WTL::acc_t acc[WA][WB];
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int r = 0; r < Sh::NACC; ++r) acc[a][b][r] = 0.f;

    // Software pipeline over k-steps (16 deep): the fragment reads of the next
    // k-step are interleaved with the MFMAs of the current one, so after the
    // prologue no LDS latency is exposed. The stage barrier sits before a
    // stage's last k-step, whose fragments are already in registers: each
    // wave first waits until its reads of the stage have returned (lgkmcnt 0)
    // and its copies of the next stage have landed (loads retire in order, so
    // only the younger stages' copies may still be outstanding); after the
    // barrier (no memory fence, which would drain every prefetch) the next
    // stage is visible to all waves and this stage's buffer is free, and the
    // copies of stage s + NST go into it.
    const int fr = lane % MF;     // operand row of this lane within a block
    const int fsw = S::sw(fr);    // fragment swizzle term, lane-only (row = wm + MF a + fr)
    bf16x8 fa[2][WA], fb[2][WB];
    // k-step kk reads chunk (KDEP / 8) kk + lane / MF of its rows
    auto fragp = [&](int64_t s, int kk) {
        return smem + (s % NST) * (2 * PANEL) + 16 * (((Sh::KDEP / 8) * kk + lane / MF) ^ fsw);
    };
    // fragment q of a k-step, in the order the MFMAs (a-major) consume them:
    // A block 0, the B blocks, then the other A blocks
    auto read_one = [&](int64_t s, int kk, int slot, int q) {
        const unsigned char* As = fragp(s, kk);
        if (q == 0) fa[slot][0] = *(const bf16x8*)(As + (wm + fr) * ROWB);
        else if (q <= WB) fb[slot][q - 1] = *(const bf16x8*)(As + PANEL + (wn + MF * (q - 1) + fr) * ROWB);
        else fa[slot][q - WB] = *(const bf16x8*)(As + (wm + MF * (q - WB) + fr) * ROWB);
    };
    auto frags = [&](int64_t s, int kk, int slot) {
#pragma unroll
        for (int q = 0; q < NR; ++q) read_one(s, kk, slot, q);
    };
    auto mfma_one = [&](int slot, int idx) {
        const int a = idx / WB, b = idx % WB;
        acc[a][b] = Sh::mfma(fa[slot][a], fb[slot][b], acc[a][b]);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < NM; ++i) mfma_one(slot, i);
    };
    // The NR reads of the next k-step ride under the first NR MFMAs of the
    // current one, one per MFMA, so the last of them has the remaining
    // NM - NR MFMAs' time to return before the next k-step needs it.
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    };

    // Past the last stage the issue repeats the last stage into the free
    // buffer, so the counts (and the waits) are the same on every iteration
    // and the loop has no joins that would force a full lgkmcnt drain.
    if (nst > 0) {
        if (copier) {
#pragma unroll
            for (int s = 0; s < NST; ++s) issue(std::min<int64_t>(s, nst - 1), s);
        }
        wait_vmcnt<(NST - 1) * 2 * PER, false>();
        __builtin_amdgcn_s_barrier();
        frags(0, 0, 0);
        auto steps = [&](int64_t s) {
#pragma unroll
            for (int kk = 0; kk + 1 < KSUB; ++kk) {
                frags(s, kk + 1, (kk + 1) & 1);
                mfmas(kk & 1);
                interleave();
            }
        };
        for (int64_t s = 0; s + 1 < nst; ++s) {
            steps(s);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(NST - 2) * 2 * PER, true>();
            __builtin_amdgcn_s_barrier();
            {
                // After the barrier: the last k-step's MFMAs, the next
                // stage's first fragment reads (one after each of the first
                // NR MFMAs) and the 2 PER copies of stage s + NST spread
                // evenly over the MFMAs, pinned in that order: a copy that
                // waits for the address unit stalls at most one MFMA's issue.
                const int64_t sl = std::min<int64_t>(s + NST, nst - 1);
                const int bl = (int)(s % NST);
                constexpr int NL = 2 * PER;
                static_for<0, NM>([&](auto mc) {
                    constexpr int m = decltype(mc)::value;
                    mfma_one(1, m);
                    if constexpr (m < NR) read_one(s + 1, 0, 0, m);
                    if (copier) static_for<m * NL / NM, (m + 1) * NL / NM>([&](auto lc) { load_one(sl, bl, lc); });
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        }
        steps(nst - 1);
        mfmas(1);
    }
    wait_vmcnt<0, true>();
    __syncthreads();
    store_tile<BMX, EPI, NW, MF>(g, acc, i0, j0, L, smem);
}

// Opt a kernel into more than 64 KB of dynamic LDS (once per instantiation).
template <int BMX, int EPI, int DKT, int NW = 4, int MF = 32>
int prepare_kernel() {
    static bool done = false;
    if (!done) {
        if constexpr (DKT > 0)
            PTQ_HIP(hipFuncSetAttribute((const void*)gemm_bf16_nt_direct_kernel<BMX, EPI, DKT, DNST<DKT>, NW, MF>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        dsmem_bytes<BMX, DKT, DNST<DKT>>()));
        else
            PTQ_HIP(hipFuncSetAttribute((const void*)gemm_bf16_nt_kernel<BMX, EPI>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, smem_bytes<BMX>()));
        done = true;
    }
    return PTQ_OK;
}

template <int BMX, int EPI, int DKT, int NW = 4, int MF = 32>
int launch_direct(const Bf16GemmArgs& g, int64_t nwork, unsigned grid, unsigned grid_y, hipStream_t st) {
    constexpr int nst = DNST<DKT>;
    constexpr int lds = dsmem_bytes<BMX, DKT, nst>();
    PTQ_TRY((prepare_kernel<BMX, EPI, DKT, NW, MF>()));
    hipLaunchKernelGGL((gemm_bf16_nt_direct_kernel<BMX, EPI, DKT, nst, NW, MF>), dim3(grid, grid_y), dim3(64 * NW),
                       lds, st, g, nwork);
    return PTQ_OK;
}

// Direct kernel at 64-deep stages and 256-wide tiles: eight waves (two per
// SIMD, 64 x 128 accumulators each) let one wave issue MFMAs while the other
// waits on a fragment read, a copy or the barrier; 16x16x32 MFMAs (16 cycles
// each, 4 accumulator registers) interleave those waits at half the grain of
// 32x32x16 ones. Measured on X^T X per 65536-row chunk: 4 waves / 32x32
// 51.3 ms, 8 / 32x32 50.1, 8 / 16x16 46.1, 4 / 16x16 58.9.
constexpr int DNW = 8;
constexpr int DMF = 16;

// Launch the direct variant when both K segments are multiples of its stage
// depth (64, else 32), the register-staged one otherwise.
template <int BMX, int EPI>
int launch_nt(const Bf16GemmArgs& g, int64_t nwork, unsigned grid_y, hipStream_t st) {
    const unsigned grid = (unsigned)(EPI == EPI_HESSIAN ? 256 * hessian_rounds(g.T) : sumsq_grid(nwork / g.tiles_n, g.tiles_n));
    if (g.M > 0 && g.N > 0 && g.K1 % 64 == 0 && g.K2 % 64 == 0) {
        PTQ_TRY((launch_direct<BMX, EPI, 64, BMX == 256 ? DNW : 4, BMX == 256 ? DMF : 32>(g, nwork, grid, grid_y, st)));
    } else if constexpr (EPI == EPI_HESSIAN) {
        // X^T X pads every chunk's depth to a multiple of 64
        set_error("X^T X tiles: depth %lld is not a multiple of 64", (long long)g.K1);
        return PTQ_EINVAL;
    } else if (g.M > 0 && g.N > 0 && g.K1 % 32 == 0 && g.K2 % 32 == 0) {
        PTQ_TRY((launch_direct<BMX, EPI, 32>(g, nwork, grid, grid_y, st)));
    } else {
        PTQ_TRY((prepare_kernel<BMX, EPI, 0>()));
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<BMX, EPI>), dim3(grid, grid_y), dim3(NTH), smem_bytes<BMX>(), st,
                           g, nwork);
    }
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

// ---------------------------------------------------------------------------
// fp32 GEMM on the bf16 MFMA. Each fp32 operand x is split into three bf16
// terms, hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid) (both
// differences are exact in fp32), so x = hi + mid + lo to about 2^-24
// relative: 24 significant bits, fp32's own. A product keeps the six term
// products down to 2^-16 (hi.hi, hi.mid, mid.hi, hi.lo, lo.hi, mid.mid) and
// drops those of order 2^-24 and below; each term product is exact and all
// six accumulate in the same fp32 MFMA accumulators, so the result carries
// fp32 GEMM accuracy at six bf16 MFMAs (16 x the fp32 MFMA's rate each) per
// block and k-step.
__device__ __forceinline__ void split3(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
    if (!(fabsf(x) <= 3.3e38f)) {   // NaN / Inf (or a value bf16 rounding would overflow): keep hi only
        h = (uint16_t)(__float_as_uint(x) >> 16) | (uint16_t)((x != x) ? 0x40 : 0);
        m = l = 0;
        return;
    }
    h = float_to_bf16_bits(x);
    const float r1 = x - bf16_bits_to_float(h);
    m = float_to_bf16_bits(r1);
    l = float_to_bf16_bits(r1 - bf16_bits_to_float(m));
}

__device__ __forceinline__ void split3_store8(const float (&v)[8], uint16_t* p, int64_t plane) {
    uint16_t h[8], m[8], l[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) split3(v[q], h[q], m[q], l[q]);
    auto pack = [](const uint16_t (&u)[8]) {
        return make_uint4((uint32_t)u[0] | ((uint32_t)u[1] << 16), (uint32_t)u[2] | ((uint32_t)u[3] << 16),
                          (uint32_t)u[4] | ((uint32_t)u[5] << 16), (uint32_t)u[6] | ((uint32_t)u[7] << 16));
    };
    *(uint4*)p = pack(h);
    *(uint4*)(p + plane) = pack(m);
    *(uint4*)(p + 2 * plane) = pack(l);
}

// Split planes are panel-blocked like the X^T X operands: element (r, k) of
// a plane sits at (r / 256) pstride + (k / 64) 256 * 64 + (r % 256) 64 + k % 64,
// so one 64-deep stage of a 256-row panel is one contiguous 32 KB block.
// Panels are padded to 256 rows (zeros) and pstride = 256 (kp + 64): one
// spare stage per panel keeps panels off power-of-two distances.
constexpr int SPLIT_PANEL = 256;
__host__ __device__ inline int64_t split3_pstride(int64_t kp) { return SPLIT_PANEL * (kp + 64); }
__device__ __forceinline__ int64_t split3_offset(int64_t r, int64_t k, int64_t pstride) {
    return (r / SPLIT_PANEL) * pstride + (k >> 6) * (SPLIT_PANEL * 64) + (r % SPLIT_PANEL) * 64 + (k & 63);
}

// P[t] (t = hi, mid, lo; plane stride plane, blocked as split3_offset) from
// S[r][k] = X[r * ldx + k] for r < R and k < K, zero for the padding rows
// R <= r < Rp and depth K <= k < kp (kp % 64 == 0).
__global__ __launch_bounds__(256) void split3_rows_kernel(const float* __restrict__ X, int64_t ldx, int64_t R,
                                                          int64_t Rp, int64_t K, int vec, uint16_t* __restrict__ P,
                                                          int64_t pstride, int64_t kp, int64_t plane) {
    const int64_t nch = kp / 8;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < Rp * nch; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / nch, k0 = 8 * (e % nch);
        float v[8];
        if (r >= R) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = 0.f;
        } else if (vec && k0 + 8 <= K) {
            const float* x = X + r * ldx + k0;
            const float4 a = *(const float4*)x, b = *(const float4*)(x + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            const float* x = X + r * ldx + k0;
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (k0 + q < K) ? x[q] : 0.f;
        }
        split3_store8(v, P + split3_offset(r, k0, pstride), plane);
    }
}

// The same from S[r][k] = X[k * ldx + r] (X stored [K][R]), through a 64 x 64
// LDS tile; grid (Rp / 64, kp / 64), kp % 64 == 0, Rp % 64 == 0.
__global__ __launch_bounds__(256) void split3_cols_kernel(const float* __restrict__ X, int64_t ldx, int64_t R,
                                                          int64_t K, uint16_t* __restrict__ P, int64_t pstride,
                                                          int64_t plane) {
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int kk = i >> 6, rr = i & 63;
        tile[kk][rr] = (k0 + kk < K && r0 + rr < R) ? X[(k0 + kk) * ldx + r0 + rr] : 0.f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 8; i += 256) {
        const int rr = i >> 3, c = i & 7;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = tile[8 * c + q][rr];
        split3_store8(v, P + split3_offset(r0 + rr, k0 + 8 * c, pstride), plane);
    }
}

// elements of one plane of R rows at depth K
int64_t split3_plane(int64_t R, int64_t K) { return cdiv(R, SPLIT_PANEL) * split3_pstride(cdiv(K, 64) * 64); }

// planes of op(X) [R, K] (trans: X stored [K][R])
int launch_split3(const float* X, int64_t ldx, bool trans, int64_t R, int64_t K, uint16_t* P, hipStream_t st) {
    const int64_t kp = cdiv(K, 64) * 64, ps = split3_pstride(kp), plane = split3_plane(R, K);
    const int64_t Rp = cdiv(R, SPLIT_PANEL) * SPLIT_PANEL;
    if (trans) {
        hipLaunchKernelGGL(split3_cols_kernel, dim3((unsigned)(Rp / 64), (unsigned)(kp / 64)), dim3(256), 0, st, X,
                           ldx, R, K, P, ps, plane);
    } else {
        const int vec = (((uintptr_t)X & 15u) == 0) && (ldx % 4 == 0);
        const int64_t items = Rp * (kp / 8);
        hipLaunchKernelGGL(split3_rows_kernel, dim3((unsigned)std::min<int64_t>(cdiv(items, 256), 16384)), dim3(256),
                           0, st, X, ldx, R, Rp, K, vec, P, ps, kp, plane);
    }
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

// MFMA flops of one split-operand launch: every computed 256 x 256 tile over
// its depth range (the kernel's triangular skips, in whole 64-deep steps),
// six bf16 term products per step.
double split3_mfma_flops(const Bf16GemmArgs& g) {
    double f = 0.0;
    for (int64_t tm = 0; tm < g.tiles_m; ++tm)
        for (int64_t tn = 0; tn < g.tiles_n; ++tn) {
            if (g.upper_only && tm > tn) continue;
            int64_t kb = 0, ke = g.K1;
            if (g.tri == TRI_A_UPPER) kb = tm * 256;
            else if (g.tri == TRI_B_UPPER_NK) kb = tn * 256;
            else if (g.tri == TRI_B_UPPER_KN) ke = std::min<int64_t>(g.K1, tn * 256 + 256);
            if (ke > kb) f += 6.0 * 2.0 * 256.0 * 256.0 * (double)(64 * ((ke - kb) / 64));
        }
    return f;
}

}  // namespace

size_t gemm_f32_split3_elems(int64_t rows, int64_t K) { return (size_t)(3 * split3_plane(rows, K)); }

namespace {
// split-operand kernel arguments of one product whose planes are pa (A) and pb (B)
Bf16GemmArgs split3_args(const GemmArgs& a, const uint16_t* pa, const uint16_t* pb) {
    const int64_t kp = cdiv(a.K, 64) * 64;
    Bf16GemmArgs g{};
    g.Ap = pa; g.Bp = pb;
    g.a_plane = split3_plane(a.M, a.K); g.b_plane = split3_plane(a.N, a.K);
    g.pstride = split3_pstride(kp);
    g.K1 = kp; g.K2 = 0;
    g.M = a.M; g.N = a.N;
    g.C = a.C; g.ldc = a.ldc;
    g.alpha = a.alpha; g.beta_one = a.beta_one; g.tri = a.tri; g.upper_only = a.upper_only;
    g.tiles_m = cdiv(a.M, 256); g.tiles_n = cdiv(a.N, 256);
    return g;
}
unsigned split3_grid(const Bf16GemmArgs& g) {
    return (unsigned)tile_order::gemm_grid(g.tiles_m, g.tiles_n, g.tri, g.upper_only, true);
}
// op(B) is A's transpose view: one set of planes serves both operands
bool same_operand(const GemmArgs& a) {
    return a.A == a.B && a.lda == a.ldb && a.M == a.N &&
           ((a.layout_a == A_MK && a.layout_b == B_NK) || (a.layout_a == A_KM && a.layout_b == B_KN));
}
}  // namespace

int launch_gemm_f32_split3_pair(const GemmArgs& a0, const GemmArgs& a1, uint16_t* pa, uint16_t* pb, hipStream_t st) {
    if (a0.A != a1.A || a0.lda != a1.lda || a0.layout_a != a1.layout_a || a0.M != a1.M || a0.K != a1.K ||
        !same_operand(a0) || a0.K <= 0 || a0.M <= 0 || a0.N <= 0 || a1.N <= 0) {
        set_error("split-operand GEMM pair: the products must share A (rows, depth, layout) and the first must be "
                  "A op(A)^T");
        return PTQ_EINVAL;
    }
    PTQ_TRY(launch_split3(a0.A, a0.lda, a0.layout_a == A_KM, a0.M, a0.K, pa, st));
    PTQ_TRY(launch_split3(a1.B, a1.ldb, a1.layout_b == B_KN, a1.N, a1.K, pb, st));
    Bf16GemmArgs g = split3_args(a0, pa, pa);
    const Bf16GemmArgs g1 = split3_args(a1, pa, pb);
    const unsigned grid0 = (unsigned)cdiv(split3_grid(g), NXCD) * NXCD, grid1 = split3_grid(g1);
    g.grid0 = grid0;
    g.Bp2 = g1.Bp; g.b_plane2 = g1.b_plane; g.N2 = g1.N; g.tiles_n2 = g1.tiles_n;
    g.C2 = g1.C; g.ldc2 = g1.ldc;
    g.alpha2 = g1.alpha; g.beta_one2 = g1.beta_one; g.tri2 = g1.tri; g.upper_only2 = g1.upper_only;
    prof_begin(PROF_SPLIT3_GEMM, st, split3_mfma_flops(g) + split3_mfma_flops(g1));
    const int rc = launch_direct<256, EPI_GEMM, 64, DNW, DMF>(g, 0, grid0 + grid1, 1, st);
    prof_end(PROF_SPLIT3_GEMM, st);
    PTQ_TRY(rc);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

int launch_gemm_f32_split3(const GemmArgs& a, uint16_t* pa, uint16_t* pb, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return PTQ_OK;
    if (a.K <= 0) return launch_gemm_f32(a, st);
    const bool same = same_operand(a);
    PTQ_TRY(launch_split3(a.A, a.lda, a.layout_a == A_KM, a.M, a.K, pa, st));
    if (!same) PTQ_TRY(launch_split3(a.B, a.ldb, a.layout_b == B_KN, a.N, a.K, pb, st));
    const Bf16GemmArgs g = split3_args(a, pa, same ? pa : pb);
    const unsigned grid = split3_grid(g);
    prof_begin(PROF_SPLIT3_GEMM, st, split3_mfma_flops(g));
    const int rc = launch_direct<256, EPI_GEMM, 64, DNW, DMF>(g, 0, grid, 1, st);
    prof_end(PROF_SPLIT3_GEMM, st);
    PTQ_TRY(rc);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

namespace {

// The transposed chunk Xt (row c of Xt = column c of X) is panel-blocked for
// the X^T X tiles: rows c of panel c / bm are stored one stage (64 chunk rows)
// at a time, so element (c, r) sits at
//   (c / bm) * pstride + (r / 64) * bm * 64 + (c % bm) * 64 + r % 64
// and one stage of one panel is a contiguous bm x 64 block (32 KB at bm = 256):
// a tile's 16-byte copies read whole 1 KB runs. Panels are padded to bm rows
// with zeros, and pstride = bm * (chunk + 64): one spare stage per panel keeps
// the panels from starting at power-of-two distances, where the same stage of
// every panel would fall into the same L2 sets.
__host__ __device__ inline int64_t xt_offset(int64_t c, int64_t r, int bm, int64_t pstride) {
    return (c / bm) * pstride + (r >> 6) * ((int64_t)bm * 64) + (c % bm) * 64 + (r & 63);
}

// Xt(c, r) = X[r0 + r][c] for r < nr and c < n; zero for nr <= r < kt or
// n <= c < npad (grid: npad / 64 x kt / 64).
__global__ void transpose_rows_kernel(const uint16_t* __restrict__ X, int64_t ldx, int64_t n, int64_t r0,
                                      int64_t nr, uint16_t* __restrict__ Xt, int bm, int64_t pstride, int64_t kt) {
    __shared__ uint16_t tile[64][66];
    const int64_t cb = (int64_t)blockIdx.x * 64, rb = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 256 threads: 64 x 4
    for (int y = ty; y < 64; y += 4) {
        const int64_t r = rb + y, c = cb + tx;
        tile[y][tx] = (r < nr && c < n) ? X[(r0 + r) * ldx + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int y = ty; y < 64; y += 4) {
        const int64_t c = cb + y, r = rb + tx;
        if (r < kt) Xt[xt_offset(c, r, bm, pstride)] = tile[tx][y];
    }
}

// Xt(c, r) = X[r0 + r][c] (zero for nr <= r < kt or n <= c) with 16-byte
// accesses on both sides: a workgroup moves a 64-column strip over TR_ROWS
// rows of the chunk through a 64 x 64 LDS tile. With dpart, it also adds up
// the fp64 squares of the strip's values over those rows, one partial per
// (row group, column) in dpart[blockIdx.y][c] (X is read once for both).
// Requires n % 8 == 0 and 16-byte aligned rows of X; grid x = npad / 64.
constexpr int TR_ROWS = 1024;
__global__ __launch_bounds__(256) void transpose_sumsq_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                              int64_t n, int64_t r0, int64_t nr,
                                                              uint16_t* __restrict__ Xt, int bm, int64_t pstride,
                                                              int64_t kt, double* __restrict__ dpart) {
    __shared__ uint32_t tile[64][33];        // 64 rows x 64 bf16 (as 32 words) + 1 word of padding
    __shared__ double red[32][65];
    const int t = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int64_t rg = (int64_t)blockIdx.y * TR_ROWS;
    const int ch = t & 7;                    // 8-column piece of the strip this thread reads
    const int rr = t >> 3;                   // row (0..31) within a half tile
    double sq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sq[j] = 0.0;
    const bool col_ok = c0 + 8 * ch < n;
    for (int64_t rb = rg; rb < std::min<int64_t>(kt, rg + TR_ROWS); rb += 64) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = rr + 32 * h;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (col_ok && rb + r < nr) v = *(const uint4*)(X + (r0 + rb + r) * ldx + c0 + 8 * ch);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                tile[r][4 * ch + j] = w[j];
                const double lo = (double)bf16_bits_to_float((uint16_t)(w[j] & 0xFFFFu));
                const double hi = (double)bf16_bits_to_float((uint16_t)(w[j] >> 16));
                sq[2 * j] += lo * lo;
                sq[2 * j + 1] += hi * hi;
            }
        }
        __syncthreads();
        // write: thread -> column c = t / 8 (+ 32), rows 8 * (t % 8) .. + 7
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = (t >> 3) + 32 * h;
            const int rw = 8 * (t & 7);
            uint16_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t word = tile[rw + j][c >> 1];
                e[j] = (uint16_t)((c & 1) ? (word >> 16) : (word & 0xFFFFu));
            }
            if (rb + rw < kt) {
                uint4 o;
                o.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
                o.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
                o.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
                o.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
                *(uint4*)(Xt + xt_offset(c0 + c, rb + rw, bm, pstride)) = o;
            }
        }
        __syncthreads();
    }
    if (!dpart) return;
    // column sums over the 32 threads that read each 8-column piece, fixed order
#pragma unroll
    for (int j = 0; j < 8; ++j) red[rr][8 * ch + j] = sq[j];
    __syncthreads();
    if (t < 64 && c0 + t < n) {
        double s = 0.0;
        for (int i = 0; i < 32; ++i) s += red[i][t];
        dpart[(int64_t)blockIdx.y * n + c0 + t] = s;
    }
}

// H[j][i] = H[i][j] for every i < j, once per accumulation (the X^T X tiles
// and the fp32 path add into the upper triangle only). One workgroup per
// 64 x 64 tile of the upper triangle (blockIdx.y = tile row <= blockIdx.x =
// tile column): the tile is read row by row in 16-byte pieces, turned
// through LDS and written row by row into its mirror position; a diagonal
// tile writes its own strictly lower half. Mirroring inside the X^T X
// epilogue instead (column-wise 4-byte stores from every tile of the last
// chunk) lengthened that launch by about 1 ms at in = 28672; this pass
// moves the 2 x 1.6 GB at HBM rate.
constexpr int MIR = 64;
__global__ __launch_bounds__(256) void mirror_upper_kernel(float* H, int64_t n) {
    const int64_t I = blockIdx.y, J = blockIdx.x;
    if (I > J) return;
    __shared__ float tile[MIR][MIR + 1];
    const int t = threadIdx.x, cq = 4 * (t % 16), rq = t / 16;
    const int64_t r0 = I * MIR, c0 = J * MIR;
    const bool full = r0 + MIR <= n && c0 + MIR <= n && n % 4 == 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = rq + 16 * p;
        const int64_t gi = r0 + r;
        if (full) {
            const float4 v = *(const float4*)(H + gi * n + c0 + cq);
            tile[r][cq] = v.x; tile[r][cq + 1] = v.y; tile[r][cq + 2] = v.z; tile[r][cq + 3] = v.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gj = c0 + cq + q;
                tile[r][cq + q] = (gi < n && gj < n) ? H[gi * n + gj] : 0.f;
            }
        }
    }
    __syncthreads();
    // mirror row c0 + c holds tile column c; its columns r0 + cq .. are tile rows cq ..
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c = rq + 16 * p;
        const int64_t gi = c0 + c;
        if (full && I < J) {
            *(float4*)(H + gi * n + r0 + cq) = make_float4(tile[cq][c], tile[cq + 1][c], tile[cq + 2][c], tile[cq + 3][c]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gj = r0 + cq + q;
                if (gi < n && gj < n && gi > gj) H[gi * n + gj] = tile[cq + q][c];
            }
        }
    }
}

int launch_mirror_upper(float* H, int64_t n, hipStream_t st) {
    const int64_t T = cdiv(n, MIR);
    if (T > 65535) {
        set_error("hessian_accumulate: in = %lld is beyond the mirror pass's grid", (long long)n);
        return PTQ_EINVAL;
    }
    hipLaunchKernelGGL(mirror_upper_kernel, dim3((unsigned)T, (unsigned)T), dim3(256), 0, st, H, n);
    PTQ_LAUNCH_CHECK();
    return PTQ_OK;
}

// H[i][j] += sum over the splits of part[s][i][j] on and above the diagonal
// (in split order); one row per blockIdx.y. The lower triangle is mirrored
// once after the last chunk (mirror_upper_kernel).
__global__ void reduce_partials_kernel(float* H, const float* part, int nsplit, int64_t n) {
    const int64_t nn = n * n;
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y)
        for (int64_t j = i + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
            const int64_t e = i * n + j;
            float v = H[e];
            for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * nn + e];
            H[e] = v;
        }
}

// fp64 column sums of squares over one slab of rows; 2 columns per thread.
template <typename T>
__global__ void colsumsq_kernel(const T* __restrict__ X, int64_t ldx, int64_t rows, int64_t n,
                                int64_t slab_rows, double* __restrict__ out, int direct) {
    const int64_t c = 2 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (c >= n) return;
    const int64_t r0 = (int64_t)blockIdx.y * slab_rows;
    const int64_t r1 = min(rows, r0 + slab_rows);
    double s0 = 0.0, s1 = 0.0;
    for (int64_t r = r0; r < r1; ++r) {
        const T* p = X + r * ldx + c;
        const float x0 = load_as_float<T>(p, 0);
        const float x1 = (c + 1 < n) ? load_as_float<T>(p, 1) : 0.f;
        s0 += (double)x0 * (double)x0;
        s1 += (double)x1 * (double)x1;
    }
    if (direct) {
        out[c] += s0;
        if (c + 1 < n) out[c + 1] += s1;
    } else {
        double* o = out + (int64_t)blockIdx.y * n;
        o[c] = s0;
        if (c + 1 < n) o[c + 1] = s1;
    }
}

__global__ void reduce_slabs_kernel(double* d, const double* part, int nslab, int64_t n) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n) return;
    double v = d[c];
    for (int s = 0; s < nslab; ++s) v += part[(int64_t)s * n + c];
    d[c] = v;
}

constexpr int64_t SLAB_ROWS = 2048;
constexpr int MAX_SLABS = 256;
constexpr int64_t CHUNK_ROWS_MAX = 65536;   // calibration rows per transposed chunk
constexpr int64_t SPLIT_ROWS_MIN = 2048;    // depth of one split of a chunk's XtX launch, at least
constexpr int64_t XT_PAD = 64;             // spare chunk rows per Xt panel (xt_offset)

struct XtxPlan {
    int bm, T, nsplit;
    int64_t chunk;        // rows per transposed chunk (multiple of 64)
    int nslab;
    int64_t slab_rows;
    int64_t ngroups;      // row groups of the fused transpose + sums, over all chunks
};

size_t plan_bytes(const XtxPlan& p, int64_t n) {
    Sizer z;
    if (p.nslab > 1) z.take<double>((size_t)p.nslab * n);
    z.take<uint16_t>((size_t)p.T * p.bm * (p.chunk + XT_PAD));
    if (p.nsplit > 1) z.take<float>((size_t)p.nsplit * n * n);
    z.take<double>((size_t)p.ngroups * n);
    return z.bytes();
}

XtxPlan plan_xtx(int64_t n, int64_t rows) {
    XtxPlan p;
    p.bm = (n >= 2048) ? 256 : 128;
    p.T = (int)cdiv(n, p.bm);
    p.chunk = std::min<int64_t>(CHUNK_ROWS_MAX, cdiv(std::max<int64_t>(rows, 1), 64) * 64);
    // Split the depth of a launch (s a power of two up to 16, each split at
    // least SPLIT_ROWS_MIN rows deep) so that its tile jobs fill the CUs: the
    // busiest XCD runs its jobs in waves of 32 (one per CU) and sets the
    // launch time. Each job costs its 64-deep stages plus an epilogue that
    // stores or adds a whole tile, and s > 1 adds a pass over s partial H, so
    // s is the one with the smallest estimate
    //   waves(s) * (stages(s) * t_stage + t_epilogue) + s * n^2 * 4 B / 5 TB/s
    // with the stage and epilogue times measured on 256-wide tiles (1.45 and
    // 48 us) and scaled by the tile area for 128-wide ones. Deeper jobs waste
    // less on epilogues, more splits fill more CUs: the 4096-wide q_proj
    // (32768 rows) takes 4 splits (0.75 ms per call against 0.99 ms with the
    // 16 that a 90%-occupancy rule gave), the 8192-wide q/k/v 4, down_proj 1.
    const int nb = (int)cdiv(p.T, SB);
    int64_t per_xcd = 0;   // tiles of the busiest XCD in one launch without splitting
    for (int P = 0; P < nb; ++P)
        for (int Q = P; Q < nb; ++Q) per_xcd += cdiv(hessian_round_tiles(P, Q, p.T), NXCD);
    const double area = (double)p.bm * p.bm / (256.0 * 256.0);
    auto estimate = [&](int64_t s) {
        const double waves = (double)cdiv(per_xcd * s, 256 / NXCD);
        const double stages = (double)p.chunk / (64.0 * (double)s);
        const double reduce = s > 1 ? (double)s * (double)n * (double)n * 4.0 / 5.0e6 : 0.0;   // us at 5 TB/s
        return waves * area * (stages * 1.45 + 48.0) + reduce;
    };
    int s = 1;
    for (int c = 2; c <= 16 && p.chunk / c >= SPLIT_ROWS_MIN; c *= 2)
        if (estimate(c) < estimate(s)) s = c;
    p.nsplit = s;
    p.slab_rows = std::max<int64_t>(SLAB_ROWS, cdiv(cdiv(rows, MAX_SLABS), 64) * 64);
    p.nslab = (int)std::max<int64_t>(1, cdiv(rows, p.slab_rows));
    p.ngroups = cdiv(std::max<int64_t>(rows, 1), TR_ROWS) + cdiv(std::max<int64_t>(rows, 1), p.chunk);
    return p;
}

}  // namespace

namespace {

// The chunk loop of H (+)= X^T X under a plan whose buffers fit `ws`. With
// per_chunk_d, the fp64 column sums of every chunk are folded into d right
// after the chunk, so the sums workspace holds one chunk's row groups only.
int run_xtx(const XtxPlan& plan, bool per_chunk_d, float* H, double* d, int64_t n, const void* X, int x_dtype,
            int64_t rows, int64_t ldx, void* ws, size_t ws_bytes, hipStream_t st) {
    XtxPlan p = plan;
    if (x_dtype == PTQ_BF16 && plan_bytes(p, n) > ws_bytes) {
        set_error("hessian_accumulate: workspace of %zu bytes, %zu needed", ws_bytes, plan_bytes(p, n));
        return PTQ_EWORKSPACE;
    }
    Arena ar(ws, ws_bytes);
    double* dpart = (p.nslab > 1 && ws) ? ar.take<double>((size_t)p.nslab * n) : nullptr;
    if (!dpart) { p.nslab = 1; p.slab_rows = rows; }
    // bf16 rows in 16-byte pieces: the transpose also produces the sums of squares
    const bool vec = (x_dtype == PTQ_BF16) && (n % 8 == 0) && (ldx % 8 == 0) && (((uintptr_t)X & 15u) == 0);

    if (d && !vec) {
        dim3 grid((unsigned)cdiv(cdiv(n, 2), 256), (unsigned)p.nslab);
        if (x_dtype == PTQ_BF16)
            hipLaunchKernelGGL(colsumsq_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)X, ldx,
                               rows, n, p.slab_rows, p.nslab > 1 ? dpart : d, p.nslab > 1 ? 0 : 1);
        else
            hipLaunchKernelGGL(colsumsq_kernel<float>, grid, dim3(256), 0, st, (const float*)X, ldx, rows,
                               n, p.slab_rows, p.nslab > 1 ? dpart : d, p.nslab > 1 ? 0 : 1);
        PTQ_LAUNCH_CHECK();
        if (p.nslab > 1) {
            hipLaunchKernelGGL(reduce_slabs_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, d, dpart,
                               p.nslab, n);
            PTQ_LAUNCH_CHECK();
        }
    }

    if (x_dtype == PTQ_F32) {
        // fp32 calibration inputs: fp32 MFMA GEMM on the upper tiles, then mirror
        GemmArgs g{};
        g.M = n; g.N = n; g.K = rows;
        g.A = (const float*)X; g.lda = ldx; g.layout_a = A_KM;
        g.B = (const float*)X; g.ldb = ldx; g.layout_b = B_KN;
        g.C = H; g.ldc = n; g.alpha = 1.f; g.beta_one = 1; g.tri = TRI_NONE; g.upper_only = 1;
        PTQ_TRY(launch_gemm_f32(g, st));
        return launch_mirror_upper(H, n, st);
    }

    uint16_t* Xt = ar.take<uint16_t>((size_t)p.T * p.bm * (p.chunk + XT_PAD));
    const int64_t npad = (int64_t)p.T * p.bm, pstride = (int64_t)p.bm * (p.chunk + XT_PAD);
    float* hpart = (p.nsplit > 1) ? ar.take<float>((size_t)p.nsplit * n * n) : nullptr;
    double* dsum = ar.take<double>((size_t)p.ngroups * n);
    const int64_t ntiles = (int64_t)p.T * (p.T + 1) / 2;
    int64_t gofs = 0;   // row groups of the fused sums so far
    for (int64_t r0 = 0; r0 < rows; r0 += p.chunk) {
        const int64_t nr = std::min<int64_t>(p.chunk, rows - r0);
        const int64_t kt = cdiv(nr, 64) * 64;     // contraction depth of this chunk (zero-padded rows)
        if (vec) {
            const int64_t ng = cdiv(kt, TR_ROWS);
            hipLaunchKernelGGL(transpose_sumsq_kernel, dim3((unsigned)(npad / 64), (unsigned)ng), dim3(256), 0,
                               st, (const uint16_t*)X, ldx, n, r0, nr, Xt, p.bm, pstride, kt,
                               d ? dsum + gofs * n : (double*)nullptr);
            gofs += ng;
        } else {
            hipLaunchKernelGGL(transpose_rows_kernel, dim3((unsigned)(npad / 64), (unsigned)(kt / 64)),
                               dim3(256), 0, st, (const uint16_t*)X, ldx, n, r0, nr, Xt, p.bm, pstride, kt);
        }
        PTQ_LAUNCH_CHECK();
        if (vec && d && per_chunk_d) {
            hipLaunchKernelGGL(reduce_slabs_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, d, dsum,
                               (int)gofs, n);
            PTQ_LAUNCH_CHECK();
            gofs = 0;
        }
        const int ns = (p.nsplit > 1 && nr >= p.nsplit * SPLIT_ROWS_MIN) ? p.nsplit : 1;
        const int64_t kper = cdiv(cdiv(kt, ns), KT) * KT;
        {
            // one launch: blockIdx.y = s takes depth [s kper, min(kt, (s+1) kper))
            Bf16GemmArgs g{};
            g.A1 = Xt; g.B1 = Xt; g.A2 = nullptr; g.B2 = nullptr;
            g.K1 = kper; g.K2 = 0; g.ktot = kt;
            g.a_batch_stride = (kper / 64) * p.bm * 64; g.b_batch_stride = g.a_batch_stride;
            g.pstride = pstride; g.lda = 64; g.ldb = 64; g.M = n; g.N = n;
            g.H = (ns > 1) ? hpart : H;
            g.h_batch_stride = n * n;
            g.ldh = n; g.T = p.T; g.store_not_add = (ns > 1) ? 1 : 0;
            prof_begin(PROF_XTX_GEMM, st, 2.0 * (double)p.bm * p.bm * (double)ntiles * (double)kt);
            const int rc = (p.bm == 256) ? launch_nt<256, EPI_HESSIAN>(g, ntiles, (unsigned)ns, st)
                                         : launch_nt<128, EPI_HESSIAN>(g, ntiles, (unsigned)ns, st);
            prof_end(PROF_XTX_GEMM, st);
            PTQ_TRY(rc);
        }
        if (ns > 1) {
            // reduce the split partials into H (upper triangle)
            hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 32),
                                                            (unsigned)std::min<int64_t>(n, 65535)),
                               dim3(256), 0, st, H, hpart, ns, n);
            PTQ_LAUNCH_CHECK();
        }
    }
    if (vec && d && gofs > 0) {
        hipLaunchKernelGGL(reduce_slabs_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, d, dsum, (int)gofs,
                           n);
        PTQ_LAUNCH_CHECK();
    }
    // every chunk added into the upper triangle only
    return launch_mirror_upper(H, n, st);
}

}  // namespace

size_t xtx_workspace_bytes(int64_t n, int64_t rows) { return plan_bytes(plan_xtx(n, rows), n); }

int launch_xtx(float* H, double* d, int64_t n, const void* X, int x_dtype, int64_t rows,
               int64_t ldx, void* ws, size_t ws_bytes, hipStream_t st) {
    if (rows == 0) return PTQ_OK;
    return run_xtx(plan_xtx(n, rows), false, H, d, n, X, x_dtype, rows, ldx, ws, ws_bytes, st);
}

// The same within a fixed scratch: no split over depth (no partial H), sums
// of squares straight into d for non-vector X, chunks of the largest multiple
// of 64 rows whose transposed copy and one chunk's fp64 row-group sums fit.
int64_t xtx_bounded_chunk(int64_t n, size_t scratch_bytes) {
    const int bm = (n >= 2048) ? 256 : 128;
    const int64_t T = cdiv(n, bm);
    // bytes of a chunk of c rows (plan_bytes with nsplit = nslab = 1, one
    // chunk's groups), plus two 256-byte alignment slacks
    auto need = [&](int64_t c) {
        return (size_t)T * bm * (c + XT_PAD) * 2 + (size_t)cdiv(c, TR_ROWS) * n * 8 + 512;
    };
    int64_t lo = 0, hi = CHUNK_ROWS_MAX / 64;   // in units of 64 rows
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (need(64 * mid) <= scratch_bytes) lo = mid;
        else hi = mid - 1;
    }
    return 64 * lo;
}

int launch_xtx_bounded(float* H, double* d, int64_t n, const void* X, int x_dtype, int64_t rows, int64_t ldx,
                       void* scratch, size_t scratch_bytes, hipStream_t st) {
    if (rows == 0) return PTQ_OK;
    XtxPlan p = plan_xtx(n, rows);
    p.nsplit = 1;
    p.nslab = 1;
    p.slab_rows = rows;
    p.chunk = std::min<int64_t>(p.chunk, xtx_bounded_chunk(n, scratch_bytes));
    if (p.chunk < 64) {
        set_error("hessian_accumulate_noalloc: in = %lld needs more than the %zu bytes of scratch", (long long)n,
                  scratch_bytes);
        return PTQ_EINVAL;
    }
    p.ngroups = cdiv(p.chunk, TR_ROWS);
    return run_xtx(p, true, H, d, n, X, x_dtype, rows, ldx, scratch, scratch_bytes, st);
}

// AWQ error GEMM: partial[z][tile] = sum over the tile of (X (hi_z + lo_z)^T)^2
int launch_awq_error_gemm(const uint16_t* X, int64_t ldx, int64_t rows, int64_t n, const uint16_t* hi,
                          const uint16_t* lo, int64_t ldw, int64_t out, int64_t batch_stride, int nbatch,
                          double* partial, int64_t* ntiles_out, hipStream_t st) {
    Bf16GemmArgs g{};
    g.A1 = X; g.B1 = hi; g.A2 = X; g.B2 = lo;
    g.K1 = n; g.K2 = n; g.lda = ldx; g.ldb = ldw; g.M = rows; g.N = out;
    g.b_batch_stride = batch_stride;
    g.tiles_n = cdiv(out, 256);
    g.ntiles = cdiv(rows, 256) * g.tiles_n;
    *ntiles_out = g.ntiles;
    g.partial = partial;
    prof_begin(PROF_AWQ_GEMM, st, 2.0 * 256.0 * 256.0 * (double)g.ntiles * (double)(g.K1 + g.K2) * nbatch);
    const int rc = launch_nt<256, EPI_SUMSQ>(g, g.ntiles, (unsigned)nbatch, st);
    prof_end(PROF_AWQ_GEMM, st);
    return rc;
}

}  // namespace ptq
