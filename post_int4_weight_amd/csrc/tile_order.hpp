// Order of the X^T X and GEMM tiles over the XCDs (pure integer code, host
// and device, so the CPU tests can check it).
#ifndef PTQ_TILE_ORDER_HPP
#define PTQ_TILE_ORDER_HPP

#include <stdint.h>

#ifndef __HIPCC__
#define __host__
#define __device__
#endif

namespace ptq {
namespace tile_order {

constexpr int NXCD = 8;   // accelerator complex dies; workgroup b runs on XCD b % 8

// Hessian tiles (upper triangle of a T x T tile grid) in rounds of 256
// workgroups; workgroup b runs on XCD b % 8 and the XCD with the most tiles
// sets the launch time, so every round deals its tiles evenly over the XCDs.
// Round r is the r-th SB x SB super-block (P <= Q, row-major), cut into eight
// 4 x 8 sub-blocks (rows 4 (s / 2).., columns 8 (s % 2)..). Its v valid tiles
// (inside the grid, on or above the diagonal) are listed sub-block by
// sub-block, row-major inside each, and XCD x takes the x-th run of
// ceil(v / 8) of them. A full off-diagonal super-block gives each XCD one
// whole sub-block: its 32 tiles read 12 panels through the XCD's own L2, and
// the 256 tiles of the round, which start together and move through k
// together, read 32 panels between them, so the die-shared last-level cache
// serves most of what the L2s miss. On a diagonal super-block the sub-blocks
// go in the order (0, 2, 1, 3, 4..7), left triangle, right square, right
// triangle, so that each XCD's run of 17 stays compact. Slots past a run
// return at once.
constexpr int SB = 16;
__host__ __device__ inline int64_t hessian_rounds(int T) {
    const int64_t nb = (T + SB - 1) / SB;
    return nb * (nb + 1) / 2;
}
// valid tiles of row ti among the 8 columns from c0
__host__ __device__ inline int hessian_row_tiles(int ti, int c0, int T) {
    if (ti >= T) return 0;
    const int hi = c0 + 8 < T ? c0 + 8 : T, lo = c0 > ti ? c0 : ti;
    return hi > lo ? hi - lo : 0;
}
// valid tiles of super-block (P, Q)
__host__ __device__ inline int hessian_round_tiles(int P, int Q, int T) {
    int v = 0;
    for (int s = 0; s < 8; ++s)
        for (int a = 0; a < 4; ++a) v += hessian_row_tiles(SB * P + 4 * (s >> 1) + a, SB * Q + 8 * (s & 1), T);
    return v;
}
__host__ __device__ inline bool hessian_tile(int64_t b, int T, int& ti, int& tj) {
    const int nb = (T + SB - 1) / SB;
    int64_t r = b / 256;
    const int w = (int)(b % 256), x = w % NXCD, i = w / NXCD;
    int P = 0;
    while (r >= nb - P) {
        r -= nb - P;
        ++P;
    }
    const int Q = P + (int)r;
    const int v = hessian_round_tiles(P, Q, T), per = (v + NXCD - 1) / NXCD;
    int c = x * per + i;
    if (i >= per || c >= v) return false;
    for (int k = 0; k < 8; ++k) {
        const int s = (k == 1) ? 2 : (k == 2) ? 1 : k;
        const int c0 = SB * Q + 8 * (s & 1);
        for (int a = 0; a < 4; ++a) {
            const int row = SB * P + 4 * (s >> 1) + a, m = hessian_row_tiles(row, c0, T);
            if (c < m) {
                ti = row;
                tj = (c0 > row ? c0 : row) + c;
                return true;
            }
            c -= m;
        }
    }
    return false;
}

// GEMM tiles (the split-operand products of gemm_bf16.hip and the fp32 MFMA
// GEMM of gemm_f32.hip) over a tiles_m x tiles_n grid. Triangular operands
// (the tri codes of common.hpp, repeated here so the header stays free of
// HIP) make a tile's depth depend on its row (A upper) or its column (B
// upper); upper_only computes the tiles on or above the diagonal only.
constexpr int TRI_NONE_ = 0, TRI_A_UP = 1, TRI_B_UP_KN = 2, TRI_B_UP_NK = 3;
enum { DEAL_SUBBLOCKS = 0, DEAL_COLUMNS = 1, DEAL_ROWS = 2, DEAL_PLAIN = 3 };
// How the tiles go to the XCDs (workgroup b runs on XCD b % 8):
//  * sub-blocks (dense products of at least 8 x 8 tiles, when the caller
//    allows them): 4 x 8 sub-blocks dealt round-robin, so the 32 tiles an
//    XCD runs side by side read 12 panels through its L2 (whole tile rows:
//    33);
//  * columns (a triangular B, at least 8 tile columns): a tile's depth
//    depends on its column only, so XCD x takes whole columns, its k-th
//    being column 8k + x for even k and 8k + 7 - x for odd k, in order of
//    decreasing depth: the last tiles to start are the shortest (dealt by
//    rows, every row would run from deep to shallow and the deep tiles of
//    the last rows would start near the end of the launch);
//  * rows (at least 8 tile rows): the same zigzag over whole tile rows,
//    which balances the products whose work falls with the row (A upper,
//    upper_only);
//  * plain row-major order otherwise.
__host__ __device__ inline int gemm_deal(int64_t tiles_m, int64_t tiles_n, int tri, int upper_only, bool subblocks) {
    if (subblocks && tiles_m >= 8 && tiles_n >= 8 && tri == TRI_NONE_ && !upper_only) return DEAL_SUBBLOCKS;
    if (tiles_n >= NXCD && (tri == TRI_B_UP_KN || tri == TRI_B_UP_NK) && !upper_only) return DEAL_COLUMNS;
    if (tiles_m >= NXCD) return DEAL_ROWS;
    return DEAL_PLAIN;
}
// workgroups one launch needs (some slots return at once)
__host__ __device__ inline int64_t gemm_grid(int64_t tiles_m, int64_t tiles_n, int tri, int upper_only, bool subblocks) {
    switch (gemm_deal(tiles_m, tiles_n, tri, upper_only, subblocks)) {
        case DEAL_SUBBLOCKS: return ((tiles_m + 3) / 4 * ((tiles_n + 7) / 8) + NXCD - 1) / NXCD * NXCD * 32;
        case DEAL_COLUMNS: return NXCD * ((tiles_n + NXCD - 1) / NXCD) * tiles_m;
        case DEAL_ROWS: return NXCD * ((tiles_m + NXCD - 1) / NXCD) * tiles_n;
        default: return tiles_m * tiles_n;
    }
}
// Tile (tm, tn) of workgroup b, or false for a slot with no tile. With B
// upper triangular in [K][N] layout the depth grows with the column, so the
// column index runs backwards and the deepest tiles start first.
__host__ __device__ inline bool gemm_tile(int64_t b, int64_t tiles_m, int64_t tiles_n, int tri, int upper_only,
                                          bool subblocks, int64_t& tm, int64_t& tn) {
    const int64_t x = b % NXCD, i = b / NXCD;
    switch (gemm_deal(tiles_m, tiles_n, tri, upper_only, subblocks)) {
        case DEAL_SUBBLOCKS: {
            const int64_t sbc = (tiles_n + 7) / 8, sbi = NXCD * (i / 32) + x, w = i % 32;
            tm = 4 * (sbi / sbc) + w / 8;
            tn = 8 * (sbi % sbc) + w % 8;
            if (tm >= tiles_m || tn >= tiles_n) return false;
            break;
        }
        case DEAL_COLUMNS: {
            const int64_t k = i / tiles_m;
            tn = NXCD * k + ((k & 1) ? NXCD - 1 - x : x);
            tm = i % tiles_m;
            if (tn >= tiles_n) return false;
            break;
        }
        case DEAL_ROWS: {
            const int64_t k = i / tiles_n;
            tm = NXCD * k + ((k & 1) ? NXCD - 1 - x : x);
            tn = i % tiles_n;
            if (tm >= tiles_m) return false;
            break;
        }
        default:
            if (b >= tiles_m * tiles_n) return false;
            tm = b / tiles_n;
            tn = b % tiles_n;
    }
    if (tri == TRI_B_UP_KN) tn = tiles_n - 1 - tn;
    return !(upper_only && tm > tn);
}

}  // namespace tile_order
}  // namespace ptq

#endif
