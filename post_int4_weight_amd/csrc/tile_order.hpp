// Order of the X^T X tiles over the XCDs (pure integer code, host and device,
// so the CPU tests can check it).
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

}  // namespace tile_order
}  // namespace ptq

#endif
