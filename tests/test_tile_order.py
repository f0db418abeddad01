"""CPU check of the tile orders in post_int4_weight_amd/csrc/tile_order.hpp.

X^T X: for every tile grid T = 1 .. 150, each tile on or above the diagonal
is dealt to exactly one workgroup slot (none twice, none missed, none below
the diagonal or outside the grid), and in every round the busiest XCD gets
ceil(v / 8) of the round's v tiles, the least any deal can give it.

GEMM tiles (split-operand and fp32 GEMMs): for every grid up to 40 x 40 and a
few large ones, every triangle code, with and without upper_only and
sub-blocks, each tile the product computes is dealt to exactly one of the
launch's slots; and where the deal goes by whole columns (triangular B) or
rows (A upper), the tiles each XCD takes come in order of non-increasing
depth, so the last tiles to start are the shortest.
The header is plain integer C++, compiled here with the host compiler.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "post_int4_weight_amd", "csrc")

PROGRAM = r"""
#include "tile_order.hpp"
#include <cstdio>
#include <vector>
using namespace ptq::tile_order;
int main() {
    int bad = 0;
    for (int T = 1; T <= 150; ++T) {
        std::vector<int> seen(T * T, 0);
        const long rounds = hessian_rounds(T);
        for (long r = 0; r < rounds; ++r) {
            int per_xcd[NXCD] = {0};
            int v = 0;
            for (int w = 0; w < 256; ++w) {
                int ti, tj;
                if (!hessian_tile(256 * r + w, T, ti, tj)) continue;
                if (ti < 0 || tj < 0 || ti >= T || tj >= T || ti > tj) { ++bad; continue; }
                ++seen[ti * T + tj];
                ++per_xcd[w % NXCD];
                ++v;
            }
            int mx = 0;
            for (int x = 0; x < NXCD; ++x) mx = per_xcd[x] > mx ? per_xcd[x] : mx;
            if (mx != (v + NXCD - 1) / NXCD) { std::printf("T=%d round %ld: busiest XCD %d of %d\n", T, r, mx, v); ++bad; }
        }
        for (int i = 0; i < T; ++i)
            for (int j = i; j < T; ++j)
                if (seen[i * T + j] != 1) { std::printf("T=%d tile (%d,%d) dealt %d times\n", T, i, j, seen[i * T + j]); ++bad; }
    }
    std::printf("bad %d\n", bad);
    return bad != 0;
}
"""


GEMM_PROGRAM = r"""
#include "tile_order.hpp"
#include <cstdio>
#include <vector>
using namespace ptq::tile_order;
// depth of tile (tm, tn) in tile units: A upper skips k < row, B upper [K][N]
// stops at the column, B upper [N][K] starts at it
static long depth(int tri, long tm, long tn, long tiles_m, long tiles_n) {
    if (tri == TRI_A_UP) return tiles_m - tm;
    if (tri == TRI_B_UP_KN) return tn + 1;
    if (tri == TRI_B_UP_NK) return tiles_n - tn;
    return 1;
}
static int check(long tiles_m, long tiles_n, int tri, int upper_only, bool sub) {
    int bad = 0;
    std::vector<int> seen(tiles_m * tiles_n, 0);
    const long grid = gemm_grid(tiles_m, tiles_n, tri, upper_only, sub);
    const int deal = gemm_deal(tiles_m, tiles_n, tri, upper_only, sub);
    std::vector<long> last(NXCD, 1L << 40);
    for (long b = 0; b < grid; ++b) {
        int64_t tm, tn;
        if (!gemm_tile(b, tiles_m, tiles_n, tri, upper_only, sub, tm, tn)) continue;
        if (tm < 0 || tn < 0 || tm >= tiles_m || tn >= tiles_n || (upper_only && tm > tn)) { ++bad; continue; }
        ++seen[tm * tiles_n + tn];
        const bool ordered = (deal == DEAL_COLUMNS) || (deal == DEAL_ROWS && tri == TRI_A_UP);
        if (ordered) {
            const long dd = depth(tri, tm, tn, tiles_m, tiles_n);
            if (dd > last[b % NXCD]) { ++bad; }
            last[b % NXCD] = dd;
        }
    }
    for (long i = 0; i < tiles_m; ++i)
        for (long j = 0; j < tiles_n; ++j) {
            const int want = (upper_only && i > j) ? 0 : 1;
            if (seen[i * tiles_n + j] != want) ++bad;
        }
    if (bad) std::printf("tiles %ld x %ld tri %d upper_only %d sub %d: %d bad\n", tiles_m, tiles_n, tri, upper_only,
                         (int)sub, bad);
    return bad;
}
int main() {
    int bad = 0;
    const long big[][2] = {{56, 56}, {112, 112}, {32, 104}, {32, 8}, {57, 9}, {9, 57}, {128, 24}};
    for (int tri = 0; tri < 4; ++tri)
        for (int uo = 0; uo < 2; ++uo)
            for (int sub = 0; sub < 2; ++sub) {
                for (long m = 1; m <= 40; ++m)
                    for (long n = 1; n <= 40; ++n) bad += check(m, n, tri, uo, sub != 0);
                for (auto& s : big) bad += check(s[0], s[1], tri, uo, sub != 0);
            }
    std::printf("bad %d\n", bad);
    return bad != 0;
}
"""


def _run(tmp_path, program, name):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / f"{name}.cpp"
    exe = tmp_path / name
    src.write_text(program)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return subprocess.run([str(exe)], capture_output=True, text=True)


def test_gemm_tile_order(tmp_path):
    r = _run(tmp_path, GEMM_PROGRAM, "gemm_tile_check")
    assert r.returncode == 0, r.stdout[-3000:]
    assert r.stdout.strip().endswith("bad 0")


def test_hessian_tile_order(tmp_path):
    r = _run(tmp_path, PROGRAM, "tile_order_check")
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad 0" in r.stdout
