"""CPU check of the X^T X tile order (post_int4_weight_amd/csrc/tile_order.hpp).

For every tile grid T = 1 .. 150: each tile on or above the diagonal is dealt
to exactly one workgroup slot (none twice, none missed, none below the
diagonal or outside the grid), and in every round the busiest XCD gets
ceil(v / 8) of the round's v tiles, the least any deal can give it.
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


def test_hessian_tile_order(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "tile_order_check.cpp"
    exe = tmp_path / "tile_order_check"
    src.write_text(PROGRAM)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad 0" in r.stdout
