"""The matrix-core grid mapping (csrc/grid_cell.hpp), checked on the host.

Every workgroup index of the launch maps to exactly one (kv head, segment,
split, query tile) cell; segments are rotated by the split only when
hkv * n_segments is a multiple of 8; and the query tiles of one (kv head,
segment, split) land on one XCD (workgroup index mod 8) whenever the
tile-to-tile stride hkv * n_segments * n_split_max is a multiple of 8.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "stream_paged_attention_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <map>
#include <tuple>
#include <vector>
#include "grid_cell.hpp"
using tfa::Cell;
using tfa::grid_cell;
int main() {
    const int HKV[] = {1, 2, 3, 4, 6, 8, 16, 32};
    const int NSEG[] = {1, 2, 3, 4, 5, 8, 16, 17, 32};
    const int NSM[] = {1, 2, 3, 7, 8, 9, 32};
    const int NQT[] = {1, 2, 5};
    long cases = 0, bad = 0, rotated = 0;
    for (int hkv : HKV) for (int nseg : NSEG) for (int nsm : NSM) for (int nqt : NQT) {
        const int n = hkv * nseg * nsm * nqt;
        std::vector<char> seen(n, 0);
        std::map<std::tuple<int, int, int>, int> xcd;
        const bool rot = (hkv * nseg) % 8 == 0;
        rotated += rot;
        for (int i = 0; i < n; ++i) {
            const Cell c = grid_cell(i, hkv, nseg, nsm);
            if (c.g < 0 || c.g >= hkv || c.seg < 0 || c.seg >= nseg || c.t < 0 || c.t >= nsm || c.qt < 0 ||
                c.qt >= nqt) { ++bad; continue; }
            const int k = ((c.qt * nsm + c.t) * nseg + c.seg) * hkv + c.g;
            if (seen[k]) ++bad;
            seen[k] = 1;
            const int col = (i / hkv) % nseg;
            const int want = rot ? ((col - c.t) % nseg + nseg) % nseg : col;
            if (c.seg != want) ++bad;
            if ((hkv * nseg * nsm) % 8 == 0) {
                auto key = std::make_tuple(c.g, c.seg, c.t);
                auto it = xcd.find(key);
                if (it == xcd.end()) xcd[key] = i % 8;
                else if (it->second != i % 8) ++bad;
            }
        }
        ++cases;
    }
    std::printf("%ld %ld %ld\n", cases, bad, rotated);
    return 0;
}
"""


def test_grid_cells_cover_every_item_once(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "cells.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "cells"
    subprocess.run([cxx, "-O1", "-std=c++17", "-D__host__=", "-D__device__=", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    cases, bad, rotated = (int(x) for x in out)
    assert cases == 8 * 9 * 7 * 3
    assert rotated > 0 and rotated < cases
    assert bad == 0
