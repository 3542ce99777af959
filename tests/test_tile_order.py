"""The workgroup -> output-tile order of tile_order.h, compiled for the host
(g++) and checked on the CPU: a bijection on every grid shape, the XCD parts
compact where the banded order applies."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "grouped_gemm_nvfp4_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "tile_order.h"
int main() {
    int tm_count, tn_count;
    while (std::scanf("%d %d", &tm_count, &tn_count) == 2) {
        const int T = tm_count * tn_count;
        for (int r = 0; r < T; ++r) {
            int tm, tn;
            nvfp4::tile_coords(r, tm_count, tn_count, &tm, &tn);
            std::printf("%d %d\n", tm, tn);
        }
        std::printf("end\n");
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def order_bin(tmp_path_factory):
    d = tmp_path_factory.mktemp("tile_order")
    src = d / "t.cpp"
    src.write_text(PROGRAM)
    exe = d / "t"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I", HEADER_DIR, "-o", str(exe), str(src)])
    return str(exe)


GRIDS = [(1, 1), (3, 5), (8, 8), (64, 32), (32, 12), (3, 12), (33, 16), (7, 9), (16, 5), (40, 24),
         (1, 64), (64, 1), (2, 36), (24, 16), (3, 16), (4, 16), (2, 8), (8, 24), (9, 16)]


def orders(exe, grids):
    text = "".join("%d %d\n" % g for g in grids)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    res, cur = [], []
    for line in out.splitlines():
        if line == "end":
            res.append(cur)
            cur = []
        else:
            cur.append(tuple(int(x) for x in line.split()))
    return res


def test_every_grid_is_covered_once(order_bin):
    for (tm_count, tn_count), coords in zip(GRIDS, orders(order_bin, GRIDS)):
        assert len(coords) == tm_count * tn_count
        assert sorted(coords) == sorted((m, n) for m in range(tm_count) for n in range(tn_count)), \
            (tm_count, tn_count)


def test_small_or_ragged_grids_keep_column_major_order(order_bin):
    grids = [(3, 5), (7, 9), (1, 1)]
    for (tm_count, tn_count), coords in zip(grids, orders(order_bin, grids)):
        assert coords == [(r % tm_count, r // tm_count) for r in range(tm_count * tn_count)]


def test_xcd_parts_are_compact(order_bin):
    """The 8192 x 8192 product in 128 x 256 tiles (64 x 32 grid): the tiles
    an XCD receives (r % 8 fixed) form one block of 32 tile rows by 8 tile
    columns, and any 64 consecutive ones of them 8 rows by 8 columns."""
    (coords,) = orders(order_bin, [(64, 32)])
    for part in range(8):
        mine = coords[part::8]
        rows = {m for m, _ in mine}
        cols = {n for _, n in mine}
        assert len(rows) == 32 and len(cols) == 8
        for start in range(0, len(mine), 64):
            window = mine[start:start + 64]
            assert len({m for m, _ in window}) == 8 and len({n for _, n in window}) == 8


def test_few_row_grids_put_each_column_on_one_xcd(order_bin):
    """Grids of at most 8 tile rows and a multiple of 8 columns: every row tile
    of a column sits at the same position mod 8 (one XCD), and each XCD
    receives whole columns."""
    grids = [(3, 16), (4, 16), (1, 64), (2, 8), (8, 24)]
    for (tm_count, tn_count), coords in zip(grids, orders(order_bin, grids)):
        for part in range(8):
            cols = {n for _, n in coords[part::8]}
            assert all(n % 8 == part for n in cols), (tm_count, tn_count)
            assert len(coords[part::8]) == tm_count * len(cols)
