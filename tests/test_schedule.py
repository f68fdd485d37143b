"""Host check of the GEMM tile visiting order (csrc/schedule.hpp).

The header is compiled into a small host program with hipcc (no GPU needed):
for many grids it checks that the order is a bijection of [0, T) onto the
tile grid, that tile_index inverts it, that the priority columns come first,
and that the grouped order matches its definition (GROUP_M rows of tiles per
group, column by column, rows fastest inside a group). The per-XCD queues
must deal every position of the sequence to exactly one queue slot, each
queue in increasing order, in blocks of Q dealt round-robin.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_collective_tile_amd", "csrc")

DRIVER = r"""
#include "schedule.hpp"
#include <cstdio>
#include <vector>
using namespace iris;
int check(int n_pm, int n_pn, int gm, int lo, int hi) {
  TileOrder o{n_pm, n_pn, gm, lo, hi};
  const int T = n_pm * n_pn;
  std::vector<int> seen(T, 0);
  const int np1 = hi - lo;
  for (int t = 0; t < T; ++t) {
    int pm, pn;
    tile_coords(o, t, pm, pn);
    if (pm < 0 || pm >= n_pm || pn < 0 || pn >= n_pn) { printf("out of grid t=%d\n", t); return 1; }
    if (seen[pm * n_pn + pn]++) { printf("repeat t=%d\n", t); return 1; }
    if (tile_index(o, pm, pn) != t) { printf("inverse t=%d\n", t); return 1; }
    const bool prio = pn >= lo && pn < hi;
    if (prio != (t < n_pm * np1)) { printf("priority t=%d\n", t); return 1; }
    // definition of the grouped order inside its part
    const int base = prio ? 0 : n_pm * np1;
    const int ncols = prio ? np1 : n_pn - np1;
    const int q = prio ? pn - lo : (pn < lo ? pn : pn - np1);
    const int r = t - base;
    const int group = r / (gm * ncols);
    const int first = group * gm;
    const int gsz = n_pm - first < gm ? n_pm - first : gm;
    const int w = r - group * gm * ncols;
    if (pm != first + w % gsz || q != w / gsz) { printf("definition t=%d\n", t); return 1; }
  }
  return 0;
}
int check_xcd(int T, int Q) {
  std::vector<int> seen(T, 0);
  for (int x = 0; x < kXcds; ++x) {
    int prev = -1;
    for (int j = 0;; ++j) {
      const int t = xcd_tile(Q, x, j);
      if (t >= T) break;
      if (t <= prev) { printf("queue %d not increasing at j=%d\n", x, j); return 1; }
      prev = t;
      if ((t / Q) % kXcds != x) { printf("block of t=%d not dealt to %d\n", t, x); return 1; }
      if (seen[t]++) { printf("t=%d twice\n", t); return 1; }
      int x2, j2;
      xcd_slot(Q, t, x2, j2);
      if (x2 != x || j2 != j) { printf("xcd_slot(%d) wrong\n", t); return 1; }
    }
  }
  for (int t = 0; t < T; ++t)
    if (!seen[t]) { printf("t=%d never dealt\n", t); return 1; }
  return 0;
}
int main() {
  const int xs[][2] = {{1, 1}, {7, 1}, {256, 32}, {688, 32}, {1000, 7}, {32768, 32}, {100, 128}, {1024, 128}};
  for (auto& s : xs)
    if (check_xcd(s[0], s[1])) { printf("T=%d Q=%d\n", s[0], s[1]); return 1; }
  const int shapes[][5] = {{1, 1, 8, 0, 0},   {16, 16, 8, 0, 0},  {16, 43, 8, 0, 6},
                           {16, 43, 8, 37, 43}, {16, 43, 8, 5, 11}, {17, 5, 4, 0, 0},
                           {3, 7, 8, 2, 3},    {512, 64, 8, 0, 0}, {33, 9, 1, 0, 9},
                           {9, 33, 16, 8, 12}, {32, 32, 8, 0, 32}};
  for (auto& s : shapes)
    if (check(s[0], s[1], s[2], s[3], s[4])) { printf("shape %d %d %d %d %d\n", s[0], s[1], s[2], s[3], s[4]); return 1; }
  printf("ok\n");
  return 0;
}
"""


def test_tile_order(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    src = tmp_path / "order.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "order"
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
