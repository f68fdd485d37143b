// Order in which GEMM tiles leave the work queue, and its inverse.
//
// Tiles are visited in GROUP_M-grouped order (iris.concurrent PR, the
// commits that keep the GROUP_M work-stealing tile swizzle): GROUP_M rows of
// tiles form a group, visited column by column, so consecutive tiles share
// B columns and a few A row blocks in L2. Column tiles [prio_lo, prio_hi)
// (the ones a reduce_scatter unit of this rank consumes) are visited first,
// all rows, then the rest in the same grouped order.
#pragma once

#include <hip/hip_runtime.h>

namespace iris {

struct TileOrder {
  int n_pm, n_pn, group_m;
  int prio_lo, prio_hi;
};

// t -> (pm, pn) on an n_pm x ncols grid.
__host__ __device__ inline void grouped(int t, int n_pm, int ncols, int gm, int& pm, int& pn) {
  const int width = gm * ncols;
  const int group = t / width;
  const int first = group * gm;
  const int gsz = n_pm - first < gm ? n_pm - first : gm;
  const int r = t - group * width;
  pm = first + r % gsz;
  pn = r / gsz;
}

// (pm, pn) -> t, the inverse of grouped().
__host__ __device__ inline int grouped_index(int pm, int pn, int n_pm, int ncols, int gm) {
  const int group = pm / gm;
  const int first = group * gm;
  const int gsz = n_pm - first < gm ? n_pm - first : gm;
  return group * gm * ncols + pn * gsz + (pm - first);
}

__host__ __device__ inline void tile_coords(const TileOrder& o, int t, int& pm, int& pn) {
  const int np1 = o.prio_hi - o.prio_lo;
  const int T1 = o.n_pm * np1;
  int q;
  if (t < T1) {
    grouped(t, o.n_pm, np1, o.group_m, pm, q);
    pn = o.prio_lo + q;
  } else {
    grouped(t - T1, o.n_pm, o.n_pn - np1, o.group_m, pm, q);
    pn = q < o.prio_lo ? q : q + np1;
  }
}

__host__ __device__ inline int tile_index(const TileOrder& o, int pm, int pn) {
  const int np1 = o.prio_hi - o.prio_lo;
  if (pn >= o.prio_lo && pn < o.prio_hi) return grouped_index(pm, pn - o.prio_lo, o.n_pm, np1, o.group_m);
  const int q = pn < o.prio_lo ? pn : pn - np1;
  return o.n_pm * np1 + grouped_index(pm, q, o.n_pm, o.n_pn - np1, o.group_m);
}

// ------------------------------------------------------- per-XCD queues
// MI355X has 8 XCDs, each with its own L2, and hands workgroups to them
// round-robin. The tile sequence above is dealt to one queue per XCD in
// blocks of Q consecutive tiles: block b goes to XCD b mod 8. With Q about
// the number of workgroups an XCD runs GEMM tiles on (grid / 8, or
// gemm_wgs / 8 beside an independent collective), the tiles an XCD runs at once form
// one compact patch of the grouped order (at Q = 32 and GROUP_M = 8, 8 row
// blocks x 4 column tiles), so their A rows and B columns meet in that XCD's
// L2 instead of being fetched by all eight.
constexpr int kXcds = 8;

// j-th tile of XCD x's queue -> position in the tile sequence. Increasing in
// j, so the queue holds exactly the j with xcd_tile(...) < T.
__host__ __device__ inline int xcd_tile(int Q, int x, int j) {
  const int blk = j / Q;
  return (blk * kXcds + x) * Q + (j - blk * Q);
}

// position t -> (XCD queue x, index j in it), the inverse of xcd_tile().
__host__ __device__ inline void xcd_slot(int Q, int t, int& x, int& j) {
  const int b = t / Q;
  x = b % kXcds;
  j = (b / kXcds) * Q + (t - b * Q);
}

}  // namespace iris
