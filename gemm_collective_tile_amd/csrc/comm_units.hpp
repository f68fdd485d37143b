// Communication units: the local data movement of one GPU's share of the
// collectives, done by ordinary workgroups with 16-byte vector loads and
// stores (bandwidth-bound, no LDS).
//
//   all_gather (Iris docs "Fused Communication and Compute Operations",
//   all_gather_matmul): shard s of rank order lands in columns
//   [s*K_local, (s+1)*K_local) of the gathered matrix. A unit copies
//   `rows_u` rows of one shard (a slice of one GEMM row block). Bit copy.
//
//   reduce (same page, matmul_reduce_scatter and matmul_all_reduce; the
//   all_reduce and reduce_scatter beside an independent GEMM of the
//   iris.concurrent PR): out = own + sum of the other ranks' partial
//   buffers, in that order, accumulated in fp32 and rounded once to fp16. A
//   unit is a rectangle of rows x columns (reduce_scatter / matmul_all_reduce)
//   or a flat chunk (the concurrent collectives).
//
//   block copy (the all_gather, all_to_all and broadcast beside an
//   independent GEMM of the iris.concurrent PR; the peer blocks of
//   matmul_all_gather on the docs page): source w, a contiguous block of
//   `blk` elements, lands at block position dst_blk[w] of the output. A unit
//   is a flat chunk of one block. Bit copy.
//
// A CU moves only a few tens of GB/s, bounded by the memory requests its
// waves keep in flight, so each thread issues all loads of a batch (up to 8
// sources x U vectors of 16 bytes) before it consumes any of them; the adds
// then run in source order. A wavefront covers 1 KiB of contiguous row per
// load and reduces its own vectors with no cross-lane traffic. Data read
// once by a reduce (partials, buffers) uses the streaming cache policy; its
// results are stored with the default policy (streaming stores ran the
// all_reduce of 8 x 64Mi fp16 at 5.1 TB/s on MI355X, default ones at 5.5).
// The all_gather copy loads with the default policy (pow2_4k's shards stay
// in the last-level cache between calls; streaming loads made that copy
// slower). It stores with the agent-coherent policy in the fused op, so that
// a unit can be published without an L2 write-back, and with the default
// policy in the sequential copy kernel.
#pragma once

#include "device_common.hpp"

namespace iris {

struct CommArgs {
  const f16* src[kMaxW];  // shards (AG) / partials (RS, AR) / buffers (concurrent)
  int32_t W;              // number of src buffers used
  f16* dst;               // gathered (AG) / out
  // all_gather
  int64_t K_local, K;     // shard row length, gathered row length
  // 2-D reduce: out[m][j] = C[m][col0 + j] + sum_p src[p][m][j]
  const f16* C;
  int64_t ldc;
  int32_t col0;           // rank * N_local (RS) or 0 (AR)
  int32_t ncols;          // N_local (RS) or N (AR): row length of src and dst
  int32_t comm_bn;        // columns per unit
  int32_t n_cc;           // column chunks per row slice
  // flat all_reduce / reduce_scatter
  int64_t elems;
  int32_t chunk;
  // block copy: W sources of blk elements, source w to block dst_blk[w]
  int64_t blk;
  int32_t n_chunk;        // chunks per block
  int32_t dst_blk[kMaxW];
  int32_t M, BM;
  int32_t rows_u;         // rows per unit (divides BM)
  int32_t n_sub;          // units per row block along M: BM / rows_u
};

// ------------------------------------------------------------- all_gather
// Unit (pm, s, q): rows [pm*BM + q*rows_u, +rows_u) of shard s. COHERENT:
// store with the agent-coherent policy, so the unit can be published without
// an L2 write-back (the fused op); the sequential copy kernel uses plain
// stores.
template <int U, bool COHERENT>
__device__ void ag_copy_unit(const CommArgs& a, int pm, int s, int q, uint32_t part = 0, uint32_t nparts = 1) {
  const int r0 = pm * a.BM + q * a.rows_u;
  const int rows = min(a.rows_u, a.M - r0);
  if (rows <= 0) return;
  const uint32_t vpr = (uint32_t)(a.K_local >> 3);  // 16-byte vectors per row
  const uint32_t total = (uint32_t)rows * vpr;
  const FastDiv fd = FastDiv::make(vpr);
  const f16* src = a.src[s] + (int64_t)r0 * a.K_local;  // rows are contiguous
  f16* dst = a.dst + (int64_t)r0 * a.K + (int64_t)s * a.K_local;
  // the unit's stores span (rows - 1) * K + K_local elements from dst; the
  // host keeps rows_u * K * 2 below 2^31 bytes
  const auto rdst = make_rsrc(dst, (uint32_t)(((int64_t)(rows - 1) * a.K + a.K_local) * 2));
  for (uint32_t base = threadIdx.x + part * kThreads * U; base < total; base += kThreads * U * nparts) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < total) v[u] = ld16(src + (int64_t)i * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < total) {
        const uint32_t r = fd.div(i);
        const uint32_t c = i - r * vpr;
        if constexpr (COHERENT)
          buf_store16_coherent(rdst, (uint32_t)(((int64_t)r * a.K + c * 8) * 2), v[u]);
        else
          st16(dst + (int64_t)r * a.K + c * 8, v[u]);
      }
    }
  }
}

__device__ __forceinline__ void add8(float acc[8], u32x4 v) {
  const f16x8 h = as_h8(v);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += (float)h[e];
}

__device__ __forceinline__ u32x4 round8(const float acc[8]) {
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (f16)acc[e];
  return as_u4(h);
}

// acc[u] += src[0][idx[u]] + src[1][idx[u]] + ... + src[n-1][idx[u]], added
// in that order; the loads of up to NB sources are all issued first.
template <int U, int NB>
__device__ __forceinline__ void accumulate(float (&acc)[U][8], const f16* const* src, int n,
                                           const int64_t (&idx)[U], const bool (&ok)[U]) {
  for (int p0 = 0; p0 < n; p0 += NB) {
    u32x4 v[NB][U];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (p0 + b < n) {
        const f16* sp = src[p0 + b];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ok[u]) v[b][u] = ld16_nt(sp + idx[u]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (p0 + b < n) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ok[u]) add8(acc[u], v[b][u]);
      }
    }
  }
}

// --------------------------------------------------------------- 2-D reduce
// Unit (pm, q, cc): rows [pm*BM + q*rows_u, +rows_u), columns
// [cc*comm_bn, +comm_bn) of the (M x ncols) output; own values come from C
// at column offset col0.
template <int U>
__device__ void reduce2d_unit(const CommArgs& a, int pm, int q, int cc, uint32_t part = 0, uint32_t nparts = 1) {
  const int r0 = pm * a.BM + q * a.rows_u;
  const int rows = min(a.rows_u, a.M - r0);
  const int j0 = cc * a.comm_bn;
  const int cols = min(a.comm_bn, a.ncols - j0);
  if (rows <= 0 || cols <= 0) return;
  const uint32_t vpr = (uint32_t)(cols >> 3);
  const uint32_t total = (uint32_t)rows * vpr;
  const FastDiv fd = FastDiv::make(vpr);
  for (uint32_t base = threadIdx.x + part * kThreads * U; base < total; base += kThreads * U * nparts) {
    float acc[U][8];
    int64_t orow[U];
    bool ok[U];
    u32x4 own[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kThreads;
      ok[u] = i < total;
      const uint32_t r = fd.div(i);
      const uint32_t c = i - r * vpr;
      orow[u] = (int64_t)(r0 + r) * a.ncols + j0 + c * 8;  // index into src/dst
      const int64_t cidx = (int64_t)(r0 + r) * a.ldc + a.col0 + j0 + c * 8;
      if (ok[u]) own[u] = ld16(a.C + cidx);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
      if (ok[u]) add8(acc[u], own[u]);
    }
    accumulate<U, 8>(acc, a.src, a.W, orow, ok);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) st16(a.dst + orow[u], round8(acc[u]));
  }
}

// ----------------------------------------------------------- flat reduce
// Unit u: elements [u*chunk, min((u+1)*chunk, elems)); dst = sum_w src[w].
// U vectors per thread, loads of NB sources in flight at a time.
template <int U, int NB>
__device__ void reduce_flat_unit(const CommArgs& a, int u, uint32_t part = 0, uint32_t nparts = 1) {
  const int64_t e0 = (int64_t)u * a.chunk;
  const int64_t n = min((int64_t)a.chunk, a.elems - e0);
  if (n <= 0) return;
  const uint32_t total = (uint32_t)(n >> 3);
  for (uint32_t base = threadIdx.x + part * kThreads * U; base < total; base += kThreads * U * nparts) {
    float acc[U][8];
    int64_t idx[U];
    bool ok[U];
#pragma unroll
    for (int v = 0; v < U; ++v) {
      ok[v] = base + v * kThreads < total;
      idx[v] = e0 + (int64_t)(base + v * kThreads) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[v][e] = 0.0f;
    }
    accumulate<U, NB>(acc, a.src, a.W, idx, ok);
#pragma unroll
    for (int v = 0; v < U; ++v)
      if (ok[v]) st16(a.dst + idx[v], round8(acc[v]));
  }
}

// ------------------------------------------------------------- block copy
// Unit (w, c): elements [c*chunk, min((c+1)*chunk, blk)) of source w.
template <int U>
__device__ void copy_block_unit(const CommArgs& a, int w, int c, uint32_t part = 0, uint32_t nparts = 1) {
  const int64_t e0 = (int64_t)c * a.chunk;
  const int64_t n = min((int64_t)a.chunk, a.blk - e0);
  if (n <= 0) return;
  const uint32_t total = (uint32_t)(n >> 3);
  const f16* src = a.src[w] + e0;
  f16* dst = a.dst + (int64_t)a.dst_blk[w] * a.blk + e0;
  for (uint32_t base = threadIdx.x + part * kThreads * U; base < total; base += kThreads * U * nparts) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < total) v[u] = ld16_nt(src + (int64_t)i * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < total) st16_nt(dst + (int64_t)i * 8, v[u]);
    }
  }
}

}  // namespace iris
