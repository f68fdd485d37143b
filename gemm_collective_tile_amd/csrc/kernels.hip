// Persistent work-stealing kernels for one GPU's share of the fused
// communication + GEMM ops, and their launchers.
//
// Scheduling follows the iris.concurrent PR ("Add iris.concurrent
// (concurrent, independent, fused comm+gemm)", description): one persistent
// kernel holds two work-stealing queues, GEMM tiles and communication units,
// each drained through an atomic counter; workgroups with
// blockIdx < gemm_wgs start on the GEMM queue, the rest on the comm queue.
// GEMM tiles are visited in GROUP_M-grouped order (same PR, commits that keep
// the GROUP_M work-stealing tile swizzle).
//
// Dependencies of the dependent ops (Iris docs "Fused Communication and
// Compute Operations": all_gather_matmul consumes the gathered A;
// reduce_scatter / all_reduce consume A @ B + bias) are carried by ready
// words in the workspace:
//   all_gather:  rows[pm] counts the finished copy units of GEMM row block
//                pm; a GEMM tile of that block waits until all W * n_sub
//                are in. With more GEMM tiles than workgroups, a second
//                counter of all finished units lets a workgroup that has
//                seen every unit done stop checking, and holds the copy
//                workgroups back until the gather is complete.
//   reduce:      flag[pm*n_pn + pn] = 1 once GEMM tile (pm, pn) is stored;
//                a reduce unit waits for the tiles covering its columns.
// A workgroup that has to wait first takes unclaimed work from the queue it
// waits on, so every wait ends even if not all workgroups are resident: a
// claimed unit is always held by a running workgroup whose own work never
// waits on the other queue. A reduce unit whose tiles are all claimed only
// spins: they are being computed, and taking another tile would hold the
// reduce back by a whole tile.
#include "launch.hpp"

#include <mutex>

namespace iris {

// ------------------------------------------------------------------ queues
// One atomic per claim. A workgroup leaves a queue the first time a claim
// comes back empty; a waiting workgroup helps with an atomic only after a
// read shows unclaimed work. A counter thus overshoots its total by a few
// claims per workgroup at most, far from int32 overflow (totals <= 2^30).
__device__ __forceinline__ int claim(int* ctr, int T, int* slot) {
  if (threadIdx.x == 0) slot[0] = fetch_add(ctr, 1);
  __syncthreads();
  const int v = slot[0];
  __syncthreads();
  return v < T ? v : -1;
}

// The XCD this workgroup runs on (hardware XCC_ID register).
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & (kXcds - 1);
}

// Lockstep of the GEMM rounds. An XCD's queue is dealt in blocks of Q
// tiles, Q being the number of workgroups that work it, so round r (tiles
// rQ .. rQ+Q-1 of the queue) is one patch of tiles whose A rows and B
// columns meet in that XCD's L2. With the lockstep on, a workgroup starts
// the tile of round r it took from its home queue only once every tile of
// round r-1 of that queue has finished (whoever ran it), so the patch's
// tiles run their K loops together. Without it the workgroups drift apart
// over the rounds by how long each tile happens to take, and how far they
// drift depended on the code around the tile loop. On MI355X, the fused g2
// op (131072 x 16384 x 16384, gemm_wgs 128) without the lockstep
// (IRIS_FLAG_NO_LOCKSTEP) read 293 GiB from beyond L2 against 118 GiB with
// it, and at about the same cycle count the chip held an 8 % lower clock for
// the extra traffic: 62.1 against 57.5 ms. The wait ends: every tile of an
// earlier round has been claimed, so it is held by a running workgroup.
__device__ __forceinline__ void wait_round(const Params& p, int home, int j) {
  if (threadIdx.x == 0) {
    const int need = (j / p.xcd_q) * p.xcd_q;
    const int* d = p.ws + kTileDone + home * kLine;
    uint32_t polls = 0;
    while (ld_relaxed(d) < need) {
      if (++polls > p.spin_limit) {
        __hip_atomic_store(p.ws + kErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// A tile taken from XCD queue q has finished (counted for the lockstep).
__device__ __forceinline__ void tile_done(const Params& p, int q) {
  if (p.lockstep && q >= 0 && threadIdx.x == 0) fetch_add(p.ws + kTileDone + q * kLine, 1);
}

// GEMM claim: this XCD's queue first (thread 0, one atomic), then the
// others. The queue a tile came from is left in slot[3] (-1 if none). `gone` (bit x: queue x seen empty) is kept in thread 0 and handed
// to wave 0 for the steal, so each queue's counter overshoots its share by at
// most one per workgroup. Once the home queue is empty, lane x of wave 0
// reads queue x's counter (one round trip for all eight) and only a queue
// that still shows unclaimed tiles gets an atomic: trying the other queues
// one atomic at a time put up to eight serial round trips at the end of
// every workgroup's GEMM phase.
__device__ __forceinline__ int claim_gemm(const Params& p, int home, uint32_t& gone, int* slot) {
  if (threadIdx.x == 0) {
    int t = -1, jh = -1;
    if (!(gone & (1u << home))) {
      const int j = fetch_add(p.ws + kCtrGemm + home * kLine, 1);
      const int c = xcd_tile(p.xcd_q, home, j);
      if (c < p.T_gemm) {
        t = c;
        jh = j;
      } else {
        gone |= 1u << home;
      }
    }
    slot[0] = t;
    slot[1] = (int)gone;
    slot[2] = jh;
    slot[3] = t >= 0 ? home : -1;
  }
  __syncthreads();
  int v = slot[0];
  if (v < 0 && threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t g = (uint32_t)slot[1];
    while (g != (1u << kXcds) - 1) {
      bool open = false;
      if (lane < kXcds && !(g & (1u << lane)))
        open = xcd_tile(p.xcd_q, lane, ld_relaxed(p.ws + kCtrGemm + lane * kLine)) < p.T_gemm;
      const uint32_t m = (uint32_t)__ballot(open) & ((1u << kXcds) - 1);
      g |= ~m & ((1u << kXcds) - 1);  // counters only grow: these stay empty
      if (m == 0) break;
      const int s = (home + 1) & (kXcds - 1);  // first open queue after home
      const uint32_t rot = ((m >> s) | (m << (kXcds - s))) & ((1u << kXcds) - 1);
      const int pick = (s + __builtin_ctz(rot)) & (kXcds - 1);
      int c = 0;
      if (lane == 0) c = xcd_tile(p.xcd_q, pick, fetch_add(p.ws + kCtrGemm + pick * kLine, 1));
      c = __shfl(c, 0);
      if (c < p.T_gemm) {
        v = c;
        if (lane == 0) slot[3] = pick;
        break;
      }
      g |= 1u << pick;
    }
    if (lane == 0) {
      gone = g;
      slot[0] = v;
    }
  }
  __syncthreads();
  v = slot[0];
  const int jh = slot[2];
  __syncthreads();
  if (p.lockstep && jh >= p.xcd_q) wait_round(p, home, jh);
  return v;
}

// Release of a unit's results to other workgroups (any XCD): every wave
// drains its stores to L2, the workgroup barriers, then one thread writes the
// XCD's L2 back (agent-scope release fence), waits for that write-back to
// finish, and only then sets the flag (or bumps the counters). The explicit
// wait matters: once the stores are drained the compiler sees nothing
// outstanding and would issue the flag store right behind the write-back.
__device__ __forceinline__ void release_begin() {
  drain_vmem();
  __syncthreads();
}

__device__ __forceinline__ void publish(int* flag) {
  release_begin();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    drain_vmem();
    __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// For data written with agent-coherent stores (buf_store16_coherent): once
// every wave's stores have completed they are visible on every XCD, so the
// counters (a, and b unless it is null) can be bumped with no L2 write-back
// in between.
__device__ __forceinline__ void publish_count_coherent(int* a, int* b) {
  release_begin();
  if (threadIdx.x == 0) {
    fetch_add(a, 1);
    if (b) fetch_add(b, 1);
  }
}

// Pause between polls of a ready word, doubling from about 0.1 us to about
// 1 us so that many waiting workgroups do not flood the line they poll.
__device__ __forceinline__ void backoff(int& n) {
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(4);
  n = n < 8 ? 2 * n : n;
}

// ------------------------------------------------------------ comm units
// Unit u; with nparts > 1 only the part-th of every nparts vector groups
// (a workgroup of the sequential comm kernel sharing the unit with others).
// WIDE: 16 vectors per thread in flight and agent-coherent stores for the
// all_gather copy, for one workgroup per CU (the persistent kernel's copy
// workgroups); otherwise 8 vectors and plain stores, for the four
// workgroups per CU of the comm-only kernel.
template <int OP, bool WIDE = true>
__device__ void run_comm_unit(const Params& p, int u, uint32_t part = 0, uint32_t nparts = 1) {
  const CommArgs& c = p.c;
  if constexpr (OP == OP_AG) {
    // u = (pm * W + s) * n_sub + q
    const int per_block = c.W * c.n_sub;
    const int pm = u / per_block;
    const int r = u - pm * per_block;
    const int s = r / c.n_sub;
    // one workgroup per CU keeps 16 vectors per thread in flight (fused
    // pow2_4k: copy window 14.7 -> 13.4 us on MI355X; 32 was slower); four
    // workgroups per CU keep 8 each (the sequential 64 MiB pow2_4k gather:
    // 3.9 TB/s, against 3.5 on one workgroup per CU)
    ag_copy_unit<(WIDE ? 16 : 8), WIDE>(c, pm, s, r - s * c.n_sub, part, nparts);
  } else if constexpr (OP == OP_RS || OP == OP_ARMM) {
    // u = (pm * n_sub + q) * n_cc + cc
    const int slice = u / c.n_cc;
    const int pm = slice / c.n_sub;
    reduce2d_unit<2>(c, pm, slice - pm * c.n_sub, u - slice * c.n_cc, part, nparts);
  } else if constexpr (OP == OP_CONC_AR) {
    // 8 vectors per thread from 2 sources at a time read the all_reduce of
    // 8 x 64Mi fp16 at 5.8 TB/s on MI355X, 2 vectors from 8 sources at 5.4;
    // a unit shared by several workgroups keeps the finer split so that
    // every share gets work
    if (nparts > 1)
      reduce_flat_unit<2, 8>(c, u, part, nparts);
    else
      reduce_flat_unit<8, 2>(c, u, part, nparts);
  } else if constexpr (OP == OP_CONC_COPY) {
    const int w = u / c.n_chunk;
    copy_block_unit<8>(c, w, u - w * c.n_chunk, part, nparts);
  }
}

__device__ __forceinline__ int ag_unit_block(const Params& p, int u) { return u / (p.c.W * p.c.n_sub); }

// all_gather: the copy unit has landed; count it for its row block
template <int OP>
__device__ __forceinline__ void finish_comm_unit(const Params& p, int u) {
  if constexpr (OP == OP_AG) {
    // the finished-unit count only serves a GEMM with more tiles than
    // workgroups (tiles that no longer check their row block; the copy
    // workgroups' wait before joining the GEMM): with a single wave every
    // workgroup has about one tile, and traffic on that one line while the
    // last units land slowed them (pow2_4k)
    if (p.fused)
      publish_count_coherent(p.ws + kFlagBase + ag_unit_block(p, u) * kLine,
                             p.T_gemm > (int)gridDim.x ? p.ws + kCommDone : nullptr);
  }
}

template <int OP, class S>
__device__ void run_gemm_tile(const Params& p, int t, int* slot, char* lds, bool& rows_ready);

// A GEMM tile of row block pm waits for the copy units of that block.
// rows_ready: this workgroup has seen every copy unit finished (and has
// acquired them), so no later tile needs to look.
template <int OP, class S>
__device__ void wait_rows(const Params& p, int pm, int* slot, bool& rows_ready) {
  if (rows_ready) return;
  const int* cnt = p.ws + kFlagBase + pm * kLine;
  const int need = p.c.W * p.c.n_sub;
  uint32_t polls = 0;
  int pause = 1;
  bool comm_left = true;  // thread 0: the comm queue may still hold units
  while (true) {
    if (threadIdx.x == 0) {
      int ready = 0, help = -1;
      const int all = p.T_gemm > (int)gridDim.x ? ld_relaxed(p.ws + kCommDone) : 0;
      const int have = ld_relaxed(cnt);
      if (all >= p.T_comm) {
        ready = 2;
      } else if (have >= need) {
        ready = 1;
      } else if (comm_left) {
        const int u = ld_relaxed(p.ws + kCtrComm) < p.T_comm ? fetch_add(p.ws + kCtrComm, 1) : p.T_comm;
        if (u < p.T_comm) help = u;
        else comm_left = false;
      } else if (++polls > p.spin_limit) {
        __hip_atomic_store(p.ws + kErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = 1;
      }
      if (ready) fence_acquire();
      slot[0] = ready;
      slot[1] = help;
    }
    __syncthreads();
    const int ready = slot[0], help = slot[1];
    __syncthreads();
    if (ready) {
      rows_ready = ready == 2;
      return;
    }
    if (help >= 0) {
      run_comm_unit<OP>(p, help);
      finish_comm_unit<OP>(p, help);
    } else {
      backoff(pause);
    }
  }
}

// all_gather with more GEMM tiles than workgroups: a workgroup that found
// the copy queue empty waits until every copy unit has finished before it
// takes GEMM tiles. Every unit is then held by a running workgroup, so the
// wait ends. The copy workgroups thus start their tiles within a poll
// interval of each other, and in every later wave the tiles that share
// operands run their K loops in step and meet in L2. Joining the GEMM queue
// one by one as each finished its last unit (up to a unit's time apart), the
// g2 all_gather_matmul (M=131072, N=K=16384) fetched 155-207 GiB from beyond
// L2 on MI355X, against 128 GiB for the same tiles started together; with
// the wait, 141. With a single wave of tiles there is no later wave to keep
// in step, and the polling of the finished-unit counter by the waiting
// workgroups slowed the last copy units (pow2_4k 4096^3: +5 us).
template <int OP>
__device__ void wait_all_units(const Params& p, bool& rows_ready) {
  if (threadIdx.x == 0) {
    uint32_t polls = 0;
    int pause = 1;
    while (ld_relaxed(p.ws + kCommDone) < p.T_comm) {
      if (++polls > p.spin_limit) {
        __hip_atomic_store(p.ws + kErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      backoff(pause);
    }
    fence_acquire();
  }
  __syncthreads();
  rows_ready = true;
}

// A reduce unit waits for the GEMM tiles covering its rows and columns.
template <int OP, class S>
__device__ void wait_tiles(const Params& p, int u, int* slot, char* lds) {
  const int pm = u / (p.c.n_cc * p.c.n_sub);
  const int cc = u % p.c.n_cc;
  const int c_lo = p.c.col0 + cc * p.c.comm_bn;
  const int c_hi = min(c_lo + p.c.comm_bn, p.c.col0 + p.c.ncols);
  const int pn_lo = c_lo / S::BN, pn_hi = (c_hi - 1) / S::BN;
  const int* f = p.ws + kFlagBase + pm * p.order.n_pn;
  bool rows_ready = false;  // unused by reduce ops
  uint32_t polls = 0;
  int pause = 1;
  bool deps_open = true;  // thread 0: some tile this unit needs may be unclaimed
  while (true) {
    if (threadIdx.x == 0) {
      int ready = 1, help = -1;
      for (int pn = pn_lo; pn <= pn_hi; ++pn)
        if (ld_relaxed(f + pn) == 0) { ready = 0; break; }
      if (ready) {
        fence_acquire();
      } else if (deps_open) {
        // a needed tile still in its XCD queue: take work from that queue
        int hx = -1;
        for (int pn = pn_lo; pn <= pn_hi && hx < 0; ++pn) {
          int x, j;
          xcd_slot(p.xcd_q, tile_index(p.order, pm, pn), x, j);
          if (ld_relaxed(p.ws + kCtrGemm + x * kLine) <= j) hx = x;
        }
        if (hx < 0) {
          deps_open = false;
        } else {
          const int t = xcd_tile(p.xcd_q, hx, fetch_add(p.ws + kCtrGemm + hx * kLine, 1));
          if (t < p.T_gemm) {
            help = t;
            slot[2] = hx;
          }
        }
      } else if (++polls > p.spin_limit) {
        __hip_atomic_store(p.ws + kErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = 1;
      }
      slot[0] = ready;
      slot[1] = help;
    }
    __syncthreads();
    const int ready = slot[0], help = slot[1];
    __syncthreads();
    if (ready) return;
    if (help >= 0) {
      const int q = slot[2];
      run_gemm_tile<OP, S>(p, help, slot, lds, rows_ready);
      tile_done(p, q);
    } else {
      backoff(pause);
    }
  }
}

template <int OP, class S>
__device__ void run_gemm_tile(const Params& p, int t, int* slot, char* lds, bool& rows_ready) {
  int pm, pn;
  tile_coords(p.order, t, pm, pn);
  if constexpr (OP == OP_AG) {
    if (p.fused) wait_rows<OP, S>(p, pm, slot, rows_ready);
  }
  gemm_tile<S>(p.g, pm * S::BM, pn * S::BN, lds);
  if constexpr (OP == OP_ARMM) {
    if (p.fused) publish(p.ws + kFlagBase + pm * p.order.n_pn + pn);
  } else if constexpr (OP == OP_RS) {
    // only the columns of this rank's slice are consumed
    if (p.fused && pn >= p.order.prio_lo && pn < p.order.prio_hi)
      publish(p.ws + kFlagBase + pm * p.order.n_pn + pn);
  }
}

// ----------------------------------------------------------------- kernels
// The persistent kernel's body. Two kernels run it: persistent_kernel for
// every op, and gather_only_kernel for the sequential all_gather's copy
// (T_gemm = 0), whose launches then show apart from the GEMM's in traces.
template <int OP, int BM, int BN>
__device__ __forceinline__ void persistent_body(const Params& p) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) char lds[S::LDS_BYTES];
  __shared__ int slot[4];
  uint64_t gs = ~0ull, ge = 0, cs = ~0ull, ce = 0;
  bool rows_ready = false;
  // shader-clock and constant-rate counters at entry (and exit, below): the
  // host divides one by the other for the clock the chip held
  __shared__ uint64_t entry[2];
  if (threadIdx.x == 0) {
    entry[0] = clock64();
    entry[1] = wall_clock64();
  }
  const int home = xcd_id();
  uint32_t gone = 0;
  const bool gemm_first = (int)blockIdx.x < p.gemm_wgs || p.T_comm == 0;
  for (int phase = 0; phase < 2; ++phase) {
    if (phase == 1 && !p.steal) break;
    const bool do_gemm = (phase == 0) == gemm_first;
    if (do_gemm) {
      if constexpr (OP == OP_AG) {
        if (p.fused && phase == 1 && p.T_gemm > (int)gridDim.x) wait_all_units<OP>(p, rows_ready);
      }
      while (true) {
        const int t = claim_gemm(p, home, gone, slot);
        if (t < 0) break;
        const int q = slot[3];
        const uint64_t t0 = stamp_now();
        gs = t0 < gs ? t0 : gs;
        run_gemm_tile<OP, S>(p, t, slot, lds, rows_ready);
        tile_done(p, q);
        ge = stamp_now();
      }
    } else {
      // From its second unit on, thread 0 claims the next unit as this one
      // starts: the atomic's round trip overlaps the unit's first loads, and
      // the claim that finds the queue empty costs nothing after the last
      // unit (g2 all_gather_matmul, 146 copy units per workgroup: 1.7 %
      // faster on MI355X). Not on the first unit: with about one unit per
      // workgroup (pow2_4k) the first workgroups to start would take two
      // units each and the copy would pile up on half of them. A unit claimed
      // ahead is held by this running workgroup, which takes it up next.
      int u = claim(p.ws + kCtrComm, p.T_comm, slot);
      bool claim_ahead = false;
      while (u >= 0) {
        int ahead = 0;
        if (claim_ahead && threadIdx.x == 0) ahead = fetch_add(p.ws + kCtrComm, 1);
        if constexpr (OP == OP_RS || OP == OP_ARMM) {
          if (p.fused) wait_tiles<OP, S>(p, u, slot, lds);
        }
        const uint64_t t0 = stamp_now();
        cs = t0 < cs ? t0 : cs;
        run_comm_unit<OP>(p, u);
        finish_comm_unit<OP>(p, u);
        ce = stamp_now();
        if (claim_ahead) {
          if (threadIdx.x == 0) slot[0] = ahead;
          __syncthreads();
          const int v = slot[0];
          __syncthreads();
          u = v < p.T_comm ? v : -1;
        } else {
          u = claim(p.ws + kCtrComm, p.T_comm, slot);
          claim_ahead = true;
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (p.T_gemm == 0) {
      // comm-only launch (the sequential gather): the comm kernel's stamp
      // layout, and the GEMM launch that follows keeps its own records
      p.comm_stamps[(size_t)blockIdx.x * 2] = cs;
      p.comm_stamps[(size_t)blockIdx.x * 2 + 1] = ce;
    } else {
      uint64_t* st = p.stamps + (size_t)blockIdx.x * 4;
      st[0] = gs;
      st[1] = ge;
      st[2] = cs;
      st[3] = ce;
      uint64_t* ck = p.stamps + (size_t)kMaxGrid * kClockOff + (size_t)blockIdx.x * 4;
      ck[0] = entry[0];
      ck[1] = entry[1];
      ck[2] = clock64();
      ck[3] = wall_clock64();
    }
    // Every counter and flag access of this workgroup was made by this
    // thread, at agent scope; once they have completed (the drain) none can
    // follow the count below, so the last workgroup's reset cannot race
    // them. A release here (an L2 write-back per workgroup, of the C tiles
    // just stored) cost about 3 us per launch and orders nothing needed: the
    // kernel's end publishes C.
    drain_vmem();
    const int done = __hip_atomic_fetch_add(p.ws + kDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    slot[0] = (done == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (slot[0]) {  // last workgroup out: leave the workspace zeroed for the next op
    // every other workgroup's accesses completed before its count (above),
    // so the error word is final here; its bit outlives the launch in the
    // status word, which only the host clears
    if (threadIdx.x == 0 && ld_relaxed(p.ws + kErr) != 0)
      __hip_atomic_fetch_or(p.ws + kStatus, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    for (int i = threadIdx.x; i < p.n_reset; i += kThreads)
      if (i != kStatus) p.ws[i] = 0;
  }
}

template <int OP, int BM, int BN>
__global__ __launch_bounds__(kThreads) void persistent_kernel(Params p) {
  persistent_body<OP, BM, BN>(p);
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gather_only_kernel(Params p) {
  persistent_body<OP_AG, BM, BN>(p);
}

// Sequential-mode comm kernel: every unit, no flags, grid-strided.
template <int OP>
__global__ __launch_bounds__(kThreads) void comm_only_kernel(Params p) {
  uint64_t cs = ~0ull, ce = 0;
  // fewer units than workgroups: each unit is shared by nparts workgroups
  const uint32_t nparts = (uint32_t)max(1, (int)gridDim.x / max(1, p.T_comm));
  const int64_t n_virtual = (int64_t)p.T_comm * nparts;
  for (int64_t v = blockIdx.x; v < n_virtual; v += gridDim.x) {
    if (cs == ~0ull) cs = stamp_now();
    const int u = (int)(v / nparts);
    run_comm_unit<OP, false>(p, u, (uint32_t)(v - (int64_t)u * nparts), nparts);
    ce = stamp_now();
  }
  if (threadIdx.x == 0) {
    p.comm_stamps[(size_t)blockIdx.x * 2] = cs;
    p.comm_stamps[(size_t)blockIdx.x * 2 + 1] = ce;
  }
}

// --------------------------------------------------------------- launchers
template <int OP, int BM, int BN>
static hipError_t launch_tile(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((persistent_kernel<OP, BM, BN>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_op(const Params& p, int grid, hipStream_t s) {
  switch (p.op) {
    case OP_GEMM: return launch_tile<OP_GEMM, BM, BN>(p, grid, s);
    case OP_AG: return launch_tile<OP_AG, BM, BN>(p, grid, s);
    case OP_RS: return launch_tile<OP_RS, BM, BN>(p, grid, s);
    case OP_ARMM: return launch_tile<OP_ARMM, BM, BN>(p, grid, s);
    case OP_CONC_AR: return launch_tile<OP_CONC_AR, BM, BN>(p, grid, s);
    case OP_CONC_COPY: return launch_tile<OP_CONC_COPY, BM, BN>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

bool tile_supported(int bm, int bn) {
  return (bm == 256 && bn == 256) || (bm == 256 && bn == 128) || (bm == 128 && bn == 128) ||
         (bm == 64 && bn == 64);
}

hipError_t launch_persistent(const Params& p, int bm, int bn, int grid, hipStream_t s) {
  if (bm == 256 && bn == 256) return launch_op<256, 256>(p, grid, s);
  if (bm == 256 && bn == 128) return launch_op<256, 128>(p, grid, s);
  if (bm == 128 && bn == 128) return launch_op<128, 128>(p, grid, s);
  if (bm == 64 && bn == 64) return launch_op<64, 64>(p, grid, s);
  return hipErrorInvalidValue;
}

template <int BM, int BN>
static hipError_t launch_gather_tile(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gather_only_kernel<BM, BN>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather_only(const Params& p, int bm, int bn, int grid, hipStream_t s) {
  if (p.op != OP_AG || p.T_gemm != 0) return hipErrorInvalidValue;
  if (bm == 256 && bn == 256) return launch_gather_tile<256, 256>(p, grid, s);
  if (bm == 256 && bn == 128) return launch_gather_tile<256, 128>(p, grid, s);
  if (bm == 128 && bn == 128) return launch_gather_tile<128, 128>(p, grid, s);
  if (bm == 64 && bn == 64) return launch_gather_tile<64, 64>(p, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_comm_only(const Params& p, int grid, hipStream_t s) {
  switch (p.op) {
    case OP_AG:
      hipLaunchKernelGGL((comm_only_kernel<OP_AG>), dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case OP_RS:
      hipLaunchKernelGGL((comm_only_kernel<OP_RS>), dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case OP_ARMM:
      hipLaunchKernelGGL((comm_only_kernel<OP_ARMM>), dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case OP_CONC_AR:
      hipLaunchKernelGGL((comm_only_kernel<OP_CONC_AR>), dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case OP_CONC_COPY:
      hipLaunchKernelGGL((comm_only_kernel<OP_CONC_COPY>), dim3(grid), dim3(kThreads), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int OP, int BM, int BN>
static int occ_tile() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)persistent_kernel<OP, BM, BN>,
                                                   kThreads, 0) != hipSuccess)
    return -1;
  return n;
}

template <int BM, int BN>
static int occ_op(int op) {
  switch (op) {
    case OP_GEMM: return occ_tile<OP_GEMM, BM, BN>();
    case OP_AG: return occ_tile<OP_AG, BM, BN>();
    case OP_RS: return occ_tile<OP_RS, BM, BN>();
    case OP_ARMM: return occ_tile<OP_ARMM, BM, BN>();
    case OP_CONC_AR: return occ_tile<OP_CONC_AR, BM, BN>();
    case OP_CONC_COPY: return occ_tile<OP_CONC_COPY, BM, BN>();
  }
  return -1;
}

// ------------------------------------------------------ static scratch
// The workspace of iris_ag_mm_noalloc, for callers that cannot allocate
// device memory (code under graph capture, allocation-free serving loops).
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory:
// host code uses only the per-device address that hipGetSymbolAddress
// returns (scratch_setup), never the array's name.
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ __launch_bounds__(kThreads) void zero_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once set up
}  // namespace

// Address of this device's scratch. On the first call for a device (which
// must be current), looks the address up and enqueues a fill kernel that
// zeroes the array on `s`, ahead of whatever the caller enqueues next (a
// kernel, not a memset node, so that a caller capturing the first call
// records a node that replays correctly).
hipError_t scratch_setup(int dev, hipStream_t s, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(kThreads), 0, s, (uint32_t*)ptr,
                       (uint32_t)(kScratchBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// The scratch address of `dev` if it has been set up, else null.
void* scratch_if_set_up(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch[dev];
}

int persistent_blocks_per_cu(int bm, int bn, int op) {
  if (bm == 256 && bn == 256) return occ_op<256, 256>(op);
  if (bm == 256 && bn == 128) return occ_op<256, 128>(op);
  if (bm == 128 && bn == 128) return occ_op<128, 128>(op);
  if (bm == 64 && bn == 64) return occ_op<64, 64>(op);
  return -1;
}

}  // namespace iris
