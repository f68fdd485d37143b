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
// flags in the workspace:
//   all_gather:  flag[pm*W + s] = 1 once shard s of row block pm is copied;
//                a GEMM tile of row block pm waits for all W flags.
//   reduce:      flag[pm*n_pn + pn] = 1 once GEMM tile (pm, pn) is stored;
//                a reduce unit waits for the tiles covering its columns.
// A workgroup that has to wait first takes unclaimed work from the queue it
// waits on, so every wait ends even if not all workgroups are resident: a
// claimed unit is always held by a running workgroup whose own work never
// waits on the other queue.
#include "launch.hpp"

namespace iris {

// ---------------------------------------------------------------- swizzle
// t -> (pm, pn) on an n_pm x ncols grid, GROUP_M rows of tiles per group,
// column-major inside a group.
__device__ __forceinline__ void grouped(int t, int n_pm, int ncols, int gm, int& pm, int& pn) {
  const int width = gm * ncols;
  const int group = t / width;
  const int first = group * gm;
  const int gsz = min(gm, n_pm - first);
  const int r = t - group * width;
  pm = first + r % gsz;
  pn = r / gsz;
}

// Column tiles [prio_lo, prio_hi) are visited first (all rows), then the rest.
__device__ __forceinline__ void tile_coords(const Params& p, int t, int& pm, int& pn) {
  const int np1 = p.prio_hi - p.prio_lo;
  const int T1 = p.n_pm * np1;
  int q;
  if (t < T1) {
    grouped(t, p.n_pm, np1, p.group_m, pm, q);
    pn = p.prio_lo + q;
  } else {
    grouped(t - T1, p.n_pm, p.n_pn - np1, p.group_m, pm, q);
    pn = q < p.prio_lo ? q : q + np1;
  }
}

// ------------------------------------------------------------------ queues
__device__ __forceinline__ int claim(int* ctr, int T, int* slot) {
  if (threadIdx.x == 0) {
    int v = T;
    if (ld_relaxed(ctr) < T) v = fetch_add(ctr, 1);
    slot[0] = v;
  }
  __syncthreads();
  const int v = slot[0];
  __syncthreads();
  return v < T ? v : -1;
}

// Release of a unit's results to other workgroups (any XCD): every wave
// drains its stores to L2, the workgroup barriers, then one thread writes the
// XCD's L2 back (agent-scope release fence), waits for that write-back to
// finish, and only then sets the flag. The explicit wait matters: once the
// stores are drained the compiler sees nothing outstanding and would issue
// the flag store right behind the write-back.
__device__ __forceinline__ void publish(int* flag) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    drain_vmem();
    __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ comm units
template <int OP>
__device__ void run_comm_unit(const Params& p, int u) {
  if constexpr (OP == OP_AG) {
    const int pm = u / p.c.W;
    ag_copy_unit<8>(p.c, pm, u - pm * p.c.W);
  } else if constexpr (OP == OP_RS || OP == OP_ARMM) {
    const int pm = u / p.c.n_cc;
    reduce2d_unit<2>(p.c, pm, u - pm * p.c.n_cc);
  } else if constexpr (OP == OP_CONC_AR) {
    reduce_flat_unit<2>(p.c, u);
  }
}

template <int OP, class S>
__device__ void run_gemm_tile(const Params& p, int t, int* slot, char* lds);

// A GEMM tile of row block pm waits for the W shard copies of that block.
template <int OP, class S>
__device__ void wait_rows(const Params& p, int pm, int* slot) {
  const int* f = p.ws + kFlagBase + pm * p.c.W;
  uint32_t polls = 0;
  while (true) {
    if (threadIdx.x == 0) {
      int ready = 1, help = -1;
      for (int s = 0; s < p.c.W; ++s)
        if (ld_relaxed(f + s) == 0) { ready = 0; break; }
      if (ready) {
        fence_acquire();
      } else if (ld_relaxed(p.ws + kCtrComm) < p.T_comm) {
        const int u = fetch_add(p.ws + kCtrComm, 1);
        if (u < p.T_comm) help = u;
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
      run_comm_unit<OP>(p, help);
      publish(p.ws + kFlagBase + help);
    } else {
      __builtin_amdgcn_s_sleep(4);
    }
  }
}

// A reduce unit waits for the GEMM tiles covering its rows and columns.
template <int OP, class S>
__device__ void wait_tiles(const Params& p, int u, int* slot, char* lds) {
  const int pm = u / p.c.n_cc;
  const int cc = u - pm * p.c.n_cc;
  const int c_lo = p.c.col0 + cc * p.c.comm_bn;
  const int c_hi = min(c_lo + p.c.comm_bn, p.c.col0 + p.c.ncols);
  const int pn_lo = c_lo / S::BN, pn_hi = (c_hi - 1) / S::BN;
  const int* f = p.ws + kFlagBase + pm * p.n_pn;
  uint32_t polls = 0;
  while (true) {
    if (threadIdx.x == 0) {
      int ready = 1, help = -1;
      for (int pn = pn_lo; pn <= pn_hi; ++pn)
        if (ld_relaxed(f + pn) == 0) { ready = 0; break; }
      if (ready) {
        fence_acquire();
      } else if (ld_relaxed(p.ws + kCtrGemm) < p.T_gemm) {
        const int t = fetch_add(p.ws + kCtrGemm, 1);
        if (t < p.T_gemm) help = t;
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
      run_gemm_tile<OP, S>(p, help, slot, lds);
    } else {
      __builtin_amdgcn_s_sleep(4);
    }
  }
}

template <int OP, class S>
__device__ void run_gemm_tile(const Params& p, int t, int* slot, char* lds) {
  int pm, pn;
  tile_coords(p, t, pm, pn);
  if constexpr (OP == OP_AG) {
    if (p.fused) wait_rows<OP, S>(p, pm, slot);
  }
  gemm_tile<S>(p.g, pm * S::BM, pn * S::BN, lds);
  if constexpr (OP == OP_RS || OP == OP_ARMM) {
    if (p.fused) publish(p.ws + kFlagBase + pm * p.n_pn + pn);
  }
}

// ----------------------------------------------------------------- kernels
template <int OP, int BM, int BN>
__global__ __launch_bounds__(kThreads) void persistent_kernel(Params p) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) char lds[S::LDS_BYTES];
  __shared__ int slot[2];
  uint64_t gs = ~0ull, ge = 0, cs = ~0ull, ce = 0;
  const bool gemm_first = (int)blockIdx.x < p.gemm_wgs || p.T_comm == 0;
  for (int phase = 0; phase < 2; ++phase) {
    if (phase == 1 && !p.steal) break;
    const bool do_gemm = (phase == 0) == gemm_first;
    if (do_gemm) {
      while (true) {
        const int t = claim(p.ws + kCtrGemm, p.T_gemm, slot);
        if (t < 0) break;
        const uint64_t t0 = stamp_now();
        gs = t0 < gs ? t0 : gs;
        run_gemm_tile<OP, S>(p, t, slot, lds);
        ge = stamp_now();
      }
    } else {
      while (true) {
        const int u = claim(p.ws + kCtrComm, p.T_comm, slot);
        if (u < 0) break;
        if constexpr (OP == OP_RS || OP == OP_ARMM) {
          if (p.fused) wait_tiles<OP, S>(p, u, slot, lds);
        }
        const uint64_t t0 = stamp_now();
        cs = t0 < cs ? t0 : cs;
        run_comm_unit<OP>(p, u);
        if constexpr (OP == OP_AG) {
          if (p.fused) publish(p.ws + kFlagBase + u);
        }
        ce = stamp_now();
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* st = p.stamps + (size_t)blockIdx.x * 4;
    st[0] = gs;
    st[1] = ge;
    st[2] = cs;
    st[3] = ce;
    // everything this workgroup did to the counters and flags precedes this
    const int done = __hip_atomic_fetch_add(p.ws + kDone, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    slot[0] = (done == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (slot[0]) {  // last workgroup out: leave the workspace zeroed for the next op
    for (int i = threadIdx.x; i < p.n_reset; i += kThreads)
      if (i != kErr) p.ws[i] = 0;
  }
}

// Sequential-mode comm kernel: every unit, no flags, grid-strided.
template <int OP>
__global__ __launch_bounds__(kThreads) void comm_only_kernel(Params p) {
  uint64_t cs = ~0ull, ce = 0;
  for (int u = blockIdx.x; u < p.T_comm; u += gridDim.x) {
    if (cs == ~0ull) cs = stamp_now();
    run_comm_unit<OP>(p, u);
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
  }
  return -1;
}

int persistent_blocks_per_cu(int bm, int bn, int op) {
  if (bm == 256 && bn == 256) return occ_op<256, 256>(op);
  if (bm == 256 && bn == 128) return occ_op<256, 128>(op);
  if (bm == 128 && bn == 128) return occ_op<128, 128>(op);
  if (bm == 64 && bn == 64) return occ_op<64, 64>(op);
  return -1;
}

}  // namespace iris
