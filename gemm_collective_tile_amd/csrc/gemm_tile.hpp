// One C tile of  C = A @ B + bias  on gfx950 matrix cores.
//
// A (M x K) and B (K x N) are row-major fp16; C is row-major fp16; the
// products accumulate in fp32 and each output is rounded once (to nearest
// even) after the bias add. The operation is the GEMM part of every op on
// the Iris docs page "Fused Communication and Compute Operations"; the tile
// decomposition, the per-tile K loop and default-cached operand loads follow
// the iris.concurrent PR ("Add iris.concurrent ...", commit that moves the
// GEMM tile onto a shared K-loop building block and keeps the default L1/L2
// caching of operands because bypassing L1 loses operand reuse).
//
// gfx950 design:
//   * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a
//     (BM/2) x (BN/2) sub-tile held in fp32 accumulators (AGPRs).
//   * v_mfma_f32_32x32x16_f16 computes 32x32 output blocks, K step 16. Lane
//     l supplies, for its row (A) or column (B) l % 32, the 8 consecutive k
//     8*(l/32) .. 8*(l/32)+7 of the 16-wide k slice.
//   * Operands go global -> LDS with buffer_load ... lds (LDS DMA): no
//     registers, no LDS write instructions. One wave instruction moves
//     1 KiB: lane l's 16 bytes land at LDS base + 16 l, so the layout in LDS
//     is chosen by which global 16-byte chunk each lane fetches.
//   * K is walked in steps of BK = 32 through a ring of NSTAGE = 4 LDS
//     stages: A as [BM][32] (64-byte rows), B as [32][BN] (row-major, as
//     stored). The 16-byte chunks of every row are XOR-swizzled by a
//     function of the row so that the fragment reads spread over the banks.
//   * A fragments: one ds_read_b128 (8 consecutive k of one row).
//     B fragments: two ds_read_b64_tr_b16. In each 16-lane group that
//     instruction returns to lane j element (j & 3) of the 8-byte chunks
//     addressed by lanes 4e + (j >> 2), e = 0..3; with lane 4e + q pointing
//     at k row kb + e, columns nb + 4q .. nb + 4q + 3 of the [k][n] stage,
//     lane j receives column nb + j at the 4 consecutive k rows kb .. kb+3.
//     Two such reads give the 8 k of an MFMA operand, in the same k order
//     as the A fragment.
//   * Masking of ragged edges: buffer loads whose offset is past the
//     resource size return zeros (M and K rows), and chunks past N or past
//     K inside a row are given an out-of-range offset.
//   * Pipeline: loads run NSTAGE - 1 steps ahead. Each K step issues the
//     loads of step t+3 and the fragment reads of slice 1 under the MFMAs of
//     slice 0; halfway through slice 1 it waits for its own loads of step
//     t+1, passes the one barrier of the step, and reads the slice-0
//     fragments of step t+1 under the rest of slice 1.
//   * The MFMA takes B as its first operand and A as its second, so each
//     lane ends up holding 4 consecutive output columns of one row: the
//     epilogue stores 8 bytes per lane after adding the bias.
#pragma once

#include "device_common.hpp"

namespace iris {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

template <int BM_, int BN_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = 32, NSTAGE = 4;
  static constexpr int WTM = BM / 2, WTN = BN / 2;    // per-wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int RA = BK * 2;                   // bytes per A row in LDS (64)
  static constexpr int RB = BN * 2;                   // bytes per B row in LDS
  static constexpr int CPR_B = BN / 8;                // 16-byte chunks per B row
  static constexpr int A_STAGE = BM * RA;
  static constexpr int B_STAGE = BK * RB;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int B_RING = NSTAGE * A_STAGE;     // LDS: [A stages | B stages]
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int A_DMA = A_STAGE / 1024 / 4;    // 1 KiB DMA instructions per wave per step
  static constexpr int B_DMA = B_STAGE / 1024 / 4;
  static constexpr int RPB = 1024 / RB;               // B rows per DMA instruction
  static_assert(FM >= 1 && FN >= 1, "tile too small for 32x32 blocks");
  static_assert(A_DMA >= 1 && B_DMA >= 1, "tile too small for 4 waves of 1 KiB loads");
};

// swizzle of the 16-byte chunks of a 64-byte A row (4 chunks)
#ifndef IRIS_SWZ_A
#define IRIS_SWZ_A 1
#endif
__device__ __forceinline__ uint32_t swz_a(uint32_t r) {
  if (IRIS_SWZ_A == 1) return (r >> 2) & 3u;
  if (IRIS_SWZ_A == 2) return r & 3u;
  if (IRIS_SWZ_A == 3) return 0u;
  if (IRIS_SWZ_A == 4) return ((r >> 1) ^ (r >> 2)) & 3u;
  return ((r >> 1) ^ (r >> 3)) & 3u;
}
// swizzle of the 16-byte chunks of a B row, by k row
#ifndef IRIS_SWZ_B_MUL
#define IRIS_SWZ_B_MUL 4
#endif
template <class S>
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
  return ((k & 3u) * IRIS_SWZ_B_MUL) & (uint32_t)(S::CPR_B - 1);
}

struct GemmArgs {
  const f16* A;
  int64_t lda;
  const f16* B;
  int64_t ldb;
  const f16* bias;
  int32_t bias_along_m;
  f16* C;
  int64_t ldc;
  int32_t M, N, K;
};

template <class S>
struct GemmPipe {
  // per-lane byte offsets of the DMA chunks within a K step's resource
  uint32_t a_off[S::A_DMA];
  uint32_t a_kc;             // k offset (elements) of this lane's A chunks
  uint32_t b_off[S::B_DMA];
  // LDS byte offsets of the fragment reads within the A / B rings
  uint32_t ra_base[2];        // A, per k slice
  uint32_t rb_base[S::FN];    // B, per 32-column block (includes B_RING)
  uint32_t wave;              // wave index, uniform (scalar)

  __device__ __forceinline__ void setup(const GemmArgs& g, int n0) {
    const uint32_t l = threadIdx.x & 63;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = w >> 1, wn = w & 1;
    wave = w;
    // A instruction b covers tile rows 16 b .. 16 b + 15: lane l takes row
    // 16 b + (l >> 2) and LDS chunk l & 3, i.e. logical chunk (l & 3) ^ swz
    // (swz_a(16 b + r) == swz_a(r), so the chunk is the same for every b)
    const uint32_t ca = (l & 3) ^ swz_a(l >> 2);
    a_kc = 8 * ca;
#pragma unroll
    for (int n = 0; n < S::A_DMA; ++n) {
      const uint32_t r = 16 * (w * S::A_DMA + n) + (l >> 2);
      a_off[n] = (uint32_t)((r * g.lda + 8 * ca) * 2);
    }
#pragma unroll
    for (int n = 0; n < S::B_DMA; ++n) {
      // B instruction b covers k rows RPB b .. RPB b + RPB - 1
      const uint32_t k = S::RPB * (w * S::B_DMA + n) + l / S::CPR_B;
      const uint32_t c = (l % S::CPR_B) ^ swz_b<S>(k);
      const bool ok = n0 + 8 * (int)c < g.N;
      b_off[n] = ok ? (uint32_t)((k * g.ldb + 8 * c) * 2) : kOob;
    }
    {
      const uint32_t r = wm * S::WTM + (l & 31);
      const uint32_t h = l >> 5;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) ra_base[sl] = r * S::RA + (((2 * sl + h) ^ swz_a(r)) << 4);
    }
    {
      const uint32_t grp = l >> 4, e = (l >> 2) & 3, q = l & 3;
      const uint32_t k = 8 * (grp >> 1) + e;
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const uint32_t c = (wn * S::WTN + 32 * j) / 8 + 2 * (grp & 1) + (q >> 1);
        rb_base[j] = S::B_RING + k * S::RB + ((c ^ swz_b<S>(k)) << 4) + 8 * (q & 1);
      }
    }
  }

  // Buffer resources of K step `step` (k0 = step * BK): rows past M and K
  // fall outside them.
  struct Rsrc {
    u32x4 a, b;
    bool kok;
  };
  __device__ __forceinline__ Rsrc rsrc(const GemmArgs& g, int m0, int n0, int step) const {
    Rsrc r;
    const int k0 = step * S::BK;
    const int rows = min(S::BM, g.M - m0);
    const int64_t abytes = (int64_t)rows * g.lda * 2 - (int64_t)k0 * 2;
    r.a = rsrc_words(g.A + (int64_t)m0 * g.lda + k0, abytes > 0 ? (uint32_t)abytes : 0u);
    const int krows = min(S::BK, g.K - k0);
    r.b = rsrc_words(g.B + (int64_t)k0 * g.ldb + n0,
                     krows > 0 ? (uint32_t)((int64_t)krows * g.ldb * 2 - (int64_t)n0 * 2) : 0u);
    r.kok = k0 + (int)a_kc < g.K;
    return r;
  }

  // DMA number D (A instructions first, then B) of a K step into ring slot ST
  template <int D>
  __device__ __forceinline__ void dma(const Rsrc& r, uint32_t lds_base, int ST) const {
    if constexpr (D < S::A_DMA) {
      dma16(r.a, lds_base + ST * S::A_STAGE + (wave * S::A_DMA + D) * 1024, r.kok ? a_off[D] : kOob);
    } else {
      constexpr int n = D - S::A_DMA;
      dma16(r.b, lds_base + S::B_RING + ST * S::B_STAGE + (wave * S::B_DMA + n) * 1024, b_off[n]);
    }
  }

  struct Frags {
    f16x8 a[S::FM];
    f16x8 b[S::FN];
  };

  // fragment read item X of k slice SL from ring slot ST: items alternate
  // a0, b0, a1, b1, ... so that the operands of the first MFMA blocks arrive
  // first
  template <int SL, int X>
  __device__ __forceinline__ void read(const char* lds, int ST, Frags& f) const {
    constexpr int NMIN = S::FM < S::FN ? S::FM : S::FN;
    constexpr bool IS_A = X < 2 * NMIN ? (X % 2 == 0) : (S::FM > S::FN);
    constexpr int IDX = X < 2 * NMIN ? X / 2 : X - NMIN;
    if constexpr (IS_A) {
      f.a[IDX] = as_h8(*(const u32x4*)(lds + ra_base[SL] + ST * S::A_STAGE + IDX * 32 * S::RA));
    } else {
      const char* p = lds + rb_base[IDX] + ST * S::B_STAGE + SL * 16 * S::RB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * S::RB));
      u32x4 v;
      v[0] = __builtin_bit_cast(u32x2, lo)[0];
      v[1] = __builtin_bit_cast(u32x2, lo)[1];
      v[2] = __builtin_bit_cast(u32x2, hi)[0];
      v[3] = __builtin_bit_cast(u32x2, hi)[1];
      f.b[IDX] = as_h8(v);
    }
  }
};

// MFMA block K of a k slice: row block K / FN, column block K % FN
template <class S, int K>
__device__ __forceinline__ void mma_block(f32x16 (&acc)[S::FM][S::FN], const typename GemmPipe<S>::Frags& f) {
  constexpr int i = K / S::FN, j = K % S::FN;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// s_waitcnt with the vector-memory counter limited to VM and the LDS counter
// to LG (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int VM, int LG = 15>
__device__ __forceinline__ void wait_cnt() {
  static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LG << 8));
}

// Slots of a K step, issued in program order:
//   region 1: slot k = MFMA block k of slice 0 (fragments f0), then fragment
//             read item k of slice 1 into f1, then DMA k of step t+3 (the
//             DMAs go first so they have the most time to land); then the first half of slice 1's MFMA blocks.
//   wait for this wave's DMAs of step t+1 and its own LDS reads; barrier.
//   region 2: the second half of slice 1's blocks, each followed by two
//             fragment reads of slice 0 of step t+1 (stage NXT) into f0.
template <class S, int K, int NM, int NR, int ND>
__device__ __forceinline__ void region1(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r,
                                        const char* lds, uint32_t lds_base, int cur, int ahead,
                                        typename GemmPipe<S>::Frags& f0, typename GemmPipe<S>::Frags& f1,
                                        f32x16 (&acc)[S::FM][S::FN]) {
  constexpr int SLOTS = NM > NR ? (NM > ND ? NM : ND) : (NR > ND ? NR : ND);
  if constexpr (K < SLOTS) {
    if constexpr (K < NM) mma_block<S, K>(acc, f0);
    if constexpr (K < NR) P.template read<1, K>(lds, cur, f1);
    constexpr int D = K;
    if constexpr (D >= 0 && D < ND) P.template dma<D>(r, lds_base, ahead);
    region1<S, K + 1, NM, NR, ND>(P, r, lds, lds_base, cur, ahead, f0, f1, acc);
  }
}

template <class S, int K, int K1, int NM>
__device__ __forceinline__ void mma_range(f32x16 (&acc)[S::FM][S::FN], const typename GemmPipe<S>::Frags& f) {
  if constexpr (K < K1 && K < NM) {
    mma_block<S, K>(acc, f);
    mma_range<S, K + 1, K1, NM>(acc, f);
  }
}

template <class S, int K, int NM, int NR, int X>
__device__ __forceinline__ void region2(const GemmPipe<S>& P, const char* lds, int nxt,
                                        typename GemmPipe<S>::Frags& f0, const typename GemmPipe<S>::Frags& f1,
                                        f32x16 (&acc)[S::FM][S::FN]) {
  if constexpr (K < NM || X < NR) {
    if constexpr (K < NM) mma_block<S, K>(acc, f1);
    if constexpr (X < NR) P.template read<0, X>(lds, nxt, f0);
    if constexpr (X + 1 < NR) P.template read<0, X + 1>(lds, nxt, f0);
    region2<S, K + 1, NM, NR, X + 2>(P, lds, nxt, f0, f1, acc);
  }
}

// Scheduling groups (masks of __builtin_amdgcn_sched_group_barrier: 0x8
// MFMA, 0x100 LDS read). Region 1: slot k = one MFMA, then the LDS reads of
// fragment item k (1 for an A item, 2 for a B item). Region 2: one MFMA, then
// the reads of two items. The DMA (inline asm) keeps its program order.
template <class S>
__device__ constexpr int item_reads(int x) {
  constexpr int NMIN = S::FM < S::FN ? S::FM : S::FN;
  if (x >= S::FM + S::FN) return 0;
  const bool is_a = x < 2 * NMIN ? (x % 2 == 0) : (S::FM > S::FN);
  return is_a ? 1 : 2;
}

template <class S, int K, int NM>
__device__ __forceinline__ void sched_region1() {
  if constexpr (K < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (item_reads<S>(K) > 0) __builtin_amdgcn_sched_group_barrier(0x100, item_reads<S>(K), 0);
    sched_region1<S, K + 1, NM>();
  }
}

template <class S, int K, int NM, int X>
__device__ __forceinline__ void sched_region2() {
  if constexpr (K < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int R = item_reads<S>(X) + item_reads<S>(X + 1);
    if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    sched_region2<S, K + 1, NM, X + 2>();
  }
}

// One K step on ring slot ST (compile-time), fragments of slice 0 already
// in f0. Loads step t+3 into slot (ST+3) % NSTAGE.
template <class S, int ST>
__device__ __forceinline__ void k_step(const GemmPipe<S>& P, const GemmArgs& g, int m0, int n0, int t,
                                       const char* lds, uint32_t lds_base, typename GemmPipe<S>::Frags& f0,
                                       typename GemmPipe<S>::Frags& f1, f32x16 (&acc)[S::FM][S::FN]) {
  constexpr int NS = S::NSTAGE;
  constexpr int CUR = ST % NS, NXT = (ST + 1) % NS, AHEAD = (ST + NS - 1) % NS;
  constexpr int NM = S::FM * S::FN, NR = S::FM + S::FN, ND = S::A_DMA + S::B_DMA;
  constexpr int H1 = NM / 2;
  // keep the scheduler from hoisting this step's reads into the previous
  // step (that would hold three fragment sets live and spill)
  __builtin_amdgcn_sched_barrier(0);
  const typename GemmPipe<S>::Rsrc r = P.rsrc(g, m0, n0, t + NS - 1);
  region1<S, 0, NM, NR, ND>(P, r, lds, lds_base, CUR, AHEAD, f0, f1, acc);
  mma_range<S, 0, H1, NM>(acc, f1);
  sched_region1<S, 0, NM + H1>();
  // step t+1 complete for this wave (t+2 and t+3 may be in flight), and
  // every fragment read of this slot done, before the barrier. The barrier
  // must carry the workgroup fences: without them the compiler may hoist the
  // next step's LDS reads above it.
  __builtin_amdgcn_sched_barrier(0);
  wait_cnt<(NS - 2) * ND, 0>();
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  region2<S, H1, NM, NR, 0>(P, lds, NXT, f0, f1, acc);
  sched_region2<S, H1, NM, 0>();
  __builtin_amdgcn_sched_barrier(0);
}

template <class S, int D, int ND>
__device__ __forceinline__ void dma_all(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r,
                                        uint32_t lds_base, int slot) {
  if constexpr (D < ND) {
    P.template dma<D>(r, lds_base, slot);
    dma_all<S, D + 1, ND>(P, r, lds_base, slot);
  }
}

template <class S, int X, int NR>
__device__ __forceinline__ void read_all(const GemmPipe<S>& P, const char* lds, int slot,
                                         typename GemmPipe<S>::Frags& f) {
  if constexpr (X < NR) {
    P.template read<0, X>(lds, slot, f);
    read_all<S, X + 1, NR>(P, lds, slot, f);
  }
}

// Computes the tile at (m0, n0) and writes it to C. `lds` must hold
// S::LDS_BYTES. Starts and ends with a workgroup barrier so callers may
// reuse the LDS around it.
template <class S>
__device__ void gemm_tile(const GemmArgs& g, int m0, int n0, char* lds) {
  using P_t = GemmPipe<S>;
  constexpr int NS = S::NSTAGE;
  constexpr int ND = S::A_DMA + S::B_DMA;  // DMA instructions per wave per step
  constexpr int NR = S::FM + S::FN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = (g.K + S::BK - 1) / S::BK;

  f32x16 acc[S::FM][S::FN];
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  P_t P;
  P.setup(g, n0);
  typename P_t::Frags f0, f1;
  // LDS byte address of the stage ring, for the DMA
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);

  __syncthreads();  // previous users of the LDS are done
  dma_all<S, 0, ND>(P, P.rsrc(g, m0, n0, 0), lds_base, 0);
  dma_all<S, 0, ND>(P, P.rsrc(g, m0, n0, 1), lds_base, 1);
  dma_all<S, 0, ND>(P, P.rsrc(g, m0, n0, 2), lds_base, 2);
  wait_cnt<(NS - 2) * ND>();  // this wave's part of step 0 has landed
  __syncthreads();
  read_all<S, 0, NR>(P, lds, 0, f0);

  // The ring has NS = 4 slots: unroll by 4 so every slot offset is a
  // constant. The step count is rounded up to a multiple of 4 (a loop with one
  // exit keeps the accumulators in place); the extra steps read only
  // out-of-range zeros and add exact zeros to accumulators that start at +0,
  // so they change no bit of the result.
  static_assert(NS == 4, "the K loop is unrolled by the ring size");
  const int nk4 = (nk + 3) & ~3;
  for (int t = 0; t < nk4; t += 4) {
    k_step<S, 0>(P, g, m0, n0, t, lds, lds_base, f0, f1, acc);
    k_step<S, 1>(P, g, m0, n0, t + 1, lds, lds_base, f0, f1, acc);
    k_step<S, 2>(P, g, m0, n0, t + 2, lds, lds_base, f0, f1, acc);
    k_step<S, 3>(P, g, m0, n0, t + 3, lds, lds_base, f0, f1, acc);
  }
  // loads issued past the last step target stages no one reads; let them
  // land before the LDS is reused
  wait_cnt<0, 0>();

  // epilogue: lane holds row m = lane & 31 of each 32x32 block and, for
  // q = 0..3, columns 8q + 4*(lane >> 5) + 0..3.
  const int khalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    const int m = m0 + wm * S::WTM + i * 32 + (lane & 31);
    if (m >= g.M) continue;
    const float bm = (g.bias && g.bias_along_m) ? (float)g.bias[m] : 0.0f;
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * S::WTN + j * 32 + 8 * q + 4 * khalf;
        if (n >= g.N) continue;
        f16x4 o;
        if (g.bias && !g.bias_along_m) {
          const f16x4 bv = *(const f16x4*)(g.bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (f16)(acc[i][j][4 * q + e] + (float)bv[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (f16)(acc[i][j][4 * q + e] + bm);
        }
        *(f16x4*)(g.C + (int64_t)m * g.ldc + n) = o;
      }
    }
  }
}

}  // namespace iris
