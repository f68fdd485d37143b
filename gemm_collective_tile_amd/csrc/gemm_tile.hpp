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
//   * K is walked in steps of BK = 64. Each thread loads its share of a
//     step's A and B tiles (16-byte buffer loads, default caching) into
//     registers two steps ahead and writes them to one of two LDS stages
//     one step ahead: A as
//     [BM][64] (128-byte rows: every load request fills a whole 128-byte
//     line; at 64-byte rows each line was fetched twice, and the operand
//     stream from L2 is bounded by the misses a CU keeps in flight), B as
//     [64][BN] (row-major, as stored). The 16-byte chunks of every row are
//     XOR-swizzled by a function of the row so that the fragment reads and
//     the LDS writes spread over the banks.
//     Loads go through registers rather than straight into LDS (the
//     buffer_load ... lds form): on gfx950 an ordinary LDS read waits for
//     every LDS-targeted load its wave still has in flight, whatever the
//     addresses, so with a load ring in flight each A fragment read would
//     wait out a global-memory latency.
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
//   * Pipeline of step t (stage t % 2 holds it, 4 k slices of 16): the
//     loads of step t+2 go out one every few MFMAs over the whole step (a
//     burst of them fills the address queue of the CU's memory pipeline and
//     stalls the wave with the MFMA pipe empty); the fragment reads of slice
//     s+1 run under the MFMAs of slice s; the registers of step t+1 (loaded
//     during step t-1) are written to the other stage, spread over the part
//     before the barrier; one barrier; the slice-0 fragments of step t+1 are
//     read under the second half of the last slice.
//   * The MFMA takes B as its first operand and A as its second, so each
//     lane ends up holding 4 consecutive output columns of one row: the
//     epilogue stores 8 bytes per lane after adding the bias.
#pragma once

#include "device_common.hpp"

namespace iris {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

template <int BM_, int BN_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NSTAGE = 2;
  static constexpr int NSL = BK / 16;                 // k slices (MFMA K steps) per K step
  static constexpr int WTM = BM / 2, WTN = BN / 2;    // per-wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int RA = BK * 2;                   // bytes per A row in LDS (128)
  static constexpr int CPR_A = BK / 8;                // 16-byte chunks per A row
  static constexpr int RB = BN * 2;                   // bytes per B row in LDS
  static constexpr int CPR_B = BN / 8;                // 16-byte chunks per B row
  static constexpr int A_STAGE = BM * RA;
  static constexpr int B_STAGE = BK * RB;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int B_RING = NSTAGE * A_STAGE;     // LDS: [A stages | B stages]
  static constexpr int STAGES_BYTES = NSTAGE * STAGE;
  // the tile's bias (BN columns or BM rows of fp16), staged for the epilogue
  static constexpr int BIAS_OFF = STAGES_BYTES;
  static constexpr int LDS_BYTES = STAGES_BYTES + 2 * (BM > BN ? BM : BN);
  static constexpr int A_LD = A_STAGE / 16 / 256;     // 16-byte chunks per thread per step
  static constexpr int B_LD = B_STAGE / 16 / 256;
  static_assert(FM >= 1 && FN >= 1, "tile too small for 32x32 blocks");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads of 16-byte loads");
};

// swizzle of the 16-byte chunks of a 128-byte A row (8 chunks): 16
// consecutive rows reading the same logical chunk land on 16 different
// 16-byte bank groups (row parity picks the half of the 256-byte bank
// cycle, (r >> 1) & 7 the slot in it)
__device__ __forceinline__ uint32_t swz_a(uint32_t r) { return (r >> 1) & 7u; }
// swizzle of the 16-byte chunks of a B row, by k row
template <class S>
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
  return ((k & 3u) * 4u) & (uint32_t)(S::CPR_B - 1);
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
  static constexpr int NLD = S::A_LD + S::B_LD;
  // per-thread byte offsets of the loaded chunks within a K step's resource,
  // and where they go in an LDS stage
  uint32_t a_off[S::A_LD];
  uint32_t a_kc;             // k offset (elements) of this thread's A chunks
  uint32_t b_off[S::B_LD];
  // LDS offsets of chunk 0; chunk n lies a fixed distance further (the
  // swizzles depend on the row only through bits that chunk n's row offset
  // leaves alone), so the distance folds into the LDS write's immediate
  uint32_t a_lds0;
  uint32_t b_lds0;           // includes B_RING
  static constexpr uint32_t A_ROWS_PER_LD = 256 / S::CPR_A;  // A rows per chunk index
  static constexpr uint32_t B_ROWS_PER_LD = 256 / S::CPR_B;  // B k rows per chunk index
  static_assert(A_ROWS_PER_LD % 16 == 0, "A chunk rows must keep the A swizzle");
  static_assert(B_ROWS_PER_LD % 4 == 0, "B chunk rows must keep the B swizzle");
  // LDS byte offsets of the fragment reads within the A / B rings
  uint32_t ra_base[S::NSL];   // A, per k slice
  uint32_t rb_base[S::FN];    // B, per 32-column block (includes B_RING)

  __device__ __forceinline__ void setup(const GemmArgs& g, int n0, uint32_t tid) {
    const uint32_t l = tid & 63;
    const uint32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = w >> 1, wn = w & 1;
    // A chunk c = tid + 256 n: row c / 8, k chunk c % 8 (= tid % 8 for every n)
    const uint32_t ca = tid & (S::CPR_A - 1);
    a_kc = 8 * ca;
#pragma unroll
    for (int n = 0; n < S::A_LD; ++n) {
      const uint32_t r = (tid + 256 * n) / S::CPR_A;
      a_off[n] = (uint32_t)((r * g.lda + 8 * ca) * 2);
    }
    a_lds0 = (tid / S::CPR_A) * S::RA + ((ca ^ swz_a(tid / S::CPR_A)) << 4);
    // B chunk c = tid + 256 n: k row c / CPR_B, column chunk c % CPR_B
#pragma unroll
    for (int n = 0; n < S::B_LD; ++n) {
      const uint32_t c = tid + 256 * n;
      const uint32_t k = c / S::CPR_B, ch = c % S::CPR_B;
      const bool ok = n0 + 8 * (int)ch < g.N;
      b_off[n] = ok ? (uint32_t)((k * g.ldb + 8 * ch) * 2) : kOob;
    }
    {
      const uint32_t k = tid / S::CPR_B, ch = tid % S::CPR_B;
      b_lds0 = S::B_RING + k * S::RB + ((ch ^ swz_b<S>(k)) << 4);
    }
    {
      const uint32_t r = wm * S::WTM + (l & 31);
      const uint32_t h = l >> 5;
#pragma unroll
      for (int sl = 0; sl < S::NSL; ++sl) ra_base[sl] = r * S::RA + (((2 * sl + h) ^ swz_a(r)) << 4);
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
    __amdgpu_buffer_rsrc_t a, b;
    bool kok;
  };
  __device__ __forceinline__ Rsrc rsrc(const GemmArgs& g, int m0, int n0, int step) const {
    Rsrc r;
    const int k0 = step * S::BK;
    const int rows = min(S::BM, g.M - m0);
    const int64_t abytes = (int64_t)rows * g.lda * 2 - (int64_t)k0 * 2;
    r.a = make_rsrc(g.A + (int64_t)m0 * g.lda + k0, abytes > 0 ? (uint32_t)abytes : 0u);
    const int krows = min(S::BK, g.K - k0);
    r.b = make_rsrc(g.B + (int64_t)k0 * g.ldb + n0,
                    krows > 0 ? (uint32_t)((int64_t)krows * g.ldb * 2 - (int64_t)n0 * 2) : 0u);
    r.kok = k0 + (int)a_kc < g.K;
    return r;
  }

  // a K step's share of this thread, in registers
  struct Regs {
    u32x4 v[NLD];
  };

  // load item D (A chunks first, then B) of a K step
  template <int D>
  __device__ __forceinline__ void load(const Rsrc& r, Regs& R) const {
    if constexpr (D < S::A_LD)
      R.v[D] = buf_load16(r.a, r.kok ? a_off[D] : kOob);
    else
      R.v[D] = buf_load16(r.b, b_off[D - S::A_LD]);
  }
  // write item D to LDS stage ST
  template <int D>
  __device__ __forceinline__ void store(char* lds, int ST, const Regs& R) const {
    if constexpr (D < S::A_LD)
      *(u32x4*)(lds + a_lds0 + (ST * S::A_STAGE + D * A_ROWS_PER_LD * S::RA)) = R.v[D];
    else
      *(u32x4*)(lds + b_lds0 + (ST * S::B_STAGE + (D - S::A_LD) * B_ROWS_PER_LD * S::RB)) = R.v[D];
  }

  struct Frags {
    f16x8 a[S::FM];
    f16x8 b[S::FN];
  };

  // fragment read item X of k slice SL from stage ST: items alternate a0,
  // b0, a1, b1, ... so that the operands of the first MFMA blocks arrive
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

// Scheduling groups (masks of __builtin_amdgcn_sched_group_barrier: 0x8
// MFMA, 0x20 global load, 0x100 LDS read, 0x200 LDS write). Every slot pins
// one MFMA, then the LDS reads of its fragment items (1 for an A item, 2 for
// a B item), then its load and its LDS write, if any.
template <class S>
__device__ constexpr int item_reads(int x) {
  constexpr int NMIN = S::FM < S::FN ? S::FM : S::FN;
  if (x >= S::FM + S::FN) return 0;
  const bool is_a = x < 2 * NMIN ? (x % 2 == 0) : (S::FM > S::FN);
  return is_a ? 1 : 2;
}

template <int MFMA, int READS, int LOADS, int WRITES>
__device__ __forceinline__ void pin_slot() {
  if constexpr (MFMA > 0) __builtin_amdgcn_sched_group_barrier(0x008, MFMA, 0);
  if constexpr (READS > 0) __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  if constexpr (LOADS > 0) __builtin_amdgcn_sched_group_barrier(0x020, LOADS, 0);
  if constexpr (WRITES > 0) __builtin_amdgcn_sched_group_barrier(0x200, WRITES, 0);
}

// Slot plan of a K step with NM MFMA blocks per k slice and NSL slices.
// Slice s owns slots s SPAN .. s SPAN + SPAN - 1, SPAN = max(NM, NR): slot
// s SPAN + b runs block b of slice s (b < NM) and reads fragment item b of
// slice s+1 (b < NR), so every read of a slice precedes its first block.
// Region 1 (before the barrier) ends after the first NM/2 blocks of the last
// slice (NSLOT slots); region 2 holds the rest of that slice (slots NSLOT ..
// NSL SPAN - 1) with the slice-0 reads of step t+1. The NLD loads of step
// t+2 go every LSP slots over the whole step, the LDS writes of step t+1
// every WSP slots over region 1. Region 1 grows extra slots without an MFMA
// when a small tile has more items than slots.
template <class S>
struct Plan {
  static constexpr int NM = S::FM * S::FN, NR = S::FM + S::FN, NLD = S::A_LD + S::B_LD;
  static constexpr int NSL = S::NSL;
  static constexpr int max2(int a, int b) { return a > b ? a : b; }
  static constexpr int SPAN = max2(NM, NR);
  static constexpr int NSLOT = (NSL - 1) * SPAN + NM / 2;
  static constexpr int NSTEP = NSL * SPAN;  // slots of the whole step
  static constexpr int LSP = NSTEP / NLD > 0 ? NSTEP / NLD : 1;
  static constexpr int WSP = NSLOT / NLD > 0 ? NSLOT / NLD : 1;
  static constexpr int W_END = WSP * (NLD - 1) + 1;
  static constexpr int READ_END = (NSL - 2) * SPAN + NR;
  static constexpr int REGION1 = max2(max2(NSLOT, READ_END), W_END);
  static constexpr bool is_mfma(int k) { return k < NSLOT && k % SPAN < NM; }
  static constexpr bool is_load(int k) { return k % LSP == 0 && k / LSP < NLD; }
  static constexpr int load_item(int k) { return k / LSP; }
  static constexpr bool is_write(int k) { return k % WSP == 0 && k / WSP < NLD; }
  static constexpr int write_item(int k) { return k / WSP; }
  static constexpr bool is_read(int k) { return k < (NSL - 1) * SPAN && k % SPAN < NR; }
  static constexpr int read_slice(int k) { return k / SPAN + 1; }
  static constexpr int read_item(int k) { return k % SPAN; }
  // loads that do not fit in the slots of the step (a small tile) go after
  // region 2
  static constexpr int LOADS_IN_STEP = NSTEP / LSP < NLD ? NSTEP / LSP : NLD;
};

// fragments of slice s live in f[s % 2]
template <class S, int SL>
__device__ __forceinline__ typename GemmPipe<S>::Frags& frag(typename GemmPipe<S>::Frags& f0,
                                                            typename GemmPipe<S>::Frags& f1) {
  if constexpr (SL % 2 == 0)
    return f0;
  else
    return f1;
}

template <class S, int K>
__device__ __forceinline__ void region1(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r, char* lds,
                                        int cur, int nxt, typename GemmPipe<S>::Regs& ahead,
                                        const typename GemmPipe<S>::Regs& next, typename GemmPipe<S>::Frags& f0,
                                        typename GemmPipe<S>::Frags& f1, f32x16 (&acc)[S::FM][S::FN]) {
  using PL = Plan<S>;
  if constexpr (K < PL::REGION1) {
    if constexpr (PL::is_mfma(K)) mma_block<S, K % PL::SPAN>(acc, frag<S, K / PL::SPAN>(f0, f1));
    constexpr bool RD = PL::is_read(K);
    if constexpr (RD)
      P.template read<PL::read_slice(K), PL::read_item(K)>(lds, cur, frag<S, PL::read_slice(K)>(f0, f1));
    constexpr bool LD = PL::is_load(K) && PL::load_item(K) < PL::LOADS_IN_STEP;
    if constexpr (LD) P.template load<PL::load_item(K)>(r, ahead);
    if constexpr (PL::is_write(K)) P.template store<PL::write_item(K)>(lds, nxt, next);
    pin_slot<PL::is_mfma(K) ? 1 : 0, RD ? item_reads<S>(PL::read_item(K)) : 0, LD ? 1 : 0,
             PL::is_write(K) ? 1 : 0>();
    region1<S, K + 1>(P, r, lds, cur, nxt, ahead, next, f0, f1, acc);
  }
}

// Region 2 (after the barrier): the second half of the last slice's blocks,
// each followed by two fragment reads of slice 0 of step t+1 (stage NXT);
// slot K (numbered as in the whole step) also carries its load, if any.
template <class S, int K, int X>
__device__ __forceinline__ void region2(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r,
                                        const char* lds, int nxt, typename GemmPipe<S>::Regs& ahead,
                                        typename GemmPipe<S>::Frags& f0, typename GemmPipe<S>::Frags& f1,
                                        f32x16 (&acc)[S::FM][S::FN]) {
  using PL = Plan<S>;
  constexpr int B = K - PL::NSLOT + PL::NM / 2;  // block of the last slice
  if constexpr (B < PL::NM || X < PL::NR) {
    if constexpr (B < PL::NM) mma_block<S, B>(acc, frag<S, PL::NSL - 1>(f0, f1));
    if constexpr (X < PL::NR) P.template read<0, X>(lds, nxt, f0);
    if constexpr (X + 1 < PL::NR) P.template read<0, X + 1>(lds, nxt, f0);
    constexpr bool LD = PL::is_load(K) && PL::load_item(K) < PL::LOADS_IN_STEP;
    if constexpr (LD) P.template load<PL::load_item(K)>(r, ahead);
    pin_slot<B < PL::NM ? 1 : 0, item_reads<S>(X) + item_reads<S>(X + 1), LD ? 1 : 0, 0>();
    region2<S, K + 1, X + 2>(P, r, lds, nxt, ahead, f0, f1, acc);
  }
}

template <class S, int D>
__device__ __forceinline__ void load_rest(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r,
                                          typename GemmPipe<S>::Regs& R) {
  if constexpr (D < GemmPipe<S>::NLD) {
    P.template load<D>(r, R);
    load_rest<S, D + 1>(P, r, R);
  }
}

// One K step t on LDS stage ST = t % 2, fragments of slice 0 already in f0.
// `next` holds step t+1 (loaded during step t-1) and is written to the other
// stage, which was last read before the previous step's barrier; `ahead`
// (written to LDS during step t-1) receives step t+2.
template <class S, int ST>
__device__ __forceinline__ void k_step(const GemmPipe<S>& P, const GemmArgs& g, int m0, int n0, int t, char* lds,
                                       typename GemmPipe<S>::Regs& ahead, const typename GemmPipe<S>::Regs& next,
                                       typename GemmPipe<S>::Frags& f0, typename GemmPipe<S>::Frags& f1,
                                       f32x16 (&acc)[S::FM][S::FN]) {
  static_assert(S::NSL % 2 == 0, "slice 0 of the next step reuses f0");
  using PL = Plan<S>;
  constexpr int CUR = ST, NXT = ST ^ 1;
  // keep the scheduler from hoisting this step's reads into the previous
  // step (that would hold three fragment sets live and spill)
  __builtin_amdgcn_sched_barrier(0);
  const typename GemmPipe<S>::Rsrc r = P.rsrc(g, m0, n0, t + 2);
  region1<S, 0>(P, r, lds, CUR, NXT, ahead, next, f0, f1, acc);
  // every wave's LDS writes of step t+1 and reads of stage CUR are done at
  // the barrier (it carries the workgroup fence, which also keeps the
  // compiler from hoisting the next reads above it)
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  region2<S, PL::NSLOT, 0>(P, r, lds, NXT, ahead, f0, f1, acc);
  if constexpr (PL::LOADS_IN_STEP < PL::NLD) load_rest<S, PL::LOADS_IN_STEP>(P, r, ahead);
  __builtin_amdgcn_sched_barrier(0);
}

template <class S, int D>
__device__ __forceinline__ void load_all(const GemmPipe<S>& P, const typename GemmPipe<S>::Rsrc& r,
                                         typename GemmPipe<S>::Regs& R) {
  if constexpr (D < GemmPipe<S>::NLD) {
    P.template load<D>(r, R);
    load_all<S, D + 1>(P, r, R);
  }
}

template <class S, int D>
__device__ __forceinline__ void store_all(const GemmPipe<S>& P, char* lds, int ST,
                                          const typename GemmPipe<S>::Regs& R) {
  if constexpr (D < GemmPipe<S>::NLD) {
    P.template store<D>(lds, ST, R);
    store_all<S, D + 1>(P, lds, ST, R);
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
// S::LDS_BYTES. Starts with a workgroup barrier so callers may reuse the LDS
// before it; the LDS writes of its last step target a stage nobody reads,
// and the caller's next use of the LDS starts with a barrier.
// The tile's bias is read from global memory at the start, next to the first
// operand loads, and parked in LDS; the epilogue takes this lane's bias
// values from there before it touches the accumulators. With a global bias
// load next to each store, the epilogue of a 256x256 tile took about 25 us
// on MI355X (load latency, and the register allocator reading out every
// accumulator up front and spilling); this way 11-16 us.
template <class S>
__device__ void gemm_tile(const GemmArgs& g, int m0, int n0, char* lds) {
  using P_t = GemmPipe<S>;
  constexpr int NR = S::FM + S::FN;
  // The thread id is made opaque here, once per tile, so that every offset
  // derived from it is recomputed per tile (a few VALU operations) instead
  // of being hoisted out of the persistent tile loop, kept live across the
  // K loop and spilled: the spilled offsets came back as about fourteen
  // serial scratch reloads in front of every K loop, each missing in L2
  // after a tile's worth of operand traffic.
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  P.setup(g, n0, tid);
  typename P_t::Frags f0, f1;
  typename P_t::Regs R0, R1;

  const int bias_n = g.bias_along_m ? S::BM : S::BN;
  f16 bias_v = (f16)0.0f;
  if (g.bias && (int)tid < bias_n) {
    const int idx = (g.bias_along_m ? m0 : n0) + (int)tid;
    if (idx < (g.bias_along_m ? g.M : g.N)) bias_v = g.bias[idx];
  }
  load_all<S, 0>(P, P.rsrc(g, m0, n0, 0), R0);
  load_all<S, 0>(P, P.rsrc(g, m0, n0, 1), R1);
  __syncthreads();  // previous users of the LDS are done
  if (g.bias && (int)tid < bias_n) ((f16*)(lds + S::BIAS_OFF))[tid] = bias_v;
  store_all<S, 0>(P, lds, 0, R0);
  __syncthreads();
  read_all<S, 0, NR>(P, lds, 0, f0);

  // Two stages and two register sets: unroll by 2 so both are named at
  // compile time. The step count is rounded up to even (a loop with one
  // exit keeps the accumulators in place); the extra step reads only
  // out-of-range zeros and adds exact zeros to accumulators that start at
  // +0, so it changes no bit of the result.
  const int nk2 = (nk + 1) & ~1;
  __builtin_assume(nk2 >= 2);  // K >= 1: the host rejects K = 0
  for (int t = 0; t < nk2; t += 2) {
    k_step<S, 0>(P, g, m0, n0, t, lds, R0, R1, f0, f1, acc);
    k_step<S, 1>(P, g, m0, n0, t + 1, lds, R1, R0, f0, f1, acc);
  }

  // epilogue: lane holds row lane & 31 of each 32x32 block and, for
  // q = 0..3, columns 8q + 4*(lane >> 5) + 0..3.
  const int khalf = lane >> 5;
  const f16* bias_l = (const f16*)(lds + S::BIAS_OFF);
  const bool col_bias = g.bias && !g.bias_along_m;
  const bool row_bias = g.bias && g.bias_along_m;
  f16x4 bn_v[S::FN][4];
#pragma unroll
  for (int j = 0; j < S::FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bn_v[j][q] = col_bias ? *(const f16x4*)(bias_l + wn * S::WTN + j * 32 + 8 * q + 4 * khalf) : f16x4{};
  // Lanes l and l + 32 hold the two 4-column halves of the same 8 columns
  // of one row. One permlane32 swap per register pair trades the upper
  // lanes' q half for the lower lanes' q + 1 half, so that each lane holds 8
  // consecutive columns (lower lanes 8q.., upper lanes 8q + 8..) and writes
  // them with one 16-byte store. The swap needs every lane active: values
  // are computed for all lanes and only the stores are masked.
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    const int r = wm * S::WTM + i * 32 + (lane & 31);
    const int m = m0 + r;
    const bool m_ok = m < g.M;
    const float bm = row_bias ? (float)bias_l[r] : 0.0f;
    f16* const crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      uint32_t w[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 o;
        if (col_bias) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (f16)(acc[i][j][4 * q + e] + (float)bn_v[j][q][e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (f16)(acc[i][j][4 * q + e] + bm);
        }
        const auto u = __builtin_bit_cast(u32x2, o);
        w[q][0] = u[0];
        w[q][1] = u[1];
      }
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto sw = __builtin_amdgcn_permlane32_swap(w[q][d], w[q + 1][d], false, false);
          w[q][d] = sw[0];
          w[q + 1][d] = sw[1];
        }
        const int n = n0 + wn * S::WTN + j * 32 + 8 * q + 8 * khalf;
        if (m_ok && n < g.N) {
          u32x4 v;
          v[0] = w[q][0];
          v[1] = w[q][1];
          v[2] = w[q + 1][0];
          v[3] = w[q + 1][1];
          *(u32x4*)(crow + n) = v;
        }
      }
    }
  }
}

}  // namespace iris
