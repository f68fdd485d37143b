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
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int A_DMA = A_STAGE / 1024 / 4;    // 1 KiB DMA instructions per wave per step
  static constexpr int B_DMA = B_STAGE / 1024 / 4;
  static constexpr int RPB = 1024 / RB;               // B rows per DMA instruction
  static_assert(FM >= 1 && FN >= 1, "tile too small for 32x32 blocks");
  static_assert(A_DMA >= 1 && B_DMA >= 1, "tile too small for 4 waves of 1 KiB loads");
};

// swizzle of the 16-byte chunks of a 64-byte A row (4 chunks)
__device__ __forceinline__ uint32_t swz_a(uint32_t r) { return ((r >> 1) ^ (r >> 3)) & 3u; }
// swizzle of the 16-byte chunks of a B row, by k row
template <class S>
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
  return ((k & 3u) << 2) & (uint32_t)(S::CPR_B - 1);
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
  // per-thread global offsets of the DMA chunks of the current tile
  uint32_t a_off[S::A_DMA];
  uint32_t a_kc[S::A_DMA];  // k offset (elements) of that chunk within a step
  uint32_t b_off[S::B_DMA];
  // LDS byte offsets within a stage of the fragment reads
  uint32_t ra_base[2];        // A, per k slice
  uint32_t rb_base[S::FN];    // B, per 32-column block

  __device__ __forceinline__ void setup(const GemmArgs& g, int n0) {
    const uint32_t l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int n = 0; n < S::A_DMA; ++n) {
      const uint32_t b = w * S::A_DMA + n;
      const uint32_t r = 16 * b + (l >> 2);
      const uint32_t c = (l & 3) ^ swz_a(r);
      a_off[n] = (uint32_t)((r * g.lda + 8 * c) * 2);
      a_kc[n] = 8 * c;
    }
#pragma unroll
    for (int n = 0; n < S::B_DMA; ++n) {
      const uint32_t b = w * S::B_DMA + n;
      const uint32_t k = S::RPB * b + l / S::CPR_B;
      const uint32_t c = (l % S::CPR_B) ^ swz_b<S>(k);
      const bool ok = n0 + 8 * (int)c < g.N;
      b_off[n] = ok ? (uint32_t)((k * g.ldb + 8 * c) * 2) : kOob;
    }
    {
      const uint32_t r = wm * S::WTM + (l & 31);
      const uint32_t h = l >> 5;
#pragma unroll
      for (int s = 0; s < 2; ++s) ra_base[s] = r * S::RA + (((2 * s + h) ^ swz_a(r)) << 4);
    }
    {
      const uint32_t grp = l >> 4, e = (l >> 2) & 3, q = l & 3;
      const uint32_t k = 8 * (grp >> 1) + e;
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const uint32_t c = (wn * S::WTN + 32 * j) / 8 + 2 * (grp & 1) + (q >> 1);
        rb_base[j] = S::A_STAGE + k * S::RB + ((c ^ swz_b<S>(k)) << 4) + 8 * (q & 1);
      }
    }
  }

  // issue the LDS DMA of K step `step` (k0 = step * BK) into `stage`
  __device__ __forceinline__ void issue(const GemmArgs& g, int m0, int n0, int step, uint32_t lds_base,
                                        uint32_t stage) const {
    const uint32_t w = threadIdx.x >> 6;
    const int k0 = step * S::BK;
    const int rows = min(S::BM, g.M - m0);
    const int64_t abytes = (int64_t)rows * g.lda * 2 - (int64_t)k0 * 2;
    const u32x4 ra = rsrc_words(g.A + (int64_t)m0 * g.lda + k0, abytes > 0 ? (uint32_t)abytes : 0u);
    const int krows = min(S::BK, g.K - k0);
    const u32x4 rb = rsrc_words(g.B + (int64_t)k0 * g.ldb + n0,
                                krows > 0 ? (uint32_t)((int64_t)krows * g.ldb * 2 - (int64_t)n0 * 2) : 0u);
#pragma unroll
    for (int n = 0; n < S::A_DMA; ++n) {
      const uint32_t off = (k0 + (int)a_kc[n] < g.K) ? a_off[n] : kOob;
      dma16(ra, lds_base + stage + (w * S::A_DMA + n) * 1024, off);
    }
#pragma unroll
    for (int n = 0; n < S::B_DMA; ++n)
      dma16(rb, lds_base + stage + S::A_STAGE + (w * S::B_DMA + n) * 1024, b_off[n]);
  }

  struct Frags {
    f16x8 a[S::FM];
    f16x8 b[S::FN];
  };

  // fragments of k slice SL (0 or 1) of the step held in `stage`
  template <int SL>
  __device__ __forceinline__ void read(const char* lds, uint32_t stage, Frags& f) const {
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
      f.a[i] = as_h8(*(const u32x4*)(lds + stage + ra_base[SL] + i * 32 * S::RA));
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const char* p = lds + stage + rb_base[j] + SL * 16 * S::RB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * S::RB));
      u32x4 v;
      v[0] = __builtin_bit_cast(u32x2, lo)[0];
      v[1] = __builtin_bit_cast(u32x2, lo)[1];
      v[2] = __builtin_bit_cast(u32x2, hi)[0];
      v[3] = __builtin_bit_cast(u32x2, hi)[1];
      f.b[j] = as_h8(v);
    }
  }
};

template <class S>
__device__ __forceinline__ void mma(f32x16 (&acc)[S::FM][S::FN], const typename GemmPipe<S>::Frags& f,
                                    int j0, int j1) {
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
      if (j >= j0 && j < j1)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Computes the tile at (m0, n0) and writes it to C. `lds` must hold
// S::LDS_BYTES. Starts and ends with a workgroup barrier so callers may
// reuse the LDS around it.
template <class S>
__device__ void gemm_tile(const GemmArgs& g, int m0, int n0, char* lds) {
  using P_t = GemmPipe<S>;
  constexpr int NS = S::NSTAGE;
  constexpr int PER_STEP = S::A_DMA + S::B_DMA;  // DMA instructions per wave per step
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
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  __syncthreads();  // previous users of the LDS are done
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) P.issue(g, m0, n0, s, lds_base, s * S::STAGE);
  wait_vmcnt<(NS - 2) * PER_STEP>();  // this wave's part of step 0 has landed
  __syncthreads();
  P.template read<0>(lds, 0, f0);

  for (int t = 0; t < nk; ++t) {
    const uint32_t cur = (uint32_t)(t % NS) * S::STAGE;
    const uint32_t nxt = (uint32_t)((t + 1) % NS) * S::STAGE;
    const uint32_t ahead = (uint32_t)((t + NS - 1) % NS) * S::STAGE;
    // slice 0: MFMAs on f0 under the loads of step t+3 and the reads of slice 1
    P.issue(g, m0, n0, t + NS - 1, lds_base, ahead);
    P.template read<1>(lds, cur, f1);
    mma<S>(acc, f0, 0, S::FN);
    // slice 1, first half
    mma<S>(acc, f1, 0, S::FN / 2);
    // step t+1 must be complete for every wave before its fragments are read;
    // the loads of steps t+2 and t+3 may still be in flight
    wait_vmcnt<(NS - 2) * PER_STEP>();
    __syncthreads();
    P.template read<0>(lds, nxt, f0);
    // slice 1, second half
    mma<S>(acc, f1, S::FN / 2, S::FN);
  }
  // loads issued past the last step target stages no one reads; let them
  // land before the LDS is reused
  wait_vmcnt<0>();

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
