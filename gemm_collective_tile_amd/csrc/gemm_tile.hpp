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
//     (BM/2) x (BN/2) sub-tile held in fp32 accumulators.
//   * v_mfma_f32_32x32x16_f16: 32x32 output blocks, K step 16. Each lane
//     feeds 8 consecutive k of one row of A and 8 consecutive k of one
//     column of B, so BOTH operands must be K-contiguous in LDS.
//   * K is walked in steps of BK = 64 through a double-buffered LDS stage:
//     A as [BM][64] and B TRANSPOSED as [BN][64], 128-byte rows whose eight
//     16-byte chunks are XOR-swizzled by the row index so that the
//     16-byte fragment reads of 8 consecutive rows and the transposed
//     writes of B hit distinct banks.
//   * B arrives row-major (N contiguous). Each thread loads an 8(k) x 8(n)
//     block with eight 16-byte loads, transposes it in registers and
//     writes eight 16-byte rows of the [n][k] stage.
//   * Global loads are raw buffer loads: an offset past the resource size
//     returns zero, which masks ragged M, N and K edges.
//   * The MFMA is issued with B as its first operand and A as its second,
//     so each lane ends up holding 4 consecutive output columns of one row:
//     the epilogue stores 8 bytes per lane after adding the bias.
#pragma once

#include "device_common.hpp"

namespace iris {

template <int BM_, int BN_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // per-wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int A_CHUNKS = BM * (BK / 8);     // 16-byte chunks per A stage
  static constexpr int A_PER_T = A_CHUNKS / kThreads;
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);  // 8x8 blocks per B stage
  static constexpr int B_PER_T = (B_BLOCKS + kThreads - 1) / kThreads;
  static constexpr int A_STAGE = BM * BK * 2;  // bytes
  static constexpr int B_STAGE = BN * BK * 2;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(A_CHUNKS % kThreads == 0, "A stage must split evenly over threads");
  static_assert(FM >= 1 && FN >= 1, "tile too small for 32x32 blocks");
};

// byte offset of 16-byte chunk c (0..7) of row r in a [rows][64] fp16 stage
__device__ __forceinline__ uint32_t lds_off(uint32_t r, uint32_t c) {
  const uint32_t sw = (r ^ (r >> 3)) & 7u;
  return (r << 7) | ((c ^ sw) << 4);
}

// Transpose an 8x8 block of fp16: in[i] holds row i (8 halves); out[j]
// holds column j. Each output dword packs two halves from adjacent rows.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = in[2 * d][w];
      const uint32_t hi = in[2 * d + 1][w];
      out[j][d] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
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
struct GemmTile {
  // registers staged between the global load and the LDS write
  u32x4 ra[S::A_PER_T];
  u32x4 rb[S::B_PER_T][8];
  // per-thread fixed parts of the load addressing for this tile
  uint32_t a_off[S::A_PER_T];
  uint32_t b_off[S::B_PER_T];
  bool b_col_ok[S::B_PER_T];

  __device__ __forceinline__ void setup(const GemmArgs& g, int n0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int p = 0; p < S::A_PER_T; ++p) {
      const int q = t + p * kThreads;
      const int r = q >> 3, c = q & 7;
      a_off[p] = (uint32_t)((r * g.lda + c * 8) * 2);
    }
#pragma unroll
    for (int p = 0; p < S::B_PER_T; ++p) {
      const int q = t + p * kThreads;
      const int nb = q % (S::BN / 8), kb = q / (S::BN / 8);
      b_off[p] = (uint32_t)(((int64_t)kb * 8 * g.ldb + nb * 8) * 2);
      b_col_ok[p] = (q < S::B_BLOCKS) && (n0 + nb * 8 < g.N);
    }
  }

  // global -> registers for k-tile starting at k0
  __device__ __forceinline__ void load(const GemmArgs& g, int m0, int n0, int k0) {
    const int t = threadIdx.x;
    const int rows = min(S::BM, g.M - m0);
    const bool ktail = (k0 + S::BK > g.K);
    {
      const f16* base = g.A + (int64_t)m0 * g.lda + k0;
      const uint32_t bytes = (uint32_t)((int64_t)rows * g.lda * 2 - (int64_t)k0 * 2);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
      for (int p = 0; p < S::A_PER_T; ++p) {
        uint32_t off = a_off[p];
        if (ktail) {
          const int c = (t + p * kThreads) & 7;
          if (k0 + c * 8 >= g.K) off = kOob;
        }
        ra[p] = buf_load16(rs, off);
      }
    }
    {
      const int krows = min(S::BK, g.K - k0);
      const f16* base = g.B + (int64_t)k0 * g.ldb + n0;
      const uint32_t bytes = (uint32_t)((int64_t)krows * g.ldb * 2 - (int64_t)n0 * 2);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
      for (int p = 0; p < S::B_PER_T; ++p) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t off = b_col_ok[p] ? b_off[p] + (uint32_t)(i * g.ldb * 2) : kOob;
          rb[p][i] = buf_load16(rs, off);
        }
      }
    }
  }

  // registers -> LDS stage
  __device__ __forceinline__ void store(char* stage) const {
    const int t = threadIdx.x;
    char* As = stage;
    char* Bs = stage + S::A_STAGE;
#pragma unroll
    for (int p = 0; p < S::A_PER_T; ++p) {
      const int q = t + p * kThreads;
      *(u32x4*)(As + lds_off(q >> 3, q & 7)) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < S::B_PER_T; ++p) {
      const int q = t + p * kThreads;
      if (S::B_BLOCKS % kThreads == 0 || q < S::B_BLOCKS) {
        const int nb = q % (S::BN / 8), kb = q / (S::BN / 8);
        u32x4 tr[8];
        transpose8x8(rb[p], tr);
#pragma unroll
        for (int j = 0; j < 8; ++j) *(u32x4*)(Bs + lds_off(nb * 8 + j, kb)) = tr[j];
      }
    }
  }
};

// Computes the tile at (m0, n0) and writes it to C. `lds` must hold
// S::LDS_BYTES. Starts and ends with a workgroup barrier so callers may
// reuse the LDS around it.
template <class S>
__device__ void gemm_tile(const GemmArgs& g, int m0, int n0, char* lds) {
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

  GemmTile<S> st;
  st.setup(g, n0);
  __syncthreads();  // previous users of the LDS are done
  st.load(g, m0, n0, 0);
  st.store(lds);
  __syncthreads();

  const uint32_t a_row0 = wm * S::WTM + (lane & 31);
  const uint32_t b_row0 = wn * S::WTN + (lane & 31);
  const uint32_t khalf = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * S::STAGE;
    const bool more = (kt + 1 < nk);
    if (more) st.load(g, m0, n0, (kt + 1) * S::BK);
    const char* As = cur;
    const char* Bs = cur + S::A_STAGE;
#pragma unroll
    for (int kk = 0; kk < S::BK / 16; ++kk) {
      const uint32_t c = kk * 2 + khalf;
      f16x8 a[S::FM], b[S::FN];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) a[i] = as_h8(*(const u32x4*)(As + lds_off(a_row0 + i * 32, c)));
#pragma unroll
      for (int j = 0; j < S::FN; ++j) b[j] = as_h8(*(const u32x4*)(Bs + lds_off(b_row0 + j * 32, c)));
#pragma unroll
      for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    if (more) st.store(lds + ((kt + 1) & 1) * S::STAGE);
    __syncthreads();
  }

  // epilogue: lane holds row m = lane & 31 of each 32x32 block and, for
  // g = 0..3, columns 8g + 4*(lane >> 5) + 0..3.
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    const int m = m0 + wm * S::WTM + i * 32 + (lane & 31);
    if (m >= g.M) continue;
    const float bm = (g.bias && g.bias_along_m) ? (float)g.bias[m] : 0.0f;
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * S::WTN + j * 32 + 8 * q + 4 * (int)khalf;
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
