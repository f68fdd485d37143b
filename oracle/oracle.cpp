/*
 * CPU oracle: plain, slow, obviously correct. TEST INFRASTRUCTURE ONLY.
 *
 * What it computes is written out from the operation definitions on the
 * Iris docs page "Fused Communication and Compute Operations" (entries
 * all_gather_matmul, matmul_reduce_scatter, matmul_all_reduce) and from the
 * iris.concurrent pull request ("Add iris.concurrent (concurrent,
 * independent, fused comm+gemm)", description: an independent GEMM beside an
 * all_reduce). Every floating-point result is the exact mathematical value
 * up to double rounding; there is no blocking, fusion or reordering of the
 * sums beyond the definitions: each dot product adds its K products in
 * ascending k, and partial buffers are added in the order given.
 *
 * The fp16 codec below is written from the IEEE-754 binary16 format
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).
 *
 * Parity pins for every function here live in the CPU test suite; none is
 * unpinned.
 */
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

/* ---------------------------------------------------------------- fp16 */

extern "C" double oracle_f16_decode(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int exp = (h >> 10) & 0x1f;
  const int frac = h & 0x3ff;
  double mag;
  if (exp == 0x1f) {
    mag = frac ? NAN : INFINITY;
  } else if (exp == 0) {
    /* subnormal: frac * 2^-24 */
    mag = std::ldexp((double)frac, -24);
  } else {
    /* normal: (1024 + frac) * 2^(exp - 15 - 10) */
    mag = std::ldexp((double)(1024 + frac), exp - 25);
  }
  return sign ? -mag : mag;
}

/* Round a non-negative double holding an exact value to the nearest integer,
 * ties to even. v < 2^52 here, so floor and the subtraction are exact. */
static double round_half_even(double v) {
  const double fl = std::floor(v);
  const double d = v - fl;
  if (d > 0.5) return fl + 1.0;
  if (d < 0.5) return fl;
  return (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

extern "C" uint16_t oracle_f16_encode(double x) {
  if (std::isnan(x)) return 0x7e00;
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  /* Largest finite binary16 is 65504 = (2 - 2^-10) * 2^15. Values at or above
   * the midpoint to the next power of two (65520) round to infinity. */
  if (a >= 65520.0) return sign | 0x7c00;
  if (a < std::ldexp(1.0, -14)) {
    /* subnormal range: the result is q * 2^-24 with integer q in [0, 1024];
     * q == 1024 is the smallest normal, whose encoding is also 1024. */
    const double q = round_half_even(std::ldexp(a, 24));
    return sign | (uint16_t)q;
  }
  int e2;
  (void)std::frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;           /* a = m * 2^e, m in [1, 2) */
  /* fraction in units of 2^(e-10): exact scaling, then one rounding */
  double q = round_half_even(std::ldexp(a, 10 - e)) - 1024.0;
  if (q >= 1024.0) { /* mantissa rounded up to 2: next binade */
    q = 0.0;
    e += 1;
  }
  const int be = e + 15;
  if (be >= 31) return sign | 0x7c00;
  return sign | (uint16_t)((be << 10) | (int)q);
}

extern "C" void oracle_f16_decode_array(const uint16_t* in, double* out,
                                        int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_decode(in[i]);
}

extern "C" void oracle_f16_encode_array(const double* in, uint16_t* out,
                                        int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_encode(in[i]);
}

/* ------------------------------------------------------------- threads */

extern "C" int oracle_default_threads(void) {
  unsigned n = std::thread::hardware_concurrency();
  return n ? (int)n : 1;
}

/* Run body(r) for r in [r0, r1) split into contiguous row ranges. */
template <class F>
static void parallel_rows(int64_t r0, int64_t r1, int nthreads, F body) {
  const int64_t rows = r1 - r0;
  if (rows <= 0) return;
  int nt = nthreads > 0 ? nthreads : oracle_default_threads();
  if (nt > rows) nt = (int)rows;
  if (nt <= 1) {
    for (int64_t r = r0; r < r1; ++r) body(r);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (rows + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    const int64_t a = r0 + t * per;
    const int64_t b = std::min(r1, a + per);
    if (a >= b) break;
    pool.emplace_back([=]() {
      for (int64_t r = a; r < b; ++r) body(r);
    });
  }
  for (auto& th : pool) th.join();
}

/* ---------------------------------------------------------------- GEMM */

static double bias_value(const uint16_t* bias, int bias_mode, int64_t m,
                         int64_t n) {
  if (bias == nullptr || bias_mode == ORACLE_BIAS_NONE) return 0.0;
  return oracle_f16_decode(bias[bias_mode == ORACLE_BIAS_ALONG_M ? m : n]);
}

/*
 * out[m - m0][n - n0] = sum_{k=0}^{K-1} A[m][k] * B[k][n]  +  bias
 * The B columns [n0, n1) are decoded to double once; then each output row
 * accumulates its K products in ascending k (acc[n] += a_mk * b_kn).
 */
extern "C" void oracle_gemm_bias(const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb,
                                 const uint16_t* bias, int bias_mode,
                                 int64_t K, int64_t m0, int64_t m1,
                                 int64_t n0, int64_t n1, double* out,
                                 int nthreads) {
  const int64_t nc = n1 - n0;
  if (m1 <= m0 || nc <= 0) return;
  std::vector<double> Bd((size_t)K * (size_t)nc);
  parallel_rows(0, K, nthreads, [&](int64_t k) {
    for (int64_t j = 0; j < nc; ++j)
      Bd[(size_t)k * nc + j] = oracle_f16_decode(B[k * ldb + n0 + j]);
  });
  parallel_rows(m0, m1, nthreads, [&](int64_t m) {
    double* acc = out + (size_t)(m - m0) * nc;
    for (int64_t j = 0; j < nc; ++j) acc[j] = 0.0;
    const uint16_t* arow = A + m * lda;
    for (int64_t k = 0; k < K; ++k) {
      const double a = oracle_f16_decode(arow[k]);
      const double* brow = Bd.data() + (size_t)k * nc;
      for (int64_t j = 0; j < nc; ++j) acc[j] += a * brow[j];
    }
    for (int64_t j = 0; j < nc; ++j)
      acc[j] += bias_value(bias, bias_mode, m, n0 + j);
  });
}

/* ---------------------------------------------------------- collectives */

extern "C" void oracle_all_gather_k(const uint16_t* const* shards, int W,
                                    int64_t M, int64_t K_local,
                                    uint16_t* gathered) {
  const int64_t K = (int64_t)W * K_local;
  for (int s = 0; s < W; ++s)
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = 0; k < K_local; ++k)
        gathered[m * K + (int64_t)s * K_local + k] = shards[s][m * K_local + k];
}

extern "C" void oracle_sum(const uint16_t* const* bufs, int nbuf, int64_t n,
                           double* out) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int w = 0; w < nbuf; ++w) s += oracle_f16_decode(bufs[w][i]);
    out[i] = s;
  }
}

/* ------------------------------------------------------------ fused ops */

extern "C" void oracle_all_gather_matmul(
    const uint16_t* const* shards, int W, int64_t M, int64_t K_local,
    const uint16_t* B, int64_t N, const uint16_t* bias, int bias_mode,
    int64_t m0, int64_t m1, int64_t n0, int64_t n1, double* out,
    int nthreads) {
  /* Step 1: all_gather(A_sharded) along K (rank order). Only rows [m0, m1)
   * of the gathered matrix enter this output region. */
  const int64_t K = (int64_t)W * K_local;
  const int64_t rows = m1 - m0;
  if (rows <= 0) return;
  std::vector<const uint16_t*> sub((size_t)W);
  for (int s = 0; s < W; ++s) sub[(size_t)s] = shards[s] + m0 * K_local;
  std::vector<uint16_t> gathered((size_t)rows * (size_t)K);
  oracle_all_gather_k(sub.data(), W, rows, K_local, gathered.data());
  (void)M;
  (void)N;
  /* Step 2: gathered @ B + bias. The gathered block starts at row m0, so
   * the bias row index must be offset back to the full matrix. */
  std::vector<uint16_t> bias_rows;
  const uint16_t* bias_use = bias;
  if (bias != nullptr && bias_mode == ORACLE_BIAS_ALONG_M) {
    bias_rows.assign(bias + m0, bias + m1);
    bias_use = bias_rows.data();
  }
  oracle_gemm_bias(gathered.data(), K, B, N, bias_use, bias_mode, K, 0, rows,
                   n0, n1, out, nthreads);
}

extern "C" void oracle_matmul_reduce_scatter(
    const uint16_t* A, const uint16_t* B, const uint16_t* bias, int bias_mode,
    const uint16_t* const* partials, int W, int rank, int64_t M, int64_t N,
    int64_t K, int64_t m0, int64_t m1, double* out, int nthreads) {
  (void)M;
  const int64_t nl = N / W;
  const int64_t rows = m1 - m0;
  if (rows <= 0 || nl <= 0) return;
  /* this rank's own partial: columns [rank*nl, (rank+1)*nl) of A@B + bias */
  oracle_gemm_bias(A, K, B, N, bias, bias_mode, K, m0, m1, rank * nl,
                   (rank + 1) * nl, out, nthreads);
  /* reduce: add the other W-1 partials for the same slice, in order */
  for (int p = 0; p < W - 1; ++p)
    for (int64_t m = m0; m < m1; ++m)
      for (int64_t j = 0; j < nl; ++j)
        out[(m - m0) * nl + j] += oracle_f16_decode(partials[p][m * nl + j]);
}

extern "C" void oracle_matmul_all_reduce(
    const uint16_t* A, const uint16_t* B, const uint16_t* bias, int bias_mode,
    const uint16_t* const* partials, int W, int64_t M, int64_t N, int64_t K,
    int64_t m0, int64_t m1, double* out, int nthreads) {
  (void)M;
  const int64_t rows = m1 - m0;
  if (rows <= 0) return;
  oracle_gemm_bias(A, K, B, N, bias, bias_mode, K, m0, m1, 0, N, out,
                   nthreads);
  for (int p = 0; p < W - 1; ++p)
    for (int64_t m = m0; m < m1; ++m)
      for (int64_t n = 0; n < N; ++n)
        out[(m - m0) * N + n] += oracle_f16_decode(partials[p][m * N + n]);
}

extern "C" void oracle_matmul_all_gather(
    const uint16_t* A, const uint16_t* B, const uint16_t* bias, int bias_mode,
    const uint16_t* const* peers, int W, int rank, int64_t M, int64_t N,
    int64_t K, int64_t m0, int64_t m1, double* out, int nthreads) {
  /* output row r belongs to the block of rank r / M; this rank's block is
   * its own A @ B + bias, every other block is that rank's stand-in result,
   * peers being listed in rank order without this rank. The requested rows
   * are taken block by block, so that the rows of this rank's block go to
   * the GEMM in one call (which shares them among its threads). */
  for (int64_t r0 = m0; r0 < m1;) {
    const int64_t q = r0 / M, row = r0 - q * M;
    const int64_t r1 = std::min(m1, (q + 1) * M); /* end of block q in range */
    double* o = out + (r0 - m0) * N;
    if (q == rank) {
      oracle_gemm_bias(A, K, B, N, bias, bias_mode, K, row, row + (r1 - r0), 0,
                       N, o, nthreads);
    } else {
      const uint16_t* src = peers[q < rank ? q : q - 1] + row * N;
      for (int64_t i = 0; i < (r1 - r0) * N; ++i) o[i] = oracle_f16_decode(src[i]);
    }
    r0 = r1;
  }
  (void)W;
}

/* ------------------------------------------------- flat collectives */

extern "C" void oracle_all_gather_flat(const uint16_t* const* bufs, int W,
                                       int64_t n, uint16_t* out) {
  for (int w = 0; w < W; ++w)
    for (int64_t i = 0; i < n; ++i) out[(int64_t)w * n + i] = bufs[w][i];
}

extern "C" void oracle_reduce_scatter_flat(const uint16_t* const* bufs, int W,
                                           int64_t n, int rank, double* out) {
  const int64_t part = n / W;
  for (int64_t i = 0; i < part; ++i) {
    double s = 0.0;
    for (int w = 0; w < W; ++w)
      s += oracle_f16_decode(bufs[w][(int64_t)rank * part + i]);
    out[i] = s;
  }
}

extern "C" void oracle_all_to_all_flat(const uint16_t* const* bufs, int W,
                                       int64_t n, int rank, uint16_t* out) {
  const int64_t part = n / W;
  for (int j = 0; j < W; ++j)
    for (int64_t i = 0; i < part; ++i)
      out[(int64_t)j * part + i] = bufs[j][(int64_t)rank * part + i];
}

extern "C" void oracle_broadcast_flat(const uint16_t* const* bufs, int W,
                                      int64_t n, int root, uint16_t* out) {
  (void)W;
  for (int64_t i = 0; i < n; ++i) out[i] = bufs[root][i];
}
