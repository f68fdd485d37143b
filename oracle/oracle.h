/*
 * CPU oracle for the one-GPU share of Iris's fused communication + GEMM ops.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this. Only the test suite, the smoke entry and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (the pages this oracle is written from):
 *   [DOCS]  Iris docs, "Fused Communication and Compute Operations":
 *           entries matmul_all_reduce, all_gather_matmul, matmul_all_gather,
 *           matmul_reduce_scatter.
 *   [PR544] ROCm/iris pull request "Add iris.concurrent (concurrent,
 *           independent, fused comm+gemm)": description and review answer
 *           (an independent GEMM running beside a collective: all_gather,
 *           all_reduce, reduce_scatter, all_to_all or broadcast).
 *
 * Conventions: fp16 values are IEEE-754 binary16 bit patterns in uint16_t.
 * Every matrix is row-major and contiguous unless a leading dimension is
 * given. All arithmetic is in double; fp16 rounding happens only where a
 * caller asks for it (oracle_f16_encode), once, at the end.
 */
#ifndef IRIS_ORACLE_H
#define IRIS_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bias_mode values */
#define ORACLE_BIAS_NONE 0
#define ORACLE_BIAS_ALONG_N 1 /* bias has one entry per output column */
#define ORACLE_BIAS_ALONG_M 2 /* bias has one entry per output row */

/* binary16 -> double, exact for every bit pattern (NaN stays NaN). */
double oracle_f16_decode(uint16_t h);
/* double -> binary16 with round-to-nearest, ties-to-even; overflow -> inf. */
uint16_t oracle_f16_encode(double x);
/* Array forms of the two conversions above. */
void oracle_f16_decode_array(const uint16_t* in, double* out, int64_t n);
void oracle_f16_encode_array(const double* in, uint16_t* out, int64_t n);

/*
 * Region [m0,m1) x [n0,n1) of  A @ B + bias, in double.
 *   A: fp16 (M x K) with leading dimension lda; B: fp16 (K x N), ldb;
 *   bias: fp16 vector selected by bias_mode (NULL allowed with BIAS_NONE).
 *   out: (m1-m0) x (n1-n0) doubles, row-major.
 * For each output element the K products are added in ascending k.
 * nthreads <= 0 means one thread per host core.                [DOCS]
 */
void oracle_gemm_bias(const uint16_t* A, int64_t lda, const uint16_t* B,
                      int64_t ldb, const uint16_t* bias, int bias_mode,
                      int64_t K, int64_t m0, int64_t m1, int64_t n0,
                      int64_t n1, double* out, int nthreads);

/*
 * all_gather of W K-shards: gathered[m][s*K_local + k] = shards[s][m][k].
 * shards is a host array of W host pointers, each (M x K_local) fp16.
 * gathered is (M x W*K_local) fp16. Pure bit copy.             [DOCS]
 */
void oracle_all_gather_k(const uint16_t* const* shards, int W, int64_t M,
                         int64_t K_local, uint16_t* gathered);

/*
 * Elementwise sum of nbuf fp16 buffers of n elements each, in double,
 * buffers added in the order given.                  [PR544], [DOCS]
 */
void oracle_sum(const uint16_t* const* bufs, int nbuf, int64_t n, double* out);

/*
 * all_gather_matmul local share: region of concat_K(shards) @ B + bias.
 * B is (W*K_local x N). out as in oracle_gemm_bias.             [DOCS]
 */
void oracle_all_gather_matmul(const uint16_t* const* shards, int W,
                              int64_t M, int64_t K_local, const uint16_t* B,
                              int64_t N, const uint16_t* bias, int bias_mode,
                              int64_t m0, int64_t m1, int64_t n0, int64_t n1,
                              double* out, int nthreads);

/*
 * matmul_reduce_scatter local share for rank `rank` of W, column slice
 * N_local = N / W:
 *   out[m][j] = (A @ B + bias)[m][rank*N_local + j] + sum_p partials[p][m][j]
 * for rows [m0,m1) and all j. partials: W-1 host pointers, each
 * (M x N_local) fp16, standing in for the other ranks' A@B+bias slices.
 * out: (m1-m0) x N_local doubles.                               [DOCS]
 */
void oracle_matmul_reduce_scatter(const uint16_t* A, const uint16_t* B,
                                  const uint16_t* bias, int bias_mode,
                                  const uint16_t* const* partials, int W,
                                  int rank, int64_t M, int64_t N, int64_t K,
                                  int64_t m0, int64_t m1, double* out,
                                  int nthreads);

/*
 * matmul_all_reduce local share:
 *   out[m][n] = (A @ B + bias)[m][n] + sum_p partials[p][m][n]
 * for rows [m0,m1); partials: W-1 host pointers, each (M x N).  [DOCS]
 */
void oracle_matmul_all_reduce(const uint16_t* A, const uint16_t* B,
                              const uint16_t* bias, int bias_mode,
                              const uint16_t* const* partials, int W,
                              int64_t M, int64_t N, int64_t K, int64_t m0,
                              int64_t m1, double* out, int nthreads);

/*
 * matmul_all_gather local share (rank `rank` of W): the (M*W x N) output is
 * all_gather along M of every rank's A @ B + bias; this rank's block (rows
 * [rank*M, (rank+1)*M)) is computed here, the other blocks are the W-1
 * stand-in results `peers` (host pointers, each M x N fp16) in rank order
 * with this rank skipped. Rows [m0, m1) of the output, as doubles (the peer
 * rows decoded exactly).                                       [DOCS]
 */
void oracle_matmul_all_gather(const uint16_t* A, const uint16_t* B,
                              const uint16_t* bias, int bias_mode,
                              const uint16_t* const* peers, int W, int rank,
                              int64_t M, int64_t N, int64_t K, int64_t m0,
                              int64_t m1, double* out, int nthreads);

/*
 * The collectives of an independent GEMM + collective, local share of rank
 * `rank` of W, each rank holding a buffer of n fp16 elements (bufs: W host
 * pointers in rank order, this rank's own buffer included).     [PR544]
 *   all_gather:     out[w*n + i] = bufs[w][i]                 (W*n, bit copy)
 *   reduce_scatter: out[i] = sum_w bufs[w][rank*n/W + i]      (n/W, double)
 *   all_to_all:     out[j*n/W + i] = bufs[j][rank*n/W + i]    (n, bit copy)
 *   broadcast:      out[i] = bufs[root][i]                    (n, bit copy)
 * (all_reduce is oracle_sum.) reduce_scatter and all_to_all need n % W == 0.
 */
void oracle_all_gather_flat(const uint16_t* const* bufs, int W, int64_t n, uint16_t* out);
void oracle_reduce_scatter_flat(const uint16_t* const* bufs, int W, int64_t n, int rank,
                                double* out);
void oracle_all_to_all_flat(const uint16_t* const* bufs, int W, int64_t n, int rank,
                            uint16_t* out);
void oracle_broadcast_flat(const uint16_t* const* bufs, int W, int64_t n, int root,
                           uint16_t* out);

/* Number of threads a call with nthreads <= 0 uses on this host. */
int oracle_default_threads(void);

#ifdef __cplusplus
}
#endif

#endif
