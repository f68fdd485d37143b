// Host-only driver for the address and undefined-behaviour sanitizer build
// of the CPU oracle and of the split predictor (test infrastructure). It
// calls every oracle entry point on small random inputs, including empty
// ranges, W = 1 and ragged shapes, and the predictor on every op with small
// and workload-sized shapes. Any out-of-bounds access, leak or undefined
// operation aborts with a sanitizer report; a clean run prints "ok".
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "iris_local.h"
#include "oracle.h"

namespace iris {
int set_error(int status, const char*) { return status; }  // the library's message store
}

static std::mt19937_64 rng(7);

static std::vector<uint16_t> rnd(size_t n) {
  std::uniform_real_distribution<double> d(-2.0, 2.0);
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = oracle_f16_encode(d(rng));
  return v;
}

static void oracle_cases() {
  for (int64_t M : {1, 7, 33})
    for (int64_t N : {8, 24})
      for (int W : {1, 2, 3}) {
        const int64_t kl = 8 * W;
        const int64_t K = kl * W;
        std::vector<std::vector<uint16_t>> sh;
        std::vector<const uint16_t*> shp;
        for (int s = 0; s < W; ++s) sh.push_back(rnd(M * kl));
        for (auto& s : sh) shp.push_back(s.data());
        auto B = rnd(K * N), bias = rnd(N > M ? N : M), A = rnd(M * K);
        std::vector<uint16_t> g(M * K);
        oracle_all_gather_k(shp.data(), W, M, kl, g.data());
        std::vector<double> out(M * N * W + 1);
        oracle_all_gather_matmul(shp.data(), W, M, kl, B.data(), N, bias.data(), ORACLE_BIAS_ALONG_N, 0, M, 0, N,
                                 out.data(), 3);
        oracle_all_gather_matmul(shp.data(), W, M, kl, B.data(), N, bias.data(), ORACLE_BIAS_ALONG_M, M / 2, M,
                                 N / 2, N, out.data(), 2);
        oracle_all_gather_matmul(shp.data(), W, M, kl, B.data(), N, nullptr, ORACLE_BIAS_NONE, 0, 0, 0, N,
                                 out.data(), 1);  // empty row range
        oracle_gemm_bias(A.data(), K, B.data(), N, bias.data(), ORACLE_BIAS_ALONG_N, K, 0, M, 0, N, out.data(), 4);
        std::vector<std::vector<uint16_t>> parts;
        std::vector<const uint16_t*> pp;
        if (N % W == 0) {
          for (int p = 0; p < W - 1; ++p) parts.push_back(rnd(M * (N / W)));
          for (auto& p : parts) pp.push_back(p.data());
          oracle_matmul_reduce_scatter(A.data(), B.data(), bias.data(), ORACLE_BIAS_ALONG_N, pp.data(), W, W - 1, M,
                                       N, K, 0, M, out.data(), 2);
        }
        parts.clear();
        pp.clear();
        for (int p = 0; p < W - 1; ++p) parts.push_back(rnd(M * N));
        for (auto& p : parts) pp.push_back(p.data());
        oracle_matmul_all_reduce(A.data(), B.data(), bias.data(), ORACLE_BIAS_ALONG_N, pp.data(), W, M, N, K, 0, M,
                                 out.data(), 2);
        oracle_matmul_all_gather(A.data(), B.data(), bias.data(), ORACLE_BIAS_ALONG_M, pp.data(), W, W / 2, M, N, K,
                                 0, M * W, out.data(), 3);
        const int64_t n = 8 * W * 5;
        std::vector<std::vector<uint16_t>> bufs;
        std::vector<const uint16_t*> bp;
        for (int w = 0; w < W; ++w) bufs.push_back(rnd(n));
        for (auto& b : bufs) bp.push_back(b.data());
        std::vector<uint16_t> o16(W * n);
        std::vector<double> o64(n);
        oracle_sum(bp.data(), W, n, o64.data());
        oracle_all_gather_flat(bp.data(), W, n, o16.data());
        oracle_reduce_scatter_flat(bp.data(), W, n, W - 1, o64.data());
        oracle_all_to_all_flat(bp.data(), W, n, 0, o16.data());
        oracle_broadcast_flat(bp.data(), W, n, W - 1, o16.data());
      }
  for (uint32_t h = 0; h < 65536; h += 7) oracle_f16_encode(oracle_f16_decode((uint16_t)h));
}

static void predict_cases() {
  struct Case {
    int op, W, rank, coll;
    int64_t M, N, K, n;
  } cases[] = {
      {IRIS_OP_AG_MM, 8, 0, 0, 4096, 4096, 512, 0},        {IRIS_OP_AG_MM, 8, 0, 0, 131072, 16384, 2048, 0},
      {IRIS_OP_AG_MM, 3, 0, 0, 300, 200, 40, 0},           {IRIS_OP_MM_RS, 8, 0, 0, 4096, 11008, 4096, 0},
      {IRIS_OP_MM_RS, 4, 3, 0, 300, 64, 40, 0},            {IRIS_OP_MM_AR, 8, 0, 0, 8192, 8192, 8192, 0},
      {IRIS_OP_CONCURRENT, 8, 0, 1, 8192, 8192, 8192, 64 << 20},
      {IRIS_OP_CONCURRENT, 4, 2, 3, 512, 512, 512, 4096}, {IRIS_OP_CONCURRENT, 4, 1, 4, 512, 512, 512, 4096},
      {IRIS_OP_CONCURRENT, 2, 1, 5, 256, 256, 256, 2048}, {IRIS_OP_CONCURRENT, 3, 0, 2, 256, 256, 256, 2048},
      {IRIS_OP_MM_AG, 8, 3, 0, 4096, 4096, 4096, 0},       {IRIS_OP_MM_AG, 1, 0, 0, 64, 64, 64, 0},
  };
  for (const Case& c : cases) {
    iris_op_args_t a{};
    a.op = c.op;
    a.W = c.W;
    a.rank = c.rank;
    a.collective = c.coll;
    a.M = c.M;
    a.N = c.N;
    a.K = c.K;
    a.comm_elems = c.n;
    for (int tile : {256, 64}) {
      a.cfg.block_m = a.cfg.block_n = tile;
      const int grid = tile == 256 ? 256 : 512;
      const int32_t cands[] = {1, grid / 8, grid / 2, (7 * grid) / 8, grid - 1};
      float ms[5];
      int32_t best = 0;
      const int st = iris_predict_gemm_wgs(&a, grid, cands, 5, nullptr, ms, &best);
      if (st != IRIS_OK) {
        std::printf("predict failed: op %d status %d\n", c.op, st);
        std::exit(1);
      }
    }
  }
  iris_op_args_t bad{};  // invalid arguments must be rejected cleanly
  const int32_t one = 1;
  bad.op = 99;
  bad.M = bad.N = bad.K = 64;
  bad.W = 1;
  if (iris_predict_gemm_wgs(&bad, 8, &one, 1, nullptr, nullptr, nullptr) == IRIS_OK) std::exit(1);
  if (iris_predict_gemm_wgs(nullptr, 8, &one, 1, nullptr, nullptr, nullptr) == IRIS_OK) std::exit(1);
}

int main() {
  oracle_cases();
  predict_cases();
  std::printf("ok\n");
  return 0;
}
