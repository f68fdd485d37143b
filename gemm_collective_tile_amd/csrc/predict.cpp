// Analytical CU-split predictor: a discrete-event simulation of the fused
// persistent work-stealing schedule for one op, used to rank gemm_wgs
// candidates before benchmarking the best few (iris.concurrent PR
// description: predict, then benchmark the top-k configurations, always
// including the static default; the predictor there is a work-stealing
// makespan simulator with per-tile atomic costs and a floor on the CUs a
// heavy collective needs).
//
// The simulation replays the kernel's own rules: workgroups below gemm_wgs
// start on the GEMM queue, the others on the comm queue, and each switches
// queues when its first one runs dry (with more tiles than workgroups, an
// all_gather_matmul copy workgroup only once every copy unit has finished);
// a GEMM tile of all_gather_matmul waits for the copy units of its row block
// and takes unclaimed copy units while it waits; a reduce unit waits for the
// GEMM tiles of its columns, taking GEMM tiles only while one it needs is
// still unclaimed. Durations come from a rate model whose constants were
// measured on MI355X:
//   * a tile costs a fixed overhead plus its FLOPs at a per-CU rate. The
//     chip's MFMA throughput is capped by power, not by CU count: with n
//     workgroups working the GEMM queue each tile runs at
//     min(r_max, r_full * grid / n), where r_full is the rate with every CU
//     on the GEMM and r_max the rate of a lone CU at its highest clock;
//   * a comm unit costs a fixed overhead plus its bytes at the per-workgroup
//     rate, capped by the chip's comm bandwidth shared by the units in
//     flight;
//   * the two slow each other: a tile started while the workgroups working
//     the comm queue could use a fraction u of the chip's comm bandwidth
//     runs (1 - gemm_slowdown * u) times as fast, and a unit started while a
//     fraction v of the grid works the GEMM queue moves
//     (1 - comm_slowdown * v) times as fast;
//   * with more tiles than workgroups, tiles that share operands reach L2
//     together only if the workgroups run in phase (every XCD runs a patch
//     of tiles whose A rows and B columns meet in its L2). A first pass of
//     the simulation gives every tile's start time; R, the length of the
//     mean of exp(2 pi i start / tile duration) over the tiles, is 1 when
//     all start in phase and near 0 when their phases are spread. The second
//     pass stretches every tile by phase_penalty * (1 - R).
// Host code only: no device call.
#include "../../include/iris_local.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <functional>
#include <queue>
#include <vector>

#include "schedule.hpp"

namespace iris {
int set_error(int status, const char* msg);  // defined beside the other entry points
}

namespace iris_predict {

constexpr double kGemmTflopsPerCu = 5.0;   // K-loop rate of a 256x256 tile, every CU on the GEMM
                                           // (fit over K = 4096..16384)
constexpr double kTileOverheadUs = 20.0;   // claim, prologue, epilogue and store drain of a tile
constexpr double kCommGbpsPerCu = 45.0;    // one 4-wave workgroup copying or reducing
constexpr double kCommGbpsChip = 5200.0;   // plain copy over the whole chip
constexpr double kUnitOverheadUs = 1.0;    // claim + release of a comm unit
// Fitted (grid search) to sixteen gemm_wgs sweeps measured on MI355X: the
// four bench workloads (pow2_4k and g2 all_gather_matmul, llama7b_gate
// reduce_scatter, the 8192^3 GEMM beside an 8 x 64Mi all_reduce) on four
// boxes. With these, the predicted best split measured within 1.1 % of the
// measured best in every sweep, and the three best predicted always held a
// split within 1 % of it.
constexpr double kGemmTflopsPerCuMax = 5.25;
constexpr double kGemmSlowdown = 0.10;
constexpr double kCommSlowdown = 0.60;
constexpr double kPhasePenalty = 0.045;

struct Work {
  int grid = 0;
  bool steal = true;
  int kind = 0;  // 1 AG, 2 RS/ARMM (comm waits on tiles), 0 independent
  std::vector<double> tile_flop;            // FLOPs of each tile
  std::vector<int> tile_pm;
  double tile_overhead_ms = 0.02;
  double r_full = kGemmTflopsPerCu * 1e12, r_max = kGemmTflopsPerCuMax * 1e12;
  double gemm_slowdown = kGemmSlowdown, comm_slowdown = kCommSlowdown, phase_penalty = kPhasePenalty;
  std::vector<double> unit_bytes;
  std::vector<int> unit_pm;                 // AG: row block the unit belongs to
  std::vector<std::vector<int>> unit_deps;  // RS/ARMM: tiles a unit needs
  int n_pm = 0;
  double comm_gbps_cu = kCommGbpsPerCu, comm_gbps_chip = kCommGbpsChip, unit_overhead_ms = 1e-3;
};

// Makespan (ms) of the schedule with gemm_wgs workgroups starting on GEMM;
// every tile is stretched by the factor `stretch`; tile start times go to
// *starts if it is not null.
double simulate(const Work& w, int gemm_wgs, double stretch, std::vector<double>* starts) {
  const int T = (int)w.tile_flop.size(), U = (int)w.unit_bytes.size();
  std::vector<double> tile_end(T, -1.0);
  int next_tile = 0, next_unit = 0;
  int on_gemm = 0, on_comm = 0;  // workgroups working each queue
  // all_gather: per row block, units not yet claimed and the latest end time
  std::vector<int> rb_left(w.n_pm, 0);
  std::vector<double> rb_end(w.n_pm, 0.0);
  if (w.kind == 1)
    for (int u = 0; u < U; ++u) ++rb_left[w.unit_pm[u]];
  // end times of comm units in flight (bandwidth sharing)
  std::priority_queue<double, std::vector<double>, std::greater<double>> active;
  auto start_unit = [&](int u, double t0) {
    while (!active.empty() && active.top() <= t0) active.pop();
    const double v = std::min(1.0, (double)on_gemm / (double)w.grid);
    const double gbps = std::min(w.comm_gbps_cu, w.comm_gbps_chip / (double)(active.size() + 1)) *
                        (1.0 - w.comm_slowdown * v);
    const double end = t0 + w.unit_overhead_ms + w.unit_bytes[u] / (gbps * 1e9) * 1e3;
    active.push(end);
    if (w.kind == 1) {
      const int pm = w.unit_pm[u];
      --rb_left[pm];
      rb_end[pm] = std::max(rb_end[pm], end);
    }
    return end;
  };
  auto start_tile = [&](int t, double t0) {
    const double n = (double)std::max(1, on_gemm);
    const double u = std::min(1.0, (double)on_comm * w.comm_gbps_cu / w.comm_gbps_chip);
    const double rate = std::min(w.r_max, w.r_full * (double)w.grid / n) * (1.0 - w.gemm_slowdown * u);
    tile_end[t] = t0 + (w.tile_overhead_ms + w.tile_flop[t] / rate * 1e3) * stretch;
    if (starts) (*starts)[t] = t0;
    return tile_end[t];
  };

  struct Worker {
    bool gemm_first;
    int phase = 0;
    int held_tile = -1, held_unit = -1;
    bool done = false;
  };
  std::vector<Worker> wk(w.grid);
  using Ev = std::pair<double, int>;
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> ev;
  for (int i = 0; i < w.grid; ++i) {
    wk[i].gemm_first = i < gemm_wgs || U == 0;
    ++(wk[i].gemm_first ? on_gemm : on_comm);
    ev.push({0.0, i});
  }
  double makespan = 0.0;
  while (!ev.empty()) {
    const auto [now, i] = ev.top();
    ev.pop();
    Worker& k = wk[i];
    makespan = std::max(makespan, now);
    if (k.held_tile >= 0) {  // all_gather: a tile waiting for its row block
      const int pm = w.tile_pm[k.held_tile];
      if (rb_left[pm] == 0) {
        ev.push({start_tile(k.held_tile, std::max(now, rb_end[pm])), i});
        k.held_tile = -1;
      } else if (next_unit < U) {
        ev.push({start_unit(next_unit++, now), i});
      } else {  // cannot happen: unclaimed units of pm would be in the queue
        ev.push({start_tile(k.held_tile, now), i});
        k.held_tile = -1;
      }
      continue;
    }
    if (k.held_unit >= 0) {  // reduce: a unit waiting for its tiles
      const auto& deps = w.unit_deps[k.held_unit];
      bool unclaimed = false;
      double ready = now;
      for (int t : deps) {
        if (tile_end[t] < 0) unclaimed = true;
        else ready = std::max(ready, tile_end[t]);
      }
      if (unclaimed && next_tile < T) {
        ev.push({start_tile(next_tile++, now), i});
      } else {
        ev.push({start_unit(k.held_unit, ready), i});
        k.held_unit = -1;
      }
      continue;
    }
    // claim from the current queue, switching once when it is empty
    for (;;) {
      const bool gemm = k.gemm_first == (k.phase == 0);
      if (gemm && next_tile < T) {
        const int t = next_tile++;
        if (w.kind == 1) {
          k.held_tile = t;
          ev.push({now, i});
        } else {
          ev.push({start_tile(t, now), i});
        }
        break;
      }
      if (!gemm && next_unit < U) {
        const int u = next_unit++;
        if (w.kind == 2) {
          k.held_unit = u;
          ev.push({now, i});
        } else {
          ev.push({start_unit(u, now), i});
        }
        break;
      }
      if (k.phase == 0 && w.steal) {
        k.phase = 1;
        // this workgroup moves to the other queue
        if (gemm) { --on_gemm; ++on_comm; } else { --on_comm; ++on_gemm; }
        if (w.kind == 1 && !k.gemm_first && T > w.grid) {
          // all_gather with more tiles than workgroups: a copy workgroup
          // joins the GEMM once every copy unit has finished (all are
          // claimed by now)
          double all_end = now;
          for (double e : rb_end) all_end = std::max(all_end, e);
          if (all_end > now) {
            ev.push({all_end, i});
            break;
          }
        }
        continue;
      }
      k.done = true;
      --(gemm ? on_gemm : on_comm);
      break;
    }
  }
  return makespan;
}

// Phase coherence R of the tile start times of a first pass (see the top of
// this file), against the median tile duration of that pass.
double phase_coherence(const std::vector<double>& starts, double period) {
  if (starts.empty() || period <= 0) return 1.0;
  double c = 0, s = 0;
  for (double t : starts) {
    const double ph = 2.0 * 3.14159265358979323846 * t / period;
    c += std::cos(ph);
    s += std::sin(ph);
  }
  return std::sqrt(c * c + s * s) / (double)starts.size();
}

double predict(const Work& w, int gemm_wgs) {
  const int T = (int)w.tile_flop.size();
  if (T <= w.grid || w.phase_penalty <= 0) return simulate(w, gemm_wgs, 1.0, nullptr);
  std::vector<double> starts(T, 0.0);
  simulate(w, gemm_wgs, 1.0, &starts);
  std::vector<double> flop(w.tile_flop);
  std::nth_element(flop.begin(), flop.begin() + T / 2, flop.end());
  const double period = w.tile_overhead_ms + flop[T / 2] / w.r_full * 1e3;
  const double R = phase_coherence(starts, period);
  return simulate(w, gemm_wgs, 1.0 + w.phase_penalty * (1.0 - R), nullptr);
}

}  // namespace iris_predict

namespace {
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}

extern "C" int iris_predict_gemm_wgs(const iris_op_args_t* a, int32_t grid, const int32_t* candidates,
                                     int32_t n_candidates, const iris_predict_params_t* params,
                                     float* predicted_ms, int32_t* best_gemm_wgs) {
  using namespace iris_predict;
  using iris::set_error;
  if (!a || !candidates || n_candidates < 1)
    return set_error(IRIS_ERR_INVALID_ARG, "predict: args and at least one candidate are required");
  if (grid < 2 || grid > 65536) return set_error(IRIS_ERR_INVALID_ARG, "predict: grid must be in [2, 65536]");
  iris_config_t c{};
  c = a->cfg;
  const int bm = c.block_m > 0 ? c.block_m : 256, bn = c.block_n > 0 ? c.block_n : 256;
  const int gm = c.group_m > 0 ? c.group_m : 8;
  const int64_t M = a->M, N = a->N, W = a->W;
  if (M <= 0 || N <= 0 || a->K <= 0 || W < 1 || W > IRIS_MAX_W || bm <= 0 || bn <= 0)
    return set_error(IRIS_ERR_INVALID_ARG, "predict: M, N, K must be positive and W in [1, IRIS_MAX_W]");
  if (a->op == IRIS_OP_MM_RS && (N % W != 0 || a->rank < 0 || a->rank >= W))
    return set_error(IRIS_ERR_INVALID_ARG, "predict: reduce_scatter needs W | N and 0 <= rank < W");
  Work w;
  w.r_full = (params && params->gemm_tflops_per_cu > 0 ? params->gemm_tflops_per_cu : kGemmTflopsPerCu) * 1e12;
  w.r_max = (params && params->gemm_tflops_per_cu_max > 0 ? params->gemm_tflops_per_cu_max : kGemmTflopsPerCuMax) *
            1e12;
  w.r_max = std::max(w.r_max, w.r_full);
  w.tile_overhead_ms = (params && params->tile_overhead_us >= 0 ? params->tile_overhead_us : kTileOverheadUs) * 1e-3;
  if (params && params->gemm_slowdown >= 0) w.gemm_slowdown = std::min(0.95, params->gemm_slowdown);
  if (params && params->comm_slowdown >= 0) w.comm_slowdown = std::min(0.95, params->comm_slowdown);
  if (params && params->phase_penalty >= 0) w.phase_penalty = params->phase_penalty;
  w.grid = grid;
  w.steal = (c.flags & IRIS_FLAG_NO_STEAL) == 0;
  if (params && params->comm_gbps_per_cu > 0) w.comm_gbps_cu = params->comm_gbps_per_cu;
  if (params && params->comm_gbps_chip > 0) w.comm_gbps_chip = params->comm_gbps_chip;
  w.unit_overhead_ms = (params && params->unit_overhead_us >= 0 ? params->unit_overhead_us : kUnitOverheadUs) * 1e-3;

  // GEMM tiles in queue order
  const int64_t K = a->op == IRIS_OP_AG_MM ? a->K * W : a->K;
  const int n_pm = (int)cdiv(M, bm), n_pn = (int)cdiv(N, bn);
  if ((int64_t)n_pm * n_pn > (1 << 26)) return set_error(IRIS_ERR_UNSUPPORTED, "predict: more than 2^26 GEMM tiles");
  iris::TileOrder o{n_pm, n_pn, gm, 0, 0};
  const int64_t nl = a->op == IRIS_OP_MM_RS ? N / W : N;
  const int64_t col0 = a->op == IRIS_OP_MM_RS ? a->rank * nl : 0;
  if (a->op == IRIS_OP_MM_RS) {
    o.prio_lo = (int)(col0 / bn);
    o.prio_hi = (int)cdiv(col0 + nl, bn);
  }
  const int T = n_pm * n_pn;
  w.tile_flop.resize(T);
  w.tile_pm.resize(T);
  w.n_pm = n_pm;
  for (int t = 0; t < T; ++t) {
    int pm, pn;
    iris::tile_coords(o, t, pm, pn);
    const double rows = (double)std::min<int64_t>(bm, M - (int64_t)pm * bm);
    const double cols = (double)std::min<int64_t>(bn, N - (int64_t)pn * bn);
    w.tile_flop[t] = 2.0 * rows * cols * (double)K;
    w.tile_pm[t] = pm;
  }

  // comm units in queue order, with the same default unit sizes as the library
  auto pow2_rows = [&](int64_t row_bytes, int64_t target) {
    int r = bm;
    while (r > 1 && (int64_t)r * row_bytes > target) r >>= 1;
    return r;
  };
  const int64_t chunk = c.comm_chunk > 0 ? c.comm_chunk : 65536;
  switch (a->op) {
    case IRIS_OP_AG_MM: {
      w.kind = 1;
      const int rows_u = c.comm_block_m > 0 ? c.comm_block_m : pow2_rows(a->K * 2, 131072);
      const int n_sub = bm / rows_u;
      for (int pm = 0; pm < n_pm; ++pm)
        for (int s = 0; s < W; ++s)
          for (int q = 0; q < n_sub; ++q) {
            const int64_t r0 = (int64_t)pm * bm + (int64_t)q * rows_u;
            const int64_t rows = std::max<int64_t>(0, std::min<int64_t>(rows_u, M - r0));
            w.unit_bytes.push_back((double)rows * (double)a->K * 4.0);  // read shard + write gathered
            w.unit_pm.push_back(pm);
          }
      break;
    }
    case IRIS_OP_MM_RS:
    case IRIS_OP_MM_AR: {
      w.kind = 2;
      const int cbn = c.comm_block_n > 0 ? c.comm_block_n : bn;
      const int rows_u = c.comm_block_m > 0 ? c.comm_block_m : pow2_rows(std::min<int64_t>(cbn, nl) * 2, 32768);
      const int n_sub = bm / rows_u;
      const int n_cc = (int)cdiv(nl, cbn);
      for (int pm = 0; pm < n_pm; ++pm)
        for (int q = 0; q < n_sub; ++q)
          for (int cc = 0; cc < n_cc; ++cc) {
            const int64_t r0 = (int64_t)pm * bm + (int64_t)q * rows_u;
            const int64_t rows = std::max<int64_t>(0, std::min<int64_t>(rows_u, M - r0));
            const int64_t j0 = (int64_t)cc * cbn, cols = std::min<int64_t>(cbn, nl - j0);
            w.unit_bytes.push_back((double)rows * (double)cols * 2.0 * (double)(W + 1));
            std::vector<int> deps;
            const int64_t c_lo = col0 + j0, c_hi = col0 + j0 + cols;
            for (int64_t pn = c_lo / bn; pn <= (c_hi - 1) / bn; ++pn)
              deps.push_back(iris::tile_index(o, pm, (int)pn));
            w.unit_deps.push_back(deps);
          }
      break;
    }
    case IRIS_OP_CONCURRENT: {
      const int coll = a->collective > 0 ? a->collective : IRIS_COLL_ALL_REDUCE;
      const int64_t n = a->comm_elems;
      if (n <= 0) return set_error(IRIS_ERR_INVALID_ARG, "predict: comm_elems must be positive");
      if (coll < IRIS_COLL_ALL_REDUCE || coll > IRIS_COLL_BROADCAST)
        return set_error(IRIS_ERR_INVALID_ARG, "predict: unknown collective");
      int64_t blocks = 1, blk = n;
      double per_elem = 4.0;  // a copy reads and writes 2 bytes
      if (coll == IRIS_COLL_ALL_REDUCE) per_elem = 2.0 * (double)(W + 1);
      if (coll == IRIS_COLL_REDUCE_SCATTER) { blk = n / W; per_elem = 2.0 * (double)(W + 1); }
      if (coll == IRIS_COLL_ALL_GATHER) blocks = W;
      if (coll == IRIS_COLL_ALL_TO_ALL) { blocks = W; blk = n / W; }
      for (int64_t b = 0; b < blocks; ++b)
        for (int64_t e0 = 0; e0 < blk; e0 += chunk)
          w.unit_bytes.push_back((double)std::min<int64_t>(chunk, blk - e0) * per_elem);
      break;
    }
    case IRIS_OP_MM_AG: {
      const int64_t blk = M * N;
      for (int64_t p = 0; p < W - 1; ++p)
        for (int64_t e0 = 0; e0 < blk; e0 += chunk)
          w.unit_bytes.push_back((double)std::min<int64_t>(chunk, blk - e0) * 4.0);
      break;
    }
    default:
      return set_error(IRIS_ERR_INVALID_ARG, "predict: unknown op");
  }
  if (w.unit_bytes.size() > ((size_t)1 << 26)) return set_error(IRIS_ERR_UNSUPPORTED, "predict: more than 2^26 comm units");

  int best = -1;
  double best_ms = 0.0;
  for (int i = 0; i < n_candidates; ++i) {
    const int gw = candidates[i];
    if (gw < 1 || gw > grid - 1) return set_error(IRIS_ERR_CONFIG, "predict: a candidate gemm_wgs is outside [1, grid-1]");
    const double ms = predict(w, gw);
    if (predicted_ms) predicted_ms[i] = (float)ms;
    if (best < 0 || ms < best_ms || (ms == best_ms && gw > best)) {
      best = gw;
      best_ms = ms;
    }
  }
  if (best_gemm_wgs) *best_gemm_wgs = best;
  return IRIS_OK;
}
