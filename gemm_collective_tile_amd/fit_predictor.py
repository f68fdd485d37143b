"""Refit the split predictor's fitted constants to measured gemm_wgs sweeps.

Host only (no GPU): the predictor is a simulation in libiris_local.so, and
this script calls it through the binding with candidate constants, scoring
each set against sweeps measured on the target GPU (a JSON file in the
format of tests/data/measured_sweeps_mi355x.json: per box, per workload, the
median milliseconds of each gemm_wgs the sweep tried).

Score of a constant set: for every sweep, how much slower (measured) the
predicted best split is than the measured best (the worst over all sweeps
is minimised first), then the mean squared log difference of the two
curves, each normalised by its own minimum (the boxes' speeds differ).

  python gemm_collective_tile_amd/fit_predictor.py [sweeps.json]

prints the best constant sets; the library's defaults are in predict.cpp.
"""
import itertools
import json
import math
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

GRID = dict(gemm_tflops_per_cu_max=[5.0, 5.25, 5.5, 6.0, 7.0], gemm_slowdown=[0.0, 0.05, 0.1, 0.2, 0.3],
            comm_slowdown=[0.3, 0.45, 0.6, 0.75, 0.9], phase_penalty=[0.0, 0.03, 0.045, 0.06, 0.1])

_DATA = None


def _load(path):
    global _DATA
    if _DATA is None:
        _DATA = json.load(open(path))
    return _DATA


def _sweeps(data):
    for run in data["runs"]:
        for name, rec in run.items():
            w = data["workloads"][name]
            shape = {k: w[k] for k in ("W", "M", "N", "K", "rank", "comm_elems") if k in w}
            yield name, w["op"], rec["grid"], {int(k): v for k, v in rec["sweep_ms"].items()}, shape


def score(params, path):
    import gemm_collective_tile_amd as il
    worst, err = 0.0, 0.0
    for name, op, grid, meas, shape in _sweeps(_load(path)):
        cands = sorted(meas)
        best, pred = il.iris_predict_gemm_wgs(op, cands, grid, params=params, **shape)
        mmin, pmin = min(meas.values()), min(pred.values())
        worst = max(worst, meas[best] / mmin - 1.0)
        err += sum((math.log(pred[c] / pmin) - math.log(meas[c] / mmin)) ** 2 for c in cands) / len(cands)
    return worst, err


def _eval(args):
    values, path = args
    params = dict(zip(GRID, values))
    return score(params, path) + (params,)


def main():
    path = sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(HERE), "tests", "data",
                                                              "measured_sweeps_mi355x.json")
    combos = [(v, path) for v in itertools.product(*GRID.values())]
    with ProcessPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        res = sorted(ex.map(_eval, combos, chunksize=8), key=lambda r: (round(r[0], 4), r[1]))
    for worst, err, params in res[:10]:
        print(f"worst miss {worst * 100:5.2f} %  shape error {err:.4f}  {params}")


if __name__ == "__main__":
    main()
