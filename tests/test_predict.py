"""The analytical CU-split predictor (host code, no GPU).

Each expected makespan below is worked out by hand from the scheduling rules
the predictor replays (workgroups below gemm_wgs start on the GEMM queue, the
rest on the comm queue, each switches queues once, an all_gather_matmul copy
workgroup with more tiles than workgroups only after the whole gather; an
all_gather_matmul tile waits for the copy units of its row block and takes
copy units meanwhile; a reduce unit waits for the tiles of its columns),
with a rate model chosen so
the durations are round numbers (the power cap, the mutual slowdowns and
the phase penalty switched off):

    GEMM tile  = 2*rows*cols*K / (1 TFLOP/s)          (no fixed cost)
    comm unit  = bytes / (1 GB/s per workgroup)       (no fixed cost)

and a chip-wide comm ceiling far above the per-workgroup rate unless a test
says otherwise.
"""
import pytest

import gemm_collective_tile_amd as il
from gemm_collective_tile_amd import Config, IrisError

UNIT = dict(gemm_tflops_per_cu=1.0, tile_overhead_us=0.0, comm_gbps_per_cu=1.0, comm_gbps_chip=1e9,
            unit_overhead_us=0.0, gemm_tflops_per_cu_max=1.0, gemm_slowdown=0.0, comm_slowdown=0.0,
            phase_penalty=0.0)


def tile_ms(rows, cols, K):
    return 2.0 * rows * cols * K / 1e12 * 1e3


def unit_ms(nbytes, gbps=1.0):
    return nbytes / (gbps * 1e9) * 1e3


def predict(op, cands, grid, config=None, params=UNIT, **shape):
    return il.iris_predict_gemm_wgs(op, cands, grid, config=config, params=params, **shape)


def test_independent_one_tile_one_unit():
    # concurrent broadcast: 1 tile beside 1 copy unit of 2048 elements (4 bytes each: read + write)
    best, ms = predict(il.IRIS_OP_CONCURRENT, [1], 2, Config(comm_chunk=2048), W=2, collective=il.IRIS_COLL_BROADCAST,
                       M=256, N=256, K=1024, comm_elems=2048)
    assert best == 1
    assert ms[1] == pytest.approx(max(tile_ms(256, 256, 1024), unit_ms(2048 * 4)), rel=1e-6)


def test_comm_workgroup_steals_gemm_tiles():
    # 8 tiles, 4 workgroups, 3 on GEMM; the comm one finishes its unit and takes tiles 3 and 7
    t, u = tile_ms(256, 256, 1024), unit_ms(2048 * 4)
    shape = dict(W=2, collective=il.IRIS_COLL_BROADCAST, M=512, N=1024, K=1024, comm_elems=2048)
    _, ms = predict(il.IRIS_OP_CONCURRENT, [3], 4, Config(comm_chunk=2048), **shape)
    assert ms[3] == pytest.approx(u + 2 * t, rel=1e-6)
    # without stealing the 3 GEMM workgroups take the 8 tiles in 3 rounds
    _, ms = predict(il.IRIS_OP_CONCURRENT, [3], 4, Config(comm_chunk=2048, flags=il.IRIS_FLAG_NO_STEAL), **shape)
    assert ms[3] == pytest.approx(3 * t, rel=1e-6)


def test_all_gather_tile_waits_for_its_row_block():
    # W=2, one 256x256 tile over K = 2*256; two copy units of 256 rows x 256 cols (read + write 2 bytes each).
    # The GEMM workgroup holds the tile and copies one unit while the other copies the second.
    _, ms = predict(il.IRIS_OP_AG_MM, [1], 2, Config(comm_block_m=256), W=2, M=256, N=256, K=256)
    assert ms[1] == pytest.approx(unit_ms(256 * 256 * 4) + tile_ms(256, 256, 512), rel=1e-6)


def test_all_gather_copy_workgroups_join_after_the_whole_gather():
    # More tiles than workgroups: a workgroup that started on the copy takes
    # GEMM tiles only once every copy unit has finished. Grid 3, gemm_wgs 1,
    # W=2, M=512 (row blocks 0 and 1), N=2048 (8 column tiles), GROUP_M 1 (row
    # block 0's tiles t0..t7 first), one 256-row copy unit per (row block,
    # shard): u0, u1 (block 0), u2, u3 (block 1), each U; a tile takes t =
    # 0.256 U. t=0: wg0 holds t0 and copies u0, wg1 copies u1, wg2 u2. t=U:
    # wg0 runs t0, wg1 copies u3 (until 2U), wg2 finds the copy queue empty
    # and waits for u3. wg0 runs t0..t3 alone (until U+4t = 2.024 U); from 2U
    # all three take tiles: wg1, wg2: t4, t5 | t7, t8 | t10, t11 | t13, t14;
    # wg0: t6, t9, t12, t15, the last ending at U + 8t. (Joining at U would
    # have given U + 7t.)
    U, t = unit_ms(256 * 256 * 4), tile_ms(256, 256, 512)
    assert t == pytest.approx(0.256 * U)
    _, ms = predict(il.IRIS_OP_AG_MM, [1], 3, Config(comm_block_m=256, group_m=1), W=2, M=512, N=2048, K=256)
    assert ms[1] == pytest.approx(U + 8 * t, rel=1e-6)


def test_reduce_scatter_units_wait_for_their_tiles():
    # W=2, rank 0: the slice is columns 0..255, tile (0,0) comes first; 4 reduce units of 64 rows x 256
    # columns (W reads + 1 write of 2 bytes) all need tile (0,0). Workgroup 1 waits for it, then reduces
    # units 0, 1, 3; workgroup 0 does tile 1, then unit 2.
    t, u = tile_ms(256, 256, 1024), unit_ms(64 * 256 * 2 * 3)
    _, ms = predict(il.IRIS_OP_MM_RS, [1], 2, W=2, rank=0, M=256, N=512, K=1024)
    assert ms[1] == pytest.approx(t + 3 * u, rel=1e-6)


def test_chip_ceiling_bounds_the_comm_time():
    # 64 copy units of 64 KiB elements on 64 comm workgroups; the chip ceiling of 4 GB/s binds.
    p = dict(UNIT, comm_gbps_chip=4.0)
    n = 64 * 65536
    _, ms = predict(il.IRIS_OP_CONCURRENT, [1], 65, params=p, W=2, collective=il.IRIS_COLL_BROADCAST,
                    M=256, N=256, K=64, comm_elems=n)
    assert ms[1] >= unit_ms(n * 4, 4.0) * (1 - 1e-6)


@pytest.mark.parametrize("op,extra", [
    (il.IRIS_OP_AG_MM, dict(W=8, M=4096, N=4096, K=512)),
    (il.IRIS_OP_MM_RS, dict(W=8, rank=3, M=8192, N=8192, K=2048)),
    (il.IRIS_OP_MM_AR, dict(W=4, M=4096, N=4096, K=4096)),
    (il.IRIS_OP_CONCURRENT, dict(W=8, collective=il.IRIS_COLL_ALL_REDUCE, M=8192, N=8192, K=8192,
                                 comm_elems=64 << 20)),
    (il.IRIS_OP_MM_AG, dict(W=8, rank=2, M=4096, N=4096, K=4096)),
])
def test_lower_bounds_with_default_rates(op, extra):
    """The makespan is at least the GEMM work over the whole grid at the
    default modelled rate (5 TFLOP/s per CU), and the best prediction is one
    of the candidates."""
    grid = 256
    cands = [16, 64, 128, 192, 224, 255]
    best, ms = il.iris_predict_gemm_wgs(op, cands, grid, **extra)
    assert best in cands and ms[best] == min(ms.values())
    M, N = extra["M"], extra["N"]
    K = extra["K"] * (extra["W"] if op == il.IRIS_OP_AG_MM else 1)
    gemm_ms = 2.0 * M * N * K / (5.0e12 * grid) * 1e3
    for v in ms.values():
        assert v >= gemm_ms * (1 - 1e-6)


def test_without_stealing_the_best_split_balances_the_queues():
    # GEMM 8192^3 (1024 tiles) beside an all_reduce of 8 x 64Mi elements (1024 units of 65536), with
    # no queue switching: the makespan is the longer of ceil(1024/g) tiles and ceil(1024/(256-g)) units,
    # which is smallest at an interior split
    p = dict(gemm_tflops_per_cu=4.4, tile_overhead_us=2.0, comm_gbps_per_cu=45.0, comm_gbps_chip=5200.0,
             unit_overhead_us=1.0, gemm_tflops_per_cu_max=4.4, gemm_slowdown=0.0, comm_slowdown=0.0,
             phase_penalty=0.0)
    t = 2e-3 + tile_ms(256, 256, 8192) / 4.4
    u = 1e-3 + unit_ms(65536 * 2 * 9, 45.0)
    cands = [32, 64, 128, 192, 224, 240, 255]
    best, ms = predict(il.IRIS_OP_CONCURRENT, cands, 256, Config(flags=il.IRIS_FLAG_NO_STEAL), params=p, W=8,
                       collective=il.IRIS_COLL_ALL_REDUCE, M=8192, N=8192, K=8192, comm_elems=64 << 20)
    assert best == 224
    for g in cands:
        nc = 256 - g
        if nc <= 115:  # below the chip ceiling every unit runs at the per-workgroup rate
            expect = max(-(-1024 // g) * t, -(-1024 // nc) * u)
            assert ms[g] == pytest.approx(expect, rel=1e-5), g


def test_ties_go_to_more_gemm_workgroups():
    # one tile and one unit: every split gives the same makespan
    best, ms = predict(il.IRIS_OP_CONCURRENT, [1, 2, 3], 4, Config(comm_chunk=2048), W=2,
                       collective=il.IRIS_COLL_BROADCAST, M=256, N=256, K=1024, comm_elems=2048)
    assert len(set(ms.values())) == 1
    assert best == 3


@pytest.mark.parametrize("kw,msg", [
    (dict(op=il.IRIS_OP_AG_MM, cands=[1], grid=1), "grid"),
    (dict(op=il.IRIS_OP_AG_MM, cands=[0], grid=8), "candidate"),
    (dict(op=il.IRIS_OP_AG_MM, cands=[8], grid=8), "candidate"),
    (dict(op=99, cands=[1], grid=8), "unknown op"),
    (dict(op=il.IRIS_OP_MM_RS, cands=[1], grid=8, N=1000, W=3), "reduce_scatter"),
    (dict(op=il.IRIS_OP_MM_RS, cands=[1], grid=8, rank=4, W=4), "reduce_scatter"),
    (dict(op=il.IRIS_OP_CONCURRENT, cands=[1], grid=8, comm_elems=0), "comm_elems"),
    (dict(op=il.IRIS_OP_CONCURRENT, cands=[1], grid=8, comm_elems=4096, collective=9), "collective"),
    (dict(op=il.IRIS_OP_AG_MM, cands=[1], grid=8, M=0), "positive"),
])
def test_invalid_arguments(kw, msg):
    shape = dict(W=2, rank=0, M=256, N=1024, K=256)
    kw = dict(kw)
    op, cands, grid = kw.pop("op"), kw.pop("cands"), kw.pop("grid")
    shape.update(kw)
    with pytest.raises(IrisError, match=msg):
        il.iris_predict_gemm_wgs(op, cands, grid, **shape)


def test_unknown_parameter_name():
    with pytest.raises(ValueError):
        il.iris_predict_gemm_wgs(il.IRIS_OP_AG_MM, [1], 8, params={"gemm_rate": 1.0}, W=2, M=256, N=256, K=256)


# ------------------------------------------------------------ rate model terms

def test_power_cap_lets_fewer_gemm_workgroups_run_faster():
    # one tile on a grid of 4 with NO_STEAL: 1 workgroup on the GEMM queue. Its tile runs at
    # min(r_max, r_full * grid / 1) = min(3, 4) = 3 TFLOP/s; with r_max = r_full it runs at 1.
    shape = dict(W=2, collective=il.IRIS_COLL_BROADCAST, M=256, N=256, K=1024, comm_elems=2048)
    cfg = Config(comm_chunk=2048, flags=il.IRIS_FLAG_NO_STEAL)
    fast = dict(UNIT, gemm_tflops_per_cu_max=3.0)
    _, ms = predict(il.IRIS_OP_CONCURRENT, [1], 4, cfg, params=fast, **shape)
    assert ms[1] == pytest.approx(max(tile_ms(256, 256, 1024) / 3.0, unit_ms(2048 * 4)), rel=1e-6)
    _, ms = predict(il.IRIS_OP_CONCURRENT, [1], 4, cfg, params=UNIT, **shape)
    assert ms[1] == pytest.approx(max(tile_ms(256, 256, 1024), unit_ms(2048 * 4)), rel=1e-6)


def test_comm_workgroups_slow_the_gemm_and_back():
    # grid 4, gemm_wgs 2, NO_STEAL: 2 workgroups on each queue. Comm rate 1 GB/s per workgroup,
    # chip 4 GB/s: the comm side could use u = 2 * 1 / 4 = 0.5 of it, so a tile runs
    # (1 - 0.2 * 0.5) = 0.9 times as fast; half the grid is on the GEMM (v = 0.5), so a unit
    # moves (1 - 0.4 * 0.5) = 0.8 times as fast.
    shape = dict(W=2, collective=il.IRIS_COLL_BROADCAST, M=256, N=256, K=1024, comm_elems=2048)
    cfg = Config(comm_chunk=2048, flags=il.IRIS_FLAG_NO_STEAL)
    prm = dict(UNIT, comm_gbps_chip=4.0, gemm_slowdown=0.2, comm_slowdown=0.4)
    _, ms = predict(il.IRIS_OP_CONCURRENT, [2], 4, cfg, params=prm, **shape)
    # one tile (2 GEMM workgroups, r_max = r_full: 1 * 4 / 2 = 2 capped at r_max = 1) and one unit
    tile = tile_ms(256, 256, 1024) / 0.9
    unit = unit_ms(2048 * 4) / 0.8
    assert ms[2] == pytest.approx(max(tile, unit), rel=1e-6)


def test_phase_penalty_only_when_workgroups_fall_out_of_phase():
    # a multi-wave GEMM alone (broadcast of one tiny unit beside it, all workgroups on the GEMM,
    # NO_STEAL so the comm workgroup never takes tiles): every wave starts in phase, R = 1, no penalty
    shape = dict(W=2, collective=il.IRIS_COLL_BROADCAST, M=1024, N=1024, K=1024, comm_elems=2048)
    cfg = Config(comm_chunk=2048, flags=il.IRIS_FLAG_NO_STEAL)
    prm = dict(UNIT, phase_penalty=0.5)
    _, ms = predict(il.IRIS_OP_CONCURRENT, [4], 5, cfg, params=prm, **shape)
    assert ms[4] == pytest.approx(4 * tile_ms(256, 256, 1024), rel=1e-6)  # 16 tiles on 4 workgroups


# ------------------------------------------------------ measured sweeps (MI355X)

def _sweeps():
    import json
    import os
    d = json.load(open(os.path.join(os.path.dirname(__file__), "data", "measured_sweeps_mi355x.json")))
    for run in d["runs"]:
        for name, rec in run.items():
            w = d["workloads"][name]
            shape = {k: w[k] for k in ("W", "M", "N", "K", "rank", "comm_elems") if k in w}
            yield name, w["op"], rec["grid"], {int(k): v for k, v in rec["sweep_ms"].items()}, shape


def test_default_model_ranks_the_measured_sweeps():
    """With its default constants the predictor's best split measured within
    1.5 % of the measured best in each of the recorded sweeps (four
    workloads on four boxes), and the three best predicted splits always hold
    one within 1 % of it, so top_k = 3 keeps a winner."""
    for name, op, grid, meas, shape in _sweeps():
        cands = sorted(meas)
        best, pred = il.iris_predict_gemm_wgs(op, cands, grid, **shape)
        mbest = min(meas.values())
        assert meas[best] <= 1.015 * mbest, (name, best, meas)
        top3 = sorted(cands, key=lambda c: (pred[c], -c))[:3]
        assert min(meas[c] for c in top3) <= 1.01 * mbest, (name, top3, meas)


def test_concurrent_prediction_is_not_flat():
    # the GEMM beside the 8 x 64Mi all_reduce: giving the comm queue more workgroups speeds the
    # all_reduce but costs GEMM throughput; the measured sweeps are U-shaped, and so is the model
    cands = [96, 128, 160, 192, 208, 224, 240, 255]
    best, pred = il.iris_predict_gemm_wgs(il.IRIS_OP_CONCURRENT, cands, 256, W=8, M=8192, N=8192, K=8192,
                                          comm_elems=64 << 20)
    assert max(pred.values()) > 1.03 * min(pred.values())
    assert 192 <= best <= 240
    assert pred[96] > pred[best] and pred[255] > pred[best]
