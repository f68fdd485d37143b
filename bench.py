"""Benchmark of one GPU's share of the fused communication + GEMM ops on MI355X.

One step = one call of the fused op on the headline workload (default g2
all_gather_matmul: W=8 K-shards (131072, 2048) gathered into (131072, 16384)
and multiplied by B (16384, 16384) plus bias), with every input already
resident in HBM. The gemm_wgs split is swept first (untimed), as the host
sweep does for any shape, then `--warmup` untimed and `--steps` timed steps
run. Prints ONE JSON line.

  value      GEMM TFLOP/s of the whole fused op: 2*M*N*K / (wall time per step)
  roofline   the fused persistent kernel against the dense fp16 MFMA peak:
             2*M*N*K / (mean kernel duration from HIP events on the op's
             stream around the timed launches). `traffic` is the kernel's
             bytes fetched from beyond L2 plus bytes written, per launch, from
             rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by what the same
             counters read for a plain device copy; read from profiles/ and
             reported only while the kernel sources still hash to the value
             recorded there (else null)
  comm       the communication units' GB/s over their in-kernel window, and
             the sequential comm kernel's; fractions of the 8 TB/s HBM peak
             only for data sets larger than the 256 MiB last-level cache
  clock      the shader clock the GPU held during the fused launch
             (iris_last_clock), next to the 2.4 GHz of the published peak
  copy_ceiling  a plain 1 GiB device-to-device copy (torch), GB/s
  cpu_baseline  the CPU oracle on a bounded sample of the headline workload
             (sampled 128x128 output tiles computed in fp64, and the whole
             gathered buffer compared bit for bit) on the CPU share of one GPU
  oracle_check  every measured workload is checked against the oracle
             outside the timed regions; any mismatch makes the exit status 1
  extra      the other workloads (pow2_4k all_gather_matmul, llama7b_gate
             reduce_scatter, concurrent 8192^3 GEMM beside an all_reduce)
             measured the same way, unless --headline-only

Only one GPU is used: --gpus above 1 exits with a message.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
MALL_BYTES = 256 << 20      # MI355X last-level (Infinity) cache
KERNEL_SOURCES = ("kernels.hip", "gemm_tile.hpp", "comm_units.hpp", "device_common.hpp", "schedule.hpp",
                  "launch.hpp")
PROFILES = os.path.join(ROOT, "profiles")
EXTRA_WORKLOADS = ("pow2_4k", "llama7b_gate", "concurrent")
CPU_TILES = 1024            # sampled 128x128 output tiles in the CPU baseline (about 10 s)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="g2")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle checks (profiling runs)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--gemm-wgs", type=int, default=0,
                    help="fixed gemm_wgs for the headline workload (no sweep)")
    ap.add_argument("--no-lockstep", action="store_true",
                    help="headline without the GEMM rounds' lockstep (IRIS_FLAG_NO_LOCKSTEP; with "
                         "--gemm-wgs, for comparison runs)")
    ap.add_argument("--kernel-hash", action="store_true", help="print the kernel source hash and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--square-gemm", type=int, default=0, metavar="N",
                    help="only compare the GEMM-only kernel with torch.matmul (hipBLASLt) on N x N x N "
                         "fp16, --steps launches each")
    ap.add_argument("--gemm-shape", default="", metavar="M,N,K",
                    help="the same comparison on M x N x K (K a multiple of 64), e.g. the g2 shape "
                         "131072,16384,16384")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Case:
    """Inputs, outputs and the step closure of one workload."""

    def __init__(self, name):
        import torch
        import workloads as wl
        import gemm_collective_tile_amd as il
        self.il, self.torch = il, torch
        self.w = w = wl.WORKLOADS[name]
        self.inp = inp = wl.make_inputs(w, seed=0, device="cuda")
        dev = dict(dtype=torch.float16, device="cuda")
        if w.op == "ag_mm":
            self.C = torch.empty(w.M, w.N, **dev)
            self.G = torch.empty(w.M, w.K, **dev)
            self.tune_kw = dict(C=self.C, out=self.G, srcs=inp["shards"], W=w.W, B=inp["B"],
                                bias=inp["bias"], M=w.M, N=w.N, K=w.K_local)
            self.op = il.IRIS_OP_AG_MM
        elif w.op == "mm_rs":
            self.C = torch.empty(w.M, w.N, **dev)
            self.out = torch.empty(w.M, w.N_local, **dev)
            self.tune_kw = dict(C=self.C, out=self.out, A=inp["A"], srcs=inp["partials"], W=w.W,
                                rank=w.rank, B=inp["B"], bias=inp["bias"], M=w.M, N=w.N, K=w.K)
            self.op = il.IRIS_OP_MM_RS
        elif w.op == "concurrent":
            self.C = torch.empty(w.M, w.N, **dev)
            self.out = torch.empty(w.comm_elems, **dev)
            self.tune_kw = dict(C=self.C, out=self.out, A=inp["A"], srcs=inp["comm_in"], W=w.W,
                                B=inp["B"], bias=inp["bias"], M=w.M, N=w.N, K=w.K,
                                comm_elems=w.comm_elems)
            self.op = il.IRIS_OP_CONCURRENT
        else:
            raise ValueError(w.op)
        self.G_wgs = il.iris_grid_size(None, op=self.op)

    def step(self, cfg):
        il, w, inp = self.il, self.w, self.inp
        if w.op == "ag_mm":
            il.iris_ag_mm(self.C, self.G, inp["shards"], inp["B"], inp["bias"], config=cfg)
        elif w.op == "mm_rs":
            il.iris_mm_rs_local(self.out, self.C, inp["A"], inp["B"], inp["partials"], w.W, rank=w.rank,
                                bias=inp["bias"], config=cfg)
        else:
            il.iris_concurrent(self.C, inp["A"], inp["B"], self.out, inp["comm_in"], bias=inp["bias"],
                               config=cfg)

    def sweep_candidates(self):
        # the listed fractions {0.5, 0.75, 0.875} of the grid, plus splits that
        # start most workgroups on the copy (1/8, 1/4; for all_gather_matmul
        # also 1) or on the GEMM (G-1);
        # the library adds its static default
        G = self.G_wgs
        fracs = [0.125, 0.25, 0.5, 0.75, 0.875]
        if self.w.op == "concurrent":
            fracs = [0.375, 0.5, 0.625, 0.75, 0.8125, 0.875, 0.9375]
        cands = {max(1, min(G - 1, int(math.floor(f * G)))) for f in fracs}
        cands.add(G - 1)
        if self.w.op == "ag_mm":
            cands.add(1)  # every workgroup but one starts on the copy
        return sorted(cands)


def time_steps(case, cfg, steps, warmup):
    """Wall time per step (host clock, synchronized on both sides) and the mean
    launch duration: HIP events on the op's stream (the stream the library
    launches on) around the whole timed region, divided by the step count.
    Steps are queued back to back, so the event span is the launches plus the
    short gaps between them, with no per-launch event packets in between."""
    torch = case.torch
    for _ in range(warmup):
        case.step(cfg)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        case.step(cfg)
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, a.elapsed_time(b) / steps


def windows(case):
    gs, ge, cs, ce = case.il.iris_last_windows()
    g = (ge - gs) / 1e6 if ge >= 0 and gs >= 0 else None
    c = (ce - cs) / 1e6 if ce >= 0 and cs >= 0 else None
    return g, c


def measure(name, steps, warmup, sweep, fixed_wgs=0, flags=0):
    il = __import__("gemm_collective_tile_amd")
    case = Case(name)
    w = case.w
    Config = il.Config
    best = fixed_wgs or None
    sweep_ms, pred_ms, pred_best = {}, {}, None
    if sweep and not fixed_wgs:
        cands = case.sweep_candidates()
        log(f"[{name}] sweeping gemm_wgs over {cands}")
        best, sweep_ms = il.iris_tune_gemm_wgs(case.op, cands, reps=5, **case.tune_kw)
        shape = {k: v for k, v in case.tune_kw.items() if k in ("W", "rank", "M", "N", "K", "comm_elems")}
        pred_best, pred_ms = il.iris_predict_gemm_wgs(case.op, cands, case.G_wgs, **shape)
    cfg = Config(gemm_wgs=best or 0, flags=flags)
    log(f"[{name}] timing fused mode, gemm_wgs={best}")
    wall_ms, mean_ms = time_steps(case, cfg, steps, warmup)
    case.step(cfg)
    gwin, cwin = windows(case)
    clock_mhz = il.iris_last_clock()
    log(f"[{name}] timing sequential mode")
    seq_cfg = Config(mode=il.IRIS_MODE_SEQUENTIAL, flags=flags)
    case.step(seq_cfg)
    case.step(seq_cfg)
    sgwin, scwin = windows(case)
    # the same comm kernel with the last-level cache (256 MiB) flushed first:
    # the warm figure above reads inputs that earlier steps left cached
    torch = case.torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(5):
        flush.fill_(1)
        case.step(seq_cfg)
        torch.cuda.synchronize()
        cold.append(windows(case)[1])
    del flush
    scwin_cold = statistics.median([c for c in cold if c]) if any(cold) else None
    # fused against sequential in alternating rounds, so that clock drift
    # (the chip's clock falls as it heats under MFMA load) hits both alike;
    # each round's figure is the event-timed mean launch (pair) duration
    n_cmp = max(3, steps // 2)
    fused_r, seq_r = [], []
    for _ in range(3):
        fused_r.append(time_steps(case, cfg, n_cmp, 1)[1])
        seq_r.append(time_steps(case, seq_cfg, n_cmp, 1)[1])
    fused_cmp, seq_cmp = statistics.median(fused_r), statistics.median(seq_r)
    two = None
    if w.op == "concurrent":
        # the independent GEMM + collective also runs as two kernels on two
        # streams; best of a few splits
        two = {}
        G = case.G_wgs
        for gw in sorted({best or (G * 7) // 8, (G * 3) // 4, (G * 7) // 8, (G * 15) // 16}):
            log(f"[{name}] timing two-stream mode, gemm_wgs={gw}")
            two[gw] = round(time_steps(case, Config(mode=il.IRIS_MODE_TWO_STREAM, gemm_wgs=gw),
                                       max(3, steps // 2), 2)[0], 4)
    il.iris_check_device_error()
    flops = w.gemm_flops
    # comm data that fits in the last-level cache stays there between steps:
    # its rates are not HBM rates
    hbm_sized = w.comm_bytes > 2 * MALL_BYTES
    res = {
        "workload": name, "op": w.op, "M": w.M, "N": w.N, "K": w.K, "W": w.W,
        "gemm_wgs": best, "grid": case.G_wgs, "tile": "256x256x64",
        "sweep_ms": {str(k): round(v, 4) for k, v in sweep_ms.items()},
        "predicted_ms": {str(k): round(v, 4) for k, v in pred_ms.items()},
        "predicted_best": pred_best,
        "fused_ms": round(wall_ms, 4), "kernel_ms": round(mean_ms, 4),
        "tflops": round(flops / (wall_ms * 1e-3) / 1e12, 2),
        "kernel_tflops": round(flops / (mean_ms * 1e-3) / 1e12, 2),
        "clock_mhz": round(clock_mhz, 1) if clock_mhz > 0 else None,
        "gemm_window_ms": round(gwin, 4) if gwin else None,
        "comm_window_ms": round(cwin, 4) if cwin else None,
        "comm_bytes": w.comm_bytes,
        "comm_hbm_sized": hbm_sized,
        "comm_gbps": round(w.comm_bytes / (cwin * 1e-3) / 1e9, 1) if cwin else None,
        "sequential_ms": round(seq_cmp, 4),
        "fused_vs_sequential_ms": [round(fused_cmp, 4), round(seq_cmp, 4)],
        "fused_rounds_ms": [round(x, 4) for x in fused_r], "sequential_rounds_ms": [round(x, 4) for x in seq_r],
        "seq_gemm_only_ms": round(sgwin, 4) if sgwin else None,
        "seq_gemm_only_tflops": round(flops / (sgwin * 1e-3) / 1e12, 2) if sgwin else None,
        "seq_comm_only_ms": round(scwin, 4) if scwin else None,
        "seq_comm_only_gbps": round(w.comm_bytes / (scwin * 1e-3) / 1e9, 1) if scwin else None,
        "seq_comm_only_cold_gbps": round(w.comm_bytes / (scwin_cold * 1e-3) / 1e9, 1) if scwin_cold else None,
        "fused_le_sequential": fused_cmp <= seq_cmp,
    }
    if two:
        res["two_stream_ms"] = two
        res["two_stream_best_ms"] = min(two.values())
    res["mfma_frac"] = round(res["kernel_tflops"] / PEAK_FP16_TFLOPS, 4)
    if clock_mhz > 0:
        # the same work against the peak at the clock the chip held
        res["mfma_frac_at_clock"] = round(res["kernel_tflops"] / (PEAK_FP16_TFLOPS * clock_mhz / 2400.0), 4)
    if hbm_sized and res["comm_gbps"]:
        res["comm_hbm_frac"] = round(res["comm_gbps"] / PEAK_HBM_GBPS, 4)
    if hbm_sized and res["seq_comm_only_gbps"]:
        res["seq_comm_only_hbm_frac"] = round(res["seq_comm_only_gbps"] / PEAK_HBM_GBPS, 4)
    if res["seq_comm_only_cold_gbps"]:
        res["seq_comm_only_cold_hbm_frac"] = round(res["seq_comm_only_cold_gbps"] / PEAK_HBM_GBPS, 4)
    return res, case


# ----------------------------------------------------------- oracle checks
# Outside every timed region. Each returns (report dict, ok).

def _tile_checks(C, tiles, ref_fn):
    """Elements outside |d| <= 1e-2 + 1e-2 |ref| over the given 128x128 tiles."""
    import numpy as np
    bad = 0
    M, N = C.shape
    for (r0, c0) in tiles:
        r1, c1 = min(M, r0 + 128), min(N, c0 + 128)
        got = C[r0:r1, c0:c1].float().cpu().numpy().astype(np.float64)
        ref = ref_fn(r0, r1, c0, c1)
        bad += int((~(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))).sum())
    return bad


def _gathered_exact(case, chunk_rows=16384):
    import numpy as np
    import oracle
    G, shards = case.G, case.inp["shards"]
    for r0 in range(0, G.shape[0], chunk_rows):
        r1 = min(G.shape[0], r0 + chunk_rows)
        ref = oracle.all_gather_k([s[r0:r1].cpu().numpy() for s in shards])
        if not np.array_equal(G[r0:r1].cpu().numpy().view(np.uint16), ref):
            return False
    return True


def _ag_tile_ref(case):
    import oracle
    inp, B_cols = case.inp, {}

    def ref(r0, r1, c0, c1):
        if c0 not in B_cols:
            B_cols[c0] = inp["B"][:, c0:c1].contiguous().cpu().numpy()
        return oracle.all_gather_matmul([s[r0:r1].cpu().numpy() for s in inp["shards"]], B_cols[c0],
                                        inp["bias"][c0:c1].cpu().numpy())
    return ref


def oracle_check(case):
    """Checks the fused op's last outputs against the oracle: copies bit for
    bit, floating-point outputs within 1e-2 + 1e-2 |ref|."""
    import numpy as np
    import oracle
    import workloads as wl
    w, inp = case.w, case.inp
    t0 = time.perf_counter()
    rep = {}
    if w.op == "ag_mm":
        if w.gemm_flops <= 2 ** 38:  # pow2_4k: the whole C
            full = oracle.all_gather_matmul([s.cpu().numpy() for s in inp["shards"]], inp["B"].cpu().numpy(),
                                            inp["bias"].cpu().numpy())
            got = case.C.float().cpu().numpy().astype(np.float64)
            rep["C_outside_tol"] = int((~(np.abs(got - full) <= 1e-2 + 1e-2 * np.abs(full))).sum())
            rep["C_checked"] = "all"
        else:
            tiles = wl.sample_tiles(w.M, w.N, 128, 64, seed=0)
            rep["C_outside_tol"] = _tile_checks(case.C, tiles, _ag_tile_ref(case))
            rep["C_checked"] = f"{len(tiles)} sampled 128x128 tiles"
        rep["gathered_bit_exact"] = _gathered_exact(case)
        ok = rep["C_outside_tol"] == 0 and rep["gathered_bit_exact"]
    elif w.op == "mm_rs":
        A, B, bias = inp["A"].cpu().numpy(), inp["B"].cpu().numpy(), inp["bias"].cpu().numpy()
        ref = oracle.matmul_reduce_scatter(A, B, [p.cpu().numpy() for p in inp["partials"]], w.W, rank=w.rank,
                                           bias=bias)
        got = case.out.float().cpu().numpy().astype(np.float64)
        rep["out_outside_tol"] = int((~(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))).sum())
        tiles = wl.sample_tiles(w.M, w.N, 128, 16, seed=0)
        rep["C_outside_tol"] = _tile_checks(
            case.C, tiles, lambda r0, r1, c0, c1: oracle.gemm_bias(A, B, bias, rows=(r0, r1), cols=(c0, c1)))
        rep["C_checked"] = f"{len(tiles)} sampled 128x128 tiles; out: all"
        ok = rep["out_outside_tol"] == 0 and rep["C_outside_tol"] == 0
    else:
        ref = oracle.all_reduce([x.cpu().numpy() for x in inp["comm_in"]])
        got = case.out.float().cpu().numpy().astype(np.float64)
        rep["all_reduce_outside_tol"] = int((~(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))).sum())
        B, bias = inp["B"].cpu().numpy(), inp["bias"].cpu().numpy()
        tiles = wl.sample_tiles(w.M, w.N, 128, 16, seed=0)
        rep["C_outside_tol"] = _tile_checks(
            case.C, tiles,
            lambda r0, r1, c0, c1: oracle.gemm_bias(inp["A"][r0:r1].cpu().numpy(), B, bias, cols=(c0, c1)))
        rep["C_checked"] = f"{len(tiles)} sampled 128x128 tiles; all_reduce: all"
        ok = rep["all_reduce_outside_tol"] == 0 and rep["C_outside_tol"] == 0
    rep["seconds"] = round(time.perf_counter() - t0, 2)
    rep["ok"] = ok
    return rep, ok


def cpu_baseline(case):
    """The oracle on a bounded sample of the headline all_gather_matmul:
    CPU_TILES sampled 128x128 output tiles (fp64 dot products over the whole
    K, plus bias) and the whole gathered buffer, on the CPU share of one GPU.
    Returns the report and whether the GPU output agreed."""
    import numpy as np
    import oracle
    import workloads as wl
    w, inp = case.w, case.inp
    threads = oracle.cpu_share()
    tiles = wl.sample_tiles(w.M, w.N, 128, CPU_TILES, seed=1)
    # operands of the sampled tiles, on the host before the clock starts
    rows = sorted({r0 for r0, _ in tiles})
    cols = sorted({c0 for _, c0 in tiles})
    A_rows = {r0: [s[r0:r0 + 128].cpu().numpy() for s in inp["shards"]] for r0 in rows}
    B_cols = {c0: inp["B"][:, c0:c0 + 128].contiguous().cpu().numpy() for c0 in cols}
    bias = inp["bias"].cpu().numpy()
    shards = [s.cpu().numpy() for s in inp["shards"]]
    log(f"[cpu_baseline] oracle: {len(tiles)} tiles of {w.name} C (K={w.K}) and the full gathered buffer "
        f"on {threads} threads")
    refs = {}
    t0 = time.perf_counter()
    for (r0, c0) in tiles:
        refs[(r0, c0)] = oracle.all_gather_matmul(A_rows[r0], B_cols[c0], bias[c0:c0 + 128], nthreads=threads)
    t_gemm = time.perf_counter() - t0
    t1 = time.perf_counter()
    gathered = oracle.all_gather_k(shards)
    t_gather = time.perf_counter() - t1
    dt = t_gemm + t_gather
    flops = 2 * 128 * 128 * w.K * len(tiles)
    gather_bytes = 4 * w.M * w.K
    bad = 0
    for (r0, c0), ref in refs.items():
        got = case.C[r0:r0 + 128, c0:c0 + 128].float().cpu().numpy().astype(np.float64)
        bad += int((~(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))).sum())
    gathered_ok = bool(np.array_equal(gathered, case.G.cpu().numpy().view(np.uint16)))
    full_s = w.gemm_flops / (flops / t_gemm) + (4 * w.M * w.K) / (gather_bytes / t_gather)
    return {
        "value": round(flops / t_gemm / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{len(tiles)} sampled 128x128 tiles of {w.name} all_gather_matmul C (fp64 dot products over "
                  f"K={w.K} + bias, {flops / 1e9:.1f} GFLOP, {t_gemm:.1f} s) and the full gathered buffer "
                  f"({gather_bytes / 2**30:.0f} GiB moved, {t_gather:.1f} s); cores = the CPU share of one GPU",
        "seconds": round(dt, 2),
        "gather_gbps": round(gather_bytes / t_gather / 1e9, 2),
        "full_problem_s_extrapolated": round(full_s, 1),
    }, bad, gathered_ok


def copy_ceiling():
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes)."""
    import torch
    n = 1 << 29
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(2 * 2 * n / (ms * 1e-3) / 1e9, 1)


def mfma_ceiling():
    """The dense fp16 MFMA rate of this GPU with no memory traffic
    (iris_mfma_ceiling): random operands switching every instruction, as on
    GEMM data, and constant ones; TFLOP/s and the clock each held."""
    import gemm_collective_tile_amd as il
    rt, rm = il.iris_mfma_ceiling(random_operands=True, iters=400000)
    ct, cm = il.iris_mfma_ceiling(random_operands=False, iters=400000)
    return {"random_operands_tflops": round(rt, 1), "random_operands_clock_mhz": round(rm, 1),
            "constant_operands_tflops": round(ct, 1), "constant_operands_clock_mhz": round(cm, 1)}


def strip_comments(src):
    """C++ source without // and /* */ comments and with runs of blank space
    collapsed, so that a comment edit leaves the hash of the code alone."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif src[i] in "\"'":  # string or character literal, copied whole
            q, j = src[i], i + 1
            while j < n and src[j] != q:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gemm_collective_tile_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


# template argument of persistent_kernel<OP, BM, BN> for each op, and the
# prefix of its profile files
KERNEL_OP = {"ag_mm": (1, "ag"), "mm_rs": (2, "rs"), "mm_ar": (3, "ar"), "concurrent": (4, "ar")}


def traffic_file(workload):
    import workloads as wl
    op = wl.WORKLOADS[workload].op if workload in wl.WORKLOADS else "ag_mm"
    return os.path.join(PROFILES, f"persistent_kernel_{KERNEL_OP[op][1]}_{workload}_traffic.txt")


def recorded_traffic(workload):
    """Bytes per launch fetched from beyond L2 plus written, recorded in
    profiles/ for this kernel build, or None. (Recorded at one gemm_wgs; the
    split moves work between queues but not the bytes the op must move.)"""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    return int(kv["traffic_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 29  # 1 GiB of fp16
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "launches": 3}))


def square_gemm(m, n, k, steps):
    """The GEMM-only kernel here against torch.matmul (the vendor library
    GEMM) on the same m x n x k fp16 operands, in one process, each run
    `steps` times back to back (library, ours, library again); prints both
    rates. Ours is the sequential all_gather_matmul of 8 K-shards: its GEMM
    launch is timed from the kernel's own stamps (the copy launch before it
    is excluded; median of the last launch of three back-to-back runs), the
    library's by HIP events."""
    import torch
    import gemm_collective_tile_amd as il
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(m, k, generator=g, device="cuda").to(torch.float16)
    b = (torch.randn(k, n, generator=g, device="cuda") / k ** 0.5).to(torch.float16)
    shards = [t.contiguous() for t in a.split(k // 8, dim=1)]
    bias = torch.zeros(n, dtype=torch.float16, device="cuda")
    C = torch.empty(m, n, dtype=torch.float16, device="cuda")
    G = torch.empty(m, k, dtype=torch.float16, device="cuda")
    seq = il.Config(mode=il.IRIS_MODE_SEQUENTIAL)
    flops = 2 * m * n * k

    def lib():
        for _ in range(2):
            torch.matmul(a, b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def ours():
        gemm = []
        for _ in range(3):  # steps back-to-back launch pairs, then the last GEMM launch's window
            for _ in range(steps):
                il.iris_ag_mm(C, G, shards, b, bias, config=seq)
            gs, ge, _, _ = il.iris_last_windows()
            gemm.append((ge - gs) / 1e6)
        return statistics.median(gemm)

    t_lib0 = lib()
    t_ours = ours()
    t_lib1 = lib()
    il.iris_check_device_error()
    ref = torch.matmul(a, b)
    ok = bool(torch.equal(C, ref)) or float((C.float() - ref.float()).abs().max()) < 1e-2
    print(json.dumps({"gemm_shape": [m, n, k], "torch_matmul_ms": [round(t_lib0, 4), round(t_lib1, 4)],
                      "torch_matmul_tflops": round(flops / (min(t_lib0, t_lib1) * 1e-3) / 1e12, 1),
                      "gemm_only_ms": round(t_ours, 4),
                      "gemm_only_tflops": round(flops / (t_ours * 1e-3) / 1e12, 1),
                      "clock_mhz": round(il.iris_last_clock(), 1), "agrees_with_torch": ok}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the fused ops on a single MI355X; "
              f"--gpus {args.gpus} is not supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.kernel_hash:
        print(kernel_source_hash())
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.square_gemm:
        square_gemm(args.square_gemm, args.square_gemm, args.square_gemm, args.steps)
        return
    if args.gemm_shape:
        m, n, k = (int(x) for x in args.gemm_shape.split(","))
        square_gemm(m, n, k, args.steps)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    failures = []
    import gemm_collective_tile_amd as il
    il_flags = il.IRIS_FLAG_NO_LOCKSTEP if args.no_lockstep else 0
    if args.no_lockstep and not args.gemm_wgs:
        print("--no-lockstep needs --gemm-wgs (the sweep runs with the lockstep)", file=sys.stderr)
        sys.exit(2)
    head, case = measure(args.workload, args.steps, args.warmup, not args.no_sweep, args.gemm_wgs, il_flags)
    if args.no_lockstep:
        head["flags"] = "IRIS_FLAG_NO_LOCKSTEP"
    cpu = None
    if not args.no_check:
        log(f"[{args.workload}] oracle check")
        head["oracle_check"], ok = oracle_check(case)
        if not ok:
            failures.append(args.workload)
    if not args.no_cpu_baseline and case.w.op == "ag_mm":
        cpu, bad, gathered_ok = cpu_baseline(case)
        cpu["C_outside_tol"], cpu["gathered_bit_exact"] = bad, gathered_ok
        if bad or not gathered_ok:
            failures.append(f"{args.workload} (cpu_baseline sample)")
    del case
    torch.cuda.empty_cache()
    ceiling = copy_ceiling()
    log("MFMA ceiling (register operands, no memory traffic)")
    mfma_ceil = mfma_ceiling()
    extra = []
    if not args.headline_only:
        for name in EXTRA_WORKLOADS + ("g2",):
            if name == args.workload:
                continue
            steps = 5 if name == "g2" else max(5, args.steps // 2)
            r, c = measure(name, steps, 2, not args.no_sweep)
            if not args.no_check:
                log(f"[{name}] oracle check")
                r["oracle_check"], ok = oracle_check(c)
                if not ok:
                    failures.append(name)
            extra.append(r)
            del c
            torch.cuda.empty_cache()
    w = head
    wl_name = "all_gather_matmul" if w["op"] == "ag_mm" else w["op"]
    line = {
        "metric": "GEMM TFLOP/s + comm-tile GB/s on 1 MI355X, as fraction of MFMA/HBM peak",
        "value": w["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": w["fused_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{w['workload']} {wl_name} local share (W={w['W']}, M={w['M']}, N={w['N']}, K={w['K']})",
            "mode": "fused", "tile": w["tile"], "gemm_wgs": w["gemm_wgs"], "grid": w["grid"],
            "accumulate": "f32",
        },
        "roofline": {
            "bound": "mfma", "achieved": w["kernel_tflops"], "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": w["mfma_frac"], "traffic": recorded_traffic(w["workload"]),
            "traffic_note": "bytes fetched from beyond L2 (HBM and last-level cache hits) plus bytes written, "
                            "per launch, rocprofv3 FETCH_SIZE/WRITE_SIZE scaled by a plain copy; "
                            + (f"profiles/{os.path.basename(traffic_file(w['workload']))}"
                               if os.path.exists(traffic_file(w["workload"])) else
                               "not recorded in this form for this workload"),
            "kernel": f"persistent_kernel<{KERNEL_OP[w['op']][0]},256,256> (fused {w['op']}), HIP-event mean over "
                      f"{args.steps} back-to-back launches: {w['kernel_ms']} ms",
            "clock_mhz": w["clock_mhz"], "frac_at_clock": w.get("mfma_frac_at_clock"),
            "mfma_ceiling": mfma_ceil,
            "frac_of_ceiling": round(w["kernel_tflops"] / mfma_ceil["random_operands_tflops"], 4),
            "ceiling_note": "mfma_ceiling: iris_mfma_ceiling, MFMAs on register operands with no memory "
                            "traffic; random fp16 operands switching every instruction (as on GEMM data) hold "
                            "the chip at its package power limit, constant ones do not",
        },
        "comm": {
            "gbps": w["comm_gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": w.get("comm_hbm_frac"),
            "window_ms": w["comm_window_ms"], "bytes": w["comm_bytes"],
            "comm_only_gbps": w["seq_comm_only_gbps"], "comm_only_frac": w.get("seq_comm_only_hbm_frac"),
            "comm_only_cold_gbps": w["seq_comm_only_cold_gbps"],
            "copy_ceiling_gbps": ceiling,
            "note": "gbps: fused comm window (per-workgroup stamps); comm_only: the sequential mode's comm "
                    "launch on all CUs (a gather beyond the 256 MiB last-level cache: gather_only_kernel, the "
                    "persistent kernel's copy workgroups alone), inputs left cached by the previous step (warm) "
                    "or after a 512 MiB "
                    "write (cold); copy_ceiling: torch device-to-device copy of 1 GiB (read + write bytes)",
        },
        "sequential_ms": w["sequential_ms"],
        "fused_vs_sequential_ms": w["fused_vs_sequential_ms"],
        "fused_le_sequential": w["fused_le_sequential"],
        "oracle_check": w.get("oracle_check"),
        "cpu_baseline": cpu,
        "detail": head,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    if failures:
        log(f"ERROR: the GPU output disagrees with the oracle on: {', '.join(failures)}")
        sys.exit(1)


if __name__ == "__main__":
    main()
