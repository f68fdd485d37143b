"""Benchmark of one GPU's share of the fused communication + GEMM ops on MI355X.

One step = one call of the fused op on the headline workload (default
pow2_4k all_gather_matmul: W=8 K-shards (4096, 512) gathered into (4096,
4096) and multiplied by B (4096, 4096) plus bias), with every input already
resident in HBM. The gemm_wgs split is swept first (untimed), as the host
sweep does for any shape, then `--warmup` untimed and `--steps` timed steps
run. Prints ONE JSON line.

  value      GEMM TFLOP/s of the whole fused op: 2*M*N*K / (wall time per step)
  roofline   the fused persistent kernel against the dense fp16 MFMA peak:
             2*M*N*K / (average kernel duration from HIP events around each
             launch on the op's stream). `traffic` is the kernel's HBM bytes
             per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by
             what the same counters read for a plain device copy; it is read
             from profiles/ and reported only while the kernel sources still
             hash to the value recorded there (else null)
  comm       the communication units' HBM GB/s over their in-kernel window
  cpu_baseline  the CPU oracle on the full headline problem (gather + GEMM +
             bias in fp64) on the host's cores; also checks the GPU output
  extra      the other workloads (llama7b_gate reduce_scatter, concurrent
             8192^3 GEMM beside an all_reduce, g2 all_gather_matmul) measured
             the same way, unless --headline-only

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
KERNEL_SOURCES = ("kernels.hip", "gemm_tile.hpp", "comm_units.hpp", "device_common.hpp", "schedule.hpp",
                  "launch.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "persistent_kernel_ag_pow2_4k_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="pow2_4k")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--gemm-wgs", type=int, default=0,
                    help="fixed gemm_wgs for the headline workload (no sweep)")
    ap.add_argument("--kernel-hash", action="store_true", help="print the kernel source hash and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter scaling)")
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


def measure(name, steps, warmup, sweep, fixed_wgs=0):
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
    cfg = Config(gemm_wgs=best or 0)
    log(f"[{name}] timing fused mode, gemm_wgs={best}")
    wall_ms, mean_ms = time_steps(case, cfg, steps, warmup)
    case.step(cfg)
    gwin, cwin = windows(case)
    log(f"[{name}] timing sequential mode")
    seq_cfg = Config(mode=il.IRIS_MODE_SEQUENTIAL)
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
    flops = w.gemm_flops
    res = {
        "workload": name, "op": w.op, "M": w.M, "N": w.N, "K": w.K, "W": w.W,
        "gemm_wgs": best, "grid": case.G_wgs, "tile": "256x256x64",
        "sweep_ms": {str(k): round(v, 4) for k, v in sweep_ms.items()},
        "predicted_ms": {str(k): round(v, 4) for k, v in pred_ms.items()},
        "predicted_best": pred_best,
        "fused_ms": round(wall_ms, 4), "kernel_ms": round(mean_ms, 4),
        "tflops": round(flops / (wall_ms * 1e-3) / 1e12, 2),
        "kernel_tflops": round(flops / (mean_ms * 1e-3) / 1e12, 2),
        "gemm_window_ms": round(gwin, 4) if gwin else None,
        "comm_window_ms": round(cwin, 4) if cwin else None,
        "comm_bytes": w.comm_bytes,
        "comm_gbps": round(w.comm_bytes / (cwin * 1e-3) / 1e9, 1) if cwin else None,
        "sequential_ms": round(seq_cmp, 4),
        "fused_vs_sequential_ms": [round(fused_cmp, 4), round(seq_cmp, 4)],
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
    if res["comm_gbps"]:
        res["comm_hbm_frac"] = round(res["comm_gbps"] / PEAK_HBM_GBPS, 4)
    if res["seq_comm_only_gbps"]:
        res["seq_comm_only_hbm_frac"] = round(res["seq_comm_only_gbps"] / PEAK_HBM_GBPS, 4)
    return res, case


def cpu_baseline(case):
    """The oracle on the full headline problem; returns the report and the
    number of output elements outside tolerance when compared to the GPU."""
    import numpy as np
    import oracle
    w = case.w
    threads = min(16, len(os.sched_getaffinity(0)))
    shards = [s.cpu().numpy() for s in case.inp["shards"]]
    B = case.inp["B"].cpu().numpy()
    bias = case.inp["bias"].cpu().numpy()
    log(f"[cpu_baseline] oracle all_gather_matmul {w.M}x{w.N}x{w.K} on {threads} threads")
    t0 = time.perf_counter()
    ref = oracle.all_gather_matmul(shards, B, bias, nthreads=threads)
    dt = time.perf_counter() - t0
    got = case.C.float().cpu().numpy().astype(np.float64)
    bad = int((~(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))).sum())
    gathered_ok = bool(np.array_equal(oracle.all_gather_k(shards), case.G.cpu().numpy().view(np.uint16)))
    return {
        "value": round(w.gemm_flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"full {w.name} all_gather_matmul (gather + {w.M}x{w.N}x{w.K} GEMM + bias, fp64), "
                  f"{dt:.1f} s",
        "seconds": round(dt, 2),
    }, bad, gathered_ok


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


def recorded_traffic(workload):
    """HBM bytes per launch recorded in profiles/ for this kernel build, or None.
    (Recorded at one gemm_wgs; the split moves work between queues but not the
    bytes the launch moves.)"""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
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
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    head, case = measure(args.workload, args.steps, args.warmup, not args.no_sweep, args.gemm_wgs)
    cpu = None
    if not args.no_cpu_baseline and case.w.op == "ag_mm" and case.w.gemm_flops <= 2 ** 38:
        cpu, bad, gathered_ok = cpu_baseline(case)
        head["oracle_check"] = {"C_outside_tol": bad, "gathered_bit_exact": gathered_ok}
        if bad or not gathered_ok:
            log(f"ERROR: GPU output disagrees with the oracle ({bad} elements, gathered {gathered_ok})")
    del case
    torch.cuda.empty_cache()
    extra = []
    if not args.headline_only:
        for name in ("llama7b_gate", "concurrent", "g2"):
            if name == args.workload:
                continue
            steps = 5 if name == "g2" else max(5, args.steps // 2)
            r, c = measure(name, steps, 2, not args.no_sweep)
            extra.append(r)
            del c
            torch.cuda.empty_cache()
    w = head
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
            "workload": f"{w['workload']} {'all_gather_matmul' if w['op'] == 'ag_mm' else w['op']} local share "
                        f"(W={w['W']}, M={w['M']}, N={w['N']}, K={w['K']})",
            "mode": "fused", "tile": w["tile"], "gemm_wgs": w["gemm_wgs"], "grid": w["grid"],
            "accumulate": "f32",
        },
        "roofline": {
            "bound": "mfma", "achieved": w["kernel_tflops"], "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": w["mfma_frac"], "traffic": recorded_traffic(w["workload"]),
            "kernel": f"persistent_kernel<1,256,256> (fused {w['op']}), HIP-event mean over {args.steps} "
                      f"back-to-back launches: {w['kernel_ms']} ms",
        },
        "comm": {
            "gbps": w["comm_gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": w.get("comm_hbm_frac"),
            "window_ms": w["comm_window_ms"], "bytes": w["comm_bytes"],
            "comm_only_gbps": w["seq_comm_only_gbps"], "comm_only_frac": w.get("seq_comm_only_hbm_frac"),
            "comm_only_cold_gbps": w["seq_comm_only_cold_gbps"],
            "note": "gbps: fused comm window; comm_only: sequential comm kernel over all CUs, inputs left in "
                    "the last-level cache by the previous step (warm) or flushed by a 512 MiB write (cold)",
        },
        "sequential_ms": w["sequential_ms"],
        "fused_le_sequential": w["fused_le_sequential"],
        "cpu_baseline": cpu,
        "detail": head,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
