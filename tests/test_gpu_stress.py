"""Bounded randomized stress of the fused kernels' flag protocol.

A fixed budget of cases (seeded, so every run draws the same ones), each a
random op (all_gather_matmul, matmul_reduce_scatter, matmul_all_reduce,
GEMM beside an all_reduce, matmul_all_gather), shape (ragged edges
included), GEMM tile, gemm_wgs split, comm unit size, W in {1, 2, 4, 8},
rank and stealing flag. Each fused result must be bit-identical to the same
op in sequential mode (the unfused kernels, no flags) with the same tile,
and within |d| <= 1e-2 + 1e-2 |ref| of the oracle; copies bit-exact. The test
stops at the first mismatch and names the case, and ends with a device-side
error check (no wait may have hit its poll bound).
"""
import random

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, assert_same_bits, empty, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
    from gemm_collective_tile_amd import Config
else:
    il = Config = None

CASES = 48
TILES = [(256, 256), (256, 128), (128, 128), (64, 64)]


def draw_case(rng):
    op = rng.choice(["ag", "rs", "ar", "conc", "mmag"])
    W = rng.choice([1, 2, 4, 8])
    bm, bn = rng.choice(TILES)
    M = rng.randint(1, 1100)
    if op == "rs":
        N = W * 8 * rng.randint(1, max(1, 1100 // (8 * W)))
    else:
        N = 8 * rng.randint(1, 140)
    kl = 8 * rng.randint(1, 48)
    K = kl * W if op == "ag" else 8 * rng.randint(1, 200)
    rank = rng.randrange(W)
    comm_bm = rng.choice([c for c in (1, 2, 4, 8, 16, 32, 64, 128, 256) if c <= bm] + [0])
    flags = il.IRIS_FLAG_NO_STEAL if rng.random() < 0.2 else 0
    return dict(op=op, W=W, bm=bm, bn=bn, M=M, N=N, K=K, kl=kl, rank=rank, comm_bm=comm_bm, flags=flags,
                frac=rng.random(), seed=rng.randrange(1 << 30))


def run_case(c, cfg):
    """Runs the op of case c with config cfg on inputs drawn from its seed;
    returns (device outputs, host inputs for the oracle)."""
    op, W, M, N, K = c["op"], c["W"], c["M"], c["N"], c["K"]
    g = torch.Generator(device="cuda").manual_seed(c["seed"])

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.float16)

    bias = rnd(N, std=0.1)
    if op == "ag":
        shards = [rnd(M, c["kl"]) for _ in range(W)]
        B = rnd(W * c["kl"], N, std=(W * c["kl"]) ** -0.5)
        C, G = empty((M, N)), empty((M, W * c["kl"]))
        il.iris_ag_mm(C, G, shards, B, bias, config=cfg)
        return (C, G), dict(shards=shards, B=B, bias=bias)
    A = rnd(M, K)
    B = rnd(K, N, std=K ** -0.5)
    if op == "rs":
        parts = [rnd(M, N // W) for _ in range(W - 1)]
        C, out = empty((M, N)), empty((M, N // W))
        il.iris_mm_rs_local(out, C, A, B, parts, W, rank=c["rank"], bias=bias, config=cfg)
        return (C, out), dict(A=A, B=B, bias=bias, parts=parts)
    if op == "ar":
        parts = [rnd(M, N) for _ in range(W - 1)]
        C, out = empty((M, N)), empty((M, N))
        il.iris_mm_ar_local(out, C, A, B, parts, W, bias=bias, config=cfg)
        return (C, out), dict(A=A, B=B, bias=bias, parts=parts)
    if op == "conc":
        n = 8 * W * (1 + (c["seed"] % 4096))
        xs = [rnd(n) for _ in range(W)]
        C, out = empty((M, N)), empty((n,))
        il.iris_concurrent(C, A, B, out, xs, bias=bias, config=cfg)
        return (C, out), dict(A=A, B=B, bias=bias, xs=xs)
    peers = [rnd(M, N) for _ in range(W - 1)]
    out = empty((M * W, N))
    il.iris_mm_ag_local(out, A, B, peers, W, rank=c["rank"], bias=bias, config=cfg)
    return (out,), dict(A=A, B=B, bias=bias, peers=peers)


def check_oracle(c, outs, inp):
    h = {k: ([host(x) for x in v] if isinstance(v, list) else host(v)) for k, v in inp.items()}
    op, W = c["op"], c["W"]
    if op == "ag":
        assert_bits_equal(outs[1], oracle.all_gather_k(h["shards"]).view(np.float16), "gathered")
        assert_close(outs[0], oracle.all_gather_matmul(h["shards"], h["B"], h["bias"]), "C")
        return
    if op == "mmag":
        assert_close(outs[0], oracle.matmul_all_gather(h["A"], h["B"], h["peers"], W, rank=c["rank"],
                                                       bias=h["bias"]), "out")
        return
    assert_close(outs[0], oracle.gemm_bias(h["A"], h["B"], h["bias"]), "C")
    if op == "rs":
        ref = oracle.matmul_reduce_scatter(h["A"], h["B"], h["parts"], W, rank=c["rank"], bias=h["bias"])
    elif op == "ar":
        ref = oracle.matmul_all_reduce(h["A"], h["B"], h["parts"], W, bias=h["bias"])
    else:
        ref = oracle.all_reduce(h["xs"])
    assert_close(outs[1], ref, "out")


def test_random_configs_match_sequential_and_oracle():
    rng = random.Random(20261203)
    il.iris_check_device_error()
    for i in range(CASES):
        c = draw_case(rng)
        opid = {"ag": il.IRIS_OP_AG_MM, "rs": il.IRIS_OP_MM_RS, "ar": il.IRIS_OP_MM_AR,
                "conc": il.IRIS_OP_CONCURRENT, "mmag": il.IRIS_OP_MM_AG}[c["op"]]
        G = il.iris_grid_size(Config(block_m=c["bm"], block_n=c["bn"]), op=opid)
        gw = max(1, min(G - 1, int(c["frac"] * G)))
        base = dict(block_m=c["bm"], block_n=c["bn"], comm_block_m=c["comm_bm"], flags=c["flags"])
        note(f"stress case {i}: {c}, gemm_wgs={gw} of {G}")
        fused, inp = run_case(c, Config(gemm_wgs=gw, **base))
        seq, _ = run_case(c, Config(mode=il.IRIS_MODE_SEQUENTIAL, **base))
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(fused, seq)):
            assert_same_bits(a, b, f"case {i} output {k}: fused vs sequential")
        check_oracle(c, fused, inp)
        del fused, seq, inp
    il.iris_check_device_error()
