"""Parity at full sizes for the ops beyond the four bench workloads: the five
collectives beside the 8192^3 GEMM of the concurrent workload (every output
element against the oracle), the concurrent op in sequential and two-stream
mode (bit-identical to fused), matmul_all_reduce at 8192^3 with W=8 and
matmul_all_gather at 4096^3 with W=8 (64 sampled 128x128 tiles against the
oracle, peer blocks bit for bit, schedules bit-identical)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, empty, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
    from gemm_collective_tile_amd import Config
else:
    il = Config = None

TILE = 128


def sampled(M, N, n, seed):
    return wl.sample_tiles(M, N, TILE, n, seed=seed)


@pytest.fixture(scope="module")
def conc():
    w = wl.WORKLOADS["concurrent"]
    inp = wl.make_inputs(w, seed=0, device="cuda")
    note("concurrent inputs: GEMM 8192^3, 8 x 64Mi buffers")
    return w, inp, [host(x) for x in inp["comm_in"]]


def out_len(coll, n, W):
    return {il.IRIS_COLL_ALL_GATHER: W * n, il.IRIS_COLL_REDUCE_SCATTER: n // W}.get(coll, n)


def test_concurrent_full_all_collectives(conc):
    w, inp, hx = conc
    n, W, rank = w.comm_elems, w.W, 3
    C_ref = None
    for name, coll in [("all_gather", il.IRIS_COLL_ALL_GATHER), ("reduce_scatter", il.IRIS_COLL_REDUCE_SCATTER),
                       ("all_to_all", il.IRIS_COLL_ALL_TO_ALL), ("broadcast", il.IRIS_COLL_BROADCAST)]:
        note(f"concurrent full: {name} rank={rank}")
        C = empty((w.M, w.N))
        out = empty((out_len(coll, n, W),))
        il.iris_concurrent(C, inp["A"], inp["B"], out, inp["comm_in"], bias=inp["bias"], collective=coll, rank=rank)
        torch.cuda.synchronize()
        if name == "all_gather":
            assert_bits_equal(out, oracle.all_gather_flat(hx).view(np.float16), name)
        elif name == "reduce_scatter":
            assert_close(out, oracle.reduce_scatter_flat(hx, rank), name)
        elif name == "all_to_all":
            assert_bits_equal(out, oracle.all_to_all_flat(hx, rank).view(np.float16), name)
        else:
            assert_bits_equal(out, oracle.broadcast_flat(hx, rank).view(np.float16), name)
        if C_ref is None:
            C_ref = C
        else:
            assert_bits_equal(C, C_ref, f"GEMM beside {name}")


def test_concurrent_full_modes_bit_identical(conc):
    w, inp, _ = conc
    outs = {}
    for mode_name, cfg in [("fused", Config()), ("sequential", Config(mode=il.IRIS_MODE_SEQUENTIAL)),
                           ("two_stream", Config(mode=il.IRIS_MODE_TWO_STREAM, gemm_wgs=224))]:
        note(f"concurrent full all_reduce, {mode_name}")
        C = empty((w.M, w.N))
        out = empty((w.comm_elems,))
        il.iris_concurrent(C, inp["A"], inp["B"], out, inp["comm_in"], bias=inp["bias"], config=cfg)
        torch.cuda.synchronize()
        outs[mode_name] = (C, out)
    for mode_name in ("sequential", "two_stream"):
        assert_bits_equal(outs[mode_name][0], outs["fused"][0], f"C {mode_name} vs fused")
        assert_bits_equal(outs[mode_name][1], outs["fused"][1], f"all_reduce {mode_name} vs fused")


def test_matmul_all_reduce_8192_w8():
    M = N = K = 8192
    W = 8
    g = wl.Workload("armm", "concurrent", M=M, N=N, K=K, W=1, a_std=1.0, b_std=K ** -0.5, comm_elems=8)
    inp = wl.make_inputs(g, seed=5, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(77)
    parts = [torch.randn(M, N, generator=gen, device="cuda").to(torch.float16) for _ in range(W - 1)]
    G = il.iris_grid_size(None, il.IRIS_OP_MM_AR)
    first = None
    for gw in sorted({G // 2, (7 * G) // 8, G - 1}):
        note(f"matmul_all_reduce 8192^3 W=8 fused gemm_wgs={gw}")
        C = empty((M, N))
        out = empty((M, N))
        il.iris_mm_ar_local(out, C, inp["A"], inp["B"], parts, W, bias=inp["bias"], config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        if first is None:
            first = (C, out)
        else:
            assert_bits_equal(C, first[0], f"C schedule invariance gemm_wgs={gw}")
            assert_bits_equal(out, first[1], f"out schedule invariance gemm_wgs={gw}")
    C, out = first
    bias = host(inp["bias"])
    for (r0, c0) in sampled(M, N, 64, seed=3):
        r1, c1 = min(M, r0 + TILE), min(N, c0 + TILE)
        A_t = host(inp["A"][r0:r1].contiguous())
        B_t = host(inp["B"][:, c0:c1].contiguous())
        P_t = [host(p[r0:r1, c0:c1].contiguous()) for p in parts]
        ref = oracle.matmul_all_reduce(A_t, B_t, P_t, W, bias=bias[c0:c1])
        assert_close(out[r0:r1, c0:c1], ref, f"out tile ({r0},{c0})")
        assert_close(C[r0:r1, c0:c1], oracle.gemm_bias(A_t, B_t, bias[c0:c1]), f"C tile ({r0},{c0})")


def test_matmul_all_gather_4096_w8():
    M = N = K = 4096
    W, rank = 8, 3
    g = wl.Workload("mmag", "concurrent", M=M, N=N, K=K, W=1, a_std=1.0, b_std=K ** -0.5, comm_elems=8)
    inp = wl.make_inputs(g, seed=9, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(91)
    peers = [torch.randn(M, N, generator=gen, device="cuda").to(torch.float16) for _ in range(W - 1)]
    G = il.iris_grid_size(None, il.IRIS_OP_MM_AG)
    first = None
    for gw in sorted({G // 4, (7 * G) // 8}):
        note(f"matmul_all_gather 4096^3 W=8 rank={rank} fused gemm_wgs={gw}")
        out = empty((M * W, N))
        il.iris_mm_ag_local(out, inp["A"], inp["B"], peers, W, rank, bias=inp["bias"], config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        if first is None:
            first = out
        else:
            assert_bits_equal(out, first, f"schedule invariance gemm_wgs={gw}")
    out = first
    for p in range(W):
        if p == rank:
            continue
        src = peers[p if p < rank else p - 1]
        assert_bits_equal(out[p * M:(p + 1) * M], src, f"peer block {p}")
    bias = host(inp["bias"])
    own = out[rank * M:(rank + 1) * M]
    for (r0, c0) in sampled(M, N, 64, seed=4):
        r1, c1 = min(M, r0 + TILE), min(N, c0 + TILE)
        ref = oracle.gemm_bias(host(inp["A"][r0:r1].contiguous()), host(inp["B"][:, c0:c1].contiguous()),
                               bias[c0:c1])
        assert_close(own[r0:r1, c0:c1], ref, f"own block tile ({r0},{c0})")
