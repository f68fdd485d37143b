"""Parity at the full workload sizes, in the launch configurations bench.py
times (default 256x256 tiles; the gemm_wgs candidates of its sweep, or at
least the split it picks, compared bit for bit with the default split).

pow2_4k's C is checked in full against the oracle; the larger GEMM outputs
on 64 sampled 128x128 tiles (always including the first and the last)
computed one by one by the oracle; the copy and reduce outputs over the whole
buffer: the gathered buffer bit for bit, the reduce_scatter slice and the
all_reduce output within tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, assert_same_bits, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
    from gemm_collective_tile_amd import Config
else:
    il = None
    Config = None

TILE = 128
NTILES = 64


def sweep_candidates(ag=True):
    """The splits bench.py's sweep tries: the fractions {0.5, 0.75, 0.875} of
    the grid the pow2_4k configuration lists, 1/8, 1/4, G-1 and, for
    all_gather_matmul, 1."""
    G = il.iris_grid_size(None)
    c = {max(1, min(G - 1, int(math.floor(f * G)))) for f in (0.125, 0.25, 0.5, 0.75, 0.875)}
    c.add(G - 1)
    if ag:
        c.add(1)
    return sorted(c)


def check_sampled_tiles(C: torch.Tensor, ref_fn, what: str) -> None:
    M, N = C.shape
    tiles = wl.sample_tiles(M, N, TILE, NTILES, seed=0)
    for (r0, c0) in tiles:
        r1, c1 = min(M, r0 + TILE), min(N, c0 + TILE)
        assert_close(C[r0:r1, c0:c1], ref_fn(r0, r1, c0, c1), f"{what} tile ({r0},{c0})")


def ag_tile_ref(inp):
    B_host = {}

    def ref(r0, r1, c0, c1):
        shards = [host(s[r0:r1]) for s in inp["shards"]]
        if c0 not in B_host:
            B_host[c0] = host(inp["B"][:, c0:c1].contiguous())
        bias = host(inp["bias"][c0:c1])
        return oracle.all_gather_matmul(shards, B_host[c0], bias)
    return ref


def check_gathered(G: torch.Tensor, shards, chunk_rows=8192):
    M = G.shape[0]
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        ref = oracle.all_gather_k([host(s[r0:r1]) for s in shards])
        assert_bits_equal(G[r0:r1], ref.view(np.float16), f"gathered rows {r0}:{r1}")


def test_pow2_4k_all_gather_matmul():
    w = wl.WORKLOADS["pow2_4k"]
    inp = wl.make_inputs(w, seed=0, device="cuda")
    first = None
    for gw in sweep_candidates():
        note(f"pow2_4k fused gemm_wgs={gw}")
        C = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
        G = torch.full((w.M, w.K), float("nan"), dtype=torch.float16, device="cuda")
        il.iris_ag_mm(C, G, inp["shards"], inp["B"], inp["bias"], config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        check_gathered(G, inp["shards"])
        if first is None:
            note("pow2_4k oracle: the full C")
            full = oracle.all_gather_matmul([host(s) for s in inp["shards"]], host(inp["B"]), host(inp["bias"]))
            assert_close(C, full, "pow2_4k C (full)")
            first = C
        else:
            assert_same_bits(C, first, f"schedule invariance gemm_wgs={gw}")


def test_llama7b_gate_reduce_scatter():
    w = wl.WORKLOADS["llama7b_gate"]
    inp = wl.make_inputs(w, seed=0, device="cuda")
    note("llama7b_gate fused reduce_scatter")
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
    out = torch.full((w.M, w.N_local), float("nan"), dtype=torch.float16, device="cuda")
    il.iris_mm_rs_local(out, C, inp["A"], inp["B"], inp["partials"], w.W, rank=w.rank, bias=inp["bias"])
    torch.cuda.synchronize()
    # the split the bench picks for this shape (every workgroup but one
    # starts on the GEMM): bit-identical to the default split
    G = il.iris_grid_size(None, op=il.IRIS_OP_MM_RS)
    note(f"llama7b_gate fused reduce_scatter gemm_wgs={G - 1}")
    C2, out2 = torch.full_like(C, float("nan")), torch.full_like(out, float("nan"))
    il.iris_mm_rs_local(out2, C2, inp["A"], inp["B"], inp["partials"], w.W, rank=w.rank, bias=inp["bias"],
                        config=Config(gemm_wgs=G - 1))
    torch.cuda.synchronize()
    assert_same_bits(out2, out, f"reduce_scatter out, gemm_wgs={G - 1} against the default split")
    assert_same_bits(C2, C, f"C, gemm_wgs={G - 1} against the default split")
    del C2, out2
    A, B, bias = host(inp["A"]), host(inp["B"]), host(inp["bias"])
    note("llama7b_gate oracle: full reduce_scatter slice")
    ref = oracle.matmul_reduce_scatter(A, B, [host(p) for p in inp["partials"]], w.W, rank=w.rank,
                                       bias=bias)
    assert_close(out, ref, "reduce_scatter out (full)")
    check_sampled_tiles(C, lambda r0, r1, c0, c1: oracle.gemm_bias(A, B, bias, rows=(r0, r1), cols=(c0, c1)),
                        "llama7b_gate C")


def test_concurrent_gemm_and_all_reduce():
    w = wl.WORKLOADS["concurrent"]
    inp = wl.make_inputs(w, seed=0, device="cuda")
    note("concurrent fused: GEMM 8192^3 beside all_reduce 8 x 64Mi")
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
    out = torch.full((w.comm_elems,), float("nan"), dtype=torch.float16, device="cuda")
    il.iris_concurrent(C, inp["A"], inp["B"], out, inp["comm_in"], bias=inp["bias"])
    torch.cuda.synchronize()
    # other splits of the bench's sweep for this op: bit-identical results
    G = il.iris_grid_size(None, op=il.IRIS_OP_CONCURRENT)
    for gw in ((G * 13) // 16, (G * 15) // 16):
        note(f"concurrent fused gemm_wgs={gw}")
        C2, out2 = torch.full_like(C, float("nan")), torch.full_like(out, float("nan"))
        il.iris_concurrent(C2, inp["A"], inp["B"], out2, inp["comm_in"], bias=inp["bias"],
                           config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_same_bits(C2, C, f"concurrent C, gemm_wgs={gw} against the default split")
        assert_same_bits(out2, out, f"all_reduce, gemm_wgs={gw} against the default split")
        del C2, out2
    note("concurrent oracle: full all_reduce")
    aref = oracle.all_reduce([host(x) for x in inp["comm_in"]])
    assert_close(out, aref, "all_reduce (full)")
    B_host = host(inp["B"])
    bias = host(inp["bias"])
    check_sampled_tiles(C, lambda r0, r1, c0, c1: oracle.gemm_bias(host(inp["A"][r0:r1]), B_host, bias,
                                                                   cols=(c0, c1)), "concurrent C")


def test_sequential_large_gather_ragged():
    """A gathered buffer beyond the 256 MiB last-level cache takes the
    sequential mode's large-gather path (the persistent kernel's copy
    workgroups alone, then the GEMM-only kernel). Here with W = 3 and ragged
    M, N and K (a 77-row last row block, a 40-column last column block, K not
    a multiple of the 64-deep K step): sequential and fused bit-identical, the
    whole gathered buffer bit-exact, sampled tiles (the ragged corner among
    them) within tolerance of the oracle."""
    K_local = 2824
    w = wl.Workload("ragged_large_gather", "ag_mm", M=16461, N=296, K=3 * K_local, W=3, a_std=1.0,
                    b_std=(3 * K_local) ** -0.5)
    assert w.M * w.K * 2 > 256 << 20
    inp = wl.make_inputs(w, seed=5, device="cuda")
    note("ragged large gather: sequential all_gather_matmul 16461x296x8472, W=3")
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
    G = torch.full((w.M, w.K), float("nan"), dtype=torch.float16, device="cuda")
    il.iris_ag_mm(C, G, inp["shards"], inp["B"], inp["bias"], config=Config(mode=il.IRIS_MODE_SEQUENTIAL))
    torch.cuda.synchronize()
    il.iris_check_device_error()
    note("ragged large gather: fused")
    C2, G2 = torch.full_like(C, float("nan")), torch.full_like(G, float("nan"))
    il.iris_ag_mm(C2, G2, inp["shards"], inp["B"], inp["bias"])
    torch.cuda.synchronize()
    il.iris_check_device_error()
    assert_same_bits(C2, C, "ragged large gather C, fused against sequential")
    assert_same_bits(G2, G, "ragged large gather gathered, fused against sequential")
    del C2, G2
    note("ragged large gather: full gathered buffer, sampled tiles of C")
    check_gathered(G, inp["shards"])
    check_sampled_tiles(C, ag_tile_ref(inp), "ragged large gather C")


def test_g2_all_gather_matmul():
    w = wl.WORKLOADS["g2"]
    inp = wl.make_inputs(w, seed=0, device="cuda")
    note("g2 fused all_gather_matmul 131072x16384x16384")
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
    G = torch.full((w.M, w.K), float("nan"), dtype=torch.float16, device="cuda")
    il.iris_ag_mm(C, G, inp["shards"], inp["B"], inp["bias"])
    torch.cuda.synchronize()
    # the split the bench picks for this shape (every workgroup but one
    # starts on the copy, and joins the GEMM after the whole gather):
    # bit-identical to the default split
    note("g2 fused all_gather_matmul gemm_wgs=1")
    C2, G2 = torch.full_like(C, float("nan")), torch.full_like(G, float("nan"))
    il.iris_ag_mm(C2, G2, inp["shards"], inp["B"], inp["bias"], config=Config(gemm_wgs=1))
    torch.cuda.synchronize()
    assert_same_bits(C2, C, "g2 C, gemm_wgs=1 against the default split")
    assert_same_bits(G2, G, "g2 gathered, gemm_wgs=1 against the default split")
    # sequential mode: the 4 GiB gather runs alone (gather_only_kernel), then
    # the GEMM-only kernel; bit-identical to the fused op
    note("g2 sequential all_gather_matmul")
    C2.fill_(float("nan"))
    G2.fill_(float("nan"))
    il.iris_ag_mm(C2, G2, inp["shards"], inp["B"], inp["bias"], config=Config(mode=il.IRIS_MODE_SEQUENTIAL))
    torch.cuda.synchronize()
    il.iris_check_device_error()
    assert_same_bits(C2, C, "g2 C, sequential against fused")
    assert_same_bits(G2, G, "g2 gathered, sequential against fused")
    del C2, G2
    note("g2: full gathered buffer")
    check_gathered(G, inp["shards"])
    note("g2: 64 sampled tiles of C")
    check_sampled_tiles(C, ag_tile_ref(inp), "g2 C")
