"""Parity of the concurrent collectives (all_gather, reduce_scatter,
all_to_all, broadcast, all_reduce beside an independent GEMM), the
matmul_all_gather local share, and the two-stream mode, through the C-ABI,
against the CPU oracle. Copies are checked bit for bit, sums within
tolerance and bit-identical across modes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, assert_exact, empty, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
    from gemm_collective_tile_amd import Config
    COLLS = {"all_reduce": il.IRIS_COLL_ALL_REDUCE, "all_gather": il.IRIS_COLL_ALL_GATHER,
             "reduce_scatter": il.IRIS_COLL_REDUCE_SCATTER, "all_to_all": il.IRIS_COLL_ALL_TO_ALL,
             "broadcast": il.IRIS_COLL_BROADCAST}
    MODES = {"fused": il.IRIS_MODE_FUSED, "sequential": il.IRIS_MODE_SEQUENTIAL,
             "two_stream": il.IRIS_MODE_TWO_STREAM}
else:
    il = Config = None
    COLLS, MODES = {}, {}

NAMES = ["all_reduce", "all_gather", "reduce_scatter", "all_to_all", "broadcast"]


def gemm_inputs(M, N, K, seed):
    g = wl.Workload("case", "concurrent", M=M, N=N, K=K, W=1, a_std=1.0, b_std=K ** -0.5, comm_elems=8)
    inp = wl.make_inputs(g, seed=seed)
    return inp["A"].cuda(), inp["B"].cuda(), inp["bias"].cuda()


def comm_buffers(W, n, seed, integer=False):
    gen = torch.Generator().manual_seed(seed)
    if integer:
        return [torch.randint(-40, 40, (n,), generator=gen).to(torch.float16).cuda() for _ in range(W)]
    return [torch.randn(n, generator=gen).to(torch.float16).cuda() for _ in range(W)]


def oracle_comm(name, xs, rank):
    hx = [host(x) for x in xs]
    if name == "all_reduce":
        return oracle.all_reduce(hx)
    if name == "all_gather":
        return oracle.all_gather_flat(hx).view(np.float16)
    if name == "reduce_scatter":
        return oracle.reduce_scatter_flat(hx, rank)
    if name == "all_to_all":
        return oracle.all_to_all_flat(hx, rank).view(np.float16)
    return oracle.broadcast_flat(hx, rank).view(np.float16)


def out_len(name, n, W):
    return {"all_gather": W * n, "reduce_scatter": n // W}.get(name, n)


@pytest.mark.parametrize("name", NAMES)
def test_concurrent_collectives_all_modes(name):
    M, N, K = 320, 256, 200
    A, B, bias = gemm_inputs(M, N, K, seed=21)
    cref = oracle.gemm_bias(host(A), host(B), host(bias))
    for W, rank in [(3, 0), (3, 2), (8, 5), (1, 0)]:
        n = 8 * W * (3 * 8192 + 37)  # several units per buffer and a ragged last one
        xs = comm_buffers(W, n, seed=100 + W + rank)
        ref = oracle_comm(name, xs, rank)
        first = None
        for mode_name, mode in MODES.items():
            for cfg in [Config(mode=mode), Config(mode=mode, block_m=64, block_n=64, comm_chunk=4096)]:
                note(f"concurrent {name} W={W} rank={rank} {mode_name} cfg={cfg}")
                C, out = empty((M, N)), empty((out_len(name, n, W),))
                il.iris_concurrent(C, A, B, out, xs, bias=bias, collective=COLLS[name], rank=rank, config=cfg)
                torch.cuda.synchronize()
                assert_close(C, cref, f"C ({name}, {mode_name})")
                if name in ("all_reduce", "reduce_scatter"):
                    assert_close(out, ref, f"{name} out ({mode_name})")
                    if first is None:
                        first = out
                    else:
                        assert_bits_equal(out, first, f"{name} invariant across modes/units")
                else:
                    assert_bits_equal(out, ref, f"{name} out ({mode_name})")


def test_concurrent_reduce_scatter_integer_exact():
    M, N, K = 128, 128, 64
    A, B, bias = gemm_inputs(M, N, K, seed=22)
    W, n = 4, 8 * 4 * 5000
    xs = comm_buffers(W, n, seed=7, integer=True)
    for rank in range(W):
        out = empty((n // W,))
        C = empty((M, N))
        il.iris_concurrent(C, A, B, out, xs, bias=bias, collective=il.IRIS_COLL_REDUCE_SCATTER, rank=rank)
        torch.cuda.synchronize()
        assert_exact(out, oracle.reduce_scatter_flat([host(x) for x in xs], rank), f"rank {rank}")


def test_concurrent_output_size_checked():
    A, B, bias = gemm_inputs(64, 64, 64, seed=23)
    xs = comm_buffers(2, 1024, seed=8)
    with pytest.raises(ValueError):
        il.iris_concurrent(empty((64, 64)), A, B, empty((1024,)), xs, collective=il.IRIS_COLL_ALL_GATHER)


@pytest.mark.parametrize("tile", [(64, 64), (256, 256), (256, 128)])
def test_mm_ag_local(tile):
    M, N, K = 300, 200, 136
    A, B, bias = gemm_inputs(M, N, K, seed=24)
    for W, rank in [(1, 0), (3, 0), (3, 2), (4, 1)]:
        gen = torch.Generator().manual_seed(W * 10 + rank)
        peers = [torch.randn(M, N, generator=gen).to(torch.float16).cuda() for _ in range(W - 1)]
        ref = oracle.matmul_all_gather(host(A), host(B), [host(p) for p in peers], W, rank=rank, bias=host(bias))
        first = None
        for mode_name, mode in MODES.items():
            note(f"mm_ag tile={tile} W={W} rank={rank} {mode_name}")
            out = empty((M * W, N))
            il.iris_mm_ag_local(out, A, B, peers, W, rank=rank, bias=bias,
                                config=Config(block_m=tile[0], block_n=tile[1], mode=mode))
            torch.cuda.synchronize()
            own = out[rank * M:(rank + 1) * M]
            assert_close(own, ref[rank * M:(rank + 1) * M], f"own block ({mode_name})")
            for q in range(W):
                if q != rank:
                    assert_bits_equal(out[q * M:(q + 1) * M], ref[q * M:(q + 1) * M].astype(np.float16),
                                      f"peer block {q} ({mode_name})")
            if first is None:
                first = out
            else:
                assert_bits_equal(out, first, f"invariant across modes ({mode_name})")


def test_mm_ag_bias_along_m_and_w1_equals_gemm():
    M, N, K = 192, 256, 128
    A, B, _ = gemm_inputs(M, N, K, seed=25)
    bias_m = torch.randn(M, generator=torch.Generator().manual_seed(3)).to(torch.float16).cuda()
    peers = [torch.randn(M, N, generator=torch.Generator().manual_seed(4)).to(torch.float16).cuda()]
    out = empty((2 * M, N))
    il.iris_mm_ag_local(out, A, B, peers, 2, rank=1, bias=bias_m,
                        config=Config(flags=il.IRIS_FLAG_BIAS_ALONG_M))
    torch.cuda.synchronize()
    ref = oracle.matmul_all_gather(host(A), host(B), [host(peers[0])], 2, rank=1, bias=host(bias_m),
                                   bias_along_m=True)
    assert_close(out[M:], ref[M:], "own block, bias along M")
    # W = 1: the output is exactly the concurrent op's GEMM
    out1, C = empty((M, N)), empty((M, N))
    il.iris_mm_ag_local(out1, A, B, [], 1, rank=0, bias=bias_m, config=Config(flags=il.IRIS_FLAG_BIAS_ALONG_M))
    xs = [torch.zeros(2048, dtype=torch.float16, device="cuda")]
    il.iris_concurrent(C, A, B, empty((2048,)), xs, bias=bias_m, config=Config(flags=il.IRIS_FLAG_BIAS_ALONG_M))
    torch.cuda.synchronize()
    assert_bits_equal(out1, C, "W=1 matmul_all_gather vs plain GEMM")


def test_two_stream_windows_and_repeats():
    M, N, K = 512, 512, 256
    A, B, bias = gemm_inputs(M, N, K, seed=26)
    xs = comm_buffers(4, 8 * 4 * 20000, seed=9)
    cfg = Config(mode=il.IRIS_MODE_TWO_STREAM)
    C0, o0 = empty((M, N)), empty((xs[0].numel(),))
    il.iris_concurrent(C0, A, B, o0, xs, bias=bias, config=cfg)
    torch.cuda.synchronize()
    gs, ge, cs, ce = il.iris_last_windows()
    note(f"two-stream windows ns: gemm [{gs:.0f}, {ge:.0f}] comm [{cs:.0f}, {ce:.0f}]")
    assert ge > gs >= 0 and ce > cs >= 0
    for i in range(4):
        C, o = empty((M, N)), empty((xs[0].numel(),))
        il.iris_concurrent(C, A, B, o, xs, bias=bias, config=cfg)
        torch.cuda.synchronize()
        assert_bits_equal(C, C0, f"repeat {i} C")
        assert_bits_equal(o, o0, f"repeat {i} all_reduce")
