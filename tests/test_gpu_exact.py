"""Bit-exact parity of the HIP path at the pow2_4k shape (M = N = K = 4096,
W = 8, the shape of the pow2_4k row of the performance table in ROCm/iris PR
"Add auto-config selection for fused AG+matmul with 28 tuned HBM buffer
configs").

Integer-exact inputs: A, B, bias, partials and buffers are integers in
{-2..2}. Every partial sum of a dot product is then an integer of magnitude
below 4 K + 2 < 2^24, exact in fp32 and in double, and every output of
magnitude <= 2048 is exact in fp16, so the GPU (any summation order) must be
bit-identical to the oracle (assert_exact checks the range on the drawn
data). This covers all_gather_matmul, matmul_reduce_scatter,
matmul_all_reduce, matmul_all_gather and the GEMM beside an all_reduce
(Iris docs "Fused Communication and Compute Operations"; ROCm/iris PR "Add
iris.concurrent ...").

Closed forms, independent of the oracle's GEMM: with B = I (K = N) the GEMM
returns the gathered A exactly, so C = fp16(A_gathered + bias) rounded once;
with A = 0, C = fp16(bias) = bias. Both are formed here from the oracle's
fp16 codec only.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_exact, empty, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
    from gemm_collective_tile_amd import Config
else:
    il = Config = None

M = N = K = 4096
W = 8


def splits(op):
    """The default split and the ones the benchmark sweep picks for this op."""
    G = il.iris_grid_size(None, op=op)
    return sorted({(7 * G) // 8, 1, G - 1})


def test_all_gather_matmul_integer_exact_pow2_4k():
    w = wl.WORKLOADS["pow2_4k"]
    inp = wl.make_inputs(w, seed=3, device="cuda", integer=True)
    shards = [host(s) for s in inp["shards"]]
    note("oracle: integer all_gather_matmul 4096^3 W=8")
    ref = oracle.all_gather_matmul(shards, host(inp["B"]), host(inp["bias"]))
    gref = oracle.all_gather_k(shards)
    for gw in splits(il.IRIS_OP_AG_MM):
        note(f"integer all_gather_matmul 4096^3 W=8 gemm_wgs={gw}")
        C, G = empty((M, N)), empty((M, K))
        il.iris_ag_mm(C, G, inp["shards"], inp["B"], inp["bias"], config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_exact(C, ref, f"C gemm_wgs={gw}")
        assert_bits_equal(G, gref.view(np.float16), f"gathered gemm_wgs={gw}")
    il.iris_check_device_error()


def test_matmul_reduce_scatter_integer_exact_pow2_4k():
    rank = 5
    w = wl.Workload("rs_int", "mm_rs", M=M, N=N, K=K, W=W, a_std=1.0, b_std=1.0, rank=rank)
    inp = wl.make_inputs(w, seed=4, device="cuda", integer=True)
    A, B, bias = host(inp["A"]), host(inp["B"]), host(inp["bias"])
    parts = [host(p) for p in inp["partials"]]
    note("oracle: integer matmul_reduce_scatter 4096^3 W=8 (slice and full C)")
    ref = oracle.matmul_reduce_scatter(A, B, parts, W, rank=rank, bias=bias)
    cref = oracle.gemm_bias(A, B, bias)
    for gw in splits(il.IRIS_OP_MM_RS):
        note(f"integer matmul_reduce_scatter rank={rank} gemm_wgs={gw}")
        C, out = empty((M, N)), empty((M, N // W))
        il.iris_mm_rs_local(out, C, inp["A"], inp["B"], inp["partials"], W, rank=rank, bias=inp["bias"],
                            config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_exact(out, ref, f"reduce_scatter out gemm_wgs={gw}")
        assert_exact(C, cref, f"C gemm_wgs={gw}")
    il.iris_check_device_error()


def test_matmul_all_reduce_integer_exact_pow2_4k():
    w = wl.Workload("ar_int", "mm_ar", M=M, N=N, K=K, W=W, a_std=1.0, b_std=1.0)
    inp = wl.make_inputs(w, seed=5, device="cuda", integer=True)
    note("oracle: integer matmul_all_reduce 4096^3 W=8")
    ref = oracle.matmul_all_reduce(host(inp["A"]), host(inp["B"]), [host(p) for p in inp["partials"]], W,
                                   bias=host(inp["bias"]))
    for gw in splits(il.IRIS_OP_MM_AR):
        note(f"integer matmul_all_reduce gemm_wgs={gw}")
        C, out = empty((M, N)), empty((M, N))
        il.iris_mm_ar_local(out, C, inp["A"], inp["B"], inp["partials"], W, bias=inp["bias"],
                            config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_exact(out, ref, f"all_reduce out gemm_wgs={gw}")
    il.iris_check_device_error()


def test_concurrent_integer_exact_pow2_4k():
    n = 16 << 20
    w = wl.Workload("conc_int", "concurrent", M=M, N=N, K=K, W=W, a_std=1.0, b_std=1.0, comm_elems=n)
    inp = wl.make_inputs(w, seed=6, device="cuda", integer=True)
    note("oracle: integer GEMM 4096^3 and all_reduce of 8 x 16Mi")
    cref = oracle.gemm_bias(host(inp["A"]), host(inp["B"]), host(inp["bias"]))
    aref = oracle.all_reduce([host(x) for x in inp["comm_in"]])
    for gw in splits(il.IRIS_OP_CONCURRENT):
        note(f"integer concurrent all_reduce gemm_wgs={gw}")
        C, out = empty((M, N)), empty((n,))
        il.iris_concurrent(C, inp["A"], inp["B"], out, inp["comm_in"], bias=inp["bias"],
                           config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_exact(C, cref, f"C gemm_wgs={gw}")
        assert_exact(out, aref, f"all_reduce gemm_wgs={gw}")
    il.iris_check_device_error()


def test_matmul_all_gather_integer_exact_pow2_4k():
    rank = 2
    w = wl.Workload("mmag_int", "mm_ar", M=M, N=N, K=K, W=W, a_std=1.0, b_std=1.0)
    inp = wl.make_inputs(w, seed=7, device="cuda", integer=True)
    peers = inp["partials"]  # W-1 (M, N) integer blocks standing in for the other ranks' results
    note("integer matmul_all_gather rank=2")
    out = empty((M * W, N))
    il.iris_mm_ag_local(out, inp["A"], inp["B"], peers, W, rank=rank, bias=inp["bias"])
    torch.cuda.synchronize()
    hp = [host(p) for p in peers]
    # one oracle call per block of M rows, so that its threads share the GEMM block
    for blk in range(W):
        note(f"oracle: integer matmul_all_gather rows of block {blk}")
        ref = oracle.matmul_all_gather(host(inp["A"]), host(inp["B"]), hp, W, rank=rank, bias=host(inp["bias"]),
                                       rows=(blk * M, (blk + 1) * M))
        assert_exact(out[blk * M:(blk + 1) * M], ref, f"matmul_all_gather out block {blk}")
    il.iris_check_device_error()


def test_identity_B_closed_form_pow2_4k():
    """B = I: C = fp16(A_gathered + bias), bit for bit, for the bench's splits."""
    w = wl.WORKLOADS["pow2_4k"]
    inp = wl.make_inputs(w, seed=8, device="cuda")
    B = torch.eye(K, dtype=torch.float16, device="cuda")
    gathered = oracle.all_gather_k([host(s) for s in inp["shards"]])
    want = oracle.f16_encode(oracle.f16_decode(gathered) + oracle.f16_decode(host(inp["bias"]))[None, :])
    for gw in splits(il.IRIS_OP_AG_MM):
        note(f"all_gather_matmul with B = I, gemm_wgs={gw}")
        C, G = empty((M, N)), empty((M, K))
        il.iris_ag_mm(C, G, inp["shards"], B, inp["bias"], config=Config(gemm_wgs=gw))
        torch.cuda.synchronize()
        assert_bits_equal(C, want.view(np.float16), f"C = fp16(A_gathered + bias), gemm_wgs={gw}")
    il.iris_check_device_error()


def test_zero_A_closed_form_pow2_4k():
    """A = 0: C = bias in every row, bit for bit (all_gather_matmul and the
    reduce_scatter's C)."""
    w = wl.WORKLOADS["pow2_4k"]
    inp = wl.make_inputs(w, seed=9, device="cuda")
    zeros = [torch.zeros_like(s) for s in inp["shards"]]
    want = np.broadcast_to(host(inp["bias"])[None, :], (M, N))
    note("all_gather_matmul with A = 0")
    C, G = empty((M, N)), empty((M, K))
    il.iris_ag_mm(C, G, zeros, inp["B"], inp["bias"])
    torch.cuda.synchronize()
    assert_bits_equal(C, np.ascontiguousarray(want), "C = bias (all_gather_matmul)")
    note("matmul_reduce_scatter with A = 0 and zero partials")
    Az = torch.zeros(M, K, dtype=torch.float16, device="cuda")
    pz = [torch.zeros(M, N // W, dtype=torch.float16, device="cuda") for _ in range(W - 1)]
    C, out = empty((M, N)), empty((M, N // W))
    il.iris_mm_rs_local(out, C, Az, inp["B"], pz, W, rank=3, bias=inp["bias"])
    torch.cuda.synchronize()
    assert_bits_equal(C, np.ascontiguousarray(want), "C = bias (matmul_reduce_scatter)")
    assert_bits_equal(out, np.ascontiguousarray(want[:, 3 * (N // W):4 * (N // W)]), "out = own slice of bias")
    il.iris_check_device_error()
