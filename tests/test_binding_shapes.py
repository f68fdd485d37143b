"""The Python binding checks every list length and tensor shape against the
M, N, K, W the library derives before it takes a single pointer, so a
caller's shape mistake raises ValueError instead of becoming an out-of-bounds
access in a kernel.

CPU tensors are used on purpose: a correctly shaped call then fails only at
the device check ("must be on a GPU"), which proves the shape checks ran
first and passed, and that nothing was launched.
"""
import pytest
import torch

import gemm_collective_tile_amd as il

F16 = dict(dtype=torch.float16)


def z(*shape):
    return torch.zeros(*shape, **F16)


def expect_shape_error(fn, what):
    with pytest.raises(ValueError) as ei:
        fn()
    msg = str(ei.value)
    assert "on a GPU" not in msg, f"{what}: reached the device check: {msg}"
    return msg


def expect_device_error(fn):
    with pytest.raises(ValueError, match="on a GPU"):
        fn()


# ------------------------------------------------------------ all_gather_matmul
M, N, KL, W = 32, 48, 16, 4


def ag(C=None, G=None, shards=None, B=None, bias=None, config=None):
    C = z(M, N) if C is None else C
    G = z(M, W * KL) if G is None else G
    shards = [z(M, KL) for _ in range(W)] if shards is None else shards
    B = z(W * KL, N) if B is None else B
    return lambda: il.iris_ag_mm(C, G, shards, B, bias, config=config)


def test_ag_mm_good_shapes_reach_the_device_check():
    expect_device_error(ag())
    expect_device_error(ag(bias=z(N)))
    expect_device_error(ag(bias=z(M), config=il.Config(flags=il.IRIS_FLAG_BIAS_ALONG_M)))
    expect_device_error(ag(bias=z(M), config={"flags": il.IRIS_FLAG_BIAS_ALONG_M}))


@pytest.mark.parametrize("case", ["C", "G", "shard", "shard_rows", "B_rows", "B_cols", "bias", "bias_m",
                                  "no_shards", "too_many"])
def test_ag_mm_shape_mismatch_raises(case):
    bad = {
        "C": ag(C=z(M, N + 8)),
        "G": ag(G=z(M, (W - 1) * KL)),
        "shard": ag(shards=[z(M, KL)] * (W - 1) + [z(M, KL + 8)]),
        "shard_rows": ag(shards=[z(M, KL)] * (W - 1) + [z(M - 1, KL)]),
        "B_rows": ag(B=z((W - 1) * KL, N)),
        "B_cols": ag(B=z(W * KL, N + 8)),
        "bias": ag(bias=z(N - 8)),
        "bias_m": ag(bias=z(N), config=il.Config(flags=il.IRIS_FLAG_BIAS_ALONG_M)),
        "no_shards": ag(shards=[]),
        "too_many": ag(shards=[z(M, KL)] * (il.IRIS_MAX_W + 1), G=z(M, (il.IRIS_MAX_W + 1) * KL),
                       B=z((il.IRIS_MAX_W + 1) * KL, N)),
    }[case]
    expect_shape_error(bad, case)


# -------------------------------------------------------- reduce_scatter / all_reduce
K = 24


def rs(out=None, C=None, A=None, B=None, partials=None, W_=W, bias=None):
    nl = N // W
    out = z(M, nl) if out is None else out
    C = z(M, N) if C is None else C
    A = z(M, K) if A is None else A
    B = z(K, N) if B is None else B
    partials = [z(M, nl) for _ in range(W - 1)] if partials is None else partials
    return lambda: il.iris_mm_rs_local(out, C, A, B, partials, W_, bias=bias)


def ar(out=None, C=None, partials=None, W_=W):
    out = z(M, N) if out is None else out
    C = z(M, N) if C is None else C
    partials = [z(M, N) for _ in range(W - 1)] if partials is None else partials
    return lambda: il.iris_mm_ar_local(out, C, z(M, K), z(K, N), partials, W_)


def test_rs_ar_good_shapes_reach_the_device_check():
    expect_device_error(rs())
    expect_device_error(rs(bias=z(N)))
    expect_device_error(ar())


@pytest.mark.parametrize("case", ["out", "C", "B_rows", "partials_short", "partials_long", "partial_shape",
                                  "N_not_divisible", "W_zero", "bias"])
def test_rs_shape_mismatch_raises(case):
    nl = N // W
    bad = {
        "out": rs(out=z(M, N)),
        "C": rs(C=z(M, nl)),
        "B_rows": rs(B=z(K + 8, N)),
        "partials_short": rs(partials=[z(M, nl)] * (W - 2)),
        "partials_long": rs(partials=[z(M, nl)] * W),
        "partial_shape": rs(partials=[z(M, nl)] * (W - 2) + [z(M, N)]),
        "N_not_divisible": rs(W_=5, partials=[z(M, nl)] * 4),
        "W_zero": rs(W_=0, partials=[]),
        "bias": rs(bias=z(nl)),
    }[case]
    expect_shape_error(bad, case)


@pytest.mark.parametrize("case", ["out", "partials_short", "partial_shape"])
def test_ar_shape_mismatch_raises(case):
    bad = {
        "out": ar(out=z(M, N // W)),
        "partials_short": ar(partials=[z(M, N)] * (W - 2)),
        "partial_shape": ar(partials=[z(M, N)] * (W - 2) + [z(M, N // W)]),
    }[case]
    expect_shape_error(bad, case)


# ---------------------------------------------------------------- concurrent
n = 64


def conc(C=None, comm_out=None, comm_in=None, coll=il.IRIS_COLL_ALL_REDUCE):
    C = z(M, N) if C is None else C
    comm_in = [z(n) for _ in range(W)] if comm_in is None else comm_in
    if comm_out is None:
        comm_out = z({il.IRIS_COLL_ALL_GATHER: W * n, il.IRIS_COLL_REDUCE_SCATTER: n // W}.get(coll, n))
    return lambda: il.iris_concurrent(C, z(M, K), z(K, N), comm_out, comm_in, collective=coll)


@pytest.mark.parametrize("coll", [il.IRIS_COLL_ALL_REDUCE, il.IRIS_COLL_ALL_GATHER, il.IRIS_COLL_REDUCE_SCATTER,
                                  il.IRIS_COLL_ALL_TO_ALL, il.IRIS_COLL_BROADCAST])
def test_concurrent_good_shapes_reach_the_device_check(coll):
    expect_device_error(conc(coll=coll))


@pytest.mark.parametrize("case", ["C", "comm_out", "comm_in_len", "gather_out"])
def test_concurrent_shape_mismatch_raises(case):
    bad = {
        "C": conc(C=z(M + 1, N)),
        "comm_out": conc(comm_out=z(n + 8)),
        "comm_in_len": conc(comm_in=[z(n)] * (W - 1) + [z(n + 8)]),
        "gather_out": conc(comm_out=z(n), coll=il.IRIS_COLL_ALL_GATHER),
    }[case]
    expect_shape_error(bad, case)


# ---------------------------------------------------------- matmul_all_gather
def mmag(out=None, peers=None, W_=W):
    out = z(M * W, N) if out is None else out
    peers = [z(M, N) for _ in range(W - 1)] if peers is None else peers
    return lambda: il.iris_mm_ag_local(out, z(M, K), z(K, N), peers, W_, rank=1)


def test_mm_ag_shapes():
    expect_device_error(mmag())
    expect_shape_error(mmag(out=z(M * (W - 1), N)), "out")
    expect_shape_error(mmag(peers=[z(M, N)] * (W - 2)), "peers short")
    expect_shape_error(mmag(peers=[z(M, N)] * (W - 2) + [z(M, N - 8)]), "peer shape")


def test_tune_validates_before_marshalling():
    with pytest.raises(ValueError, match="A_shards holds"):
        il.iris_tune_gemm_wgs(il.IRIS_OP_AG_MM, [1], C=z(M, N), out=z(M, W * KL), srcs=[z(M, KL)] * (W - 1),
                              W=W, B=z(W * KL, N), M=M, N=N, K=KL)
