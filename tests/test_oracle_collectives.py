"""Pins of the oracle's matmul_all_gather and flat collectives (all_gather,
reduce_scatter, all_to_all, broadcast) against library formulations,
invariants, the already-pinned GEMM and sum, and hand-computed fixtures."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float16)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


@pytest.mark.parametrize("W,n", [(1, 8), (2, 16), (3, 24), (5, 40), (4, 0)])
def test_all_gather_flat_is_concatenation(W, n):
    xs = [rnd(n, 10 + w) for w in range(W)]
    got = oracle.all_gather_flat(xs)
    assert np.array_equal(got, np.concatenate([bits(x) for x in xs]))


@pytest.mark.parametrize("W,n", [(1, 8), (2, 16), (4, 32), (8, 64)])
def test_all_to_all_matches_block_transpose_and_is_an_involution(W, n):
    xs = [rnd(n, 20 + w) for w in range(W)]
    part = n // W
    # stack (source rank, block, element); rank r receives the r-th block of every source
    T = np.stack([bits(x).reshape(W, part) for x in xs])
    ys = []
    for r in range(W):
        y = oracle.all_to_all_flat(xs, r)
        assert np.array_equal(y, T[:, r, :].reshape(-1))
        ys.append(y.view(np.float16))
    # exchanging twice returns every rank its own buffer
    for r in range(W):
        assert np.array_equal(oracle.all_to_all_flat(ys, r), bits(xs[r]))


@pytest.mark.parametrize("W,n", [(1, 8), (2, 16), (3, 24), (8, 64)])
def test_reduce_scatter_flat_is_the_rank_slice_of_the_sum(W, n):
    xs = [rnd(n, 30 + w) for w in range(W)]
    part = n // W
    full = np.sum(np.stack([x.astype(np.float64) for x in xs]), axis=0)
    pieces = []
    for r in range(W):
        got = oracle.reduce_scatter_flat(xs, r)
        np.testing.assert_allclose(got, full[r * part:(r + 1) * part], rtol=0, atol=1e-12)
        pieces.append(got)
    # the W slices together are the all_reduce
    np.testing.assert_array_equal(np.concatenate(pieces), oracle.sum_buffers(xs))


def test_reduce_scatter_flat_integer_exact():
    rng = np.random.default_rng(3)
    xs = [rng.integers(-50, 50, 64).astype(np.float16) for _ in range(4)]
    got = oracle.reduce_scatter_flat(xs, 3)
    # Python integer sums of the last quarter of every buffer
    want = [sum(int(x[48 + i]) for x in xs) for i in range(16)]
    assert got.tolist() == want


@pytest.mark.parametrize("W", [1, 2, 5])
def test_broadcast_flat_returns_the_root_buffer(W):
    xs = [rnd(24, 40 + w) for w in range(W)]
    for root in range(W):
        assert np.array_equal(oracle.broadcast_flat(xs, root), bits(xs[root]))


@pytest.mark.parametrize("W,rank", [(1, 0), (2, 0), (3, 1), (4, 3)])
def test_matmul_all_gather_blocks(W, rank):
    M, N, K = 5, 7, 6
    A, B, bias = rnd((M, K), 1), rnd((K, N), 2, K ** -0.5), rnd(N, 3, 0.1)
    peers = [rnd((M, N), 50 + p) for p in range(W - 1)]
    got = oracle.matmul_all_gather(A, B, peers, W, rank=rank, bias=bias)
    assert got.shape == (M * W, N)
    # this rank's block is the (pinned) GEMM + bias
    np.testing.assert_array_equal(got[rank * M:(rank + 1) * M], oracle.gemm_bias(A, B, bias))
    # the other blocks are the peers, exactly, in rank order
    others = [q for q in range(W) if q != rank]
    for p, q in enumerate(others):
        np.testing.assert_array_equal(got[q * M:(q + 1) * M], peers[p].astype(np.float64))
    # row sub-ranges agree with the whole
    np.testing.assert_array_equal(oracle.matmul_all_gather(A, B, peers, W, rank=rank, bias=bias,
                                                           rows=(M - 2, M * W - 1)), got[M - 2:M * W - 1])


def test_matmul_all_gather_bias_along_m_and_numpy():
    M, N, K, W, rank = 4, 3, 8, 2, 1
    A, B, bias = rnd((M, K), 4), rnd((K, N), 5), rnd(M, 6)
    got = oracle.matmul_all_gather(A, B, [rnd((M, N), 7)], W, rank=rank, bias=bias, bias_along_m=True)
    ref = A.astype(np.float64) @ B.astype(np.float64) + bias.astype(np.float64)[:, None]
    np.testing.assert_allclose(got[M:], ref, rtol=1e-12, atol=1e-12)


def test_golden_matmul_all_gather():
    g = json.load(open(os.path.join(GOLDEN, "matmul_all_gather_w3_rank1.json")))
    A = np.array(g["A"], np.float16)
    B = np.array(g["B"], np.float16)
    bias = np.array(g["bias"], np.float16)
    peers = [np.array(p, np.float16) for p in g["peers"]]
    got = oracle.matmul_all_gather(A, B, peers, g["W"], rank=g["rank"], bias=bias)
    assert np.array_equal(got, np.array(g["expected"]))


def test_golden_all_to_all():
    g = json.load(open(os.path.join(GOLDEN, "all_to_all_w2.json")))
    bufs = [np.array(b, np.float16) for b in g["bufs"]]
    for r in (0, 1):
        got = oracle.all_to_all_flat(bufs, r).view(np.float16).astype(np.float64)
        assert np.array_equal(got, np.array(g[f"expected_rank{r}"], np.float64))
