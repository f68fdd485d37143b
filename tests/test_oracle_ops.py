"""Pins for the oracle's GEMM and collective arithmetic (CPU only).

Each pin checks the oracle against something other than itself:
  - exact rational arithmetic (fractions.Fraction) on tiny inputs,
  - Python integer arithmetic on integer-valued inputs,
  - numpy's float64 matmul / concatenate (library routines),
  - closed forms: B = I, A = 0, W = 1, all-equal and all-zero partials,
  - invariants: region slices, permutation of partials.
Shapes are deliberately non-square so that a transposed operand, a swapped
index, a wrong shard order, a wrong rank slice or the bias on the wrong axis
changes the result.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(20260101)


def f16(shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float16)


def ints(shape, lo=-2, hi=2):
    return RNG.integers(lo, hi + 1, size=shape).astype(np.float16)


def exact_gemm(A, B, bias=None, along_m=False):
    """Exact rational A @ B + bias (pure Python, tiny sizes only)."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(A[m, k])) for k in range(K)] for m in range(M)]
    Bf = [[Fraction(float(B[k, n])) for n in range(N)] for k in range(K)]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            s = sum((Af[m][k] * Bf[k][n] for k in range(K)), Fraction(0))
            if bias is not None:
                s += Fraction(float(bias[m if along_m else n]))
            row.append(s)
        out.append(row)
    return out


def assert_close_exact(got, exact, rel=1e-14):
    """|got - exact| within a few double ulps of the sum of magnitudes."""
    for i, row in enumerate(exact):
        for j, v in enumerate(row):
            err = abs(Fraction(float(got[i, j])) - v)
            assert err <= Fraction(rel) * (abs(v) + 1), (i, j, float(got[i, j]), float(v))


# ----------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 5, 2), (4, 7, 6), (6, 3, 5)])
@pytest.mark.parametrize("along_m", [False, True])
def test_gemm_bias_brute_force(M, K, N, along_m):
    A, B = f16((M, K)), f16((K, N))
    bias = f16((M if along_m else N,), 0.1)
    got = oracle.gemm_bias(A, B, bias, bias_along_m=along_m)
    assert_close_exact(got, exact_gemm(A, B, bias, along_m))


def test_gemm_no_bias_brute_force():
    A, B = f16((5, 9)), f16((9, 4))
    assert_close_exact(oracle.gemm_bias(A, B, None), exact_gemm(A, B))


@pytest.mark.parametrize("M,K,N", [(37, 53, 29), (64, 136, 48), (17, 256, 96)])
def test_gemm_integer_exact(M, K, N):
    A, B, bias = ints((M, K)), ints((K, N)), ints((N,))
    got = oracle.gemm_bias(A, B, bias)
    Ai = A.astype(np.int64)
    Bi = B.astype(np.int64)
    want = Ai @ Bi + bias.astype(np.int64)[None, :]
    assert np.array_equal(got, want.astype(np.float64))


@pytest.mark.parametrize("M,K,N", [(37, 53, 29), (130, 200, 70)])
def test_gemm_matches_numpy_float64(M, K, N):
    A, B, bias = f16((M, K)), f16((K, N), 0.1), f16((N,), 0.1)
    got = oracle.gemm_bias(A, B, bias, nthreads=3)
    ref = A.astype(np.float64) @ B.astype(np.float64) + bias.astype(np.float64)
    mag = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)) + 1
    assert np.all(np.abs(got - ref) <= 1e-13 * mag)


def test_gemm_region_is_slice_of_full():
    A, B, bias = f16((50, 40)), f16((40, 60)), f16((50,), 0.1)
    full = oracle.gemm_bias(A, B, bias, bias_along_m=True)
    part = oracle.gemm_bias(A, B, bias, bias_along_m=True, rows=(7, 33), cols=(11, 59))
    assert np.array_equal(part, full[7:33, 11:59])


def test_gemm_identity_and_zero_closed_forms():
    M, K = 24, 32
    A, bias = f16((M, K)), f16((K,), 0.1)
    eye = np.eye(K, dtype=np.float16)
    got = oracle.gemm_bias(A, eye, bias)
    assert np.array_equal(got, A.astype(np.float64) + bias.astype(np.float64)[None, :])
    zeros = np.zeros((M, K), np.float16)
    B = f16((K, 20))
    b20 = f16((20,), 0.1)
    got0 = oracle.gemm_bias(zeros, B, b20)
    assert np.array_equal(got0, np.broadcast_to(b20.astype(np.float64), (M, 20)))


def test_gemm_threads_do_not_change_bits():
    A, B, bias = f16((70, 90)), f16((90, 33)), f16((33,))
    a = oracle.gemm_bias(A, B, bias, nthreads=1)
    b = oracle.gemm_bias(A, B, bias, nthreads=7)
    assert np.array_equal(a, b)


# ----------------------------------------------------------- all_gather

def test_all_gather_matches_numpy_concatenate():
    shards = [f16((9, 16)) for _ in range(3)]
    got = oracle.all_gather_k(shards)
    want = np.concatenate(shards, axis=1).view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("along_m", [False, True])
def test_all_gather_matmul_brute_force(along_m):
    W, M, kl, N = 3, 5, 2, 4
    shards = [f16((M, kl)) for _ in range(W)]
    B = f16((W * kl, N))
    bias = f16((M if along_m else N,), 0.1)
    got = oracle.all_gather_matmul(shards, B, bias, bias_along_m=along_m)
    assert_close_exact(got, exact_gemm(np.concatenate(shards, 1), B, bias, along_m))


def test_all_gather_matmul_region_with_row_offset():
    W, M, kl, N = 2, 12, 8, 10
    shards = [f16((M, kl)) for _ in range(W)]
    B, bias = f16((W * kl, N)), f16((M,), 0.1)
    full = oracle.all_gather_matmul(shards, B, bias, bias_along_m=True)
    part = oracle.all_gather_matmul(shards, B, bias, bias_along_m=True, rows=(5, 11), cols=(3, 9))
    assert np.array_equal(part, full[5:11, 3:9])
    exact = exact_gemm(np.concatenate(shards, 1)[5:11], B[:, 3:9], bias[5:11], True)
    assert_close_exact(part, exact)


def test_all_gather_matmul_w1_is_plain_gemm():
    A, B, bias = f16((33, 40)), f16((40, 24)), f16((24,))
    assert np.array_equal(oracle.all_gather_matmul([A], B, bias), oracle.gemm_bias(A, B, bias))


def test_all_gather_matmul_integer_exact():
    W, M, kl, N = 8, 40, 16, 24
    shards = [ints((M, kl)) for _ in range(W)]
    B, bias = ints((W * kl, N)), ints((N,))
    got = oracle.all_gather_matmul(shards, B, bias)
    A = np.concatenate(shards, 1).astype(np.int64)
    want = A @ B.astype(np.int64) + bias.astype(np.int64)
    assert np.array_equal(got, want.astype(np.float64))


# -------------------------------------------------------- reduce_scatter

@pytest.mark.parametrize("rank", [0, 1, 2])
def test_reduce_scatter_brute_force(rank):
    W, M, K, N = 3, 4, 5, 6
    A, B, bias = f16((M, K)), f16((K, N)), f16((N,), 0.1)
    nl = N // W
    parts = [f16((M, nl)) for _ in range(W - 1)]
    got = oracle.matmul_reduce_scatter(A, B, parts, W, rank=rank, bias=bias)
    own = exact_gemm(A, B[:, rank * nl:(rank + 1) * nl], bias[rank * nl:(rank + 1) * nl])
    exact = [[own[m][j] + sum(Fraction(float(p[m, j])) for p in parts) for j in range(nl)]
             for m in range(M)]
    assert_close_exact(got, exact)


def test_reduce_scatter_integer_exact_and_rows():
    W, M, K, N, rank = 8, 24, 64, 64, 5
    A, B, bias = ints((M, K)), ints((K, N)), ints((N,))
    nl = N // W
    parts = [ints((M, nl)) for _ in range(W - 1)]
    want = (A.astype(np.int64) @ B.astype(np.int64) + bias.astype(np.int64))[:, rank * nl:(rank + 1) * nl]
    want = want + sum(p.astype(np.int64) for p in parts)
    got = oracle.matmul_reduce_scatter(A, B, parts, W, rank=rank, bias=bias)
    assert np.array_equal(got, want.astype(np.float64))
    rows = oracle.matmul_reduce_scatter(A, B, parts, W, rank=rank, bias=bias, rows=(3, 17))
    assert np.array_equal(rows, got[3:17])


def test_reduce_scatter_zero_partials_is_own_slice():
    W, M, K, N = 4, 10, 12, 16
    A, B, bias = f16((M, K)), f16((K, N)), f16((N,))
    parts = [np.zeros((M, N // W), np.float16) for _ in range(W - 1)]
    got = oracle.matmul_reduce_scatter(A, B, parts, W, rank=2, bias=bias)
    own = oracle.gemm_bias(A, B, bias, cols=(8, 12))
    assert np.array_equal(got, own)


def test_reduce_scatter_partial_permutation_invariant():
    W, M, K, N = 8, 16, 32, 64
    A, B, bias = f16((M, K)), f16((K, N)), f16((N,))
    parts = [f16((M, N // W)) for _ in range(W - 1)]
    a = oracle.matmul_reduce_scatter(A, B, parts, W, bias=bias)
    b = oracle.matmul_reduce_scatter(A, B, parts[::-1], W, bias=bias)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------ all_reduce

def test_matmul_all_reduce_brute_force_and_w1():
    W, M, K, N = 3, 3, 4, 5
    A, B, bias = f16((M, K)), f16((K, N)), f16((M,), 0.1)
    parts = [f16((M, N)) for _ in range(W - 1)]
    got = oracle.matmul_all_reduce(A, B, parts, W, bias=bias, bias_along_m=True)
    own = exact_gemm(A, B, bias, True)
    exact = [[own[m][n] + sum(Fraction(float(p[m, n])) for p in parts) for n in range(N)]
             for m in range(M)]
    assert_close_exact(got, exact)
    assert np.array_equal(oracle.matmul_all_reduce(A, B, [], 1, bias=bias, bias_along_m=True),
                          oracle.gemm_bias(A, B, bias, bias_along_m=True))


def test_all_reduce_sum_exact_and_closed_forms():
    bufs = [f16((1000,)) for _ in range(8)]
    got = oracle.all_reduce(bufs)
    exact = [sum(Fraction(float(b[i])) for b in bufs) for i in range(1000)]
    assert all(abs(Fraction(float(g)) - e) <= Fraction(1, 2**40) * (abs(e) + 1)
               for g, e in zip(got, exact))
    x = f16((500,))
    same = oracle.all_reduce([x] * 8)
    assert np.array_equal(same, 8 * x.astype(np.float64))
    # order of the buffers does not matter beyond rounding
    assert np.allclose(oracle.all_reduce(bufs[::-1]), got, rtol=1e-14, atol=1e-14)
