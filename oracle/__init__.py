"""ctypes front end of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke entry and
by the benchmark's CPU-baseline leg; never by the product package. Shares no
code with the HIP library. What each function computes is stated, with its
source on the pages, in oracle/oracle.h and oracle/oracle.cpp:
  - Iris docs "Fused Communication and Compute Operations" (all_gather_matmul,
    matmul_reduce_scatter, matmul_all_reduce),
  - ROCm/iris PR "Add iris.concurrent (concurrent, independent, fused
    comm+gemm)" (independent GEMM beside an all_reduce).

Inputs are numpy uint16 arrays holding binary16 bit patterns (or float16
arrays, viewed as uint16). Float results come back as float64 arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BIAS_NONE = 0
BIAS_ALONG_N = 1
BIAS_ALONG_M = 2

_lib = None
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("IRIS_ORACLE_LIB")  # a test may point at another build
    if not path:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_f16_decode.restype = ctypes.c_double
    lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_encode.restype = ctypes.c_uint16
    lib.oracle_f16_encode.argtypes = [ctypes.c_double]
    lib.oracle_f16_decode_array.argtypes = [_u16p, _f64p, _i64]
    lib.oracle_f16_encode_array.argtypes = [_f64p, _u16p, _i64]
    lib.oracle_gemm_bias.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, ctypes.c_int,
                                     _i64, _i64, _i64, _i64, _i64, _f64p, ctypes.c_int]
    lib.oracle_all_gather_k.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, _i64, _u16p]
    lib.oracle_sum.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, _f64p]
    lib.oracle_all_gather_matmul.argtypes = [
        ctypes.POINTER(_u16p), ctypes.c_int, _i64, _i64, _u16p, _i64, _u16p, ctypes.c_int,
        _i64, _i64, _i64, _i64, _f64p, ctypes.c_int]
    lib.oracle_matmul_reduce_scatter.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.POINTER(_u16p), ctypes.c_int, ctypes.c_int,
        _i64, _i64, _i64, _i64, _i64, _f64p, ctypes.c_int]
    lib.oracle_matmul_all_reduce.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.POINTER(_u16p), ctypes.c_int,
        _i64, _i64, _i64, _i64, _i64, _f64p, ctypes.c_int]
    lib.oracle_matmul_all_gather.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.POINTER(_u16p), ctypes.c_int, ctypes.c_int,
        _i64, _i64, _i64, _i64, _i64, _f64p, ctypes.c_int]
    lib.oracle_all_gather_flat.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, _u16p]
    lib.oracle_reduce_scatter_flat.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, ctypes.c_int, _f64p]
    lib.oracle_all_to_all_flat.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, ctypes.c_int, _u16p]
    lib.oracle_broadcast_flat.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _i64, ctypes.c_int, _u16p]
    lib.oracle_default_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    return _load().oracle_default_threads()


def cpu_share() -> int:
    """Threads a call with nthreads=0 uses: IRIS_ORACLE_THREADS if set, else
    the cores this process may run on, at most 16 (the CPU share of one GPU
    on the machines the tests and the benchmark run on)."""
    env = os.environ.get("IRIS_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _nt(nthreads: int) -> int:
    return nthreads if nthreads > 0 else cpu_share()


def _u16(a):
    """Contiguous uint16 view of an fp16/uint16 numpy array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16/uint16 array, got {a.dtype}")
    return a


def _p16(a):
    return None if a is None else a.ctypes.data_as(_u16p)


def _ptr_array(arrs):
    return (_u16p * len(arrs))(*[a.ctypes.data_as(_u16p) for a in arrs])


def _bias_mode(bias, along_m):
    if bias is None:
        return BIAS_NONE
    return BIAS_ALONG_M if along_m else BIAS_ALONG_N


# ------------------------------------------------------------------ fp16 codec

def f16_decode(bits) -> np.ndarray:
    b = _u16(np.asarray(bits))
    out = np.empty(b.shape, np.float64)
    _load().oracle_f16_decode_array(b.ctypes.data_as(_u16p), out.ctypes.data_as(_f64p), b.size)
    return out


def f16_encode(x) -> np.ndarray:
    """double -> binary16 bits (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f16_encode_array(x.ctypes.data_as(_f64p), out.ctypes.data_as(_u16p), x.size)
    return out


# ------------------------------------------------------------------ GEMM + ops

def gemm_bias(A, B, bias=None, bias_along_m=False, rows=None, cols=None, nthreads=0):
    """Region of A @ B + bias in float64. A (M,K), B (K,N) fp16."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    m0, m1 = rows if rows is not None else (0, M)
    n0, n1 = cols if cols is not None else (0, N)
    bias = None if bias is None else _u16(bias)
    out = np.empty((m1 - m0, n1 - n0), np.float64)
    _load().oracle_gemm_bias(_p16(A), K, _p16(B), N, _p16(bias), _bias_mode(bias, bias_along_m),
                             K, m0, m1, n0, n1, out.ctypes.data_as(_f64p), _nt(nthreads))
    return out


def all_gather_k(shards) -> np.ndarray:
    """Concatenate W (M, K_local) fp16 shards along K in rank order (bit copy)."""
    shards = [_u16(s) for s in shards]
    M, kl = shards[0].shape
    out = np.empty((M, kl * len(shards)), np.uint16)
    _load().oracle_all_gather_k(_ptr_array(shards), len(shards), M, kl, _p16(out))
    return out


def sum_buffers(bufs) -> np.ndarray:
    """Elementwise float64 sum of fp16 buffers (same shape), in the given order."""
    bufs = [_u16(b) for b in bufs]
    out = np.empty(bufs[0].shape, np.float64)
    _load().oracle_sum(_ptr_array(bufs), len(bufs), bufs[0].size, out.ctypes.data_as(_f64p))
    return out


def all_gather_matmul(shards, B, bias=None, bias_along_m=False, rows=None, cols=None,
                      nthreads=0):
    """Region of concat_K(shards) @ B + bias in float64."""
    shards = [_u16(s) for s in shards]
    B = _u16(B)
    M, kl = shards[0].shape
    W = len(shards)
    assert B.shape[0] == W * kl
    N = B.shape[1]
    m0, m1 = rows if rows is not None else (0, M)
    n0, n1 = cols if cols is not None else (0, N)
    bias = None if bias is None else _u16(bias)
    out = np.empty((m1 - m0, n1 - n0), np.float64)
    _load().oracle_all_gather_matmul(_ptr_array(shards), W, M, kl, _p16(B), N, _p16(bias),
                                     _bias_mode(bias, bias_along_m), m0, m1, n0, n1,
                                     out.ctypes.data_as(_f64p), _nt(nthreads))
    return out


def matmul_reduce_scatter(A, B, partials, W, rank=0, bias=None, bias_along_m=False,
                          rows=None, nthreads=0):
    """This rank's (rows, N/W) slice of reduce_scatter(A @ B + bias), float64.

    partials: W-1 fp16 (M, N/W) buffers standing in for the other ranks."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N = B.shape[1]
    assert len(partials) == W - 1 and N % W == 0
    partials = [_u16(p) for p in partials]
    m0, m1 = rows if rows is not None else (0, M)
    bias = None if bias is None else _u16(bias)
    out = np.empty((m1 - m0, N // W), np.float64)
    pp = _ptr_array(partials) if partials else None
    _load().oracle_matmul_reduce_scatter(_p16(A), _p16(B), _p16(bias),
                                         _bias_mode(bias, bias_along_m), pp, W, rank,
                                         M, N, K, m0, m1, out.ctypes.data_as(_f64p), _nt(nthreads))
    return out


def matmul_all_reduce(A, B, partials, W, bias=None, bias_along_m=False, rows=None,
                      nthreads=0):
    """Rows of all_reduce(A @ B + bias) with W-1 stand-in (M, N) partials, float64."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N = B.shape[1]
    assert len(partials) == W - 1
    partials = [_u16(p) for p in partials]
    m0, m1 = rows if rows is not None else (0, M)
    bias = None if bias is None else _u16(bias)
    out = np.empty((m1 - m0, N), np.float64)
    pp = _ptr_array(partials) if partials else None
    _load().oracle_matmul_all_reduce(_p16(A), _p16(B), _p16(bias), _bias_mode(bias, bias_along_m),
                                     pp, W, M, N, K, m0, m1, out.ctypes.data_as(_f64p), _nt(nthreads))
    return out


def all_reduce(bufs) -> np.ndarray:
    """Elementwise sum of W fp16 buffers (the all_reduce beside an independent GEMM)."""
    return sum_buffers(bufs)


def matmul_all_gather(A, B, peers, W, rank=0, bias=None, bias_along_m=False, rows=None, nthreads=0):
    """Rows of all_gather along M of every rank's A @ B + bias, (M*W, N) float64.

    peers: W-1 fp16 (M, N) buffers standing in for the other ranks' results,
    in rank order without this rank."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N = B.shape[1]
    assert len(peers) == W - 1 and 0 <= rank < W
    peers = [_u16(p) for p in peers]
    m0, m1 = rows if rows is not None else (0, M * W)
    bias = None if bias is None else _u16(bias)
    out = np.empty((m1 - m0, N), np.float64)
    pp = _ptr_array(peers) if peers else None
    _load().oracle_matmul_all_gather(_p16(A), _p16(B), _p16(bias), _bias_mode(bias, bias_along_m),
                                     pp, W, rank, M, N, K, m0, m1, out.ctypes.data_as(_f64p), _nt(nthreads))
    return out


def all_gather_flat(bufs) -> np.ndarray:
    """all_gather of W flat fp16 buffers of n elements: their concatenation in rank order."""
    bufs = [_u16(b).reshape(-1) for b in bufs]
    n = bufs[0].size
    out = np.empty(len(bufs) * n, np.uint16)
    _load().oracle_all_gather_flat(_ptr_array(bufs), len(bufs), n, _p16(out))
    return out


def reduce_scatter_flat(bufs, rank) -> np.ndarray:
    """This rank's n/W slice of the elementwise sum of W flat fp16 buffers, float64."""
    bufs = [_u16(b).reshape(-1) for b in bufs]
    W, n = len(bufs), bufs[0].size
    assert n % W == 0 and 0 <= rank < W
    out = np.empty(n // W, np.float64)
    _load().oracle_reduce_scatter_flat(_ptr_array(bufs), W, n, rank, out.ctypes.data_as(_f64p))
    return out


def all_to_all_flat(bufs, rank) -> np.ndarray:
    """Block j of the result is block `rank` of rank j's buffer (W blocks of n/W)."""
    bufs = [_u16(b).reshape(-1) for b in bufs]
    W, n = len(bufs), bufs[0].size
    assert n % W == 0 and 0 <= rank < W
    out = np.empty(n, np.uint16)
    _load().oracle_all_to_all_flat(_ptr_array(bufs), W, n, rank, _p16(out))
    return out


def broadcast_flat(bufs, root) -> np.ndarray:
    """The root rank's buffer."""
    bufs = [_u16(b).reshape(-1) for b in bufs]
    assert 0 <= root < len(bufs)
    out = np.empty(bufs[0].size, np.uint16)
    _load().oracle_broadcast_flat(_ptr_array(bufs), len(bufs), bufs[0].size, root, _p16(out))
    return out
