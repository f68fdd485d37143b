"""Python binding of libiris_local.so: one GPU's share of Iris-style fused
communication + GEMM ops on MI355X (gfx950).

Argument marshalling only: every step of every op runs in the library's HIP
kernels. PyTorch supplies device memory (tensors) and the stream. The
functions carry the names of the C entry points declared in
include/iris_local.h, which states each operation, its source on the pages,
argument layouts, ownership and error behaviour:

  iris_ag_mm          all_gather(A shards along K) -> gathered buffer; C = gathered @ B + bias
  iris_mm_rs_local    C = A @ B + bias; out = C[:, rank slice] + sum(partials)
  iris_mm_ar_local    C = A @ B + bias; out = C + sum(partials)
  iris_concurrent     C = A @ B + bias beside an independent all_reduce of W buffers

There is no fallback: if the library is missing or fails to load, importing
this package raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiris_local.so")

IRIS_MAX_W = 16
IRIS_MODE_FUSED = 0
IRIS_MODE_SEQUENTIAL = 1
IRIS_MODE_TWO_STREAM = 2
IRIS_FLAG_NO_STEAL = 1
IRIS_FLAG_BIAS_ALONG_M = 2
IRIS_FLAG_NO_LOCKSTEP = 4
IRIS_OP_AG_MM = 1
IRIS_OP_MM_RS = 2
IRIS_OP_MM_AR = 3
IRIS_OP_CONCURRENT = 4
IRIS_OP_MM_AG = 5
IRIS_COLL_ALL_REDUCE = 1
IRIS_COLL_ALL_GATHER = 2
IRIS_COLL_REDUCE_SCATTER = 3
IRIS_COLL_ALL_TO_ALL = 4
IRIS_COLL_BROADCAST = 5

STATUS = {
    0: "IRIS_OK", 1: "IRIS_ERR_INVALID_ARG", 2: "IRIS_ERR_UNSUPPORTED", 3: "IRIS_ERR_CONFIG",
    4: "IRIS_ERR_ALIGNMENT", 5: "IRIS_ERR_NO_MEMORY", 6: "IRIS_ERR_HIP", 7: "IRIS_ERR_WORKSPACE",
    8: "IRIS_ERR_NO_DEVICE", 9: "IRIS_ERR_DEVICE_TIMEOUT",
}


class IrisError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "block_m", "block_n", "block_k", "group_m", "gemm_wgs", "comm_block_m", "comm_block_n", "comm_chunk",
        "mode", "flags")]


@dataclass
class Config:
    """iris_config_t; a field <= 0 means automatic (tuned cache, else default)."""
    block_m: int = 0
    block_n: int = 0
    block_k: int = 0
    group_m: int = 0
    gemm_wgs: int = 0
    comm_block_m: int = 0
    comm_block_n: int = 0
    comm_chunk: int = 0
    mode: int = IRIS_MODE_FUSED
    flags: int = 0

    def _c(self) -> _Config:
        return _Config(*[int(getattr(self, f.name)) for f in fields(self)])


class _OpArgs(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("C", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("srcs", ctypes.POINTER(ctypes.c_void_p)),
        ("W", ctypes.c_int32), ("rank", ctypes.c_int32), ("collective", ctypes.c_int32), ("B", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
        ("K", ctypes.c_int64), ("comm_elems", ctypes.c_int64), ("cfg", _Config),
    ]


class _PredictParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in (
        "gemm_tflops_per_cu", "tile_overhead_us", "comm_gbps_per_cu", "comm_gbps_chip", "unit_overhead_us",
        "gemm_tflops_per_cu_max", "gemm_slowdown", "comm_slowdown", "phase_penalty")]


class _DeviceInfo(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("clock_khz", ctypes.c_int32), ("memory_clock_khz", ctypes.c_int32),
                ("lds_bytes_per_cu", ctypes.c_int32), ("global_mem_bytes", ctypes.c_int64),
                ("arch", ctypes.c_char * 64), ("peak_fp16_tflops", ctypes.c_double),
                ("peak_hbm_gbps", ctypes.c_double)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          f"python gemm_collective_tile_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    vpp = ctypes.POINTER(ctypes.c_void_p)
    cfgp = ctypes.POINTER(_Config)
    sig = {
        "iris_ag_mm": [vp, vp, vpp, i32, vp, vp, i64, i64, i64, cfgp, vp, sz, vp],
        "iris_ag_mm_noalloc": [vp, vp, vpp, i32, vp, vp, i64, i64, i64, cfgp, vp],
        "iris_mm_rs_local": [vp, vp, vp, vp, vp, vpp, i32, i32, i64, i64, i64, cfgp, vp, sz, vp],
        "iris_mm_ar_local": [vp, vp, vp, vp, vp, vpp, i32, i64, i64, i64, cfgp, vp, sz, vp],
        "iris_concurrent": [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vpp, i32, i64, cfgp, vp, sz, vp],
        "iris_mm_ag_local": [vp, vp, vp, vp, vpp, i32, i32, i64, i64, i64, cfgp, vp, sz, vp],
        "iris_grid_size": [ctypes.c_int32, cfgp],
        "iris_tune_gemm_wgs": [ctypes.POINTER(_OpArgs), ctypes.POINTER(i32), i32, i32, i32,
                               ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float), vp],
        "iris_predict_gemm_wgs": [ctypes.POINTER(_OpArgs), i32, ctypes.POINTER(i32), i32,
                                  ctypes.POINTER(_PredictParams), ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(i32)],
        "iris_last_windows": [vp, vp] + [ctypes.POINTER(ctypes.c_double)] * 4,
        "iris_check_device_error": [vp, vp],
        "iris_last_clock": [vp, vp, ctypes.POINTER(ctypes.c_double)],
        "iris_mfma_ceiling": [i32, i32, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
        "iris_device_info": [i32, ctypes.POINTER(_DeviceInfo)],
        "iris_status_str": [i32],
        "iris_last_error_message": [],
        "iris_finalize": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.iris_workspace_size.argtypes = [i32, i64, i64, i64, i32, cfgp]
    lib.iris_workspace_size.restype = sz
    lib.iris_status_str.restype = ctypes.c_char_p
    lib.iris_last_error_message.restype = ctypes.c_char_p
    return lib


_lib = _load()


# --------------------------------------------------------------- marshalling

def _check(status: int) -> None:
    if status != 0:
        raise IrisError(status, _lib.iris_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor], name: str, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16:
        raise TypeError(f"{name} must be a float16 torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    return ctypes.c_void_p(t.data_ptr())


def _ptr_array(ts: Sequence[torch.Tensor], name: str):
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t, f"{name}[{i}]").value
    return arr


def _cfg(config) -> Optional[ctypes.pointer]:
    if config is None:
        return None
    if isinstance(config, dict):
        config = Config(**config)
    return ctypes.pointer(config._c())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ws(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _shape2(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return t.shape


# Shape checks. They run before any pointer is taken: a tensor whose shape
# does not match the M, N, K, W the library derives would be read or written
# past its end by the kernels.

def _want_shape(t, shape, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _want_numel(t, n: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n}")


def _want_count(ts, n: int, name: str) -> None:
    if len(ts) != n:
        raise ValueError(f"{name} holds {len(ts)} tensors, expected {n}")


def _bias_along_m(config) -> bool:
    if config is None:
        return False
    flags = config.get("flags", 0) if isinstance(config, dict) else config.flags
    return bool(int(flags) & IRIS_FLAG_BIAS_ALONG_M)


def _want_bias(bias, M: int, N: int, config) -> None:
    if bias is not None:
        _want_numel(bias, M if _bias_along_m(config) else N, "bias")


def _want_w(W: int) -> None:
    if not 1 <= int(W) <= IRIS_MAX_W:
        raise ValueError(f"W must be in [1, {IRIS_MAX_W}] (got {W})")


def _validate(op, config, C=None, out=None, A=None, srcs=(), W=1, B=None, bias=None, M=0, N=0, K=0,
              comm_elems=0, collective=IRIS_COLL_ALL_REDUCE):
    """Checks every tensor of op `op` against the shape the library derives
    (K is K_local for all_gather_matmul)."""
    _want_w(W)
    if op == IRIS_OP_AG_MM:
        _want_count(srcs, W, "A_shards")
        for s, t in enumerate(srcs):
            _want_shape(t, (M, K), f"A_shards[{s}]")
        _want_shape(B, (W * K, N), "B")
        _want_shape(C, (M, N), "C")
        _want_shape(out, (M, W * K), "A_gathered")
    elif op in (IRIS_OP_MM_RS, IRIS_OP_MM_AR):
        if op == IRIS_OP_MM_RS and N % W != 0:
            raise ValueError(f"N ({N}) must be divisible by W ({W})")
        cols = N // W if op == IRIS_OP_MM_RS else N
        _want_shape(A, (M, K), "A")
        _want_shape(B, (K, N), "B")
        _want_shape(C, (M, N), "C")
        _want_shape(out, (M, cols), "out")
        _want_count(srcs, W - 1, "partials")
        for p, t in enumerate(srcs):
            _want_shape(t, (M, cols), f"partials[{p}]")
    elif op == IRIS_OP_CONCURRENT:
        _want_shape(A, (M, K), "A")
        _want_shape(B, (K, N), "B")
        _want_shape(C, (M, N), "C")
        _want_count(srcs, W, "comm_in")
        for w, t in enumerate(srcs):
            _want_numel(t, comm_elems, f"comm_in[{w}]")
        if collective in _COMM_OUT_LEN:
            _want_numel(out, _COMM_OUT_LEN[collective](comm_elems, W), "comm_out")
    elif op == IRIS_OP_MM_AG:
        _want_shape(A, (M, K), "A")
        _want_shape(B, (K, N), "B")
        _want_shape(out, (M * W, N), "out")
        _want_count(srcs, W - 1, "peers")
        for p, t in enumerate(srcs):
            _want_shape(t, (M, N), f"peers[{p}]")
    else:
        raise ValueError(f"unknown op {op}")
    _want_bias(bias, M, N, config)


_COMM_OUT_LEN = {
    IRIS_COLL_ALL_REDUCE: lambda n, W: n, IRIS_COLL_ALL_GATHER: lambda n, W: W * n,
    IRIS_COLL_REDUCE_SCATTER: lambda n, W: n // W, IRIS_COLL_ALL_TO_ALL: lambda n, W: n,
    IRIS_COLL_BROADCAST: lambda n, W: n,
}


# ----------------------------------------------------------------------- ops

def iris_ag_mm(C, A_gathered, A_shards, B, bias=None, config=None, workspace=None, stream=None):
    """all_gather_matmul local share: A_gathered = concat_K(A_shards); C = A_gathered @ B + bias."""
    W = len(A_shards)
    if W < 1:
        raise ValueError("A_shards is empty")
    M, K_local = _shape2(A_shards[0], "A_shards[0]")
    N = _shape2(B, "B")[1]
    _validate(IRIS_OP_AG_MM, config, C=C, out=A_gathered, srcs=A_shards, W=W, B=B, bias=bias, M=M, N=N,
              K=K_local)
    ws, wsb = _ws(workspace)
    _check(_lib.iris_ag_mm(_ptr(C, "C"), _ptr(A_gathered, "A_gathered"), _ptr_array(A_shards, "A_shards"),
                           W, _ptr(B, "B"), _ptr(bias, "bias", True), M, N, K_local, _cfg(config),
                           ws, wsb, _stream(stream)))


def iris_ag_mm_noalloc(C, A_gathered, A_shards, B, bias=None, config=None, stream=None):
    """iris_ag_mm on the library's static device scratch (no workspace, no
    allocation); calls that overlap in time on one GPU race."""
    W = len(A_shards)
    if W < 1:
        raise ValueError("A_shards is empty")
    M, K_local = _shape2(A_shards[0], "A_shards[0]")
    N = _shape2(B, "B")[1]
    _validate(IRIS_OP_AG_MM, config, C=C, out=A_gathered, srcs=A_shards, W=W, B=B, bias=bias, M=M, N=N,
              K=K_local)
    _check(_lib.iris_ag_mm_noalloc(_ptr(C, "C"), _ptr(A_gathered, "A_gathered"),
                                   _ptr_array(A_shards, "A_shards"), W, _ptr(B, "B"), _ptr(bias, "bias", True),
                                   M, N, K_local, _cfg(config), _stream(stream)))


def iris_mm_rs_local(out, C, A, B, partials, W, rank=0, bias=None, config=None, workspace=None,
                     stream=None):
    """matmul_reduce_scatter local share: C = A @ B + bias; out = C[:, rank*N/W:(rank+1)*N/W] + sum(partials)."""
    M, K = _shape2(A, "A")
    N = _shape2(B, "B")[1]
    _validate(IRIS_OP_MM_RS, config, C=C, out=out, A=A, srcs=partials, W=W, B=B, bias=bias, M=M, N=N, K=K)
    ws, wsb = _ws(workspace)
    _check(_lib.iris_mm_rs_local(_ptr(out, "out"), _ptr(C, "C"), _ptr(A, "A"), _ptr(B, "B"),
                                 _ptr(bias, "bias", True), _ptr_array(partials, "partials"), W, rank,
                                 M, N, K, _cfg(config), ws, wsb, _stream(stream)))


def iris_mm_ar_local(out, C, A, B, partials, W, bias=None, config=None, workspace=None, stream=None):
    """matmul_all_reduce local share: C = A @ B + bias; out = C + sum(partials)."""
    M, K = _shape2(A, "A")
    N = _shape2(B, "B")[1]
    _validate(IRIS_OP_MM_AR, config, C=C, out=out, A=A, srcs=partials, W=W, B=B, bias=bias, M=M, N=N, K=K)
    ws, wsb = _ws(workspace)
    _check(_lib.iris_mm_ar_local(_ptr(out, "out"), _ptr(C, "C"), _ptr(A, "A"), _ptr(B, "B"),
                                 _ptr(bias, "bias", True), _ptr_array(partials, "partials"), W,
                                 M, N, K, _cfg(config), ws, wsb, _stream(stream)))


def iris_concurrent(C, A, B, comm_out, comm_in, bias=None, collective=IRIS_COLL_ALL_REDUCE, rank=0,
                    config=None, workspace=None, stream=None):
    """C = A @ B + bias, and independently the local share of `collective`
    over the W buffers comm_in (every rank's buffer, own included) into
    comm_out; `rank` is this rank (the root for broadcast)."""
    M, K = _shape2(A, "A")
    N = _shape2(B, "B")[1]
    W = len(comm_in)
    if W < 1:
        raise ValueError("comm_in is empty")
    n = comm_in[0].numel()
    _validate(IRIS_OP_CONCURRENT, config, C=C, out=comm_out, A=A, srcs=comm_in, W=W, B=B, bias=bias, M=M, N=N,
              K=K, comm_elems=n, collective=collective)
    ws, wsb = _ws(workspace)
    _check(_lib.iris_concurrent(_ptr(C, "C"), _ptr(A, "A"), _ptr(B, "B"), _ptr(bias, "bias", True),
                                M, N, K, collective, rank, _ptr(comm_out, "comm_out"),
                                _ptr_array(comm_in, "comm_in"), W, n, _cfg(config),
                                ws, wsb, _stream(stream)))


def iris_mm_ag_local(out, A, B, peers, W, rank=0, bias=None, config=None, workspace=None, stream=None):
    """matmul_all_gather local share: out (M*W, N) holds every rank's A @ B + bias
    along M; this rank's block is computed, the W-1 `peers` (M, N) are copied."""
    M, K = _shape2(A, "A")
    N = _shape2(B, "B")[1]
    _validate(IRIS_OP_MM_AG, config, out=out, A=A, srcs=peers, W=W, B=B, bias=bias, M=M, N=N, K=K)
    ws, wsb = _ws(workspace)
    _check(_lib.iris_mm_ag_local(_ptr(out, "out"), _ptr(A, "A"), _ptr(B, "B"), _ptr(bias, "bias", True),
                                 _ptr_array(peers, "peers"), W, rank, M, N, K, _cfg(config), ws, wsb,
                                 _stream(stream)))


# ------------------------------------------------------------------- helpers

def iris_workspace_size(op, M, N, K, W, config=None) -> int:
    return int(_lib.iris_workspace_size(op, M, N, K, W, _cfg(config)))


def iris_grid_size(config=None, op=IRIS_OP_AG_MM) -> int:
    """Workgroups of the fused persistent launch of `op` for this config."""
    g = _lib.iris_grid_size(op, _cfg(config))
    if g < 0:
        _check(-g)
    return g


def _op_args(op, config, C=None, out=None, A=None, srcs=(), W=1, rank=0, collective=0, B=None, bias=None,
             M=0, N=0, K=0, comm_elems=0):
    keep = _ptr_array(list(srcs), "srcs")
    a = _OpArgs()
    a.op = op
    a.C = _ptr(C, "C", True)
    a.out = _ptr(out, "out", True)
    a.A = _ptr(A, "A", True)
    a.srcs = ctypes.cast(keep, ctypes.POINTER(ctypes.c_void_p))
    a.W, a.rank, a.collective = W, rank, collective
    a.B = _ptr(B, "B", True)
    a.bias = _ptr(bias, "bias", True)
    a.M, a.N, a.K, a.comm_elems = M, N, K, comm_elems
    a.cfg = (config if isinstance(config, Config) else Config(**(config or {})))._c()
    return a, keep


def iris_tune_gemm_wgs(op, candidates, reps=5, config=None, stream=None, *, top_k=0, C=None, out=None, A=None,
                       srcs=(), W=1, rank=0, collective=0, B=None, bias=None, M=0, N=0, K=0, comm_elems=0):
    """Sweep gemm_wgs over `candidates` (the static default is always added),
    cache and return (best, {candidate: median ms}). With top_k > 0 only the
    top_k candidates the predictor ranks best are run (the others read -1)."""
    _validate(op, config, C=C, out=out, A=A, srcs=srcs, W=W, B=B, bias=bias, M=M, N=N, K=K,
              comm_elems=comm_elems, collective=collective or IRIS_COLL_ALL_REDUCE)
    a, keep = _op_args(op, config, C, out, A, srcs, W, rank, collective, B, bias, M, N, K, comm_elems)
    cands = (ctypes.c_int32 * max(1, len(candidates)))(*candidates)
    ms = (ctypes.c_float * max(1, len(candidates)))()
    best = ctypes.c_int32(0)
    _check(_lib.iris_tune_gemm_wgs(ctypes.byref(a), cands, len(candidates), reps, top_k, ctypes.byref(best),
                                   ms, _stream(stream)))
    del keep
    return best.value, {c: ms[i] for i, c in enumerate(candidates)}


def iris_predict_gemm_wgs(op, candidates, grid, config=None, params=None, *, W=1, rank=0, collective=0,
                          M=0, N=0, K=0, comm_elems=0):
    """Predicted makespan (ms) of the fused schedule for each gemm_wgs
    candidate on a grid of `grid` workgroups; returns (best, {candidate: ms}).
    Host only: needs the shapes, no tensors. `params` is a dict of the
    model's constants (gemm_tflops_per_cu, tile_overhead_us, comm_gbps_per_cu,
    comm_gbps_chip, unit_overhead_us, gemm_tflops_per_cu_max, gemm_slowdown,
    comm_slowdown, phase_penalty); missing ones take the defaults."""
    a, keep = _op_args(op, config, W=W, rank=rank, collective=collective, M=M, N=N, K=K, comm_elems=comm_elems)
    pp = _PredictParams(*[-1.0] * len(_PredictParams._fields_))
    for k, v in (params or {}).items():
        if k not in dict(_PredictParams._fields_):
            raise ValueError(f"unknown predictor parameter {k!r}")
        setattr(pp, k, float(v))
    cands = (ctypes.c_int32 * max(1, len(candidates)))(*candidates)
    ms = (ctypes.c_float * max(1, len(candidates)))()
    best = ctypes.c_int32(0)
    _check(_lib.iris_predict_gemm_wgs(ctypes.byref(a), grid, cands, len(candidates), ctypes.byref(pp), ms,
                                      ctypes.byref(best)))
    del keep
    return best.value, {c: ms[i] for i, c in enumerate(candidates)}


def iris_last_windows(workspace=None, stream=None):
    """(gemm_start, gemm_end, comm_start, comm_end) in ns of the last fused launch; -1 if none."""
    vals = [ctypes.c_double() for _ in range(4)]
    ws, _ = _ws(workspace)
    _check(_lib.iris_last_windows(ws, _stream(stream), *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)


def iris_last_clock(workspace=None, stream=None) -> float:
    """Shader clock (MHz) held during the last persistent launch on this
    workspace (-1 if none was recorded)."""
    v = ctypes.c_double()
    ws, _ = _ws(workspace)
    _check(_lib.iris_last_clock(ws, _stream(stream), ctypes.byref(v)))
    return v.value


def iris_mfma_ceiling(random_operands: bool = True, iters: int = 400000, stream=None):
    """(TFLOP/s, MHz): the dense fp16 MFMA rate of the current GPU with no
    memory traffic, operands random (switching as on GEMM data) or constant,
    and the shader clock it held. Waits for the run."""
    t, m = ctypes.c_double(), ctypes.c_double()
    _check(_lib.iris_mfma_ceiling(1 if random_operands else 0, int(iters), _stream(stream), ctypes.byref(t),
                                  ctypes.byref(m)))
    return t.value, m.value


def iris_check_device_error(workspace=None, stream=None) -> None:
    """Waits for the stream; raises IrisError (IRIS_ERR_DEVICE_TIMEOUT) if a
    device-side wait of a fused op on this workspace gave up since the last
    check (the outputs of those ops are then not to be trusted)."""
    ws, _ = _ws(workspace)
    _check(_lib.iris_check_device_error(ws, _stream(stream)))


def iris_device_info(device: int = 0) -> dict:
    info = _DeviceInfo()
    _check(_lib.iris_device_info(device, ctypes.byref(info)))
    return {f[0]: (getattr(info, f[0]).decode() if f[0] == "arch" else getattr(info, f[0]))
            for f in _DeviceInfo._fields_}


def iris_finalize() -> None:
    _check(_lib.iris_finalize())


def library_path() -> str:
    return LIB_PATH
