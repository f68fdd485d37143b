"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments with the documented status codes before touching the GPU.

No test here launches work: pointers passed are non-NULL placeholders that
are only checked for NULL-ness and alignment, which the library does before
any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iris_local.h")


@pytest.fixture(scope="module")
def lib():
    from gemm_collective_tile_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"\b(iris_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_the_four_ops():
    names = declared_functions()
    for op in ("iris_ag_mm", "iris_mm_rs_local", "iris_mm_ar_local", "iris_concurrent", "iris_mm_ag_local"):
        assert op in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_oracle_symbol_in_product_library():
    out = os.popen(f"nm -D --defined-only {ROOT}/gemm_collective_tile_amd/libiris_local.so").read()
    assert "oracle_" not in out
    exported = set(re.findall(r"\b(iris_[a-z_0-9]+)\b", out))
    assert exported >= set(declared_functions())


# placeholder "device" pointers: non-NULL and 16-byte aligned, never dereferenced
P = ctypes.c_void_p(0x100000)
MIS = ctypes.c_void_p(0x100008)


def ptrs(n, p=P):
    return (ctypes.c_void_p * max(1, n))(*([p.value] * n))


def status(lib, s):
    return lib.iris_status_str(s).decode()


def test_status_strings(lib):
    assert status(lib, 0) == "IRIS_OK"
    assert status(lib, 3) == "IRIS_ERR_CONFIG"
    assert status(lib, 99) == "IRIS_ERR_UNKNOWN"


def test_ag_mm_argument_errors(lib):
    shards = ptrs(2)
    ok = dict(C=P, G=P, S=shards, W=2, B=P, bias=None, M=256, N=256, K=256)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.iris_ag_mm(a["C"], a["G"], a["S"], a["W"], a["B"], a["bias"], a["M"], a["N"], a["K"],
                              None, None, 0, None)
    assert call(C=None) == 1
    assert call(W=0) == 1
    assert call(W=17, S=ptrs(17)) == 1
    assert call(S=ptrs(2, MIS)) == 4
    assert call(C=MIS) == 4
    assert call(K=12) == 4          # K_local % 8
    assert b"K_local" in lib.iris_last_error_message()
    assert call(N=100) == 4         # N % 8
    assert call(M=0) == 1
    assert call(M=-256) == 1
    assert call(bias=MIS) == 4
    assert b"bias" in lib.iris_last_error_message()
    # size limits (buffer resources and tile indices are 32-bit): rejected
    # before any device call
    assert call(M=(1 << 30) + 256) == 2
    assert call(N=(1 << 21) + 8) == 2
    assert call(K=(1 << 20) + 8) == 2   # W * K_local = K past 2^21
    assert b"too large" in lib.iris_last_error_message()
    assert call(M=1 << 30, N=1 << 21) == 2  # 2^22 * 2^13 tiles past 2^30


def test_rs_ar_concurrent_argument_errors(lib):
    parts = ptrs(7)
    # rank outside [0, W)
    assert lib.iris_mm_rs_local(P, P, P, P, None, parts, 8, 8, 4096, 11008, 4096, None, None, 0, None) == 1
    # N not divisible by W
    assert lib.iris_mm_rs_local(P, P, P, P, None, ptrs(2), 3, 0, 64, 64, 64, None, None, 0, None) == 1
    # N/W not a multiple of 8
    assert lib.iris_mm_rs_local(P, P, P, P, None, ptrs(3), 4, 0, 64, 48, 64, None, None, 0, None) == 4
    assert lib.iris_mm_ar_local(P, None, P, P, None, ptrs(1), 2, 64, 64, 64, None, None, 0, None) == 1
    # unknown collective
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 6, 0, P, ptrs(2), 2, 1024, None, None, 0, None) == 2
    # comm_elems % 8
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 1, 0, P, ptrs(2), 2, 1001, None, None, 0, None) == 4
    # reduce_scatter / all_to_all: comm_elems % (8 W); rank range for the ranked collectives
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 3, 0, P, ptrs(4), 4, 1040, None, None, 0, None) == 4
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 4, 0, P, ptrs(4), 4, 1040, None, None, 0, None) == 4
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 5, 2, P, ptrs(2), 2, 1024, None, None, 0, None) == 1
    assert lib.iris_concurrent(P, P, P, None, 64, 64, 64, 3, -1, P, ptrs(2), 2, 1024, None, None, 0, None) == 1
    # matmul_all_gather: rank range, peer pointers
    assert lib.iris_mm_ag_local(P, P, P, None, ptrs(2), 3, 3, 64, 64, 64, None, None, 0, None) == 1
    assert lib.iris_mm_ag_local(P, P, P, None, ptrs(2, MIS), 3, 0, 64, 64, 64, None, None, 0, None) == 4


def test_two_stream_mode_only_for_independent_ops(lib):
    from gemm_collective_tile_amd import IRIS_MODE_TWO_STREAM, Config
    c = ctypes.pointer(Config(mode=IRIS_MODE_TWO_STREAM)._c())
    # the all_gather feeds the GEMM: refused before any device call
    assert lib.iris_ag_mm(P, P, ptrs(2), 2, P, None, 256, 256, 256, c, None, 0, None) == 3
    assert b"two-stream" in lib.iris_last_error_message()
    assert lib.iris_mm_rs_local(P, P, P, P, None, ptrs(1), 2, 0, 64, 64, 64, c, None, 0, None) == 3


def test_config_errors_before_any_device_call(lib):
    from gemm_collective_tile_amd import Config
    shards = ptrs(2)
    for cfg, code in [(Config(block_m=96, block_n=96), 3), (Config(block_k=32), 3),
                      (Config(mode=7), 3), (Config(flags=64), 3), (Config(comm_block_n=12), 3),
                      (Config(comm_chunk=1000), 3), (Config(comm_block_m=96), 3)]:
        c = ctypes.pointer(cfg._c())
        assert lib.iris_ag_mm(P, P, shards, 2, P, None, 256, 256, 256, c, None, 0, None) == code, cfg


def test_workspace_size_is_host_only(lib):
    from gemm_collective_tile_amd import (IRIS_OP_AG_MM, IRIS_OP_CONCURRENT, IRIS_OP_MM_RS,
                                          iris_workspace_size)
    a = iris_workspace_size(IRIS_OP_AG_MM, 131072, 16384, 2048, 8)
    r = iris_workspace_size(IRIS_OP_MM_RS, 4096, 11008, 4096, 8)
    c = iris_workspace_size(IRIS_OP_CONCURRENT, 8192, 8192, 8192, 8)
    assert a > c > 0 and r > c
    # AG: one ready counter per row block (ceil(M/256)), each on its own
    # 128-byte line; RS: one flag per GEMM tile (16 x 43); concurrent: none
    # (the fixed counter words and the 256-byte rounding are in all three)
    assert a - c >= 512 * 128 - 256
    assert r - c >= 16 * 43 * 4 - 256
    assert iris_workspace_size(99, 1, 1, 1, 1) == 0
    assert iris_workspace_size(IRIS_OP_AG_MM, 0, 8, 8, 1) == 0


def test_python_binding_rejects_cpu_tensors():
    import torch
    from gemm_collective_tile_amd import iris_ag_mm
    x = torch.zeros(8, 8, dtype=torch.float16)
    with pytest.raises((ValueError, TypeError)):
        iris_ag_mm(x, x, [x], x)


def test_grid_size_rejects_unknown_op(lib):
    # the op is checked before the device is queried
    assert lib.iris_grid_size(99, None) == -1
    assert "unknown op" in lib.iris_last_error_message().decode()


def test_mfma_ceiling_checks_arguments_before_any_device_call(lib):
    t, m = ctypes.c_double(7.0), ctypes.c_double(7.0)
    for iters in (0, -1, (1 << 22) + 1):
        assert lib.iris_mfma_ceiling(1, iters, None, ctypes.byref(t), ctypes.byref(m)) == 1
        assert t.value == -1.0 and m.value == -1.0
    assert lib.iris_mfma_ceiling(1, 10, None, None, ctypes.byref(m)) == 1
    assert "NULL" in lib.iris_last_error_message().decode()
