"""The oracle against hand-computed examples (tests/golden/*.json).

The pages print no worked numeric example, so each fixture is a tiny case
computed by hand from the operation definition it cites; every value is
exactly representable, so the comparison is exact.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


def h(x):
    return np.asarray(x, dtype=np.float16)


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden(path):
    with open(path) as f:
        g = json.load(f)
    assert g["citation"]
    op = g["op"]
    bias = h(g["bias"]) if g.get("bias") is not None else None
    along_m = g.get("bias_along_m", False)
    if op == "all_gather_matmul":
        shards = [h(s) for s in g["shards"]]
        gathered = oracle.all_gather_k(shards).view(np.float16).astype(np.float64)
        assert np.array_equal(gathered, np.asarray(g["expected_gathered"], np.float64))
        got = oracle.all_gather_matmul(shards, h(g["B"]), bias, bias_along_m=along_m)
    elif op == "matmul_reduce_scatter":
        got = oracle.matmul_reduce_scatter(h(g["A"]), h(g["B"]), [h(p) for p in g["partials"]],
                                           g["W"], rank=g["rank"], bias=bias,
                                           bias_along_m=along_m)
    elif op == "matmul_all_reduce":
        got = oracle.matmul_all_reduce(h(g["A"]), h(g["B"]), [h(p) for p in g["partials"]],
                                       g["W"], bias=bias, bias_along_m=along_m)
    elif op == "concurrent":
        got = oracle.gemm_bias(h(g["A"]), h(g["B"]), bias, bias_along_m=along_m)
        comm = oracle.all_reduce([h(x) for x in g["comm_in"]])
        assert np.array_equal(comm, np.asarray(g["expected_comm"], np.float64))
    elif op == "matmul_all_gather":
        got = oracle.matmul_all_gather(h(g["A"]), h(g["B"]), [h(p) for p in g["peers"]], g["W"],
                                       rank=g["rank"], bias=bias, bias_along_m=along_m)
    elif op == "all_to_all":
        bufs = [h(b) for b in g["bufs"]]
        for r in (0, 1):
            got_r = oracle.all_to_all_flat(bufs, r).view(np.float16).astype(np.float64)
            assert np.array_equal(got_r, np.asarray(g[f"expected_rank{r}"], np.float64))
        return
    else:
        raise AssertionError(op)
    assert np.array_equal(got, np.asarray(g["expected"], np.float64))
    # the fp16 outputs are the same exact values
    enc = oracle.f16_encode(got).view(np.float16).astype(np.float64)
    assert np.array_equal(enc, np.asarray(g["expected"], np.float64))
