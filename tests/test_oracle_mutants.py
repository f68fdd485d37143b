"""Planted mistakes in the oracle must each fail at least one pin.

Each case copies oracle/oracle.cpp, plants one plausible mistake (a dropped
term, a wrong sign or index, a wrong axis, a wrong shard order or rank
slice, a wrong rounding rule), builds the copy on the CPU, and runs the pin
suites against it in a child process. The child must fail. This shows that
the pins constrain every part of the oracle, not only that the oracle
passes them.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
PINS = ["tests/test_oracle_fp16.py", "tests/test_oracle_ops.py", "tests/test_oracle_golden.py",
        "tests/test_oracle_collectives.py"]

MUTANTS = {
    "dropped_bias": ("acc[j] += bias_value(bias, bias_mode, m, n0 + j);", "(void)0;"),
    "bias_wrong_axis": ("bias_mode == ORACLE_BIAS_ALONG_M ? m : n", "bias_mode == ORACLE_BIAS_ALONG_M ? n : m"),
    "product_sign": ("acc[j] += a * brow[j];", "acc[j] -= a * brow[j];"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k < K - 1; ++k) {"),
    "b_column_offset": ("oracle_f16_decode(B[k * ldb + n0 + j])", "oracle_f16_decode(B[k * ldb + j])"),
    "shard_order": ("gathered[m * K + (int64_t)s * K_local + k]", "gathered[m * K + (int64_t)(W - 1 - s) * K_local + k]"),
    "rank_slice": ("K, m0, m1, rank * nl,\n                   (rank + 1) * nl", "K, m0, m1, 0,\n                   nl"),
    "dropped_partial": ("for (int p = 0; p < W - 1; ++p)\n    for (int64_t m = m0; m < m1; ++m)\n      for (int64_t j = 0; j < nl; ++j)",
                        "for (int p = 1; p < W - 1; ++p)\n    for (int64_t m = m0; m < m1; ++m)\n      for (int64_t j = 0; j < nl; ++j)"),
    "sum_skips_first": ("for (int w = 0; w < nbuf; ++w)", "for (int w = 1; w < nbuf; ++w)"),
    "ties_round_up": ("return (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "subnormal_scale": ("mag = std::ldexp((double)frac, -24);", "mag = std::ldexp((double)frac, -23);"),
    "exponent_bias": ("const int be = e + 15;", "const int be = e + 14;"),
    "row_bias_offset": ("bias_rows.assign(bias + m0, bias + m1);", "bias_rows.assign(bias, bias + (m1 - m0));"),
    "mmag_peer_order": ("peers[q < rank ? q : q - 1]", "peers[(W - 2) - (q < rank ? q : q - 1)]"),
    "mmag_own_block": ("if (q == rank) {", "if (q == 0) {"),
    "ag_flat_order": ("out[(int64_t)w * n + i] = bufs[w][i];", "out[(int64_t)(W - 1 - w) * n + i] = bufs[w][i];"),
    "rs_flat_slice": ("s += oracle_f16_decode(bufs[w][(int64_t)rank * part + i]);", "s += oracle_f16_decode(bufs[w][i]);"),
    "a2a_source_block": ("out[(int64_t)j * part + i] = bufs[j][(int64_t)rank * part + i];",
                         "out[(int64_t)j * part + i] = bufs[j][(int64_t)j * part + i];"),
    "bcast_root": ("for (int64_t i = 0; i < n; ++i) out[i] = bufs[root][i];", "for (int64_t i = 0; i < n; ++i) out[i] = bufs[0][i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "oracle_mutant.cpp"
    mutant_src.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    obuild.build(src=str(mutant_src), out=lib)
    env = dict(os.environ, IRIS_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
