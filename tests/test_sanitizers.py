"""Host address and undefined-behaviour sanitizer runs of the CPU oracle and
of the split predictor (host code only; no GPU). Both are built with g++,
-fsanitize=address,undefined and no recovery, linked with a driver that
calls every oracle entry point and the predictor on small, ragged and
workload-sized inputs (tests/native/sanitize_main.cpp). A sanitizer finding
aborts the driver with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_and_predictor_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_main")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "native", "sanitize_main.cpp"), os.path.join(ROOT, "oracle", "oracle.cpp"),
           os.path.join(ROOT, "gemm_collective_tile_amd", "csrc", "predict.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
