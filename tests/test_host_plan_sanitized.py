"""Host planning code under ASan and UBSan (CPU only).

csrc/host_plan.cpp is plain C++ (no HIP) so that its arithmetic can be
checked on its own: tests/host_plan_check.cpp sweeps the shapes check_shape
admits up to its limits with n_max and M around every planner threshold and
checks each plan's invariants, built here with g++ and
-fsanitize=address,undefined (any out-of-bounds access or signed overflow
aborts the run).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_long_kv_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "host_plan.cpp"), os.path.join(ROOT, "tests", "host_plan_check.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
                                UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host plan checks passed" in r.stdout
