"""The host code of libhinm (hinm_plan.cpp: region counts, per-tile plans,
workspace sizes, launch options, status strings) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and driven over many random
and malformed arguments by tests/sanitize/plan_driver.cpp (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "plan_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "structured_sparse_gemm_amd", "csrc"),
           os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
           os.path.join(ROOT, "structured_sparse_gemm_amd", "csrc", "hinm_plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HINM_PREFILL_SPLITS="2", HINM_DECODE_WGS="x")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "all checks passed" in r.stdout
