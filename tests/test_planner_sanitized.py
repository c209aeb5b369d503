"""The host planner (fa_plan.cpp: validation, int64 clamping, overflow guards, tile and work-item
planning, workspace layouts) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
CPU and driven over edge-case arguments. Any out-of-bounds access, overflow of a signed integer,
invalid shift or similar finding aborts the child process and fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planner_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    so = tmp_path / "libfa_plan_sanitized.so"
    cmd = [gxx, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "masked_attention_forward_amd", "csrc", "fa_plan.cpp"), "-o", str(so)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gxx, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (asan, ubsan) if os.path.exists(p))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_planner_driver.py"), str(so)],
                         env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "planner sanitized run ok" in res.stdout
