"""The library's host layer (config validation, kernel selection, workspace
planning: hlta_host.cpp, which includes no HIP) built with g++ together with
tests/host/host_checks.cpp under AddressSanitizer and UndefinedBehaviorSanitizer,
then run: status strings, the measured workloads' plans, one invalid field at a
time, and a seeded sweep over 200,000 configs with edge values. No GPU."""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_host_layer_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "host_checks"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           str(ROOT / "tests" / "host" / "host_checks.cpp"),
           str(ROOT / "hybrid_linear_temporal_amd" / "csrc" / "hlta_host.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed: 200000 configs" in r.stdout
