"""The launch planner and the per-step launch sequence on the CPU, under
AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_check/planner_check.cpp compiles runtime.cpp for the host with
every HIP runtime call and kernel launcher replaced by stubs.  Each stubbed
launch checks that every access its kernel would make (table entries, rows
and columns of W, G and M, partials, counters, Newton-Schulz workspaces and
tiles) lies in a buffer the harness registered, and that tiles fit the padded
shapes.  It runs the DiT-1.3B, DiT-4B, MuonBP and DiT-15B plans (host copies of
the tables at a fake base address) in several configurations, and a ragged
and a MuonBP set through muon_init, muon_step (with a pointer change),
muon_step_noalloc and the other entry points, with host memory behind them.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_asan_ubsan(tmp_path):
    exe = tmp_path / "planner_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "matrix_aware_optimizer_periodic_amd", "csrc"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "host_check", "planner_check.cpp"),
           "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "failures 0" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
