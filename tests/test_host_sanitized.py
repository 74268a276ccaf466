"""The host runtime (lf_host.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer against host stand-ins of the device side
(tests/host_sanitize): argument validation, the state layout and work list,
the start-up of the recent-slot ring, handles over one and several layers,
both resets (with and without new budgets), the state checks and the prefill
entry points run with every memory access and integer operation checked.  No
GPU and no HIP runtime are involved."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


def test_host_runtime_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "lf_host_san"
    srcs = [os.path.join(ROOT, "kv_cache_eviction_lf_amd", "csrc", "lf_host.cpp"),
            os.path.join(HERE, "stub_device.cpp"), os.path.join(HERE, "drive.cpp")]
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", *srcs, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "ok: 0 failed checks" in r.stdout
