"""The scratch pool (gemm_tiled_amd/csrc/workspace.hpp) on the CPU, under a
mock device that runs each stream's operations in order and the streams in a
random interleaving (tests/workspace_selftest.cpp): no launch on a freed or
not yet allocated buffer, no free under queued work, no two calls interleaving
launches on one buffer, the cap on kept slots, nothing allocated or queried
under stream capture, and captured slots never reused or freed.  Built with
g++ twice: optimised, and with ThreadSanitizer for the threaded scenario."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "workspace_selftest.cpp")
INC = os.path.join(ROOT, "gemm_tiled_amd", "csrc")
BUILD = os.path.join(ROOT, "_build", "selftest")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build_and_run(name, extra):
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread", "-Wall", "-Wextra", "-I" + INC, SRC,
           "-o", exe, *extra]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and extra:
        pytest.skip(f"g++ {' '.join(extra)} unavailable: {res.stderr[-300:]}")
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr


def test_scratch_pool_lifetime_rules():
    _build_and_run("workspace_selftest", [])


def test_scratch_pool_under_thread_sanitizer():
    _build_and_run("workspace_selftest_tsan", ["-fsanitize=thread"])
