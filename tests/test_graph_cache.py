"""The graph-cache bookkeeping (LRU order and eviction, zero capacity,
prefix-bucket choice and validation; vla_flow_matching_amd/csrc/
ae_graph_cache.h) checked on the host by tests/host/graph_cache_check.cpp.
Plain C++: needs a host compiler, no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_graph_cache_host(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "graph_cache_check")
    src = os.path.join(ROOT, "tests", "host", "graph_cache_check.cpp")
    cmd = [cxx, "-O1", "-std=c++17", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-I", os.path.join(ROOT, "vla_flow_matching_amd", "csrc"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failed checks: 0" in r.stdout
