"""The key-block K / V cache layout (KvLayout, vla_flow_matching_amd/csrc/
ae_device.h) checked on the host: a bijection onto the cache that keeps keys
in their blocks and matches the fragment views the attention kernels read
(tests/host/kv_layout_check.cpp).  Host code only; needs hipcc, no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_kv_layout_host(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "kv_layout_check")
    src = os.path.join(ROOT, "tests", "host", "kv_layout_check.cpp")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "vla_flow_matching_amd", "csrc"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "violations: 0" in r.stdout
