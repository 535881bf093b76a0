"""The C ABI's host-side argument validation under AddressSanitizer and
UBSan: every HIP source of the library is compiled with the sanitizers on
its host code only (the device code is built as usual), linked with
tests/host/abi_validation_check.cpp, and run.  It drives every entry point's
checks that must reject a call before any HIP work (invalid and unsupported
configs, null arguments, out-of-range enumerator values), so it needs no GPU:
a valid config then ends in AE_ERR_HIP (or, with a GPU, in a handle that is
created and destroyed).  Any sanitizer report fails the test."""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vla_flow_matching_amd", "csrc")
SOURCES = ["ae_gemm", "ae_tgemm", "ae_attention", "ae_misc", "ae_persist", "ae_runtime", "ae_testing"]


def _tool(*names):
    for n in names:
        if n and os.path.exists(n):
            return n
    return None


def test_abi_validation_under_host_sanitizers(tmp_path):
    hipcc = _tool(os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc") or "")
    clang = _tool("/opt/rocm/llvm/bin/clang++")
    if hipcc is None or clang is None:
        pytest.skip("no HIP toolchain")
    # sanitizers on the host side of each HIP source only
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(name):
        obj = str(tmp_path / f"{name}.o")
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] if name == "ae_attention" else []
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
               "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    check_obj = str(tmp_path / "check.o")
    exe = str(tmp_path / "abi_validation_check")
    r = subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "host", "abi_validation_check.cpp"), "-o", check_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([clang, "-fsanitize=address,undefined", check_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "failed checks: 0" in r.stdout
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
