"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/ae.h declares, rejects bad configs before touching HIP, and
reports the missing device as AE_ERR_HIP."""

import ctypes
import os
import re
import sys

import pytest

from vla_flow_matching_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="ae.h", prefix="ae_"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^\s*(?:ae_status|const char\*|void)\s+(" + prefix + r"\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from vla_flow_matching_amd import build
        build.build(verbose=False)
    return binding.load()


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_library_exports_test_entry_points(lib):
    """include/ae_testing.h: the test-only entry points of the fp8 path."""
    names = _declared("ae_testing.h", "aetest_")
    assert len(names) == 5
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.ae_status_string(0) == b"ok"
    assert lib.ae_status_string(2) == b"shape mismatch"
    assert lib.ae_status_string(99) == b"unknown status"


def _create(lib, **changes):
    cfg = binding.make_config(synth.workload("c1"))
    for k, v in changes.items():
        setattr(cfg, k, v)
    h = ctypes.c_void_p()
    st = lib.ae_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("width", 100), ("width", 0), ("n_kv_heads", 3), ("mlp_dim", 48),
    ("action_dim", 65), ("max_batch", 0), ("max_steps", 0), ("max_steps", 65),
    ("max_prefix_len", -1), ("act_dtype", 7), ("rope_theta", 0.0), ("use_graphs", 2),
    ("exec_path", 3), ("exec_path", -1),
])
def test_invalid_config_rejected_before_hip(lib, field, value):
    st, h = _create(lib, **{field: value})
    assert st == binding.AE_ERR_INVALID_ARGUMENT
    assert not h.value


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("head_dim", 32)])
def test_unsupported_config(lib, field, value):
    st, h = _create(lib, **{field: value})
    assert st == binding.AE_ERR_UNSUPPORTED
    assert not h.value


def test_fp8_projection_configs(lib):
    """fp8 e4m3 projections need bf16 activations and 128-multiple GEMM
    widths; a valid fp8 config passes every check and then finds no device."""
    st, h = _create(lib, proj_weight_dtype=binding.AE_FP8_E4M3)
    assert st == binding.AE_ERR_UNSUPPORTED and not h.value
    st, h = _create(lib, proj_weight_dtype=binding.AE_FP8_E4M3, act_dtype=binding.AE_BF16, width=192)
    assert st == binding.AE_ERR_UNSUPPORTED and not h.value
    st, h = _create(lib, proj_weight_dtype=binding.AE_FP8_E4M3, act_dtype=binding.AE_BF16)
    assert st == binding.AE_ERR_HIP and not h.value


def test_null_arguments(lib):
    assert lib.ae_create(None, None) == binding.AE_ERR_INVALID_ARGUMENT
    h = ctypes.c_void_p()
    assert lib.ae_create(None, ctypes.byref(h)) == binding.AE_ERR_INVALID_ARGUMENT
    assert lib.ae_load_weights(None, None, 0, None) == binding.AE_ERR_INVALID_ARGUMENT
    assert lib.ae_set_prefix_kv(None, 1, 0, None, None, None, None) == binding.AE_ERR_INVALID_ARGUMENT
    assert lib.ae_denoise(None, None, 1, 1, None, None) == binding.AE_ERR_INVALID_ARGUMENT
    assert lib.ae_get_stats(None, None) == binding.AE_ERR_INVALID_ARGUMENT
    lib.ae_destroy(None)


def test_no_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = _create(lib)
    assert st == binding.AE_ERR_HIP
    assert not h.value


@pytest.mark.parametrize("field,value", [("graph_cache_size", -1), ("graph_cache_size", 65),
                                         ("graph_cache_evict", 2)])
def test_invalid_graph_cache_config(lib, field, value):
    st, h = _create(lib, **{field: value})
    assert st == binding.AE_ERR_INVALID_ARGUMENT and not h.value


def _unopened(name="c2", **kw):
    """An ActionExpert whose argument checks run without a device handle:
    the binding checks shapes and dtypes before any pointer reaches the ABI."""
    ex = binding.ActionExpert.__new__(binding.ActionExpert)
    ex.lib = binding.load()
    ex.cfg = binding.make_config(synth.workload(name, **kw))
    ex.h = None
    return ex


def test_binding_rejects_wrong_prefix_shapes(lib):
    import torch
    ex = _unopened("c2", n_layers=2)
    L, P = 2, 712
    good = torch.zeros((L, 1, P, 1, 256), dtype=torch.bfloat16)
    mask = torch.ones((1, P), dtype=torch.uint8)
    cases = [
        (torch.zeros((L, 1, P, 1, 128), dtype=torch.bfloat16), good, mask),   # head_dim
        (torch.zeros((L + 1, 1, P, 1, 256), dtype=torch.bfloat16), good, mask),  # layers
        (good, torch.zeros((L, 1, P - 1, 1, 256), dtype=torch.bfloat16), mask),  # V shorter
        (good.float(), good, mask),                                            # dtype
        (good, good, torch.ones((1, P), dtype=torch.int32)),                   # mask dtype
        (good, good, torch.ones((P,), dtype=torch.uint8)),                     # mask rank
    ]
    for K, V, m in cases:
        with pytest.raises(binding.AeError) as e:
            ex.set_prefix_kv(K, V, m)
        assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH


def test_binding_rejects_wrong_noise_shapes(lib):
    import torch
    ex = _unopened("c2")
    for noise in (torch.zeros((1, 50, 31)), torch.zeros((1, 49, 32)), torch.zeros((50, 32)),
                  torch.zeros((1, 50, 32), dtype=torch.float64)):
        with pytest.raises(binding.AeError) as e:
            ex.denoise(noise, 10)
        assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH
    with pytest.raises(binding.AeError) as e:
        ex.denoise(torch.zeros((2, 50, 32)), 10, out=torch.zeros((1, 50, 32)))
    assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH


@pytest.mark.parametrize("changes", [
    dict(context_width=100), dict(context_width=-64), dict(context_width=8256),
    dict(state_dim=14),                      # a state needs a context width
    dict(context_width=64, state_dim=65),
])
def test_invalid_context_config(lib, changes):
    st, h = _create(lib, **changes)
    assert st == binding.AE_ERR_INVALID_ARGUMENT and not h.value


def test_context_needs_bf16(lib):
    st, h = _create(lib, context_width=128)  # the c1 workload is fp32
    assert st == binding.AE_ERR_UNSUPPORTED and not h.value


def test_dit_block_configs(lib):
    """The DiT-style block: block_type outside {0, 1} is invalid; it needs
    bf16 weights and projections and 128-multiple widths; the c2 shapes in
    bf16 pass every check and then find no device."""
    st, h = _create(lib, block_type=2)
    assert st == binding.AE_ERR_INVALID_ARGUMENT and not h.value
    st, h = _create(lib, block_type=binding.AE_BLOCK_DIT)  # the c1 workload is fp32
    assert st == binding.AE_ERR_UNSUPPORTED and not h.value
    cfg = binding.make_config(synth.workload("c2", block="dit"))
    assert cfg.block_type == binding.AE_BLOCK_DIT
    for k, v in (("proj_weight_dtype", binding.AE_FP8_E4M3), ("width", 960)):
        c = binding.make_config(synth.workload("c2", block="dit"))
        setattr(c, k, v)
        h = ctypes.c_void_p()
        assert lib.ae_create(ctypes.byref(c), ctypes.byref(h)) == binding.AE_ERR_UNSUPPORTED and not h.value
    h = ctypes.c_void_p()
    assert lib.ae_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.AE_ERR_HIP and not h.value


def test_fp8_rowwise_configs(lib):
    """Row-wise fp8 and the fp8 output projection: flags are 0 or 1, need fp8
    projections, and the fp8 output projection needs the row-wise recipe; a
    valid row-wise config passes every check and then finds no device."""
    base = dict(proj_weight_dtype=binding.AE_FP8_E4M3, act_dtype=binding.AE_BF16)
    for bad in (dict(fp8_rowwise=2), dict(fp8_oproj=-1), dict(fp8_rowwise=1, proj_weight_dtype=binding.AE_BF16,
                                                              act_dtype=binding.AE_BF16)):
        st, h = _create(lib, **{**base, **bad})
        assert st == binding.AE_ERR_INVALID_ARGUMENT and not h.value, bad
    st, h = _create(lib, **base, fp8_oproj=1)  # output projection without the row-wise recipe
    assert st == binding.AE_ERR_UNSUPPORTED and not h.value
    st, h = _create(lib, **base, fp8_rowwise=1, fp8_oproj=1)
    assert st == binding.AE_ERR_HIP and not h.value
    cfg = binding.make_config(synth.workload("c5fp8r"))
    assert cfg.fp8_rowwise == 1 and cfg.fp8_oproj == 1


def test_bench_refuses_to_report_after_device_errors(monkeypatch, capsys):
    """bench.py prints no JSON line and exits with status 3 when a timed
    workload reports device errors (a whole-call wait that timed out)."""
    import bench

    def boom(*a, **k):
        raise bench.DeviceErrors("c2: 1 whole-call launch(es) timed out; their results are invalid")

    monkeypatch.setattr(bench, "run_gpu", boom)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-cpu-baseline"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 3
    out = capsys.readouterr()
    assert '"metric"' not in out.out and "timed out" in out.err


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors of ae_config, ae_tensor_view and ae_stats have the
    C header's size and field offsets (a shorter Stats would let
    ae_get_stats write past the Python buffer)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"ae_config": binding.Config, "ae_tensor_view": binding.TensorView, "ae_stats": binding.Stats}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "ae.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([cc, "-I", os.path.join(root, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
