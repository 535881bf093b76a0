"""The allocation-free entry point ae_denoise_static (through the C ABI)
against ae_denoise on the same handle and inputs: the same kernels with
their scratch in the library's static device array instead of the handle's.

Two calls in a row, the second with a smaller input, on the whole-call
kernel (batch * T <= 64) and on the per-phase kernels; the results must equal
ae_denoise's (the same kernels, plans and reduction orders: bitwise), and the
device's free memory must not move across the static calls.  A call whose
scratch exceeds the static array is rejected with AE_ERR_UNSUPPORTED."""

import dataclasses
import sys

import numpy as np
import pytest

from vla_flow_matching_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(ex, w, K, V, m, x0, static):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ex.set_prefix_kv(torch.from_numpy(np.ascontiguousarray(K)).to("cuda", dt),
                     torch.from_numpy(np.ascontiguousarray(V)).to("cuda", dt),
                     torch.from_numpy(np.ascontiguousarray(m)).cuda())
    x = torch.from_numpy(np.ascontiguousarray(x0)).cuda()
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    ex.denoise(x, w.n_steps, out=out, static_scratch=static)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert ex.stats()["device_errors"] == 0
    return out.cpu().numpy(), free0 - free1


@pytest.mark.parametrize("name,first,second,fields", [
    # whole-call kernel: 3 requests (48 rows), then 1
    ("c4", 3, 1, dict(n_layers=2, n_steps=3)),
    # per-phase kernels: 3 requests of 50 rows, then 2
    ("c5", 3, 2, dict(n_layers=2, n_steps=2, prefix_len=640)),
    # fp32 whole-call kernel: 8 requests (64 rows), then 2
    ("c1", 8, 2, dict()),
    # the DiT-style block (per-phase kernels, split K at 16-row requests): 2 requests, then 1
    ("c4dit", 2, 1, dict(n_layers=2, n_steps=2)),
    # row-wise e4m3 with the fp8 output projection: 3 requests, then 1
    ("c5fp8r", 3, 1, dict(n_layers=2, n_steps=2, prefix_len=640)),
])
def test_static_equals_denoise(name, first, second, fields):
    from vla_flow_matching_amd import binding
    _need_gpu()
    wmax = synth.workload(name, batch=first, **fields)
    say(f"[case] ae_denoise_static vs ae_denoise: {name} batch {first} then {second}")
    W = synth.make_weights(wmax)
    # (the cases named for the whole-call kernel ask for it; the rest run
    # the per-phase kernels whatever the path)
    with binding.ActionExpert(binding.make_config(wmax, exec_path=binding.AE_PATH_WHOLE_CALL)) as ex:
        ex.load_weights(binding.weights_to_device(W, wmax.dtype))
        for b in (first, second):
            w = dataclasses.replace(wmax, batch=b)
            m = synth.valid_masks(w)
            K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
            x0 = synth.make_noise(w)
            ref, _ = _run(ex, w, K, V, m, x0, static=False)
            got, grown = _run(ex, w, K, V, m, x0, static=True)
            again, grown2 = _run(ex, w, K, V, m, x0, static=True)
            err = float(np.abs(got - ref).max())
            say(f"[no-alloc] {name} batch {b}: max|static - denoise| = {err:.3e}; "
                f"device memory taken by the static calls: {grown} / {grown2} bytes")
            assert np.isfinite(got).all()
            assert np.array_equal(got, ref)
            assert np.array_equal(again, ref)
            assert grown2 == 0


def test_static_rejects_oversize_scratch():
    """The per-phase attention of 32 Pi0.5-shaped requests keeps two key
    splits of partials per query group: ~30 MB, past the 24 MiB array."""
    from vla_flow_matching_amd import binding
    _need_gpu()
    w = synth.workload("c5", batch=32, n_layers=1, n_steps=1, prefix_len=700)
    say("[case] ae_denoise_static: a call whose scratch exceeds the static array")
    W = synth.make_weights(w)
    with binding.ActionExpert(binding.make_config(w)) as ex:
        ex.load_weights(binding.weights_to_device(W, w.dtype))
        m = np.ones((32, 700), np.uint8)
        K = torch.zeros((1, 32, 700, 1, 256), dtype=torch.bfloat16, device="cuda")
        ex.set_prefix_kv(K, K, torch.from_numpy(m).cuda())
        x = torch.zeros((32, 50, 32), dtype=torch.float32, device="cuda")
        with pytest.raises(binding.AeError) as e:
            ex.denoise(x, 1, static_scratch=True)
        assert e.value.status == binding.AE_ERR_UNSUPPORTED
        say(f"[no-alloc] rejected: {e.value}")
        out = ex.denoise(x, 1)  # the allocating entry point still serves it
        torch.cuda.synchronize()
        assert torch.isfinite(out).all().item()
