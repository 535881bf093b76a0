"""GPU parity of the DiT-style block (block_type AE_BLOCK_DIT, through the C
ABI) against the oracle's DiT block (MolmoBot PR Part 2: the block hands the
cached context K/V to its second attention; the correctness table lists
cross_attn and self_attn apart).

* MolmoBot-shaped expert (c4: 12 layers, 12/4 heads x 64, width 768), full
  depth and 10 steps, at the pages' 1621-1634 visible-token range: each
  request against the oracle at the bf16 contract (2e-2).
* Several requests with different visible counts, one of them with every
  prefix row masked (attn2 adds nothing), each against the oracle, and the
  batched result against each request run alone.
* Masked rows are never read: NaN garbage there gives bitwise the same
  actions.
* Pi0.5-shaped expert (8/1 heads x 256) at reduced depth.
* The context prepared on the GPU (ae_prepare_prefix, with the robot state)
  feeding the DiT block, against the oracle that re-projects every step.
* The DiT block never runs the whole-call kernel; graph replays equal direct
  launches bitwise.
"""

import dataclasses
import sys

import numpy as np
import pytest

from oracle import ae_oracle as O
from vla_flow_matching_amd import synth

import oracle_pool

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16)


class Dit:
    def __init__(self, w, W, extra=None, **cfg_kw):
        from vla_flow_matching_amd import binding
        self.w = w
        self.ex = binding.ActionExpert(binding.make_config(w, **cfg_kw))
        dev = binding.weights_to_device(W, w.dtype)
        if extra:
            dev.update(binding.weights_to_device(extra, w.dtype))
        self.ex.load_weights(dev)

    def run(self, K, V, m, x0, steps=None):
        self.ex.set_prefix_kv(bf16(K), bf16(V), torch.from_numpy(np.ascontiguousarray(m)).cuda())
        out = self.ex.denoise(torch.from_numpy(np.ascontiguousarray(x0)).cuda(),
                              self.w.n_steps if steps is None else steps)
        torch.cuda.synchronize()
        st = self.ex.stats()
        assert st["device_errors"] == 0
        assert st["persistent_calls"] == 0  # the DiT block runs the per-phase kernels
        return out.cpu().numpy()


def check(gpu, ref, tol, label):
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    say(f"[parity] {label}: max|gpu-oracle| = {err:.3e} (tol {tol:g}, |ref|max {np.abs(ref).max():.3f})")
    assert np.isfinite(gpu).all(), label
    assert err <= tol, label
    return err


def test_dit_molmobot_full():
    _need_gpu()
    w = synth.workload("c4", block="dit", batch=2)
    say("[case] DiT block, MolmoBot-shaped: 12 layers, 12/4 heads x 64, prefix 2048, 2 requests")
    W = synth.make_weights(w)
    m = synth.valid_masks(w, n_valid=(1622, 1635))
    K, V, _ = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    g = Dit(w, W)
    out = g.run(K, V, m, x0)
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(2))
    for b, (ref, _) in enumerate(refs):
        check(out[b:b + 1], ref, TOL_BF16, f"DiT c4 request {b} (n={int(m[b].sum())})")
    g.ex.close()


def test_dit_requests_empty_prefix_and_garbage():
    """Four requests (64 action rows), one with every prefix row masked;
    NaN in masked rows is bitwise invisible; batched == alone."""
    _need_gpu()
    w = synth.workload("c4", block="dit", batch=4, n_layers=3, n_steps=3, prefix_len=600)
    say("[case] DiT block, 4 requests (n = 600, 0, 417, 1), 3 layers, 3 steps")
    W = synth.make_weights(w)
    m = synth.valid_masks(w, n_valid=(600, 0, 417, 1))
    K, V, _ = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    g = Dit(w, W)
    out = g.run(K, V, m, x0)
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(4))
    for b, (ref, _) in enumerate(refs):
        check(out[b:b + 1], ref, TOL_BF16, f"DiT request {b} (n={int(m[b].sum())})")
    Kg, Vg = K.copy(), V.copy()
    synth.fill_garbage(w, Kg, Vg, m, "nan")
    assert np.array_equal(g.run(Kg, Vg, m, x0), out), "masked garbage changed the actions"
    g.ex.close()
    w1 = dataclasses.replace(w, batch=1)
    g1 = Dit(w1, W, max_batch=4)
    for b in range(4):
        alone = g1.run(K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1])
        d = float(np.abs(alone - out[b:b + 1]).max())
        say(f"[parity] DiT request {b} batched vs alone: {d:.3e}")
        assert d <= TOL_BF16
    g1.ex.close()


def test_dit_empty_prefix_is_attn1_and_mlp():
    """An empty prefix (prefix_len 0): attn2 has no key and adds nothing;
    against the oracle with no prefix."""
    _need_gpu()
    w = synth.workload("c4", block="dit", n_layers=2, n_steps=2, prefix_len=0)
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    g = Dit(w, W, max_prefix_len=64)
    out = g.run(K, V, m, x0)
    ref = O.Expert(W, O.Params.like(w)).denoise(x0, K, V, m, w.n_steps)
    check(out, ref, TOL_BF16, "DiT empty prefix")
    g.ex.close()


def test_dit_pi05_shaped():
    _need_gpu()
    w = synth.workload("c2", block="dit", n_layers=3, n_steps=3)
    say("[case] DiT block, Pi0.5-shaped: 8/1 heads x 256, prefix 712, 3 layers")
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    g = Dit(w, W)
    out = g.run(K, V, m, x0)
    ref = O.Expert(W, O.Params.like(w)).denoise(x0, K, V, m, w.n_steps)
    check(out, ref, TOL_BF16, "DiT Pi0.5-shaped")
    g.ex.close()


def test_dit_graph_equals_direct():
    _need_gpu()
    w = synth.workload("c4", block="dit", n_layers=2, n_steps=3, prefix_len=256)
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    a = Dit(w, W)
    b = Dit(w, W, use_graphs=False)
    first = a.run(K, V, m, x0)
    for _ in range(3):
        assert np.array_equal(a.run(K, V, m, x0), first)
    assert np.array_equal(b.run(K, V, m, x0), first)
    assert a.ex.stats()["graph_replays"] >= 3
    a.ex.close()
    b.ex.close()


def test_dit_with_prepared_context_and_state():
    """ae_prepare_prefix (context 2560 wide, 14-D state) feeding the DiT
    block, against the oracle re-projecting the context every step."""
    _need_gpu()
    w = synth.workload("c4", block="dit", batch=2, n_layers=3, n_steps=3, prefix_len=2047)
    Dc, S = 2560, 14
    say(f"[case] DiT block with GPU context preparation: context {Dc} wide, {S}-D state")
    W = synth.make_weights(w)
    CW = synth.make_context_weights(w, Dc, S)
    m = np.zeros((2, 2047), np.uint8)
    m[0, :1629] = 1
    m[1, :1600] = 1
    m[1, 700:760] = 0
    H, _ = synth.make_context(w, Dc, mask=m, garbage="nan")
    state = synth.make_state(w, S)
    x0 = synth.make_noise(w)
    g = Dit(w, W, extra=CW, max_prefix_len=2048, context_width=Dc, state_dim=S)
    g.ex.prepare_prefix(bf16(H), torch.from_numpy(m).cuda(), torch.from_numpy(state).cuda())
    out = g.ex.denoise(torch.from_numpy(x0).cuda(), w.n_steps).cpu().numpy()
    torch.cuda.synchronize()
    assert g.ex.stats()["device_errors"] == 0
    g.ex.close()
    L = w.n_layers
    wk = np.stack([CW[f"layers.{l}.ctx_k"] for l in range(L)]).astype(np.float64)
    wv = np.stack([CW[f"layers.{l}.ctx_v"] for l in range(L)]).astype(np.float64)
    E = O.Expert(W, O.Params.like(dataclasses.replace(w, batch=1)))
    for b in range(2):
        hs = O.encode_state(state[b:b + 1], CW["state_in.w"], CW["state_in.b"])

        def kv(l, _b, b=b, hs=hs):
            K, V, m2 = O.prepare_prefix(np.nan_to_num(H[l:l + 1, b:b + 1], nan=0.0), wk[l:l + 1], wv[l:l + 1],
                                        m[b:b + 1], w.n_kv_heads, w.rope_theta, hs)
            idx = np.nonzero(m2[0])[0]
            return K[0, 0, idx], V[0, 0, idx]

        n = np.array([int(m[b].sum()) + 1])
        ref = E.integrate(x0[b:b + 1], kv, n, w.n_steps)
        check(out[b:b + 1], ref, TOL_BF16, f"DiT prepared context request {b}")


def test_dit_past_one_row_tile():
    """The DiT block at 5 MolmoBot-shaped requests (80 action rows: several
    GEMM row tiles, and attention items of several requests), each request
    against the oracle."""
    _need_gpu()
    w = synth.workload("c4", block="dit", batch=5, n_layers=2, n_steps=2, prefix_len=512)
    say("[case] DiT block, 5 requests (80 action rows)")
    W = synth.make_weights(w)
    m = synth.valid_masks(w, n_valid=(512, 300, 17, 0, 450))
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    g = Dit(w, W)
    out = g.run(K, V, m, x0)
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(5))
    for b, (ref, _) in enumerate(refs):
        check(out[b:b + 1], ref, TOL_BF16, f"DiT request {b} of 5 (n={int(m[b].sum())})")
    g.ex.close()
