"""GPU parity of the HIP denoise loop (through the C ABI) against the CPU oracle.

Tolerances: max-abs 2e-2 on the actions for bf16 workloads (the contract;
the MolmoBot PR reports a bf16 padding delta of 0.0033 for context), 1e-4
for the fp32 workload.  Properties that hold bitwise on the GPU are checked
bitwise: compaction of the visible prefix rows makes masked / garbage /
pruned-slot inputs produce the same kernel inputs, and the kernels reduce in
fixed orders (graph replays, A-B-A, graph vs direct launches).
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
TOL_F32 = 1e-4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dt(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


# the paths a config can ask for (ae_path): the tests pick one where it
# matters; AE_PATH_AUTO is the library's default
AUTO, WHOLE_CALL, PER_PHASE = 0, 1, 2


class Gpu:
    """A library handle with one workload's weights loaded; unless a test
    says otherwise, calls that fit the whole-call kernel take it (the
    per-phase kernels take the rest)."""

    def __init__(self, w, W, **cfg_kw):
        from vla_flow_matching_amd import binding
        self.w = w
        cfg_kw.setdefault("exec_path", WHOLE_CALL)
        self.exec_path = cfg_kw["exec_path"]
        self.ex = binding.ActionExpert(binding.make_config(w, **cfg_kw))
        self.ex.load_weights(binding.weights_to_device(W, w.dtype))

    def run(self, K, V, m, x0, steps=None):
        dt = _dt(self.w)
        Kt = torch.from_numpy(np.ascontiguousarray(K)).to("cuda", dt)
        Vt = torch.from_numpy(np.ascontiguousarray(V)).to("cuda", dt)
        mt = torch.from_numpy(np.ascontiguousarray(m)).cuda()
        self.ex.set_prefix_kv(Kt, Vt, mt)
        x = torch.from_numpy(np.ascontiguousarray(x0)).cuda()
        out = self.ex.denoise(x, self.w.n_steps if steps is None else steps)
        torch.cuda.synchronize()
        assert self.ex.stats()["device_errors"] == 0, "a whole-call kernel wait timed out"
        return out.cpu().numpy()


def oracle(w, W, K, V, m, x0, steps=None):
    return O.Expert(W, O.Params.like(w)).denoise(x0, K, V, m, w.n_steps if steps is None else steps)


def check(gpu, ref, tol, label):
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    say(f"[parity] {label}: max|gpu-oracle| = {err:.3e} (tol {tol:g}, |ref|max {np.abs(ref).max():.3f})")
    assert np.isfinite(gpu).all(), label
    assert err <= tol, label
    return err


# --------------------------------------------------------------------------
# fixtures: one weight set per workload, shared by the tests
# --------------------------------------------------------------------------

@pytest.fixture(scope="module", params=[WHOLE_CALL, PER_PHASE], ids=["whole-call", "per-phase"])
def c1(request):
    _need_gpu()
    w = synth.workload("c1")
    W = synth.make_weights(w)
    return w, W, Gpu(w, W, exec_path=request.param)


@pytest.fixture(scope="module", params=[WHOLE_CALL, PER_PHASE], ids=["whole-call", "per-phase"])
def c2small(request):
    """The Pi0.5 shape at 2 layers, 2 steps, on each path."""
    _need_gpu()
    w = synth.workload("c2", n_layers=2, n_steps=2)
    W = synth.make_weights(w)
    return w, W, Gpu(w, W, max_prefix_len=1018, max_steps=4, exec_path=request.param)


@pytest.fixture(scope="module")
def c2full():
    """The Pi0.5 shape, the library's own choice of path (a step streams
    623 MB of layer weights, past the last-level cache: the whole-call
    kernel)."""
    _need_gpu()
    w = synth.workload("c2")
    W = synth.make_weights(w)
    return w, W, Gpu(w, W, max_prefix_len=1018, exec_path=AUTO)


# --------------------------------------------------------------------------
# parity
# --------------------------------------------------------------------------

def test_c1_fp32_parity(c1):
    w, W, g = c1
    say("[case] c1 fp32 full")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    check(g.run(K, V, m, x0), oracle(w, W, K, V, m, x0), TOL_F32, "c1")


def test_c1_fp32_batched_per_phase():
    """fp32 with 12 requests (96 action rows): past the whole-call kernel's
    64-row tile, so the per-phase kernels run (the fp32 GEMM, the attention
    kernel, action-in over 128 columns with half of each workgroup idle,
    action-out with one column per thread); every request against the
    oracle."""
    _need_gpu()
    w = synth.workload("c1", batch=12)
    say("[case] c1 fp32, 12 requests (per-phase kernels)")
    W = synth.make_weights(w)
    g = Gpu(w, W)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    check(g.run(K, V, m, x0), oracle(w, W, K, V, m, x0), TOL_F32, "c1 batch 12")


def test_c1_euler_closed_form(c1):
    """Constant-velocity head: x_N = x_0 + N dt v = x_0 - v."""
    w, W, g1 = c1
    say("[case] c1 constant-velocity head")
    W2 = dict(W)
    vel = np.random.default_rng(3).standard_normal(w.action_dim).astype(np.float32)
    W2["action_out.w"] = np.zeros_like(W["action_out.w"])
    W2["action_out.b"] = vel
    g = Gpu(w, W2, exec_path=g1.exec_path)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    out = g.run(K, V, m, x0)
    check(out, x0.astype(np.float64) - vel, 1e-5, "c1 euler closed form")


def test_c2_small_parity(c2small):
    w, W, g = c2small
    say("[case] c2 shape, 2 layers, 2 steps")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    check(g.run(K, V, m, x0), oracle(w, W, K, V, m, x0), TOL_BF16, "c2 small")


@pytest.mark.parametrize("n_valid", [520, 521, 575, 576, 577, 640, 711, 712])
def test_c2_ragged_valid_counts(c2small, n_valid):
    w, W, g = c2small
    say(f"[case] c2 small, n_valid={n_valid}")
    m = synth.valid_masks(w, n_valid=(n_valid,))
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, m == 0] = 0.0
    Vc[:, m == 0] = 0.0
    check(g.run(K, V, m, x0), oracle(w, W, Kc, Vc, m, x0), TOL_BF16, f"c2 n={n_valid}")


@pytest.mark.parametrize("steps", [1, 3])
def test_step_counts(c2small, steps):
    w, W, g = c2small
    say(f"[case] c2 small, steps={steps}")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    check(g.run(K, V, m, x0, steps), oracle(w, W, K, V, m, x0, steps), TOL_BF16, f"steps={steps}")


def test_empty_prefix(c2small):
    w, W, g = c2small
    say("[case] c2 small, empty prefix")
    w0 = synth.workload("c2", n_layers=2, n_steps=2, prefix_len=0)
    K = np.zeros((2, 1, 0, 1, 256), np.float32)
    m = np.zeros((1, 0), np.uint8)
    x0 = synth.make_noise(w)
    check(g.run(K, K, m, x0), oracle(w0, W, K, K, m, x0), TOL_BF16, "empty prefix")


def test_all_masked_prefix(c2small):
    w, W, g = c2small
    say("[case] c2 small, every prefix row masked")
    m = np.zeros((1, 712), np.uint8)
    K, V, _ = synth.make_prefix(w, mask=m, garbage="huge")
    x0 = synth.make_noise(w)
    check(g.run(K, V, m, x0), oracle(w, W, K, V, m, x0), TOL_BF16, "all masked")


@pytest.mark.parametrize("kind", ["nan", "inf", "huge"])
def test_masked_garbage_is_bitwise_invisible(c2small, kind):
    w, W, g = c2small
    say(f"[case] c2 small, {kind} in masked rows")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    clean = g.run(K, V, m, x0)
    Kg, Vg = K.copy(), V.copy()
    synth.fill_garbage(w, Kg, Vg, m, kind)
    assert np.array_equal(g.run(Kg, Vg, m, x0), clean)


def test_c2_full_parity(c2full):
    w, W, g = c2full
    say("[case] c2 full: 18 layers, 10 steps, bf16")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    before = g.ex.stats()["persistent_calls"]
    check(g.run(K, V, m, x0), oracle(w, W, K, V, m, x0), TOL_BF16, "c2 full")
    assert g.ex.stats()["persistent_calls"] == before + 1  # AE_PATH_AUTO's choice at this shape


@pytest.mark.parametrize("slot", [2, 1])
def test_c3_masked_slot_equals_c2_pruned(c2full, slot):
    """Three-camera prefix with one slot masked == the two-camera prefix
    (LoongForge blog section 1): bitwise on the GPU (the visible rows are
    compacted identically), and within tolerance of the oracle."""
    w2, W, g = c2full
    say(f"[case] c3 (slot {slot} masked) vs c2")
    w3 = synth.workload("c3")
    K2, V2, m2 = synth.make_prefix(w2)
    K3, V3, m3 = synth.insert_camera_slot(w3, K2, V2, m2, slot=slot, garbage="nan")
    x0 = synth.make_noise(w2)
    a2 = g.run(K2, V2, m2, x0)
    a3 = g.run(K3, V3, m3, x0)
    assert np.array_equal(a2, a3)
    if slot == 2:
        Kc, Vc = K3.copy(), V3.copy()
        Kc[:, m3 == 0] = 0
        Vc[:, m3 == 0] = 0
        check(a3, oracle(w3, W, Kc, Vc, m3, x0), TOL_BF16, "c3 vs oracle")


def test_c4_full_parity():
    _need_gpu()
    w = synth.workload("c4")
    say("[case] c4 full: 12 layers, 12/4 heads, head_dim 64, prefix 2048, both paths")
    W = synth.make_weights(w)
    # the library's choice (208 MB of layer weights, within the last-level
    # cache: the per-phase kernels) and the whole-call kernel
    auto, whole = Gpu(w, W, exec_path=AUTO), Gpu(w, W, exec_path=WHOLE_CALL)
    for n in (1622, 1628, 1635):  # the pages' 1621-1634 visible tokens, plus the state row
        m = synth.valid_masks(w, n_valid=(n,))
        K, V, _ = synth.make_prefix(w, mask=m)
        x0 = synth.make_noise(w)
        ref = oracle(w, W, K, V, m, x0)
        check(auto.run(K, V, m, x0), ref, TOL_BF16, f"c4 n={n} (per-phase kernels)")
        check(whole.run(K, V, m, x0), ref, TOL_BF16, f"c4 n={n} (whole-call kernel)")
    assert auto.ex.stats()["persistent_calls"] == 0
    assert whole.ex.stats()["persistent_calls"] == 3


@pytest.mark.parametrize("name,batch", [("c4", 4), ("c1", 8), ("c4", 3)])
def test_whole_call_kernel_several_requests(name, batch):
    """Batches whose action rows fit one 64-row tile (c4: 4 x 16, c1: 8 x 8,
    and a part-filled tile of 3 x 16) run the whole-call kernel: its
    per-request indexing (request of a row, each request's visible count and
    RoPE rows, one attention item per request and KV head) against the oracle
    for every request, and each request against the same one run alone."""
    _need_gpu()
    w = synth.workload(name, batch=batch)
    if name == "c4":
        w = synth.workload(name, batch=batch, n_layers=3, n_steps=3)
    say(f"[case] whole-call kernel, {name} x {batch} requests ({batch * w.action_horizon} rows)")
    W = synth.make_weights(w)
    g = Gpu(w, W)
    m = np.zeros((batch, w.prefix_len), np.uint8)
    for b in range(batch):  # different visible counts, the last request's with a hole
        m[b, :w.prefix_len - 7 * b - 1] = 1
        if b == batch - 1:
            m[b, 5:9] = 0
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    out = g.run(K, V, m, x0)
    st = g.ex.stats()
    assert st["persistent_calls"] >= 1, st
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(batch))
    for b, (ref, _) in enumerate(refs):
        check(out[b:b + 1], ref, tol, f"{name} request {b} of {batch} (n={int(m[b].sum())})")
    g1 = Gpu(dataclasses.replace(w, batch=1), W)
    for b in (0, batch - 1):
        alone = g1.run(K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1])
        err = float(np.abs(alone - out[b:b + 1]).max())
        say(f"[parity] {name} request {b}: batched vs alone {err:.3e}")
        assert err <= tol


@pytest.mark.parametrize("name,fields", [
    ("c2fp8r", dict(n_layers=2, n_steps=2)),              # fp8 projections
    ("c4dit", dict(n_layers=2, n_steps=2)),               # the DiT-style block
    ("c4", dict(batch=5, n_layers=2, n_steps=2)),         # 80 action rows
])
def test_whole_call_request_outside_its_reach(name, fields):
    """A handle that asks for the whole-call kernel runs the per-phase kernels
    for calls the whole-call kernel does not cover (fp8, the DiT block, more
    than 64 action rows): bitwise the same actions as the library's own
    choice, and no whole-call launch."""
    _need_gpu()
    w = synth.workload(name, **fields)
    say(f"[case] exec_path whole-call on {name} {fields}: the per-phase kernels")
    W = synth.make_weights(w)
    m = synth.valid_masks(w)
    K, V, _ = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    forced, auto = Gpu(w, W, exec_path=WHOLE_CALL), Gpu(w, W, exec_path=AUTO)
    a, b = forced.run(K, V, m, x0), auto.run(K, V, m, x0)
    assert forced.ex.stats()["persistent_calls"] == 0
    assert np.array_equal(a, b)


def test_graph_cache_lru_and_capacity(c2small):
    """The bounded graph cache (sglang PR summary, items 3 and 5): capacity 2
    with eviction keeps the two most recently used signatures, evicts the
    least recently used one and counts hits, misses and evictions; capacity 0
    captures nothing; a full cache without eviction runs new signatures
    directly.  Every result is bitwise that of direct launches."""
    w, W, g = c2small
    path = g.exec_path  # (every handle here on the fixture's path: results compared bitwise)
    say("[case] graph cache: LRU eviction, zero capacity, no-evict fallback")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    direct = Gpu(w, W, max_prefix_len=1018, max_steps=4, use_graphs=False, exec_path=path)
    want = {n: direct.run(K, V, m, x0, n) for n in (1, 2, 3)}
    lru = Gpu(w, W, max_prefix_len=1018, max_steps=4, graph_cache_size=2, exec_path=path)
    for n in (1, 2, 1, 3, 1, 2):  # misses 1, 2; hit 1; miss 3 evicts 2; hit 1; miss 2 evicts 3
        assert np.array_equal(lru.run(K, V, m, x0, n), want[n]), n
    st = lru.ex.stats()
    say(f"[stats] {st}")
    assert (st["graph_hits"], st["graph_misses"], st["graph_evictions"]) == (2, 4, 2)
    assert st["graph_captures"] == 4 and st["graphs_cached"] == 2 and st["eager_runs"] == 0
    off = Gpu(w, W, max_prefix_len=1018, max_steps=4, graph_cache_size=0, exec_path=path)
    assert np.array_equal(off.run(K, V, m, x0, 2), want[2])
    st = off.ex.stats()
    assert st["graph_captures"] == 0 and st["eager_runs"] == 1
    full = Gpu(w, W, max_prefix_len=1018, max_steps=4, graph_cache_size=1, graph_cache_evict=False,
               exec_path=path)
    for n in (2, 3, 2):
        assert np.array_equal(full.run(K, V, m, x0, n), want[n]), n
    st = full.ex.stats()
    assert (st["graph_captures"], st["graph_hits"], st["graph_evictions"], st["eager_runs"]) == (1, 1, 0, 1)


def test_prefix_buckets(c2small):
    """Prefix buckets (sglang PR summary, items 4-5): a prefix takes the
    smallest bucket that holds it, the key splits and the graph key follow
    the bucket, and the result matches the oracle (the split layout changes
    the rounding order only); bucket lists that are not strictly increasing
    or exceed the capacity are rejected and leave the handle unchanged."""
    from vla_flow_matching_amd import binding
    w, W, g0 = c2small
    say("[case] prefix buckets")
    g = Gpu(w, W, max_prefix_len=1018, max_steps=4, exec_path=g0.exec_path)
    g.ex.set_prefix_buckets([128, 576, 712])
    for bad in ([576, 576], [600, 128], [0, 64], [64, 2000]):
        with pytest.raises(binding.AeError) as e:
            g.ex.set_prefix_buckets(bad)
        assert e.value.status == binding.AE_ERR_INVALID_ARGUMENT
    x0 = synth.make_noise(w)
    for P, n, bucket in ((712, 600, 712), (560, 540, 576), (100, 100, 128), (900, 700, 1018)):
        wp = synth.workload("c2", n_layers=2, n_steps=2, prefix_len=P)
        mk = np.zeros((1, P), np.uint8)
        mk[0, :n] = 1
        K, V, _ = synth.make_prefix(wp, mask=mk, garbage="nan")
        out = g.run(K, V, mk, x0)
        st = g.ex.stats()
        assert st["prefix_bucket"] == bucket, st
        Kc, Vc = K.copy(), V.copy()
        Kc[:, mk == 0] = 0
        Vc[:, mk == 0] = 0
        check(out, oracle(wp, W, Kc, Vc, mk, x0), TOL_BF16, f"prefix {P} ({n} visible) in bucket {bucket}")
    assert g.ex.stats()["graph_captures"] == 4


def test_c5_batched_full():
    """16 requests with their own prefixes (valid 700..1024 of 1024): every
    request against the oracle run alone, and the batched rows against the
    same request run at batch 1 on the GPU."""
    _need_gpu()
    w = synth.workload("c5")
    say("[case] c5 full: batch 16, prefix 1024, bf16")
    W = synth.make_weights(w)
    g = Gpu(w, W)
    m = synth.valid_masks(w)
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    out = g.run(K, V, m, x0)
    assert np.isfinite(out).all()
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(w.batch))
    errs = []
    for b, (ref, _) in enumerate(refs):
        errs.append(check(out[b:b + 1], ref, TOL_BF16, f"c5 request {b} (n={int(m[b].sum())})"))
    say(f"[parity] c5 all {w.batch} requests: max {max(errs):.3e}")
    w1 = synth.workload("c5", batch=1)
    g1 = Gpu(w1, W)
    b = 7
    alone = g1.run(K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1])
    err = float(np.abs(alone - out[b:b + 1]).max())
    say(f"[parity] c5 batched vs alone, request {b}: {err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("name,batch", [("c5", 2), ("c5", 3), ("c5fp8", 3), ("c5fp8r", 3), ("c5fp8r", 1),
                                        ("c5fp8", 1), ("c2fp8r", 1)])
def test_batched_tiles_small(name, batch):
    """The batched path at reduced depth: 100 / 150 action rows leave a ragged
    32-row tile and a part-filled 8-row action-in group; every request
    against the oracle (fp8: the oracle's e4m3 emulation with per-request
    activation scales; c5fp8r: scales per row and per weight column, and the
    output projection in fp8 too).  Batch 1 runs the fp8 variants on a single
    request (fp8 never takes the whole-call kernel); c2fp8r is the c2 request
    (712-row prefix, 663 visible) in row-wise fp8.  With c2's weights the
    oracle's own output moves by 1.25e-2 when its noise is perturbed by a
    relative 1e-6 at this depth already, so that case is held to the derived
    fp8 tolerance (fp8_tolerance, here ~2.5e-2) and its error is printed
    against 2e-2."""
    _need_gpu()
    w = synth.workload(name, batch=batch, n_layers=2, n_steps=2)
    say(f"[case] {name} batch {batch}, 2 layers, 2 steps")
    W = synth.make_weights(w)
    g = Gpu(w, W)
    m = synth.valid_masks(w)
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, m == 0] = 0.0
    Vc[:, m == 0] = 0.0
    ref = oracle(w, W, Kc, Vc, m, x0)
    tol = fp8_tolerance(w, W, Kc, Vc, m, x0, ref) if name == "c2fp8r" else TOL_BF16
    err = check(g.run(K, V, m, x0), ref, tol, f"{name} batch {batch}")
    if tol > TOL_BF16:
        say(f"[fp8] {name}: {err:.3e} against the 2e-2 contract: {'within' if err <= TOL_BF16 else 'above'}")


_COVER = [(dt, dh, b, "same", 7) for dt in ("f32", "bf16") for dh in (64, 128, 256) for b in (1, 3)] + [
    ("bf16", 128, 3, "fp8", 7),    # fp8 projections away from the Pi0.5 shape
    ("bf16", 128, 1, "same", 40),  # action_dim above 32: the per-phase kernels at batch 1
]


@pytest.mark.parametrize("dtype,dh,batch,proj,adim", _COVER)
def test_head_dim_dtype_path_coverage(dtype, dh, batch, proj, adim):
    """Every head_dim and activation dtype the library accepts, on both
    paths (batch 1 x 24 rows: the whole-call kernel; batch 3 x 24 = 72 rows,
    or action_dim 40: the per-phase kernels), with grouped heads (4 query /
    2 KV) and a ragged prefix whose visible rows have a masked hole.  The
    gates' bias is raised to 0.5 so the residual branches carry weight: the
    prefix V then moves the actions by 0.3-0.6, and hiding one more key row
    moves them by 0.03-0.05, above the bf16 tolerance (with the plain
    initialisation the attention branch moves them by under 0.04)."""
    _need_gpu()
    w = synth.Workload("hd", n_layers=2, width=256, n_q_heads=4, n_kv_heads=2, head_dim=dh,
                       mlp_dim=512, action_horizon=24, action_dim=adim, n_steps=2, batch=batch,
                       prefix_len=150, dtype=dtype, proj_dtype=proj, index=7, gate_bias=0.5)
    label = f"{dtype} dh={dh} batch={batch} proj={proj} A={adim}"
    say(f"[case] {label}")
    W = synth.make_weights(w)
    m = np.zeros((batch, w.prefix_len), dtype=np.uint8)
    for b in range(batch):
        m[b, :40 + 17 * b] = 1
        m[b, 70:130 - 5 * b] = 1
    K, V, m = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    out = Gpu(w, W).run(K, V, m, x0)
    ref = oracle(w, W, K, V, m, x0)
    if proj == "fp8":
        tol = fp8_tolerance(w, W, K, V, m, x0, ref)
    else:
        tol = TOL_F32 if dtype == "f32" else TOL_BF16
    check(out, ref, tol, label)


_LIMITS = [
    # (label, workload fields): the largest action_dim, step count and width
    # the library accepts, on both paths
    ("A=64, 64 steps (per-phase kernels)",
     dict(n_layers=1, width=64, n_q_heads=1, n_kv_heads=1, head_dim=64, mlp_dim=64, action_horizon=8,
          action_dim=64, n_steps=64, batch=1, prefix_len=40)),
    ("A=32, 64 steps (whole-call kernel)",
     dict(n_layers=1, width=64, n_q_heads=1, n_kv_heads=1, head_dim=64, mlp_dim=64, action_horizon=8,
          action_dim=32, n_steps=64, batch=1, prefix_len=40)),
    ("width 4096 (whole-call kernel)",
     dict(n_layers=1, width=4096, n_q_heads=8, n_kv_heads=1, head_dim=128, mlp_dim=256, action_horizon=8,
          action_dim=7, n_steps=2, batch=1, prefix_len=40)),
    ("width 4096 (per-phase kernels)",
     dict(n_layers=1, width=4096, n_q_heads=8, n_kv_heads=1, head_dim=128, mlp_dim=256, action_horizon=8,
          action_dim=7, n_steps=2, batch=9, prefix_len=40)),
    # degenerate shapes: one action token of one dimension, heads not grouped
    ("T=1, A=1, MHA (whole-call kernel)",
     dict(n_layers=1, width=64, n_q_heads=2, n_kv_heads=2, head_dim=64, mlp_dim=64, action_horizon=1,
          action_dim=1, n_steps=3, batch=1, prefix_len=40)),
    ("T=1, A=1, MHA, batch 65 (per-phase kernels; requests 14+ see no prefix)",
     dict(n_layers=1, width=64, n_q_heads=2, n_kv_heads=2, head_dim=64, mlp_dim=64, action_horizon=1,
          action_dim=1, n_steps=3, batch=65, prefix_len=40)),
]


@pytest.mark.parametrize("label,fields", _LIMITS, ids=[c[0] for c in _LIMITS])
def test_size_limits(label, fields):
    """The configuration limits (action_dim 64, 64 Euler steps, width 4096)
    and degenerate shapes (one action token, ungrouped heads, requests with
    an empty prefix) against the oracle, with a ragged prefix (bf16)."""
    _need_gpu()
    w = synth.Workload("lim", dtype="bf16", proj_dtype="same", index=8, gate_bias=0.5, **fields)
    say(f"[case] {label}")
    W = synth.make_weights(w)
    m = np.zeros((w.batch, w.prefix_len), dtype=np.uint8)
    for b in range(w.batch):
        m[b, :max(0, w.prefix_len - 3 * b)] = 1
    K, V, m = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    out = Gpu(w, W).run(K, V, m, x0)
    ref = oracle(w, W, K, V, m, x0)
    check(out, ref, bf16_tolerance(w, W, K, V, m, x0, ref), label)


def bf16_tolerance(w, W, K, V, m, x0, ref):
    """The contract's bf16 tolerance, or, where a configuration is more
    sensitive to bf16 rounding than the named workloads (width 4096 with
    weighted residual branches), the oracle's own response to a relative
    2^-9 perturbation (half a bf16 ulp, random sign) of every weight: the
    size of the rounding the GPU applies to each product input.  At the
    c2 shape that response is ~7e-3, well inside the contract's figure."""
    rng = np.random.default_rng(12)
    W2 = {k: (v * (1.0 + 2.0 ** -9 * rng.choice([-1.0, 1.0], size=v.shape))).astype(v.dtype)
          for k, v in W.items()}
    floor = float(np.abs(oracle(w, W2, K, V, m, x0) - ref).max())
    say(f"[bf16] oracle response to a half-ulp weight perturbation: {floor:.3e}")
    return max(TOL_BF16, floor)


def fp8_tolerance(w, W, K, V, m, x0, ref):
    """Tolerance for a whole fp8 denoise call, derived from the arithmetic:
    every projection input is re-coded to e4m3 each layer, so a difference
    far below bf16 resolution upstream flips codes near rounding midpoints
    and the flips compound over layers and steps.  The oracle's own output
    moves by the returned floor / 2 when the noise is perturbed by a relative
    1e-6 (the bf16 loop moves by ~1e-6 under the same perturbation); an
    implementation whose intermediates differ from the oracle's by rounding
    is held to twice that floor, and never to less than the bf16 tolerance."""
    rng = np.random.default_rng(11)
    x1 = (x0 * (1.0 + 1e-6 * rng.standard_normal(x0.shape))).astype(np.float32)
    floor = float(np.abs(oracle(w, W, K, V, m, x1) - ref).max())
    say(f"[fp8] oracle response to a 1e-6 relative noise perturbation: {floor:.3e}")
    return max(TOL_BF16, 2.0 * floor)


@pytest.mark.parametrize("name", ["c5fp8", "c5fp8r"])
def test_c5_fp8_full(name):
    """c5 with e4m3 QKV / gate-up / down weights (static per tensor) and
    per-request dynamic activation scales (c5fp8r: a scale per weight column
    and per activation row, and the output projection in e4m3 too): every
    request against the oracle's emulation, and a request batched against
    the same one alone.

    Each request is held to twice the oracle's own response to a relative
    1e-6 perturbation of its noise (never less than 2e-2; see fp8_tolerance);
    the error is also reported against the 2e-2 contract itself, which the
    full-size fp8 loop does not meet for every request."""
    _need_gpu()
    w = synth.workload(name)
    say(f"[case] {name} full: batch 16, prefix 1024")
    W = synth.make_weights(w)
    g = Gpu(w, W)
    m = synth.valid_masks(w)
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    out = g.run(K, V, m, x0)
    assert np.isfinite(out).all()
    refs = oracle_pool.per_request(w, W, K, V, m, x0, range(w.batch), perturb=1e-6)
    tols, errs = [], []
    for b, (ref, floor) in enumerate(refs):
        tols.append(max(TOL_BF16, 2.0 * floor))
        say(f"[fp8] request {b}: oracle response to a 1e-6 relative noise perturbation {floor:.3e}")
        errs.append(check(out[b:b + 1], ref, tols[-1], f"{name} request {b} (n={int(m[b].sum())})"))
    over = [b for b, e in enumerate(errs) if e > TOL_BF16]
    say(f"[fp8] {name} all {w.batch} requests: max error {max(errs):.3e}; "
        f"{len(over)} of {w.batch} above the 2e-2 contract: {over}")
    w1 = synth.workload(name, batch=1)
    g1 = Gpu(w1, W)
    b = 7
    alone = g1.run(K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1])
    err = float(np.abs(alone - out[b:b + 1]).max())
    say(f"[parity] {name} batched vs alone, request {b}: {err:.3e} (tol {tols[b]:.3e})")
    assert err <= tols[b]


# --------------------------------------------------------------------------
# reproducibility (MolmoBot PR "Correctness": replay stability, A-B-A)
# --------------------------------------------------------------------------

def test_replay_stability(c2small):
    w, W, g = c2small
    say("[case] replay stability x20")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    first = g.run(K, V, m, x0)
    x = torch.from_numpy(x0).cuda()
    outs = [g.ex.denoise(x, w.n_steps) for _ in range(20)]
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), first)
    st = g.ex.stats()
    say(f"[stats] {st}")
    assert st["graph_replays"] + st["eager_runs"] >= 21
    assert st["device_errors"] == 0


def test_aba_stale_memory(c2small):
    w, W, g = c2small
    say("[case] A-B-A prefixes of different lengths")
    mA = synth.valid_masks(w, n_valid=(600,))
    KA, VA, _ = synth.make_prefix(w, mask=mA)
    w3 = synth.workload("c3", n_layers=2, n_steps=2)
    mB = np.zeros((1, 1018), np.uint8)
    mB[0, :900] = 1
    KB, VB, _ = synth.make_prefix(w3, mask=mB, seed=555)
    x0 = synth.make_noise(w)
    a1 = g.run(KA, VA, mA, x0)
    b1 = g.run(KB, VB, mB, x0)
    a2 = g.run(KA, VA, mA, x0)
    assert not np.array_equal(a1, b1)
    assert np.array_equal(a1, a2)


def test_graph_equals_direct_launch(c2small):
    w, W, g = c2small
    say("[case] graph replay vs direct launches")
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    direct = Gpu(w, W, max_prefix_len=1018, max_steps=4, use_graphs=False, exec_path=g.exec_path)
    assert np.array_equal(g.run(K, V, m, x0), direct.run(K, V, m, x0))
    assert direct.ex.stats()["graph_captures"] == 0
    # launches in the replayed graph: the whole-call kernel and its counter
    # fill, or several per layer; none reported for direct launches
    nodes = g.ex.stats()["graph_nodes"]
    assert nodes == 2 if g.ex.stats()["persistent_calls"] > 0 else nodes > 2 * w.n_layers * w.n_steps
    assert direct.ex.stats()["graph_nodes"] == 0


# --------------------------------------------------------------------------
# error conventions through the ABI
# --------------------------------------------------------------------------

def test_error_paths_leave_state_unchanged(c2small):
    from vla_flow_matching_amd import binding
    w, W, g = c2small
    say("[case] error paths")
    fresh = binding.ActionExpert(binding.make_config(w, max_prefix_len=1018, max_steps=4))
    x = torch.from_numpy(synth.make_noise(w)).cuda()
    with pytest.raises(binding.AeError) as e:
        fresh.denoise(x, 2)
    assert e.value.status == binding.AE_ERR_NOT_READY
    bad = binding.weights_to_device(W, w.dtype)
    bad["layers.1.o"] = bad["layers.1.o"][:, :512].contiguous()
    with pytest.raises(binding.AeError) as e:
        fresh.load_weights(bad)
    assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH
    del bad["layers.1.o"]
    with pytest.raises(binding.AeError) as e:
        fresh.load_weights(bad)
    assert e.value.status == binding.AE_ERR_INVALID_ARGUMENT
    # the loaded handle: a wrong batch, too many steps, an oversize prefix
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    ref = g.run(K, V, m, x0)
    x2 = torch.from_numpy(np.concatenate([x0, x0])).cuda()
    with pytest.raises(binding.AeError) as e:
        g.ex.denoise(x2, 2)
    assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH
    with pytest.raises(binding.AeError) as e:
        g.ex.denoise(torch.from_numpy(x0).cuda(), 5)
    assert e.value.status == binding.AE_ERR_INVALID_ARGUMENT
    big = torch.zeros((2, 1, 1100, 1, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.AeError) as e:
        g.ex.set_prefix_kv(big, big, torch.ones((1, 1100), dtype=torch.uint8, device="cuda"))
    assert e.value.status == binding.AE_ERR_SHAPE_MISMATCH
    # K / V of the right shape and dtype but 2 bytes off a 16-byte boundary
    n = int(np.prod(K.shape))
    flat = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")
    Kmis = flat[1:n + 1].view(K.shape)
    assert Kmis.is_contiguous() and Kmis.data_ptr() % 16 != 0
    with pytest.raises(binding.AeError) as e:
        g.ex.set_prefix_kv(Kmis, Kmis, torch.from_numpy(m).cuda())
    assert e.value.status == binding.AE_ERR_INVALID_ARGUMENT
    out = g.ex.denoise(torch.from_numpy(x0).cuda(), 2)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
