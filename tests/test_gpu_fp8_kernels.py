"""The fp8 e4m3 projection path piece by piece on the GPU (test-only entry
points, include/ae_testing.h) against the oracle on identical codes and
scales (MolmoBot PR Part 3: per-tensor dynamic fp8, amax -> cast -> scaled
matmul; LoongForge blog section 7).

* The quantiser: bit-exact codes and scales per request, including exact
  midpoints between e4m3 values (ties to even), the subnormal range and an
  all-zero request.
* The adaRMS-then-quantise pass: the GPU's fp32 u against the oracle's fp64
  u may only differ at near-ties: almost every code equal, the others one
  code step apart.
* The down, gate/up and q|k|v products through their own epilogues, fed the
  oracle's activation codes: element-wise against (codes_x . codes_w) s_x s_w
  with each logical tensor's own scale.  The products of e4m3 codes are
  exact; the sum over K is accumulated in fp32 in an order the MFMA units
  choose, so an output may differ by a small multiple of fp32 rounding of
  the sum of its terms' magnitudes: the bound is 2^-16 of that sum (256
  fp32 ulps of it; the measured error is below a tenth of the bound).  A
  wrong scale, weight code or column pairing moves outputs by far more
  (by 1e-3 of |y| and up).  The q|k|v outputs are stored as bf16, so half a
  bf16 ulp (at most 2^-8 relative: 8 significant bits) is added there.

These take the whole loop's amplification out of the fp8 check: a wrong
scale, code or column pairing shows up directly."""

import ctypes
import sys

import numpy as np
import pytest

from oracle import ae_oracle as O

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    L = binding.load()
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.aetest_fp8_quantize.argtypes = [vp, ci, ci, ci, vp, vp, vp]
    L.aetest_fp8_norm_quantize.argtypes = [vp, ci, ci, ci, vp, vp, cf, vp, vp, vp, vp]
    L.aetest_fp8_down.argtypes = [vp, vp, ci, ci, vp, ci, vp, vp, ci, vp]
    L.aetest_fp8_gate_up.argtypes = [vp, vp, ci, ci, vp, vp, ci, vp, vp, ci, vp]
    L.aetest_fp8_qkv.argtypes = [vp, vp, ci, ci, vp, vp, vp, ci, ci, ci, vp, vp, vp, vp, ci, vp]
    for f in ("aetest_fp8_quantize", "aetest_fp8_norm_quantize", "aetest_fp8_down", "aetest_fp8_gate_up",
              "aetest_fp8_qkv"):
        getattr(L, f).restype = ci
    return L


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def decode(codes_u8):
    """e4m3 bytes (torch uint8, device) -> float64 values on the host."""
    return codes_u8.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()


def encode(values):
    """float64 e4m3 values (exactly representable) -> uint8 bytes on the device."""
    t = torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn)
    back = t.to(torch.float64).numpy()
    assert np.array_equal(back, np.asarray(values, np.float64)), "not e4m3 values"
    return t.view(torch.uint8).cuda()


def bf16_weight(rng, K, N, scale=1.0):
    """Random weights as bf16 (torch, device) and the same values as fp32."""
    w = (rng.standard_normal((K, N)).astype(np.float32) * np.float32(0.02 * scale))
    t = torch.from_numpy(w).to(torch.bfloat16)
    return t.cuda(), t.to(torch.float32).numpy()


def oracle_codes(x, T):
    """Per-request codes (float64 values) and fp32 scales of x [M][K]."""
    M = x.shape[0]
    codes = np.empty(x.shape)
    sx = np.empty(M, np.float32)
    for r0 in range(0, M, T):
        c, s = O.quantize_tensor(x[r0:r0 + T])
        codes[r0:r0 + T] = c
        sx[r0:r0 + T] = np.float32(s)
    return codes, sx


def e4m3_values():
    v = sorted({float(x) for x in torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn)
                .to(torch.float64)})
    return np.array(v)


def test_quantizer_bit_exact(lib):
    rng = np.random.default_rng(21)
    T, K = 50, 4096
    # request 0: N(0, 1); 1: N(0, 100^2); 2: amax 448 (multiplier exactly 1)
    # holding every e4m3 value and every midpoint between neighbours (ties to
    # even), subnormals included; 3: all zero (amax floor)
    x = np.zeros((4 * T, K), np.float32)
    x[:T] = rng.standard_normal((T, K))
    x[T:2 * T] = rng.standard_normal((T, K)) * 100
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    special = np.concatenate([vals, mids, -vals, -mids]).astype(np.float32)
    blk = np.resize(special, (T, K))
    blk[0, 0] = 448.0
    x[2 * T:3 * T] = blk
    xt = dev(x)
    codes = torch.empty((4 * T, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty(4 * T, dtype=torch.float32, device="cuda")
    assert lib.aetest_fp8_quantize(ptr(xt), 4 * T, K, T, ptr(codes), ptr(sx), stream()) == 0
    want_codes, want_sx = oracle_codes(x, T)
    got = decode(codes)
    bad = int((got != want_codes).sum())
    say(f"[fp8] quantiser: {bad} of {got.size} codes differ; scales {sx[::T].tolist()}")
    assert bad == 0
    assert np.array_equal(sx.cpu().numpy(), want_sx)
    assert np.all(got[3 * T:] == 0)


def test_quantizer_rejects_bad_sizes(lib):
    z = torch.zeros(64, dtype=torch.float32, device="cuda")
    c = torch.zeros(64, dtype=torch.uint8, device="cuda")
    assert lib.aetest_fp8_quantize(ptr(z), 1, 63, 1, ptr(c), ptr(z), stream()) == 1
    assert lib.aetest_fp8_quantize(ptr(z), 3, 64, 2, ptr(c), ptr(z), stream()) == 1


@pytest.mark.parametrize("T", [50, 1])
def test_norm_then_quantize(lib, T):
    """adaRMS rows then codes: the fp32 GPU u and the fp64 oracle u differ by
    rounding, so a code may differ only where u lands next to a midpoint.
    T = 1: the row-wise recipe (each row its own scale, the one-pass kernel)."""
    rng = np.random.default_rng(22)
    D, M = 1024, 150
    h = rng.standard_normal((M, D)).astype(np.float32) * np.float32(3.0)
    sc = (rng.standard_normal(D) * 0.3).astype(np.float32)
    sh = (rng.standard_normal(D) * 0.1).astype(np.float32)
    eps = 1e-6
    codes = torch.empty((M, D), dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    r = torch.empty(M, dtype=torch.float32, device="cuda")
    ht, sct, sht = dev(h), dev(sc), dev(sh)
    assert lib.aetest_fp8_norm_quantize(ptr(ht), M, D, T, ptr(sct), ptr(sht), eps, ptr(codes), ptr(sx), ptr(r),
                                        stream()) == 0
    u = O.ada_rms(h.astype(np.float64), sc.astype(np.float64), sh.astype(np.float64), eps)
    want_codes, want_sx = oracle_codes(u, T)
    r_ref = 1.0 / np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1) + eps)
    assert np.allclose(r.cpu().numpy(), r_ref, rtol=2e-6, atol=0)
    assert np.allclose(sx.cpu().numpy(), want_sx, rtol=2e-6, atol=0)
    got = decode(codes)
    diff = got != want_codes
    say(f"[fp8] norm + quantiser (T={T}): {int(diff.sum())} of {got.size} codes differ (near-ties)")
    assert diff.mean() <= 1e-3
    # a differing code is a neighbour: within one e4m3 step of the other
    vals = e4m3_values()
    gi = np.searchsorted(vals, np.abs(got[diff]))
    wi = np.searchsorted(vals, np.abs(want_codes[diff]))
    assert np.all(np.abs(gi - wi) <= 1) and np.all(np.sign(got[diff]) * np.sign(want_codes[diff]) >= 0)


ACC_REL = 2.0 ** -16  # of the sum of the terms' magnitudes (fp32 accumulation)


def product_ref(xcodes, sx, wf32, per_column=False):
    """(reference y, fp32 weight scale(s), per-element accumulation bound);
    per_column: the row-wise recipe's scale per weight column."""
    if per_column:
        wc, s_w = O.quantize_columns(wf32)
        scale = sx[:, None].astype(np.float64) * s_w[None, :]
        s_out = s_w.astype(np.float32)
    else:
        wc, s_w = O.quantize_tensor(wf32)
        scale = sx[:, None].astype(np.float64) * s_w
        s_out = np.float32(s_w)
    y = (xcodes @ wc) * scale
    mag = (np.abs(xcodes) @ np.abs(wc)) * scale
    return y, s_out, ACC_REL * mag + 1e-30


def worst(got, ref, bound):
    return float((np.abs(got - ref) / bound).max())


def col_spread(rng, wf, wt):
    """Give the weight columns widely different scales (so a per-tensor scale
    in place of per-column ones, or a column map error, shows)."""
    f = np.float32(2.0) ** rng.integers(-4, 5, size=wf.shape[1]).astype(np.float32)
    wf = (wf * f[None, :]).astype(np.float32)
    return torch.from_numpy(wf).to(torch.bfloat16).cuda(), wf


@pytest.mark.parametrize("M,per_column", [(100, 0), (800, 0), (800, 1)])
def test_down_product(lib, M, per_column):
    rng = np.random.default_rng(23)
    T, K, N = 50, 4096, 1024
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[T:2 * T] *= np.float32(7.0)
    xc, sxr = oracle_codes(x, 1 if per_column else T)
    wt, wf = bf16_weight(rng, K, N)
    if per_column:
        wt, wf = col_spread(rng, wf, wt)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sw = torch.empty(N if per_column else 1, dtype=torch.float32, device="cuda")
    assert lib.aetest_fp8_down(ptr(encode(xc)), ptr(dev(sxr)), M, K, ptr(wt), N, ptr(y), ptr(sw), per_column,
                               stream()) == 0
    ref, s_w, bound = product_ref(xc, sxr, wf, per_column)
    got = y.cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    w = worst(got, ref, bound)
    say(f"[fp8] down {M}x{K}x{N} ({'per column' if per_column else 'per tensor'}): max err {err:.2e} of max|y|; "
        f"worst error / bound {w:.3f}")
    assert np.array_equal(sw.cpu().numpy(), np.atleast_1d(s_w))
    assert w <= 1.0


@pytest.mark.parametrize("per_column", [0, 1])
def test_gate_up_product(lib, per_column):
    rng = np.random.default_rng(24)
    T, K, F, M = 50, 1024, 4096, 150
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[2 * T:] *= np.float32(0.1)
    xc, sxr = oracle_codes(x, 1 if per_column else T)
    wg, wgf = bf16_weight(rng, K, F)
    wu, wuf = bf16_weight(rng, K, F, scale=5.0)  # up's scale differs from gate's
    if per_column:
        wg, wgf = col_spread(rng, wgf, wg)
        wu, wuf = col_spread(rng, wuf, wu)
    act = torch.empty((M, F), dtype=torch.float32, device="cuda")
    sw = torch.empty(2 * F if per_column else 2, dtype=torch.float32, device="cuda")
    assert lib.aetest_fp8_gate_up(ptr(encode(xc)), ptr(dev(sxr)), M, K, ptr(wg), ptr(wu), F, ptr(act), ptr(sw),
                                  per_column, stream()) == 0
    g, sg, bg = product_ref(xc, sxr, wgf, per_column)
    u, su, bu = product_ref(xc, sxr, wuf, per_column)
    ref = O.gelu_tanh(g) * u
    # each factor within its own bound (|gelu'| <= 1.13), plus fp32 rounding
    # of the gelu (tanhf) and the product
    bound = 1.13 * np.abs(u) * bg + np.abs(O.gelu_tanh(g)) * bu + 4e-6 * np.abs(ref) + 1e-30
    got = act.cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    w = worst(got, ref, bound)
    say(f"[fp8] gate/up {M}x{K}x2*{F} ({'per column' if per_column else 'per tensor'}): max err {err:.2e} of "
        f"max|act|; worst error / bound {w:.3f}")
    assert np.array_equal(sw.cpu().numpy(), np.concatenate([np.atleast_1d(sg), np.atleast_1d(su)]))
    assert w <= 1.0


@pytest.mark.parametrize("Hq,Hkv,dh,per_column", [(8, 1, 256, 0), (12, 4, 64, 0), (8, 1, 256, 1),
                                                  (12, 4, 64, 1)])
def test_qkv_product(lib, Hq, Hkv, dh, per_column):
    rng = np.random.default_rng(25)
    K, M = 1024, 50
    x = rng.standard_normal((M, K)).astype(np.float32)
    xc, sxr = oracle_codes(x, 1 if per_column else M)
    wq, wqf = bf16_weight(rng, K, Hq * dh)
    wk, wkf = bf16_weight(rng, K, Hkv * dh, scale=3.0)
    wv, wvf = bf16_weight(rng, K, Hkv * dh, scale=0.25)
    if per_column:
        wq, wqf = col_spread(rng, wqf, wq)
        wk, wkf = col_spread(rng, wkf, wk)
        wv, wvf = col_spread(rng, wvf, wv)
    q = torch.empty((M, Hq * dh), dtype=torch.float32, device="cuda")
    k = torch.empty((M, Hkv * dh), dtype=torch.float32, device="cuda")
    v = torch.empty((M, Hkv * dh), dtype=torch.float32, device="cuda")
    sw = torch.empty((Hq + 2 * Hkv) * dh if per_column else 3, dtype=torch.float32, device="cuda")
    assert lib.aetest_fp8_qkv(ptr(encode(xc)), ptr(dev(sxr)), M, K, ptr(wq), ptr(wk), ptr(wv), Hq, Hkv, dh,
                              ptr(q), ptr(k), ptr(v), ptr(sw), per_column, stream()) == 0
    scales = []
    for name, got, wf in (("q", q, wqf), ("k", k, wkf), ("v", v, wvf)):
        ref, s, acc = product_ref(xc, sxr, wf, per_column)
        scales.append(s)
        g = got.cpu().numpy()
        # stored as bf16: half an ulp (<= 2^-8 relative) plus accumulation rounding
        bound = 2.0 ** -8 * np.abs(ref) + acc
        w = worst(g, ref, bound)
        say(f"[fp8] qkv {name} (Hq {Hq}, Hkv {Hkv}, dh {dh}, {'per column' if per_column else 'per tensor'}): "
            f"worst error / bound {w:.3f}")
        assert w <= 1.0, name
    assert np.array_equal(sw.cpu().numpy(), np.concatenate([np.atleast_1d(x) for x in scales]))
