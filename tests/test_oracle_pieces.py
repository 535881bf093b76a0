"""Pins of the oracle's pieces against closed forms and library routines.

Each test fixes a fact the oracle must get right independently of how the
oracle itself computes it: a textbook identity, a value at a special point, or
a PyTorch float64 routine that computes the same definition by another route.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ae_oracle as O

RNG = np.random.default_rng(12345)


# --------------------------------------------------------------------------
# Euler grid (spec update x += dt * v; t from 1 to 0)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 4, 10, 37])
def test_timestep_grid_endpoints(n):
    t, dt = O.timestep_grid(n)
    assert t[0] == 1.0
    assert t[-1] == pytest.approx(1.0 / n, abs=0)
    assert dt * n == pytest.approx(-1.0, abs=1e-15)
    # consecutive grid points differ by exactly |dt| (t_k = t_0 + k dt)
    assert np.allclose(np.diff(t), dt, atol=1e-15)


# --------------------------------------------------------------------------
# Sinusoidal time embedding
# --------------------------------------------------------------------------

def test_sinusoid_at_zero_is_zeros_then_ones():
    e = O.sinusoid(np.array([0.0]), 128)[0]
    assert np.array_equal(e[:64], np.zeros(64))
    assert np.array_equal(e[64:], np.ones(64))


def test_sinusoid_period_endpoints():
    D = 256
    half = D // 2
    # channel 0 has period 4e-3: one full turn at t = 4e-3
    e = O.sinusoid(np.array([4e-3]), D)[0]
    assert abs(e[0]) < 1e-12 and abs(e[half] - 1.0) < 1e-12
    # the last channel has period 4.0: a quarter turn at t = 1
    e = O.sinusoid(np.array([1.0]), D)[0]
    assert abs(e[half - 1] - 1.0) < 1e-12 and abs(e[D - 1]) < 1e-12
    # periods are geometric: channel i has period 4e-3 * 1000^(i/(half-1))
    i = 37
    period = 4e-3 * 1000.0 ** (i / (half - 1))
    e = O.sinusoid(np.array([period / 4]), D)[0]
    assert abs(e[i] - 1.0) < 1e-12


def test_sinusoid_unit_circle():
    t = RNG.uniform(0, 1, 9)
    e = O.sinusoid(t, 64)
    assert np.allclose(e[:, :32] ** 2 + e[:, 32:] ** 2, 1.0, atol=1e-14)


# --------------------------------------------------------------------------
# Activations, linear layout, norm
# --------------------------------------------------------------------------

def test_silu_matches_torch():
    x = RNG.standard_normal(1000) * 6
    assert np.allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=0, atol=1e-14)


def test_gelu_tanh_matches_torch():
    x = RNG.standard_normal(1000) * 6
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(O.gelu_tanh(x), ref, rtol=0, atol=1e-14)
    # and it is the tanh form, not the erf form
    erf = F.gelu(torch.from_numpy(x)).numpy()
    assert np.abs(O.gelu_tanh(x) - erf).max() > 1e-5


def test_linear_is_in_by_out():
    """Weights are stored [in, out]: a single 1 at W[i, j] copies input i to output j."""
    x = RNG.standard_normal((3, 5))
    W = np.zeros((5, 7))
    W[2, 6] = 1.0
    y = O.linear(x, W, np.arange(7.0))
    assert np.array_equal(y[:, 6], x[:, 2] + 6.0)
    assert np.array_equal(y[:, :6], np.broadcast_to(np.arange(6.0), (3, 6)))


def test_ada_rms_matches_torch_rms_norm():
    h = RNG.standard_normal((6, 96)) * 3
    scale = RNG.standard_normal(96) * 0.1
    shift = RNG.standard_normal(96) * 0.1
    ref = F.rms_norm(torch.from_numpy(h), (96,), eps=1e-6).numpy() * (1 + scale) + shift
    assert np.allclose(O.ada_rms(h, scale, shift, 1e-6), ref, rtol=0, atol=1e-13)


def test_ada_rms_scale_invariant_and_shift_only_when_h_zero():
    h = RNG.standard_normal((4, 64))
    s, b = RNG.standard_normal(64), RNG.standard_normal(64)
    a1 = O.ada_rms(h, s, b, 0.0)
    a2 = O.ada_rms(7.5 * h, s, b, 0.0)
    assert np.allclose(a1, a2, atol=1e-13)
    assert np.array_equal(O.ada_rms(np.zeros((2, 64)), s, b, 1e-6), np.broadcast_to(b, (2, 64)))


def test_time_condition_structure():
    """Two linears with bias, SiLU after each: with one-hot weights the chain
    reduces to silu(silu(e_i + b1_j) + b2_k) on the chosen channels."""
    D = 16
    W = {k: np.zeros(s) for k, s in {"time_mlp.1.w": (D, D), "time_mlp.1.b": (D,),
                                      "time_mlp.2.w": (D, D), "time_mlp.2.b": (D,)}.items()}
    W["time_mlp.1.w"][3, 5] = 1.0
    W["time_mlp.1.b"][5] = 0.25
    W["time_mlp.2.w"][5, 9] = 2.0
    W["time_mlp.2.b"][9] = -0.5
    t = np.array([0.3, 0.9])
    e = O.sinusoid(t, D)
    c = O.time_condition(t, W)
    silu = lambda z: z / (1 + np.exp(-z))
    assert np.allclose(c[:, 9], silu(2.0 * silu(e[:, 3] + 0.25) - 0.5), atol=1e-15)
    # channels with zero weights and bias sit at silu(silu(0) * 0 + 0) = 0
    assert np.array_equal(c[:, 0], np.zeros(2))


# --------------------------------------------------------------------------
# RoPE (rotate_half form)
# --------------------------------------------------------------------------

def test_rope_is_complex_rotation():
    """(x_j, x_{j+dh/2}) as the complex number x_j + i x_{j+dh/2}, multiplied by e^{i phi}."""
    dh, T = 64, 11
    x = RNG.standard_normal((T, 3, dh))
    pos = RNG.integers(0, 3000, T)
    cos, sin = O.rope_cos_sin(pos, dh, 10000.0)
    y = O.apply_rope(x, cos, sin)
    z = (x[..., :32] + 1j * x[..., 32:]) * np.exp(1j * (pos[:, None] * 10000.0 ** (-np.arange(32) / 32)))[:, None, :]
    assert np.allclose(y[..., :32], z.real, atol=1e-11)
    assert np.allclose(y[..., 32:], z.imag, atol=1e-11)


def test_rope_frequencies_closed_form():
    # theta^(-2j/dh) with theta = 1e4, dh = 64: j=0 -> 1 rad per position, j=16 -> 0.01
    cos, sin = O.rope_cos_sin(np.array([1.0, 100.0]), 64, 10000.0)
    assert math.isclose(math.atan2(sin[0, 0], cos[0, 0]), 1.0, abs_tol=1e-14)
    assert math.isclose(math.atan2(sin[0, 16], cos[0, 16]), 0.01, abs_tol=1e-14)
    assert math.isclose(math.atan2(sin[1, 16], cos[1, 16]), 1.0, abs_tol=1e-12)


def test_rope_identity_norm_relative():
    dh = 256
    q = RNG.standard_normal((1, 1, dh))
    k = RNG.standard_normal((1, 1, dh))
    c0, s0 = O.rope_cos_sin(np.array([0]), dh, 10000.0)
    assert np.array_equal(O.apply_rope(q, c0, s0), q)
    dots = []
    for p in (0, 17, 900):
        cq, sq = O.rope_cos_sin(np.array([p + 5]), dh, 10000.0)
        ck, sk = O.rope_cos_sin(np.array([p]), dh, 10000.0)
        rq, rk = O.apply_rope(q, cq, sq), O.apply_rope(k, ck, sk)
        assert np.isclose(np.linalg.norm(rq), np.linalg.norm(q), rtol=1e-13)
        dots.append(float((rq * rk).sum()))
    assert np.allclose(dots, dots[0], atol=1e-10)


# --------------------------------------------------------------------------
# Masked GQA attention vs torch SDPA (float64, boolean mask, enable_gqa)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,dh,P,T", [(8, 1, 32, 40, 6), (12, 4, 16, 33, 5), (2, 1, 64, 64, 8), (4, 4, 8, 7, 3)])
def test_attention_matches_torch_sdpa(Hq, Hkv, dh, P, T):
    q = RNG.standard_normal((T, Hq, dh))
    kp = RNG.standard_normal((P, Hkv, dh))
    vp = RNG.standard_normal((P, Hkv, dh))
    ka = RNG.standard_normal((T, Hkv, dh))
    va = RNG.standard_normal((T, Hkv, dh))
    mask = RNG.integers(0, 2, P).astype(bool)
    mask[0] = True
    keys = np.concatenate([kp[mask], ka])
    vals = np.concatenate([vp[mask], va])
    ours = O.attention(q, keys, vals)
    # torch: full padded key set, boolean mask over [prefix | actions]
    Kt = torch.from_numpy(np.concatenate([kp, ka])).permute(1, 0, 2)[None]
    Vt = torch.from_numpy(np.concatenate([vp, va])).permute(1, 0, 2)[None]
    Qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    am = torch.from_numpy(np.concatenate([mask, np.ones(T, bool)]))[None, None, None, :].expand(1, Hq, T, P + T)
    ref = F.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=am, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(ours, ref, rtol=0, atol=1e-12)


def test_attention_single_key_returns_its_value():
    q = RNG.standard_normal((4, 2, 8))
    k = RNG.standard_normal((1, 1, 8))
    v = RNG.standard_normal((1, 1, 8))
    o = O.attention(q, k, v)
    assert np.array_equal(o, np.broadcast_to(v[0, 0], o.shape))


def test_attention_uniform_when_keys_equal():
    q = RNG.standard_normal((3, 4, 8))
    k = np.broadcast_to(RNG.standard_normal((1, 2, 8)), (9, 2, 8)).copy()
    v = RNG.standard_normal((9, 2, 8))
    o = O.attention(q, k, v)
    # heads 0,1 read kv head 0; heads 2,3 read kv head 1 (contiguous groups)
    assert np.allclose(o[:, 0], v[:, 0].mean(0), atol=1e-14)
    assert np.allclose(o[:, 1], v[:, 0].mean(0), atol=1e-14)
    assert np.allclose(o[:, 3], v[:, 1].mean(0), atol=1e-14)


# --------------------------------------------------------------------------
# fp8 e4m3 (OCP e4m3fn)
# --------------------------------------------------------------------------

def _all_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    v = codes.to(torch.float64).numpy()
    return v[np.isfinite(v)]


def test_e4m3_fixed_points_are_all_finite_codes():
    v = _all_e4m3_values()
    assert len(np.unique(v)) == 253  # 254 finite codes, +0 and -0 compare equal
    assert np.array_equal(O.e4m3(v), v)
    assert v.max() == 448.0 and v[v > 0].min() == 2.0 ** -9


def test_e4m3_midpoints_round_to_even():
    v = np.unique(_all_e4m3_values())
    pos = v[v >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    got = O.e4m3(mids)
    codes = torch.from_numpy(pos).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    lo_even = codes[:-1] % 2 == 0
    want = np.where(lo_even, pos[:-1], pos[1:])
    assert np.array_equal(got, want)
    assert np.array_equal(O.e4m3(-mids), -want)


def test_e4m3_saturates_and_matches_torch_on_clamped_inputs():
    assert O.e4m3(np.array([1e6, -500.0, 464.0, 465.0]))[0] == 448.0
    assert np.array_equal(O.e4m3(np.array([-500.0, 464.0, 465.0])), [-448.0, 448.0, 448.0])
    x = np.concatenate([RNG.standard_normal(20000) * 50, RNG.standard_normal(20000) * 1e-2,
                        RNG.uniform(-448, 448, 20000)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3(np.clip(x, -448, 448)), ref)


def test_quantize_tensor_amax_maps_to_448():
    x = RNG.standard_normal((5, 40)).astype(np.float32)
    codes, s = O.quantize_tensor(x)
    assert np.abs(codes).max() == 448.0
    # dequantised values are within half an e4m3 spacing (relative 2^-4) of the input
    assert np.all(np.abs(codes * s - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * s)
    z, sz = O.quantize_tensor(np.zeros((2, 3), np.float32))
    assert np.array_equal(z, np.zeros((2, 3))) and sz == pytest.approx(1e-12 / 448)
