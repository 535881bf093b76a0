"""CPU oracle for the flow-matching action-expert denoise loop.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; both sides only take the same seeded inputs.

A plain, slow, obviously-correct NumPy implementation in float64.  Inputs are
the exact fp32 / bf16-representable values the GPU receives, widened to fp64;
no intermediate is rounded to bf16 (the GPU's bf16 intermediates are what the
parity tolerance covers).  The only places where fp32 is used on purpose are
the decisions of the fp8 emulation (scale and code selection), which the
kernel takes in fp32.

What it follows (page titles as given on the pages):

* MolmoBot PR "Inference optimization for MolmoBot VLA: torch.compile + CUDA
  graphs + action-expert KV cache", Part 2: the VLM runs once, the action
  expert is integrated for ``num_steps`` Euler steps, and only the action-token
  queries and the flow timestep change between steps; the context K/V are
  projected once per query and reused by every step.  Part 3: per-tensor
  dynamic fp8 e4m3 (amax -> cast -> scaled matmul).
* LoongForge blog "How to Speed Up VLA Training Step by Step: A 3x
  Acceleration Case Study on Pi0.5": section 1 (masked camera slot is
  invisible; pad tokens do not advance position ids), section 2 (adaRMS in
  fp32: square, mean, rsqrt, scale/shift/gate; gated residuals; gelu*up; RoPE
  as q*cos + rotate_half(q)*sin), section 3 (actions see every valid prefix
  token and each other, padding rows/columns masked; the single KV head is
  broadcast to every query head), section 5.3 (time MLP, action input and
  output projections, final norm as separate small pieces), section 7 (fp8
  GEMM: quantise inputs and weights, restore with the scales).
* sglang PR 34599 summary, implementation items 1-2: Q/K/V and gate/up are
  merged projections (shard order q, k, v); mask, positions and the sinusoidal
  time scaling are computed once per call and reused by every step.

Readings where the pages leave a step open (each a plain choice the rest of
the pages support):

* time runs from t=1 (noise) to t=0; step k evaluates the velocity at
  t_k = (N-k)/N and applies x += dt*v with dt = -1/N;
* sinusoidal embedding: [sin(2*pi*t/P_i) | cos(2*pi*t/P_i)], i < D/2, with
  periods P_i geometric from 4e-3 to 4.0;
* time MLP: two D x D linears with bias, SiLU after each;
* adaRMS: u = h / sqrt(mean(h^2) + eps) * (1 + scale) + shift, eps = 1e-6, no
  learned gain; one [D, 6D] modulation per layer chunked [scale_a, shift_a,
  gate_a, scale_m, shift_m, gate_m]; gated residual h + gate * branch;
* final norm: adaRMS with (scale_f, shift_f) from a [D, 2D] modulation;
* RoPE: half-split (rotate_half) form, theta = 10000, whole head rotated;
  prefix K arrives already rotated; action token i of a request sits at
  position n_valid + i (the count of valid prefix rows, since pads do not
  advance positions);
* attention: scale 1/sqrt(head_dim), action block bidirectional, query head
  h reads KV head floor(h * Hkv / Hq); masked prefix rows take no part at all
  (they are skipped, so NaN or inf there cannot leak);
* MLP: gelu (tanh form) on the gate half, times the up half;
* fp8: OCP e4m3fn, round to nearest even, saturating at +-448; weights
  static per logical tensor (q, k, v, gate, up, down), activations dynamic per
  request; s = max(amax, 1e-12)/448, code = e4m3(x * (448/amax)) in fp32,
  y = (codes_x . codes_w) * s_x * s_w.  The row-wise variant (the MolmoBot
  PR reports it unsupported on its GPU, so the pages fix no more of it than
  its name) takes the plainest reading: one scale per input row (token) and
  one per weight output column (channel), y[i, j] = (codes_x[i] .
  codes_w[:, j]) s_x[i] s_w[j]; the attention output projection may be
  quantised the same way (fp8_o);
* context preparation: each layer's context K/V = the context hidden states
  times that layer's context K and V projections, K rotated at the row's
  count position; the robot state enters through one linear layer as one
  more visible row after the context rows;
* DiT-style block (the MolmoBot expert's attn1 / attn2): nine modulation
  chunks per layer (scale, shift, gate of the self-attention, the
  cross-attention and the MLP); attn1 over the action tokens only, attn2 of
  separate q2 / o2 projections over the visible prefix only, each with its
  own softmax; an empty prefix gives attn2 no contribution.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, library routines, brute force or invariants; none is
left unpinned.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

F64 = np.float64

P_MIN = 4e-3
P_MAX = 4.0
FP8_MAX = 448.0
AMAX_FLOOR = 1e-12


@dataclasses.dataclass(frozen=True)
class Params:
    """Shape and scalar hyper-parameters of the expert (weights carry the rest)."""
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    fp8: bool = False
    block: str = "joint"  # "joint": one attention over [prefix | actions]; "dit": attn1 + attn2
    fp8_rowwise: bool = False  # fp8 scales per input row and per weight column (else per request / tensor)
    fp8_o: bool = False        # the attention output projection in fp8 too

    @staticmethod
    def like(obj, fp8: Optional[bool] = None) -> "Params":
        f = getattr(obj, "proj_dtype", "same") == "fp8" if fp8 is None else fp8
        return Params(obj.n_q_heads, obj.n_kv_heads, obj.head_dim,
                      float(obj.rope_theta), float(obj.rms_eps), f, getattr(obj, "block", "joint"),
                      f and getattr(obj, "fp8_scaling", "tensor") == "rowwise",
                      f and bool(getattr(obj, "fp8_o", False)))


def to64(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=F64) for k, v in weights.items()}


def n_layers_of(W: Dict[str, np.ndarray]) -> int:
    n = 0
    while f"layers.{n}.q" in W:
        n += 1
    return n


# ---------------------------------------------------------------------------
# Time path (hoisted out of the step loop: sglang PR summary, item 2)
# ---------------------------------------------------------------------------

def timestep_grid(n_steps: int) -> Tuple[np.ndarray, float]:
    """Euler grid: t_k = (N - k)/N for k < N, dt = -1/N (t from 1 to 0)."""
    k = np.arange(n_steps, dtype=F64)
    return (n_steps - k) / n_steps, -1.0 / n_steps


def sinusoid(t: np.ndarray, width: int) -> np.ndarray:
    """[len(t), width]: sin half then cos half, periods geometric 4e-3..4.0."""
    t = np.atleast_1d(np.asarray(t, dtype=F64))
    half = width // 2
    frac = np.arange(half, dtype=F64) / (half - 1)
    period = P_MIN * (P_MAX / P_MIN) ** frac
    ang = 2.0 * np.pi * t[:, None] / period[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x @ W (+ b), weights stored [in, out]."""
    y = x @ w
    return y if b is None else y + b


def time_condition(t: np.ndarray, W: Dict[str, np.ndarray]) -> np.ndarray:
    """c = SiLU(W2 . SiLU(W1 . e(t) + b1) + b2), one row per time value."""
    D = W["time_mlp.1.w"].shape[0]
    e = sinusoid(t, D)
    z = silu(linear(e, W["time_mlp.1.w"], W["time_mlp.1.b"]))
    return silu(linear(z, W["time_mlp.2.w"], W["time_mlp.2.b"]))


def layer_modulation(c: np.ndarray, W: Dict[str, np.ndarray], layer: int):
    """The [.., D] chunks of a layer's modulation: six (scale_a, shift_a,
    gate_a, scale_m, shift_m, gate_m) for the joint block, nine (scale, shift,
    gate of the self-attention, the cross-attention and the MLP) for the
    DiT-style block."""
    wm = W[f"layers.{layer}.mod.w"]
    m = linear(c, wm, W[f"layers.{layer}.mod.b"])
    return np.split(m, wm.shape[1] // wm.shape[0], axis=-1)


def final_modulation(c: np.ndarray, W: Dict[str, np.ndarray]):
    m = linear(c, W["final_mod.w"], W["final_mod.b"])
    return np.split(m, 2, axis=-1)


# ---------------------------------------------------------------------------
# Layer pieces
# ---------------------------------------------------------------------------

def ada_rms(h: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * (1 + scale) + shift over the last axis."""
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h * r * (1.0 + scale) + shift


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float):
    """cos, sin of phi = p * theta^(-2j/dh), j < dh/2; [len(p), dh/2]."""
    half = head_dim // 2
    omega = theta ** (-2.0 * np.arange(half, dtype=F64) / head_dim)
    phi = np.asarray(positions, dtype=F64)[:, None] * omega[None, :]
    return np.cos(phi), np.sin(phi)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x [T, H, dh]; pair (x_j, x_{j+dh/2}) rotated by phi_j of the row's position."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """q [T, Hq, dh]; keys, values [S, Hkv, dh] (only visible rows).

    o_h = softmax(q_h . K_g^T / sqrt(dh)) . V_g with g = floor(h * Hkv / Hq)."""
    T, Hq, dh = q.shape
    Hkv = keys.shape[1]
    if keys.shape[0] == 0:  # no visible key (a cross-attention over an empty prefix): no contribution
        return np.zeros_like(q)
    o = np.empty_like(q)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (q[:, h, :] @ keys[:, g, :].T) / np.sqrt(dh)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        o[:, h, :] = (p @ values[:, g, :]) / p.sum(axis=1, keepdims=True)
    return o


# ---------------------------------------------------------------------------
# fp8 e4m3 emulation (MolmoBot PR Part 3; LoongForge blog section 7)
# ---------------------------------------------------------------------------

def e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3fn value (ties to even), saturated to +-448, as fp64.

    Normal binades have 3 fraction bits, so the spacing in [2^e, 2^(e+1)) is
    2^(e-3); below 2^-6 the spacing is the subnormal step 2^-9."""
    x = np.asarray(x, dtype=F64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                 # ax = m * 2^e, m in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    q = np.rint(ax / quantum) * quantum  # rint: half to even; exact in fp64
    q = np.minimum(q, FP8_MAX)
    return np.copysign(q, x)


def fp8_scale(amax) -> Tuple[np.float32, np.float32]:
    """(multiplier into the fp8 range, dequantisation scale), both fp32."""
    a = np.maximum(np.float32(amax), np.float32(AMAX_FLOOR))
    return np.float32(FP8_MAX) / a, a / np.float32(FP8_MAX)


def quantize_tensor(x: np.ndarray) -> Tuple[np.ndarray, float]:
    """Per-tensor: codes = e4m3(fp32(x) * fp32(448/amax)), scale = amax/448."""
    x32 = np.asarray(x, dtype=np.float32)
    mul, s = fp8_scale(np.max(np.abs(x32)))
    return e4m3((x32 * mul).astype(np.float32)), float(s)


def fp8_linear(x: np.ndarray, w_codes: np.ndarray, w_scale: float) -> np.ndarray:
    """x [T, K] of ONE request: dynamic per-request activation scale."""
    xq, xs = quantize_tensor(x)
    return (xq @ w_codes) * xs * w_scale


def quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per row (token): each row quantised as its own tensor (the per-tensor
    rule applied to every row at once, element by element in fp32); scales
    [rows]."""
    x32 = np.asarray(x, dtype=np.float32)
    a = np.maximum(np.max(np.abs(x32), axis=1), np.float32(AMAX_FLOOR))
    mul, s = np.float32(FP8_MAX) / a, a / np.float32(FP8_MAX)
    return e4m3((x32 * mul[:, None]).astype(np.float32)), s.astype(F64)


def quantize_columns(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per output column (channel) of a [K, N] weight; scales [N]."""
    c, s = quantize_rows(np.asarray(w).T)
    return c.T.copy(), s


def fp8_linear_rowwise(x: np.ndarray, w_codes: np.ndarray, w_scales: np.ndarray) -> np.ndarray:
    """x [T, K]: y[i, j] = (codes_x[i] . codes_w[:, j]) s_x[i] s_w[j]."""
    xq, xs = quantize_rows(x)
    return (xq @ w_codes) * xs[:, None] * w_scales[None, :]


# ---------------------------------------------------------------------------
# One velocity evaluation and the Euler loop
# ---------------------------------------------------------------------------

def prefix_visible(K: np.ndarray, V: np.ndarray, mask: np.ndarray, layer: int, b: int):
    """Valid prefix rows of request b in layer ``layer``, in prefix order."""
    idx = np.nonzero(np.asarray(mask[b]) != 0)[0]
    return K[layer, b, idx].astype(F64), V[layer, b, idx].astype(F64)


class Expert:
    """Weights (fp64) + hyper-parameters; fp8 codes prepared once if asked."""

    def __init__(self, weights: Dict[str, np.ndarray], params: Params):
        self.W = to64(weights)
        self.p = params
        self.L = n_layers_of(self.W)
        self.q8: Dict[str, tuple] = {}
        if params.fp8:
            names = ("q", "k", "v", "gate", "up", "down") + (("o",) if params.fp8_o else ())
            quant = quantize_columns if params.fp8_rowwise else quantize_tensor
            for l in range(self.L):
                for nm in names:
                    key = f"layers.{l}.{nm}"
                    self.q8[key] = quant(weights[key])

    def proj(self, x: np.ndarray, key: str) -> np.ndarray:
        """A projection of one request's rows [T, K]; the fp8 variant quantises
        q, k, v, gate, up, down (and o with fp8_o)."""
        if key in self.q8:
            codes, s = self.q8[key]
            if self.p.fp8_rowwise:
                return fp8_linear_rowwise(x, codes, s)
            return fp8_linear(x, codes, s)
        return x @ self.W[key]

    def velocity(self, x: np.ndarray, c: np.ndarray, kv_of_layer, n_valid: np.ndarray) -> np.ndarray:
        """v(x, t) for a batch.  x [B, T, A]; c [D] the time condition of this
        step; kv_of_layer(l, b) -> (keys, values) visible prefix rows."""
        if self.p.block == "dit":
            return self.velocity_dit(x, c, kv_of_layer, n_valid)
        W, p = self.W, self.p
        B, T, _ = x.shape
        Hq, Hkv, dh = p.n_q_heads, p.n_kv_heads, p.head_dim
        h = linear(x, W["action_in.w"], W["action_in.b"])  # [B, T, D]
        for l in range(self.L):
            sa, ha, ga, sm, hm, gm = layer_modulation(c, W, l)
            pre = f"layers.{l}."
            u = ada_rms(h, sa, ha, p.rms_eps)
            o = np.empty((B, T, Hq * dh))
            for b in range(B):
                q = self.proj(u[b], pre + "q").reshape(T, Hq, dh)
                k = self.proj(u[b], pre + "k").reshape(T, Hkv, dh)
                v = self.proj(u[b], pre + "v").reshape(T, Hkv, dh)
                cos, sin = rope_cos_sin(n_valid[b] + np.arange(T), dh, p.rope_theta)
                q, k = apply_rope(q, cos, sin), apply_rope(k, cos, sin)
                pk, pv = kv_of_layer(l, b)
                keys = np.concatenate([pk, k], axis=0)
                vals = np.concatenate([pv, v], axis=0)
                o[b] = attention(q, keys, vals).reshape(T, Hq * dh)
            h = h + ga * np.stack([self.proj(o[b], pre + "o") for b in range(B)])
            u2 = ada_rms(h, sm, hm, p.rms_eps)
            a = np.empty((B, T, W[pre + "gate"].shape[1]))
            for b in range(B):
                a[b] = gelu_tanh(self.proj(u2[b], pre + "gate")) * self.proj(u2[b], pre + "up")
            d = np.stack([self.proj(a[b], pre + "down") for b in range(B)])
            h = h + gm * d
        sf, hf = final_modulation(c, W)
        return linear(ada_rms(h, sf, hf, p.rms_eps), W["action_out.w"], W["action_out.b"])

    def velocity_dit(self, x: np.ndarray, c: np.ndarray, kv_of_layer, n_valid: np.ndarray) -> np.ndarray:
        """v(x, t) with the DiT-style block of the MolmoBot action expert
        (MolmoBot PR Part 2: ActionExpertBlock passes the cached context K/V
        to attn2; Correctness table: cross_attn and self_attn): per layer
        h += gate1 * attn1(adaRMS(h)) over the action tokens only (q, k, v, o),
        h += gate2 * attn2(adaRMS(h)) of the action queries (q2, o2) over the
        visible prefix K/V only, h += gate3 * MLP(adaRMS(h)); each attention
        has its own softmax.  Action token i sits at position n_valid + i in
        both (only position differences matter inside attn1)."""
        W, p = self.W, self.p
        B, T, _ = x.shape
        Hq, Hkv, dh = p.n_q_heads, p.n_kv_heads, p.head_dim
        h = linear(x, W["action_in.w"], W["action_in.b"])
        for l in range(self.L):
            s1, b1, g1, s2, b2, g2, s3, b3, g3 = layer_modulation(c, W, l)
            pre = f"layers.{l}."
            u = ada_rms(h, s1, b1, p.rms_eps)
            o = np.empty((B, T, Hq * dh))
            for b in range(B):
                q = self.proj(u[b], pre + "q").reshape(T, Hq, dh)
                k = self.proj(u[b], pre + "k").reshape(T, Hkv, dh)
                v = self.proj(u[b], pre + "v").reshape(T, Hkv, dh)
                cos, sin = rope_cos_sin(n_valid[b] + np.arange(T), dh, p.rope_theta)
                o[b] = attention(apply_rope(q, cos, sin), apply_rope(k, cos, sin), v).reshape(T, Hq * dh)
            h = h + g1 * np.stack([self.proj(o[b], pre + "o") for b in range(B)])
            u2 = ada_rms(h, s2, b2, p.rms_eps)
            o2 = np.empty((B, T, Hq * dh))
            for b in range(B):
                q2 = (u2[b] @ W[pre + "q2"]).reshape(T, Hq, dh)
                cos, sin = rope_cos_sin(n_valid[b] + np.arange(T), dh, p.rope_theta)
                pk, pv = kv_of_layer(l, b)
                o2[b] = attention(apply_rope(q2, cos, sin), pk, pv).reshape(T, Hq * dh)
            h = h + g2 * (o2 @ W[pre + "o2"])
            u3 = ada_rms(h, s3, b3, p.rms_eps)
            a = np.empty((B, T, W[pre + "gate"].shape[1]))
            for b in range(B):
                a[b] = gelu_tanh(self.proj(u3[b], pre + "gate")) * self.proj(u3[b], pre + "up")
            d = np.stack([self.proj(a[b], pre + "down") for b in range(B)])
            h = h + g3 * d
        sf, hf = final_modulation(c, W)
        return linear(ada_rms(h, sf, hf, p.rms_eps), W["action_out.w"], W["action_out.b"])

    def denoise(self, noise: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray,
                n_steps: int) -> np.ndarray:
        """x_N after N Euler steps from x_0 = noise [B, T, A]; K, V
        [L, B, P, Hkv, dh] (prefix K already rotated); mask [B, P]."""
        mask = np.asarray(mask)
        n_valid = (mask != 0).sum(axis=1)
        cache = {}

        def kv(l, b):
            if (l, b) not in cache:
                cache[(l, b)] = prefix_visible(K, V, mask, l, b)
            return cache[(l, b)]

        return self.integrate(noise, kv, n_valid, n_steps)

    def integrate(self, noise, kv_of_layer, n_valid, n_steps):
        t, dt = timestep_grid(n_steps)
        c = time_condition(t, self.W)  # [N, D], once per call
        x = np.asarray(noise, dtype=F64).copy()
        for k in range(n_steps):
            x = x + dt * self.velocity(x, c[k], kv_of_layer, n_valid)
        return x


def denoise(weights, params: Params, noise, K, V, mask, n_steps: int) -> np.ndarray:
    return Expert(weights, params).denoise(noise, K, V, mask, n_steps)


# ---------------------------------------------------------------------------
# Prepare-side helpers (MolmoBot PR Part 2: context K/V projected from the
# VLM's per-layer hidden states, once per query)
# ---------------------------------------------------------------------------

def prefix_positions(mask_row: np.ndarray) -> np.ndarray:
    """Position of each valid prefix row = number of valid rows before it."""
    m = (np.asarray(mask_row) != 0).astype(np.int64)
    return np.cumsum(m) - m


def project_prefix_kv(hidden: np.ndarray, wk: np.ndarray, wv: np.ndarray, mask: np.ndarray,
                      n_kv_heads: int, theta: float):
    """hidden [B, P, Dc] of one layer -> K (rotated at its own positions), V,
    each [B, P, Hkv, dh]; masked rows are projected too (and stay invisible)."""
    B, P, _ = hidden.shape
    dh = wk.shape[1] // n_kv_heads
    K = np.empty((B, P, n_kv_heads, dh))
    V = np.empty((B, P, n_kv_heads, dh))
    for b in range(B):
        k = (hidden[b] @ wk).reshape(P, n_kv_heads, dh)
        cos, sin = rope_cos_sin(prefix_positions(mask[b]), dh, theta)
        K[b] = apply_rope(k, cos, sin)
        V[b] = (hidden[b] @ wv).reshape(P, n_kv_heads, dh)
    return K, V


def encode_state(state: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The robot state's context row: one linear layer, state [B, S] ->
    [B, Dc] (MolmoBot PR Part 2: the state is part of the context computed
    once per query; the pages do not give the encoder's form, and one linear
    layer is the plainest reading)."""
    return linear(np.asarray(state, dtype=F64), w, b)


def prepare_prefix(hidden: np.ndarray, wk: np.ndarray, wv: np.ndarray, mask: np.ndarray,
                   n_kv_heads: int, theta: float, state_hidden: Optional[np.ndarray] = None):
    """The context K/V of one query, every layer at once (MolmoBot PR Part 2:
    prepare_cross_context / precompute_kv, run once before the flow steps).

    hidden [L, B, P, Dc], wk / wv [L, Dc, Hkv*dh], mask [B, P].  With
    state_hidden [B, Dc] one more visible row follows the P context rows:
    the state, projected by every layer like a context row and rotated at
    its own position, the count of visible context rows.
    Returns K, V [L, B, P(+1), Hkv, dh] and the mask [B, P(+1)]."""
    hidden = np.asarray(hidden, dtype=F64)
    mask = np.asarray(mask)
    L, B, P, Dc = hidden.shape
    if state_hidden is not None:
        sh = np.asarray(state_hidden, dtype=F64)[None, :, None, :]
        hidden = np.concatenate([hidden, np.broadcast_to(sh, (L, B, 1, Dc))], axis=2)
        mask = np.concatenate([mask, np.ones((B, 1), mask.dtype)], axis=1)
    KV = [project_prefix_kv(hidden[l], wk[l], wv[l], mask, n_kv_heads, theta) for l in range(L)]
    return np.stack([k for k, _ in KV]), np.stack([v for _, v in KV]), mask
