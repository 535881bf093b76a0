"""Seeded synthetic inputs for the action-expert denoise loop.

This module only *draws* inputs: workload shapes, random weights, prefix K/V,
valid masks and noise.  It holds none of the method's arithmetic, so both the
CPU oracle (through the tests) and the HIP path take their inputs from here.

Workloads (shapes from the pages' models):

* ``c1`` tiny fp32 expert: 2 layers, width 128, 2 query heads / 1 KV head,
  head_dim 64, MLP 512, prefix 64 rows with the last 16 masked, 8x7 action
  chunk, 4 Euler steps.
* ``c2`` Pi0.5-shaped bf16 expert (LoongForge blog, section 1: two 256-token
  cameras + a 200-token instruction; 50 action tokens): 18 layers, width 1024,
  8/1 heads, head_dim 256, MLP 4096; prefix 712 rows = 512 image rows (valid)
  + 200 text rows of which the first 8..200 are valid; 50x32 actions, 10 steps.
* ``c3`` the c2 expert with three fixed camera slots (LoongForge blog,
  section 1): 1018 rows = cam0, cam1, cam2 (masked, 256 rows) + 250 text rows.
* ``c4`` MolmoBot-shaped expert (MolmoBot PR, Part 1: ~1600 image tokens + a
  few instruction tokens + a 14-D state, padded to 2048): 12 layers, width 768,
  12/4 heads, head_dim 64, MLP 3072; 16x14 actions, 10 steps.
* ``c5`` the c2 expert, 16 requests, prefix 1024 rows each with 700..1024
  valid; bf16 or fp8 e4m3 projection weights.

Seeds for workload ``cN``: weights 100N+1, prefix K/V 100N+2, noise 100N+3,
valid lengths 100N+4, garbage in masked rows 100N+5, context hidden states
100N+6, robot state 100N+7.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    width: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    action_horizon: int
    action_dim: int
    n_steps: int
    batch: int
    prefix_len: int
    dtype: str            # "f32" or "bf16": weights, prefix K/V and activations
    proj_dtype: str       # "same" or "fp8": QKV / gate-up / down weights
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    index: int = 0        # N in the seed formula 100N+k
    gate_bias: float = 0.0  # offset on the gate chunks of every layer's modulation bias
    block: str = "joint"    # "joint" attention over [prefix | actions], or "dit" (attn1 + attn2)
    fp8_scaling: str = "tensor"  # fp8 scales per request / tensor, or "rowwise" (per row / column)
    fp8_o: bool = False          # the attention output projection in fp8 too

    def seed(self, k: int) -> int:
        return 100 * self.index + k

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


_PI05 = dict(n_layers=18, width=1024, n_q_heads=8, n_kv_heads=1, head_dim=256,
             mlp_dim=4096, action_horizon=50, action_dim=32, n_steps=10)

WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", n_layers=2, width=128, n_q_heads=2, n_kv_heads=1, head_dim=64,
                   mlp_dim=512, action_horizon=8, action_dim=7, n_steps=4, batch=1,
                   prefix_len=64, dtype="f32", proj_dtype="same", index=1),
    "c2": Workload("c2", batch=1, prefix_len=712, dtype="bf16", proj_dtype="same", index=2, **_PI05),
    "c3": Workload("c3", batch=1, prefix_len=1018, dtype="bf16", proj_dtype="same", index=3, **_PI05),
    "c4": Workload("c4", n_layers=12, width=768, n_q_heads=12, n_kv_heads=4, head_dim=64,
                   mlp_dim=3072, action_horizon=16, action_dim=14, n_steps=10, batch=1,
                   prefix_len=2048, dtype="bf16", proj_dtype="same", index=4, gate_bias=0.1),
    # the c4 shapes and inputs with the DiT-style block (its extra weights drawn after c4's)
    "c4dit": Workload("c4dit", n_layers=12, width=768, n_q_heads=12, n_kv_heads=4, head_dim=64,
                      mlp_dim=3072, action_horizon=16, action_dim=14, n_steps=10, batch=1,
                      prefix_len=2048, dtype="bf16", proj_dtype="same", index=4, gate_bias=0.1, block="dit"),
    # the c2 request with row-wise fp8 scales and the fp8 output projection (one request in e4m3)
    "c2fp8r": Workload("c2fp8r", batch=1, prefix_len=712, dtype="bf16", proj_dtype="fp8", index=2,
                       fp8_scaling="rowwise", fp8_o=True, **_PI05),
    "c5": Workload("c5", batch=16, prefix_len=1024, dtype="bf16", proj_dtype="same", index=5, **_PI05),
    "c5fp8": Workload("c5fp8", batch=16, prefix_len=1024, dtype="bf16", proj_dtype="fp8", index=5, **_PI05),
    # the c5 batch with row-wise fp8 scales and the attention output projection in fp8 as well
    "c5fp8r": Workload("c5fp8r", batch=16, prefix_len=1024, dtype="bf16", proj_dtype="fp8", index=5,
                       fp8_scaling="rowwise", fp8_o=True, **_PI05),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller test shapes)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


# ----------------------------------------------------------------------------
# bf16 encoding of inputs (round to nearest even), used to hand both sides the
# same representable values.
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even, NaN kept NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot overflow 32 bits here; NaN is patched below
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------

def weight_shapes(w: Workload) -> Dict[str, Tuple[int, ...]]:
    """Logical weights, all stored [in_features, out_features] (y = x @ W + b)."""
    D, A, F = w.width, w.action_dim, w.mlp_dim
    qd, kd = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    shapes: Dict[str, Tuple[int, ...]] = {
        "time_mlp.1.w": (D, D), "time_mlp.1.b": (D,),
        "time_mlp.2.w": (D, D), "time_mlp.2.b": (D,),
        "action_in.w": (A, D), "action_in.b": (D,),
        "action_out.w": (D, A), "action_out.b": (A,),
        "final_mod.w": (D, 2 * D), "final_mod.b": (2 * D,),
    }
    nmod = 9 if w.block == "dit" else 6
    for l in range(w.n_layers):
        p = f"layers.{l}."
        shapes.update({
            p + "q": (D, qd), p + "k": (D, kd), p + "v": (D, kd), p + "o": (qd, D),
            p + "gate": (D, F), p + "up": (D, F), p + "down": (F, D),
            p + "mod.w": (D, nmod * D), p + "mod.b": (nmod * D,),
        })
        if w.block == "dit":
            shapes.update({p + "q2": (D, qd), p + "o2": (qd, D)})
    return shapes


def _normal(seed_words, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) fp32 draws from the PCG64 stream seeded by ``seed_words``."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed_words)))
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_weights(w: Workload, seed: Optional[int] = None, std: float = 0.02,
                 gate_bias: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Random-init weights: every matrix and bias ~ N(0, std^2), drawn in fp32
    and encoded in the workload dtype.  Tensor number i (in the order of
    ``weight_shapes``) draws from the stream seeded by (seed, i), so tensors
    can be drawn in parallel and any one can be redrawn alone.

    ``gate_bias`` is added to the gate chunks (3rd and 6th of six) of every
    ``layers.l.mod.b`` before encoding; 0 keeps the plain N(0, std^2) init.
    By default it is the workload's own (0.1 for c4, whose 1600+ visible
    prefix rows otherwise average the prefix's influence on the actions down
    below five times the parity tolerance; 0 elsewhere)."""
    base = w.seed(1) if seed is None else seed
    if gate_bias is None:
        gate_bias = w.gate_bias
    D = w.width
    items = list(weight_shapes(w).items())

    def draw(i: int) -> np.ndarray:
        name, shape = items[i]
        x = _normal((base, i), shape, std)
        if gate_bias and name.endswith("mod.b"):
            for chunk in range(2, x.shape[0] // D, 3):  # the gate of every (scale, shift, gate)
                x[chunk * D:(chunk + 1) * D] += np.float32(gate_bias)
        return _encode(x, w.dtype)

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        arrays = list(ex.map(draw, range(len(items))))
    return {name: a for (name, _), a in zip(items, arrays)}


# ----------------------------------------------------------------------------
# Prefix K/V, valid masks
# ----------------------------------------------------------------------------

def valid_masks(w: Workload, seed: Optional[int] = None,
                n_valid: Optional[Tuple[int, ...]] = None) -> np.ndarray:
    """[batch, prefix_len] uint8 masks following each workload's layout.

    ``n_valid`` (one entry per request) fixes the valid count instead of
    drawing it: for c2/c3 it is the total valid count (512 image rows + text),
    for c4 the total including the state row, for c5 the valid prefix rows."""
    rng = np.random.default_rng(w.seed(4) if seed is None else seed)
    B, P = w.batch, w.prefix_len
    m = np.zeros((B, P), dtype=np.uint8)
    for b in range(B):
        nv = None if n_valid is None else int(n_valid[b])
        if w.name == "c1":
            nv = 48 if nv is None else nv
            m[b, :nv] = 1
        elif w.name in ("c2", "c3", "c2fp8r"):
            n_text = int(rng.integers(8, 201)) if nv is None else nv - 512
            if w.name != "c3" or P == 712:
                m[b, :512] = 1
                m[b, 512:512 + n_text] = 1
            else:  # three camera slots, cam2 masked, 250 text slots
                m[b, :512] = 1
                m[b, 768:768 + n_text] = 1
        elif w.name in ("c4", "c4dit"):
            n_instr = int(rng.integers(21, 35)) if nv is None else nv - 1601
            m[b, :1600 + n_instr + 1] = 1
        else:  # c5 / c5fp8 / generic: right padding
            nv = int(rng.integers(700, 1025)) if nv is None else nv
            nv = min(nv, P)
            m[b, :nv] = 1
    return m


def make_prefix(w: Workload, mask: Optional[np.ndarray] = None, seed: Optional[int] = None,
                garbage: Optional[str] = None, garbage_seed: Optional[int] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Prefix K (already rotated, as the VLM's cache holds it) and V, each
    [L, B, P, Hkv, dh] ~ N(0, 1) in the workload dtype, plus the mask.

    ``garbage`` overwrites the masked rows: ``"huge"`` ~ N(0, 100^2),
    ``"nan"`` NaN, ``"inf"`` +-inf alternating."""
    if mask is None:
        mask = valid_masks(w)
    base = w.seed(2) if seed is None else seed
    shape = (w.n_layers, w.batch, w.prefix_len, w.n_kv_heads, w.head_dim)
    # layer l of K draws from stream (seed, 0, l), of V from (seed, 1, l)
    jobs = [(j, l) for j in range(2) for l in range(w.n_layers)]
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda jl: _encode(_normal((base, jl[0], jl[1]), shape[1:]), w.dtype), jobs))
    K = np.stack(parts[:w.n_layers])
    V = np.stack(parts[w.n_layers:])
    if garbage is not None:
        fill_garbage(w, K, V, mask, garbage, garbage_seed)
    return K, V, mask


def fill_garbage(w: Workload, K: np.ndarray, V: np.ndarray, mask: np.ndarray,
                 kind: str, seed: Optional[int] = None) -> None:
    rng = np.random.default_rng(w.seed(5) if seed is None else seed)
    sel = mask == 0  # [B, P]
    for X in (K, V):
        sub = X[:, sel]  # [L, n_masked, Hkv, dh]
        if kind == "huge":
            g = rng.standard_normal(sub.shape, dtype=np.float32) * np.float32(100.0)
            X[:, sel] = _encode(g, w.dtype)
        elif kind == "nan":
            X[:, sel] = np.nan
        elif kind == "inf":
            g = np.where(rng.integers(0, 2, sub.shape) == 0, np.inf, -np.inf).astype(np.float32)
            X[:, sel] = g
        else:
            raise ValueError(kind)


# ----------------------------------------------------------------------------
# Context preparation inputs: per-layer context hidden states, the robot
# state, and the context K/V / state projections (MolmoBot PR Part 2: the
# VLM's hidden states and the state are turned into the expert's context
# K/V once per query)
# ----------------------------------------------------------------------------

def context_weight_shapes(w: Workload, context_width: int, state_dim: int) -> Dict[str, Tuple[int, ...]]:
    kd = w.n_kv_heads * w.head_dim
    shapes: Dict[str, Tuple[int, ...]] = {}
    for l in range(w.n_layers):
        shapes[f"layers.{l}.ctx_k"] = (context_width, kd)
        shapes[f"layers.{l}.ctx_v"] = (context_width, kd)
    if state_dim:
        shapes["state_in.w"] = (state_dim, context_width)
        shapes["state_in.b"] = (context_width,)
    return shapes


def make_context_weights(w: Workload, context_width: int, state_dim: int = 0,
                         std: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Context K/V projections (and the state's input layer) ~ N(0, std^2),
    std = 1/sqrt(context_width) by default so projected keys and values have
    unit scale like the prefix K/V of the other workloads; drawn from the
    weight seed's streams (seed, 10000 + i), encoded in the workload dtype."""
    base = w.seed(1)
    sd = (1.0 / np.sqrt(context_width)) if std is None else std
    out = {}
    for i, (name, shape) in enumerate(context_weight_shapes(w, context_width, state_dim).items()):
        x = _normal((base, 10000 + i), shape, sd)
        out[name] = _encode(x, w.dtype)
    return out


def make_context(w: Workload, context_width: int, mask: Optional[np.ndarray] = None,
                 seed: Optional[int] = None, garbage: Optional[str] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-layer context hidden states [L, B, P, Dc] ~ N(0, 1) in the workload
    dtype (layer l from stream (seed, l)), and the mask.  ``garbage="nan"``
    fills the masked rows with NaN."""
    if mask is None:
        mask = valid_masks(w)
    base = w.seed(6) if seed is None else seed
    shape = (w.batch, w.prefix_len, context_width)
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda l: _encode(_normal((base, l), shape), w.dtype), range(w.n_layers)))
    H = np.stack(parts)
    if garbage == "nan":
        H[:, mask == 0] = np.nan
    elif garbage is not None:
        raise ValueError(garbage)
    return H, mask


def make_state(w: Workload, state_dim: int, seed: Optional[int] = None) -> np.ndarray:
    """Robot state [B, S] ~ N(0, 1), fp32."""
    rng = np.random.default_rng(w.seed(7) if seed is None else seed)
    return rng.standard_normal((w.batch, state_dim), dtype=np.float32)


def make_noise(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Initial action chunk x_0 ~ N(0, 1), [B, T, A] fp32 (the loop state is fp32)."""
    rng = np.random.default_rng(w.seed(3) if seed is None else seed)
    return rng.standard_normal((w.batch, w.action_horizon, w.action_dim), dtype=np.float32)


def insert_camera_slot(w3: Workload, K2: np.ndarray, V2: np.ndarray, mask2: np.ndarray,
                       slot: int = 2, garbage: Optional[str] = "huge",
                       seed: Optional[int] = None):
    """Build a three-camera (1018-row) prefix from a two-camera (712-row) one:
    the extra 256-row camera slot is inserted at slot ``slot`` (0..2) and
    masked, and the text segment grows from 200 to 250 rows with the extra rows
    masked.  Pruning the masked rows gives back exactly the 712-row instance's
    valid rows, in the same order."""
    L, B, P2, H, dh = K2.shape
    assert P2 == 712
    rng = np.random.default_rng(w3.seed(5) if seed is None else seed)
    K3 = np.zeros((L, B, 1018, H, dh), np.float32)
    V3 = np.zeros_like(K3)
    m3 = np.zeros((B, 1018), np.uint8)
    cams = [(0, 256), (256, 512)]
    dst_cam = [s for s in range(3) if s != slot]
    for (s0, s1), d in zip(cams, dst_cam):
        K3[:, :, d * 256:(d + 1) * 256] = K2[:, :, s0:s1]
        V3[:, :, d * 256:(d + 1) * 256] = V2[:, :, s0:s1]
        m3[:, d * 256:(d + 1) * 256] = mask2[:, s0:s1]
    K3[:, :, 768:968] = K2[:, :, 512:712]
    V3[:, :, 768:968] = V2[:, :, 512:712]
    m3[:, 768:968] = mask2[:, 512:712]
    # the empty slot and the extra text slots: masked, holding garbage
    for X in (K3, V3):
        fillshape = X[:, :, slot * 256:(slot + 1) * 256].shape
        X[:, :, slot * 256:(slot + 1) * 256] = _encode(
            rng.standard_normal(fillshape, dtype=np.float32) * np.float32(100.0), w3.dtype)
        X[:, :, 968:1018] = _encode(
            rng.standard_normal(X[:, :, 968:1018].shape, dtype=np.float32), w3.dtype)
    # masked rows of the 2-camera instance (its text padding) may hold garbage too
    if garbage == "nan":
        sel = m3 == 0
        K3[:, sel] = np.nan
        V3[:, sel] = np.nan
    return K3, V3, m3
