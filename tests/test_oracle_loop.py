"""Whole-loop pins of the oracle: brute force, closed forms and the pages'
invariants (MolmoBot PR "Correctness" table; LoongForge blog section 1).

* brute force: a scalar pure-Python twin with an explicit [T, P+T] visibility
  mask and -inf logits (the oracle instead drops masked rows);
* Euler closed form: a constant-velocity head gives x_N = x_0 + N dt v = x_0 - v;
* zero gates: with the gate chunks of every modulation zeroed the residual
  stream never changes, so each step is a closed-form map of x;
* masked / padded / pruned prefix rows leave the actions unchanged;
* context K/V projected once == re-projected every step;
* batched requests == each request alone;
* the prefix matters: redrawing it moves the actions by far more than the
  GPU parity tolerance, so the tolerance-level checks are not vacuous.
"""

import cmath
import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ae_oracle as O
from vla_flow_matching_amd import synth


def tiny(**kw):
    base = dict(n_layers=2, width=8, n_q_heads=2, n_kv_heads=1, head_dim=4, mlp_dim=6,
                action_horizon=3, action_dim=2, n_steps=2, batch=2, prefix_len=5,
                dtype="f32", proj_dtype="same", index=9)
    base.update(kw)
    return synth.Workload("tiny", **base)


def small_c2(layers=2, steps=2, batch=1, **kw):
    return synth.workload("c2", n_layers=layers, n_steps=steps, batch=batch, **kw)


def run(w, W, K, V, m, x0, fp8=False):
    return O.Expert(W, O.Params.like(w, fp8=fp8)).denoise(x0, K, V, m, w.n_steps)


def run_params(W, p, K, V, m, x0, n_steps):
    return O.Expert(W, p).denoise(x0, K, V, m, n_steps)


# --------------------------------------------------------------------------
# Brute-force scalar twin
# --------------------------------------------------------------------------

def _e4m3_table():
    """Every finite non-negative OCP e4m3fn value with its code, from the
    format's definition: exponent field e (4 bits, bias 7) and mantissa m
    (3 bits); e = 0 is subnormal, m * 2^-9; code 0x7F is NaN, so 0x7E = 448
    is the largest."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append((m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7), code))
    return vals


_E4M3 = _e4m3_table()


def _e4m3_scalar(v):
    """Nearest e4m3 value by scanning the whole table; a tie goes to the even
    code (even mantissa); magnitudes past 448 saturate."""
    a = abs(v)
    best, best_code = None, None
    for val, code in _E4M3:
        if best is None or abs(a - val) < abs(a - best) or (
                abs(a - val) == abs(a - best) and code % 2 == 0):
            best, best_code = val, code
    return math.copysign(best, v)


def _fp8_rows(rows, wcodes, wscale):
    """Rows of ONE request through a per-tensor fp8 linear: the request's
    amax over every element of its rows, the multiplier 448 / amax and each
    code decided in fp32, the product of codes summed in fp64 and scaled by
    both scales."""
    f32 = np.float32
    amax = f32(max(abs(f32(v)) for r in rows for v in r))
    amax = max(amax, f32(1e-12))
    mul, sx = f32(448.0) / amax, amax / f32(448.0)
    out = []
    for r in rows:
        codes = [_e4m3_scalar(float(f32(f32(v) * mul))) for v in r]
        acc = [0.0] * wcodes.shape[1]
        for j in range(wcodes.shape[1]):
            t = 0.0
            for i in range(len(codes)):
                t += codes[i] * wcodes[i, j]
            acc[j] = t * float(sx) * wscale
        out.append(acc)
    return out


def _fp8_rows_rowwise(rows, wcodes, wscales):
    """Rows through a row-wise fp8 linear: each row's own amax, multiplier and
    codes in fp32; each weight column its own scale."""
    f32 = np.float32
    out = []
    for r in rows:
        amax = max(max(abs(f32(v)) for v in r), f32(1e-12))
        mul, sx = f32(448.0) / amax, amax / f32(448.0)
        codes = [_e4m3_scalar(float(f32(f32(v) * mul))) for v in r]
        acc = []
        for j in range(wcodes.shape[1]):
            t = 0.0
            for i in range(len(codes)):
                t += codes[i] * wcodes[i, j]
            acc.append(t * float(sx) * float(wscales[j]))
        out.append(acc)
    return out


def _fp8_weight_cols(Wt):
    """One weight tensor, each output column with its own amax and codes."""
    f32 = np.float32
    w32 = np.asarray(Wt, dtype=np.float32)
    codes = np.empty(w32.shape)
    scales = []
    for j in range(w32.shape[1]):
        amax = max(f32(np.abs(w32[:, j]).max()), f32(1e-12))
        mul = f32(448.0) / amax
        scales.append(amax / f32(448.0))
        codes[:, j] = [_e4m3_scalar(float(f32(v * mul))) for v in w32[:, j]]
    return codes, scales


def _fp8_weight(Wt):
    """One logical weight tensor: amax over the whole tensor, codes in fp32."""
    f32 = np.float32
    w32 = np.asarray(Wt, dtype=np.float32)
    amax = max(f32(np.abs(w32).max()), f32(1e-12))
    mul, s = f32(448.0) / amax, amax / f32(448.0)
    codes = np.array([[_e4m3_scalar(float(f32(v * mul))) for v in row] for row in w32])
    return codes, float(s)


def _bf_denoise(w, W, K, V, mask, x0, fp8=False, rowwise=False, fp8_o=False):
    """Scalar loops only; explicit visibility mask; independent of the oracle.
    fp8: the q, k, v, gate, up and down projections quantised per logical
    tensor (weights) and per request (inputs); rowwise: per weight column and
    per input row instead; fp8_o: the output projection o as well."""
    L, D, Hq, Hkv, dh, Fd = w.n_layers, w.width, w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim
    T, A, N, B, P = w.action_horizon, w.action_dim, w.n_steps, w.batch, w.prefix_len
    g = lambda name: np.asarray(W[name], dtype=np.float64)
    q8 = {}
    if fp8:
        for l in range(L):
            for nm in ("q", "k", "v", "gate", "up", "down") + (("o",) if fp8_o else ()):
                q8[f"layers.{l}.{nm}"] = (_fp8_weight_cols if rowwise else _fp8_weight)(W[f"layers.{l}.{nm}"])

    def mv(vec, mat, bias=None):  # vec [in] @ mat [in, out]
        out = [0.0] * mat.shape[1]
        for j in range(mat.shape[1]):
            acc = 0.0
            for i in range(mat.shape[0]):
                acc += vec[i] * mat[i, j]
            out[j] = acc + (0.0 if bias is None else bias[j])
        return out

    def silu(z):
        return z / (1.0 + math.exp(-z))

    def norm(vec, scale, shift):
        ms = sum(v * v for v in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + w.rms_eps)
        return [vec[i] * r * (1.0 + scale[i]) + shift[i] for i in range(len(vec))]

    def rot(vec, p):
        half = len(vec) // 2
        out = list(vec)
        for j in range(half):
            ang = p * w.rope_theta ** (-2.0 * j / len(vec))
            a, b = vec[j], vec[j + half]
            out[j] = a * math.cos(ang) - b * math.sin(ang)
            out[j + half] = b * math.cos(ang) + a * math.sin(ang)
        return out

    x = [[[float(x0[b, i, a]) for a in range(A)] for i in range(T)] for b in range(B)]
    for k in range(N):
        t = 1.0 - k / N
        half = D // 2
        e = [0.0] * D
        for i in range(half):
            period = 4e-3 * (4.0 / 4e-3) ** (i / (half - 1))
            e[i] = math.sin(2 * math.pi * t / period)
            e[half + i] = math.cos(2 * math.pi * t / period)
        c = [silu(z) for z in mv([silu(z) for z in mv(e, g("time_mlp.1.w"), g("time_mlp.1.b"))],
                                 g("time_mlp.2.w"), g("time_mlp.2.b"))]
        for b in range(B):
            nv = int(sum(int(mask[b, j] != 0) for j in range(P)))
            h = [mv(x[b][i], g("action_in.w"), g("action_in.b")) for i in range(T)]
            for l in range(L):
                mod = mv(c, g(f"layers.{l}.mod.w"), g(f"layers.{l}.mod.b"))
                ch = [mod[j * D:(j + 1) * D] for j in range(6)]
                u = [norm(h[i], ch[0], ch[1]) for i in range(T)]

                def proj(rows, nm):
                    key = f"layers.{l}.{nm}"
                    if key in q8:
                        return (_fp8_rows_rowwise if rowwise else _fp8_rows)(rows, *q8[key])
                    return [mv(r, g(key)) for r in rows]

                qs, ks, vs = proj(u, "q"), proj(u, "k"), proj(u, "v")
                o = [[0.0] * (Hq * dh) for _ in range(T)]
                for hd in range(Hq):
                    kv = hd // (Hq // Hkv)
                    # all P + T keys, visibility by mask
                    keys, vals, vis = [], [], []
                    for j in range(P):
                        keys.append([float(K[l, b, j, kv, d]) for d in range(dh)])
                        vals.append([float(V[l, b, j, kv, d]) for d in range(dh)])
                        vis.append(mask[b, j] != 0)
                    for j in range(T):
                        keys.append(rot(ks[j][kv * dh:(kv + 1) * dh], nv + j))
                        vals.append(vs[j][kv * dh:(kv + 1) * dh])
                        vis.append(True)
                    for i in range(T):
                        qv = rot(qs[i][hd * dh:(hd + 1) * dh], nv + i)
                        logits = []
                        for j in range(P + T):
                            if vis[j]:
                                logits.append(sum(qv[d] * keys[j][d] for d in range(dh)) / math.sqrt(dh))
                            else:
                                logits.append(-math.inf)
                        mx = max(logits)
                        ws = [math.exp(s - mx) if s != -math.inf else 0.0 for s in logits]
                        tot = sum(ws)
                        for d in range(dh):
                            acc = 0.0
                            for j in range(P + T):
                                if ws[j] != 0.0:
                                    acc += ws[j] * vals[j][d]
                            o[i][hd * dh + d] = acc / tot
                obs = proj(o, "o")
                for i in range(T):
                    h[i] = [h[i][d] + ch[2][d] * obs[i][d] for d in range(D)]
                u2 = [norm(h[i], ch[3], ch[4]) for i in range(T)]
                gts, ups = proj(u2, "gate"), proj(u2, "up")
                acts = []
                for i in range(T):
                    gt, up = gts[i], ups[i]
                    acts.append([0.5 * gt[f] * (1 + math.tanh(math.sqrt(2 / math.pi) * (gt[f] + 0.044715 * gt[f] ** 3)))
                                 * up[f] for f in range(Fd)])
                dns = proj(acts, "down")
                for i in range(T):
                    h[i] = [h[i][d] + ch[5][d] * dns[i][d] for d in range(D)]
            fm = mv(c, g("final_mod.w"), g("final_mod.b"))
            for i in range(T):
                vv = mv(norm(h[i], fm[:D], fm[D:]), g("action_out.w"), g("action_out.b"))
                x[b][i] = [x[b][i][a] - vv[a] / N for a in range(A)]
    return np.array(x)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2)])
def test_oracle_matches_brute_force(hq, hkv):
    w = tiny(n_q_heads=hq, n_kv_heads=hkv, width=8 if hq == 2 else 16)
    W = synth.make_weights(w, std=0.3)
    mask = np.array([[1, 0, 1, 1, 0], [0, 1, 1, 1, 1]], np.uint8)
    K, V, _ = synth.make_prefix(w, mask=mask, garbage="huge")
    x0 = synth.make_noise(w)
    ours = run(w, W, K, V, mask, x0)
    ref = _bf_denoise(w, W, K, V, mask, x0)
    assert np.abs(ours - x0).max() > 0.05  # the loop moved the actions
    assert np.allclose(ours, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2)])
def test_oracle_fp8_matches_brute_force(hq, hkv):
    """The fp8 recipe (MolmoBot PR Part 3: per-tensor dynamic e4m3, amax ->
    cast -> scaled matmul) against the scalar twin, whose e4m3 rounding is a
    nearest-value scan of the format's code table: per-request activation
    amax, codes decided in fp32, y = (codes_x . codes_w) s_x s_w, a separate
    weight scale per logical tensor.  Two requests whose inputs differ in
    scale make a batch-wide amax, or one weight scale shared by q, k and v,
    fail it; so does dropping either scale."""
    w = tiny(n_q_heads=hq, n_kv_heads=hkv, width=8 if hq == 2 else 16)
    W = synth.make_weights(w, std=0.3)
    # per-tensor scales that differ widely between q, k and v, and gate, up
    for l in range(w.n_layers):
        for nm, f in (("k", 3.0), ("v", 0.25), ("up", 5.0), ("down", 0.5)):
            W[f"layers.{l}.{nm}"] = (W[f"layers.{l}.{nm}"] * np.float32(f)).astype(np.float32)
    mask = np.array([[1, 0, 1, 1, 0], [0, 1, 1, 1, 1]], np.uint8)
    K, V, _ = synth.make_prefix(w, mask=mask, garbage="huge")
    x0 = synth.make_noise(w)
    x0[1] *= np.float32(6.0)  # request 1's inputs on another scale than request 0's
    ours = run(w, W, K, V, mask, x0, fp8=True)
    ref = _bf_denoise(w, W, K, V, mask, x0, fp8=True)
    plain = run(w, W, K, V, mask, x0)
    assert np.abs(ours - plain).max() > 1e-3  # quantisation is visible at this size
    assert np.allclose(ours, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fp8_o", [False, True])
def test_oracle_fp8_rowwise_matches_brute_force(fp8_o):
    """The row-wise fp8 variant against the scalar twin: every input row its
    own amax, every weight column its own scale, y = (codes_x . codes_w)
    s_x[row] s_w[col]; with fp8_o the attention output projection too.  One
    row of request 1 and one weight column scaled far from the rest make a
    per-request or per-tensor scale fail it."""
    w = tiny(n_q_heads=2, n_kv_heads=1, width=8)
    W = synth.make_weights(w, std=0.3)
    for l in range(w.n_layers):
        for nm in ("q", "up", "down", "o"):
            wt = W[f"layers.{l}.{nm}"].copy()
            wt[:, 1] *= np.float32(9.0)
            W[f"layers.{l}.{nm}"] = wt
    mask = np.array([[1, 0, 1, 1, 0], [0, 1, 1, 1, 1]], np.uint8)
    K, V, _ = synth.make_prefix(w, mask=mask, garbage="huge")
    x0 = synth.make_noise(w)
    x0[1, 2] *= np.float32(7.0)
    p = dataclasses.replace(O.Params.like(w, fp8=True), fp8_rowwise=True, fp8_o=fp8_o)
    ours = run_params(W, p, K, V, mask, x0, w.n_steps)
    ref = _bf_denoise(w, W, K, V, mask, x0, fp8=True, rowwise=True, fp8_o=fp8_o)
    tensor = run(w, W, K, V, mask, x0, fp8=True)
    assert np.abs(ours - tensor).max() > 1e-4  # the granularity is visible
    assert np.allclose(ours, ref, rtol=0, atol=1e-12)


def test_rowwise_scaling_invariances():
    """Row-wise scales make rows and columns independent: a power-of-two
    factor on one input row leaves its codes unchanged and scales its scale
    (and its output row) by the same factor, exactly, and leaves every other
    output row bit-identical; likewise for one weight column.  The per-request
    recipe does not have the row property (its other rows' codes move)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    wt = (rng.standard_normal((64, 24)) * 0.1).astype(np.float32)
    wc, ws = O.quantize_columns(wt)
    y = O.fp8_linear_rowwise(x, wc, ws)
    x2 = x.copy()
    x2[3] *= np.float32(64.0)
    y2 = O.fp8_linear_rowwise(x2, wc, ws)
    assert np.array_equal(np.delete(y2, 3, 0), np.delete(y, 3, 0))
    assert np.array_equal(y2[3], y[3] * 64.0)
    c1, s1 = O.quantize_rows(x)
    c2, s2 = O.quantize_rows(x2)
    assert np.array_equal(c1, c2) and s2[3] == s1[3] * 64.0
    wt2 = wt.copy()
    wt2[:, 5] *= np.float32(0.25)
    wc2, ws2 = O.quantize_columns(wt2)
    y3 = O.fp8_linear_rowwise(x, wc2, ws2)
    assert np.array_equal(np.delete(y3, 5, 1), np.delete(y, 5, 1))
    assert np.array_equal(y3[:, 5], y[:, 5] * 0.25)
    # a single row is its own tensor
    ct, st = O.quantize_tensor(x[2])
    assert np.array_equal(ct, c1[2]) and st == s1[2]
    # per request: scaling row 3 moves the codes of the rows that set the amax with it
    t1, _ = O.quantize_tensor(x)
    t2, _ = O.quantize_tensor(x2)
    assert not np.array_equal(np.delete(t1, 3, 0), np.delete(t2, 3, 0))


def test_e4m3_twin_table_agrees_with_torch():
    """The twin's table-scan rounding against torch.float8_e4m3fn on values
    spread over every binade, the midpoints between codes and saturation."""
    vals = [v for v, _ in _E4M3]
    probes = set(vals)
    for a, b in zip(vals, vals[1:]):
        probes.update({(a + b) / 2, a + (b - a) / 3, b - (b - a) / 5})
    probes.update({500.0, 448.0 + 16.0, 1e-4, 3e-3})
    probes = sorted(probes)
    x = torch.tensor(probes + [-v for v in probes], dtype=torch.float32)
    got = [_e4m3_scalar(float(v)) for v in x]
    want = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64).tolist()
    assert got == want


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2small"])
def test_constant_velocity_head_euler_closed_form(name):
    w = synth.workload("c1") if name == "c1" else small_c2()
    W = synth.make_weights(w)
    vel = np.random.default_rng(7).standard_normal(w.action_dim)
    W["action_out.w"] = np.zeros_like(W["action_out.w"])
    W["action_out.b"] = vel.astype(np.float32)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    xN = run(w, W, K, V, m, x0)
    # x_N = x_0 + N * dt * v = x_0 - v
    assert np.allclose(xN, x0 - vel.astype(np.float32).astype(np.float64), rtol=0, atol=1e-14)


def test_zero_gates_closed_form():
    w = synth.workload("c1")
    W = synth.make_weights(w)
    D = w.width
    for l in range(w.n_layers):
        for ch in (2, 5):
            W[f"layers.{l}.mod.w"][:, ch * D:(ch + 1) * D] = 0
            W[f"layers.{l}.mod.b"][ch * D:(ch + 1) * D] = 0
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    xN = run(w, W, K, V, m, x0)
    # independent recursion with torch float64 pieces: h = x W_in + b_in never
    # changes through the layers, v = rms_norm(h) (1 + s_f) + sh_f, W_out, b_out
    tt = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = tt(x0)
    for k in range(w.n_steps):
        t = 1.0 - k / w.n_steps
        half = D // 2
        i = torch.arange(half, dtype=torch.float64)
        period = 4e-3 * 1000.0 ** (i / (half - 1))
        e = torch.cat([torch.sin(2 * math.pi * t / period), torch.cos(2 * math.pi * t / period)])
        c = F.silu(F.silu(e @ tt(W["time_mlp.1.w"]) + tt(W["time_mlp.1.b"])) @ tt(W["time_mlp.2.w"]) + tt(W["time_mlp.2.b"]))
        fm = c @ tt(W["final_mod.w"]) + tt(W["final_mod.b"])
        h = x @ tt(W["action_in.w"]) + tt(W["action_in.b"])
        u = F.rms_norm(h, (D,), eps=1e-6) * (1 + fm[:D]) + fm[D:]
        x = x - (u @ tt(W["action_out.w"]) + tt(W["action_out.b"])) / w.n_steps
    assert np.allclose(xN, x.numpy(), rtol=0, atol=1e-13)
    # and the prefix is then irrelevant
    K2, V2, _ = synth.make_prefix(w, mask=m, seed=4242)
    assert np.array_equal(run(w, W, K2, V2, m, x0), xN)


# --------------------------------------------------------------------------
# Invariants (pages' correctness properties)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["huge", "nan", "inf"])
def test_masked_rows_are_invisible(kind):
    w = synth.workload("c1")
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    base = run(w, W, K, V, m, x0)
    Kg, Vg = K.copy(), V.copy()
    synth.fill_garbage(w, Kg, Vg, m, kind)
    assert not np.array_equal(Kg, K)
    assert np.array_equal(run(w, W, Kg, Vg, m, x0), base)


def test_padding_is_invisible():
    """MolmoBot PR Part 1: padding the prefix to a fixed length changes nothing."""
    w = synth.workload("c1")
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    base = run(w, W, K, V, m, x0)
    w2 = synth.workload("c1", prefix_len=160)
    K2 = np.full((w.n_layers, 1, 160, 1, 64), np.nan, np.float32)
    V2 = np.full_like(K2, np.nan)
    K2[:, :, :64], V2[:, :, :64] = K, V
    m2 = np.zeros((1, 160), np.uint8)
    m2[:, :64] = m
    assert np.array_equal(run(w2, W, K2, V2, m2, x0), base)


@pytest.mark.parametrize("slot", [2, 1])
def test_masked_camera_slot_equals_pruned(slot):
    """LoongForge blog section 1: a masked 256-row camera slot (at the end of
    the image block, or in the middle of it) gives the same actions as the
    prefix with the slot pruned, since pads do not advance positions."""
    w2 = small_c2(layers=2, steps=2)
    w3 = synth.workload("c3", n_layers=2, n_steps=2)
    W = synth.make_weights(w2)
    K2, V2, m2 = synth.make_prefix(w2)
    K3, V3, m3 = synth.insert_camera_slot(w3, K2, V2, m2, slot=slot)
    x0 = synth.make_noise(w2)
    a2 = run(w2, W, K2, V2, m2, x0)
    a3 = run(w3, W, K3, V3, m3, x0)
    assert m3.sum() == m2.sum()
    assert np.array_equal(a2, a3)


def test_kv_projected_once_equals_reprojected_every_step():
    """MolmoBot PR Part 2 / Correctness: the per-query context K/V cache is
    bitwise equal to re-projecting the context on every flow step."""
    w = synth.workload("c1")
    W = synth.make_weights(w)
    rng = np.random.default_rng(77)
    Dc = 96
    hidden = [rng.standard_normal((1, w.prefix_len, Dc)) for _ in range(w.n_layers)]
    wk = [rng.standard_normal((Dc, 64)) * 0.1 for _ in range(w.n_layers)]
    wv = [rng.standard_normal((Dc, 64)) * 0.1 for _ in range(w.n_layers)]
    m = synth.valid_masks(w)
    m[0, 5] = 0  # a hole in the middle: positions must skip it
    KV = [O.project_prefix_kv(hidden[l], wk[l], wv[l], m, 1, 10000.0) for l in range(w.n_layers)]
    K = np.stack([k for k, _ in KV])
    V = np.stack([v for _, v in KV])
    x0 = synth.make_noise(w)
    E = O.Expert(synth.make_weights(w), O.Params.like(w))
    once = E.denoise(x0, K, V, m, w.n_steps)
    calls = []

    def reproject(l, b):
        calls.append((l, b))
        k, v = O.project_prefix_kv(hidden[l], wk[l], wv[l], m, 1, 10000.0)
        idx = np.nonzero(m[b])[0]
        return k[b, idx], v[b, idx]

    every = E.integrate(x0, reproject, m.sum(1), w.n_steps)
    assert len(calls) == w.n_steps * w.n_layers
    assert np.array_equal(once, every)
    # positions of the prefix skip the masked row
    pos = O.prefix_positions(m[0])
    assert pos[4] == 4 and pos[6] == 5


@pytest.mark.parametrize("fp8", [False, True])
def test_batched_equals_unbatched(fp8):
    w = small_c2(layers=2, steps=2, batch=3)
    w = synth.Workload(**{**w.__dict__, "name": "c5", "prefix_len": 640})
    W = synth.make_weights(w)
    m = synth.valid_masks(w, n_valid=(640, 521, 600))
    K, V, _ = synth.make_prefix(w, mask=m, garbage="nan")
    x0 = synth.make_noise(w)
    batched = run(w, W, K, V, m, x0, fp8=fp8)
    w1 = synth.Workload(**{**w.__dict__, "batch": 1})
    for b in range(3):
        alone = run(w1, W, K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1], fp8=fp8)
        # numpy's stacked matmul may block rows differently: rounding-level only
        assert np.allclose(batched[b:b + 1], alone, rtol=0, atol=1e-12)


def test_fp8_close_to_bf16():
    """Context: MolmoBot PR Part 3 reports 0.39 % max / 0.11 % mean action
    delta for fp8 on the LLM blocks.  Quantising this expert's QKV / MLP
    weights and inputs moves the actions by a few percent at most."""
    w = small_c2(layers=4, steps=4)
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    a = run(w, W, K, V, m, x0)
    b = run(w, W, K, V, m, x0, fp8=True)
    d = np.abs(a - b)
    assert 0 < d.max() < 0.1 * np.abs(a).max()


@pytest.mark.slow
def test_prefix_matters_at_full_size():
    """Guard: at the full Pi0.5-shaped (c2) and MolmoBot-shaped (c4) sizes,
    redrawing every visible prefix row moves the actions by more than five
    times the 2e-2 parity tolerance."""
    for name in ("c2", "c4"):
        w = synth.workload(name)
        W = synth.make_weights(w)
        K, V, m = synth.make_prefix(w)
        x0 = synth.make_noise(w)
        E = O.Expert(W, O.Params.like(w))
        a = E.denoise(x0, K, V, m, w.n_steps)
        K2, V2, _ = synth.make_prefix(w, mask=m, seed=99)
        b = E.denoise(x0, K2, V2, m, w.n_steps)
        assert np.abs(a - b).max() > 0.1, name


# --------------------------------------------------------------------------
# Context preparation (MolmoBot PR Part 2: prepare_cross_context /
# precompute_kv, once per query)
# --------------------------------------------------------------------------

def _rotate_complex(vec, pos, theta):
    """RoPE as a complex rotation: pair (x_j, x_{j+dh/2}) is the complex
    number x_j + i x_{j+dh/2}, multiplied by exp(i pos theta^(-2j/dh))."""
    dh = len(vec)
    half = dh // 2
    out = [0.0] * dh
    for j in range(half):
        z = complex(vec[j], vec[j + half]) * cmath.exp(1j * pos * theta ** (-2.0 * j / dh))
        out[j], out[j + half] = z.real, z.imag
    return out


def test_project_prefix_kv_is_a_complex_rotation_at_count_positions():
    """Each visible context row's key is its projection rotated by its count
    position (the number of visible rows before it: pads do not advance
    positions, LoongForge blog section 1); values are not rotated."""
    rng = np.random.default_rng(5)
    B, P, Dc, Hkv, dh, theta = 2, 9, 6, 2, 8, 10000.0
    hidden = rng.standard_normal((B, P, Dc))
    wk = rng.standard_normal((Dc, Hkv * dh))
    wv = rng.standard_normal((Dc, Hkv * dh))
    mask = np.array([[1, 1, 0, 1, 0, 0, 1, 1, 1], [0, 1, 1, 1, 1, 0, 1, 0, 1]], np.uint8)
    K, V = O.project_prefix_kv(hidden, wk, wv, mask, Hkv, theta)
    for b in range(B):
        pos = 0
        for r in range(P):
            kr = [sum(hidden[b, r, c] * wk[c, j] for c in range(Dc)) for j in range(Hkv * dh)]
            vr = [sum(hidden[b, r, c] * wv[c, j] for c in range(Dc)) for j in range(Hkv * dh)]
            for g in range(Hkv):
                want = _rotate_complex(kr[g * dh:(g + 1) * dh], pos, theta)
                assert np.allclose(K[b, r, g], want, rtol=0, atol=1e-12)
                assert np.allclose(V[b, r, g], vr[g * dh:(g + 1) * dh], rtol=0, atol=1e-12)
            pos += int(mask[b, r] != 0)


def test_prepare_prefix_appends_the_state_row():
    """With a robot state, one more visible row follows the context rows:
    its hidden state is the state through one linear layer (checked by
    loops), its key is rotated at the count of visible context rows."""
    rng = np.random.default_rng(6)
    L, B, P, Dc, Hkv, dh, S, theta = 2, 2, 7, 5, 1, 4, 3, 10000.0
    hidden = rng.standard_normal((L, B, P, Dc))
    wk = rng.standard_normal((L, Dc, Hkv * dh))
    wv = rng.standard_normal((L, Dc, Hkv * dh))
    ws, bs = rng.standard_normal((S, Dc)), rng.standard_normal(Dc)
    state = rng.standard_normal((B, S))
    mask = np.array([[1, 1, 1, 0, 1, 0, 0], [1, 0, 1, 1, 1, 1, 0]], np.uint8)
    hs = O.encode_state(state, ws, bs)
    for b in range(B):
        for c in range(Dc):
            assert abs(hs[b, c] - (sum(state[b, i] * ws[i, c] for i in range(S)) + bs[c])) < 1e-12
    K, V, m2 = O.prepare_prefix(hidden, wk, wv, mask, Hkv, theta, state_hidden=hs)
    assert K.shape == (L, B, P + 1, Hkv, dh) and m2.shape == (B, P + 1)
    assert np.array_equal(m2[:, :P], mask) and np.all(m2[:, P] == 1)
    for l in range(L):
        k0, v0 = O.project_prefix_kv(hidden[l], wk[l], wv[l], mask, Hkv, theta)
        assert np.array_equal(K[l, :, :P], k0) and np.array_equal(V[l, :, :P], v0)
        for b in range(B):
            kr = [sum(hs[b, c] * wk[l, c, j] for c in range(Dc)) for j in range(dh)]
            want = _rotate_complex(kr, int(mask[b].sum()), theta)
            assert np.allclose(K[l, b, P, 0], want, rtol=0, atol=1e-12)


def test_prepared_context_once_equals_every_step():
    """Context (and state) projected once per query == re-projected on every
    flow step (MolmoBot PR Part 2 / Correctness table), bitwise."""
    w = synth.workload("c1", n_layers=2, n_steps=3)
    W = synth.make_weights(w)
    Dc, S = 48, 14
    CW = synth.make_context_weights(w, Dc, S)
    H, m = synth.make_context(w, Dc)
    m[0, 7] = 0
    st = synth.make_state(w, S)
    wk = np.stack([CW[f"layers.{l}.ctx_k"] for l in range(w.n_layers)])
    wv = np.stack([CW[f"layers.{l}.ctx_v"] for l in range(w.n_layers)])
    hs = O.encode_state(st, CW["state_in.w"], CW["state_in.b"])
    K, V, m2 = O.prepare_prefix(H, wk, wv, m, w.n_kv_heads, w.rope_theta, hs)
    x0 = synth.make_noise(w)
    E = O.Expert(W, O.Params.like(w))
    once = E.denoise(x0, K, V, m2, w.n_steps)

    def reproject(l, b):
        hsl = O.encode_state(st, CW["state_in.w"], CW["state_in.b"])
        k, v, mm = O.prepare_prefix(H[l:l + 1], wk[l:l + 1], wv[l:l + 1], m, w.n_kv_heads, w.rope_theta, hsl)
        idx = np.nonzero(mm[b])[0]
        return k[0, b, idx], v[0, b, idx]

    every = E.integrate(x0, reproject, m2.sum(1), w.n_steps)
    assert np.array_equal(once, every)
    assert np.abs(once - E.denoise(x0, K[:, :, :-1], V[:, :, :-1], m, w.n_steps)).max() > 1e-3  # the state row counts


# --------------------------------------------------------------------------
# DiT-style block (MolmoBot PR Part 2: attn2 reads the cached context K/V;
# Correctness table: cross_attn & self_attn)
# --------------------------------------------------------------------------

def _bf_denoise_dit(w, W, K, V, mask, x0):
    """Scalar twin of the DiT-style block: per layer a self-attention over
    the action tokens (explicit all-visible key list), a cross-attention of
    separate q2 / o2 projections over the prefix with an explicit visibility
    list and -inf logits for invisible rows (an empty visible set adds
    nothing), and the MLP; nine modulation chunks."""
    L, D, Hq, Hkv, dh, Fd = w.n_layers, w.width, w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim
    T, A, N, B, P = w.action_horizon, w.action_dim, w.n_steps, w.batch, w.prefix_len
    g = lambda name: np.asarray(W[name], dtype=np.float64)

    def mv(vec, mat, bias=None):
        out = [0.0] * mat.shape[1]
        for j in range(mat.shape[1]):
            acc = 0.0
            for i in range(mat.shape[0]):
                acc += vec[i] * mat[i, j]
            out[j] = acc + (0.0 if bias is None else bias[j])
        return out

    silu = lambda z: z / (1.0 + math.exp(-z))

    def norm(vec, scale, shift):
        r = 1.0 / math.sqrt(sum(v * v for v in vec) / len(vec) + w.rms_eps)
        return [vec[i] * r * (1.0 + scale[i]) + shift[i] for i in range(len(vec))]

    def rot(vec, p):
        half = len(vec) // 2
        out = list(vec)
        for j in range(half):
            ang = p * w.rope_theta ** (-2.0 * j / len(vec))
            out[j] = vec[j] * math.cos(ang) - vec[j + half] * math.sin(ang)
            out[j + half] = vec[j + half] * math.cos(ang) + vec[j] * math.sin(ang)
        return out

    def attend(qv, keys, vals, vis):
        logits = [sum(qv[d] * kk[d] for d in range(dh)) / math.sqrt(dh) if vv else -math.inf
                  for kk, vv in zip(keys, vis)]
        if not any(vis):
            return [0.0] * dh
        mx = max(logits)
        ws = [math.exp(s - mx) if s != -math.inf else 0.0 for s in logits]
        tot = sum(ws)
        return [sum(ws[j] * vals[j][d] for j in range(len(keys)) if ws[j] != 0.0) / tot for d in range(dh)]

    x = [[[float(x0[b, i, a]) for a in range(A)] for i in range(T)] for b in range(B)]
    for k in range(N):
        t = 1.0 - k / N
        half = D // 2
        e = [math.sin(2 * math.pi * t / (4e-3 * 1000.0 ** (i / (half - 1)))) for i in range(half)]
        e += [math.cos(2 * math.pi * t / (4e-3 * 1000.0 ** (i / (half - 1)))) for i in range(half)]
        c = [silu(z) for z in mv([silu(z) for z in mv(e, g("time_mlp.1.w"), g("time_mlp.1.b"))],
                                 g("time_mlp.2.w"), g("time_mlp.2.b"))]
        for b in range(B):
            nv = int(sum(int(mask[b, j] != 0) for j in range(P)))
            h = [mv(x[b][i], g("action_in.w"), g("action_in.b")) for i in range(T)]
            for l in range(L):
                mod = mv(c, g(f"layers.{l}.mod.w"), g(f"layers.{l}.mod.b"))
                ch = [mod[j * D:(j + 1) * D] for j in range(9)]
                pre = f"layers.{l}."
                # attn1: the action tokens among themselves
                u = [norm(h[i], ch[0], ch[1]) for i in range(T)]
                qs = [mv(r, g(pre + "q")) for r in u]
                ks = [mv(r, g(pre + "k")) for r in u]
                vs = [mv(r, g(pre + "v")) for r in u]
                o = [[0.0] * (Hq * dh) for _ in range(T)]
                for hd in range(Hq):
                    kv = hd // (Hq // Hkv)
                    keys = [rot(ks[j][kv * dh:(kv + 1) * dh], nv + j) for j in range(T)]
                    vals = [vs[j][kv * dh:(kv + 1) * dh] for j in range(T)]
                    for i in range(T):
                        o[i][hd * dh:(hd + 1) * dh] = attend(rot(qs[i][hd * dh:(hd + 1) * dh], nv + i),
                                                             keys, vals, [True] * T)
                for i in range(T):
                    ob = mv(o[i], g(pre + "o"))
                    h[i] = [h[i][d] + ch[2][d] * ob[d] for d in range(D)]
                # attn2: the action queries over the prefix
                u2 = [norm(h[i], ch[3], ch[4]) for i in range(T)]
                q2 = [mv(r, g(pre + "q2")) for r in u2]
                o2 = [[0.0] * (Hq * dh) for _ in range(T)]
                for hd in range(Hq):
                    kv = hd // (Hq // Hkv)
                    keys = [[float(K[l, b, j, kv, d]) for d in range(dh)] for j in range(P)]
                    vals = [[float(V[l, b, j, kv, d]) for d in range(dh)] for j in range(P)]
                    vis = [mask[b, j] != 0 for j in range(P)]
                    for i in range(T):
                        o2[i][hd * dh:(hd + 1) * dh] = attend(rot(q2[i][hd * dh:(hd + 1) * dh], nv + i),
                                                              keys, vals, vis)
                for i in range(T):
                    ob = mv(o2[i], g(pre + "o2"))
                    h[i] = [h[i][d] + ch[5][d] * ob[d] for d in range(D)]
                # MLP
                for i in range(T):
                    u3 = norm(h[i], ch[6], ch[7])
                    gt, up = mv(u3, g(pre + "gate")), mv(u3, g(pre + "up"))
                    act = [0.5 * gt[f] * (1 + math.tanh(math.sqrt(2 / math.pi) * (gt[f] + 0.044715 * gt[f] ** 3)))
                           * up[f] for f in range(Fd)]
                    dn = mv(act, g(pre + "down"))
                    h[i] = [h[i][d] + ch[8][d] * dn[d] for d in range(D)]
            fm = mv(c, g("final_mod.w"), g("final_mod.b"))
            for i in range(T):
                vv = mv(norm(h[i], fm[:D], fm[D:]), g("action_out.w"), g("action_out.b"))
                x[b][i] = [x[b][i][a] - vv[a] / N for a in range(A)]
    return np.array(x)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2)])
def test_oracle_dit_matches_brute_force(hq, hkv):
    """With request 1's prefix entirely masked its cross-attention adds
    nothing (and NaN there must not leak)."""
    w = tiny(n_q_heads=hq, n_kv_heads=hkv, width=8 if hq == 2 else 16, block="dit")
    W = synth.make_weights(w, std=0.3)
    mask = np.array([[1, 0, 1, 1, 0], [0, 0, 0, 0, 0]], np.uint8)
    K, V, _ = synth.make_prefix(w, mask=mask, garbage="nan")
    x0 = synth.make_noise(w)
    ours = run(w, W, K, V, mask, x0)
    ref = _bf_denoise_dit(w, W, K, V, mask, x0)
    assert np.abs(ours - x0).max() > 0.05
    assert np.allclose(ours, ref, rtol=0, atol=1e-11)


def test_dit_without_cross_attention_is_the_joint_block_without_prefix():
    """With o2 = 0 the DiT block is attn1 + MLP: the joint block over an
    empty prefix whose six chunks are the DiT's (attn1, MLP) chunks; the
    prefix cannot matter (only position differences enter attn1)."""
    wd = synth.workload("c1", block="dit", n_layers=2, n_steps=3)
    Wd = synth.make_weights(wd)
    D = wd.width
    for l in range(wd.n_layers):
        Wd[f"layers.{l}.o2"] = np.zeros_like(Wd[f"layers.{l}.o2"])
    wj = synth.workload("c1", n_layers=2, n_steps=3, prefix_len=0)
    Wj = {k: v for k, v in Wd.items() if not (k.endswith(".q2") or k.endswith(".o2"))}
    keep = [0, 1, 2, 6, 7, 8]
    for l in range(wd.n_layers):
        mw, mb = Wd[f"layers.{l}.mod.w"], Wd[f"layers.{l}.mod.b"]
        Wj[f"layers.{l}.mod.w"] = np.concatenate([mw[:, c * D:(c + 1) * D] for c in keep], axis=1)
        Wj[f"layers.{l}.mod.b"] = np.concatenate([mb[c * D:(c + 1) * D] for c in keep])
    K, V, m = synth.make_prefix(wd)
    x0 = synth.make_noise(wd)
    dit = run(wd, Wd, K, V, m, x0)
    joint = run(wj, Wj, K[:, :, :0], V[:, :, :0], m[:, :0], x0)
    assert np.allclose(dit, joint, rtol=0, atol=1e-10)


def test_dit_invariants():
    """Masked rows and garbage are invisible, batched == alone, and a single
    visible prefix row makes attn2 return that row's V for every query."""
    w = small_c2(layers=2, steps=2, batch=2)
    w = synth.Workload(**{**w.__dict__, "block": "dit", "name": "c5", "prefix_len": 600})
    W = synth.make_weights(w)
    m = synth.valid_masks(w, n_valid=(600, 530))
    K, V, _ = synth.make_prefix(w, mask=m)
    x0 = synth.make_noise(w)
    a = run(w, W, K, V, m, x0)
    Kg, Vg = K.copy(), V.copy()
    synth.fill_garbage(w, Kg, Vg, m, "nan")
    assert np.array_equal(run(w, W, Kg, Vg, m, x0), a)
    w1 = synth.Workload(**{**w.__dict__, "batch": 1})
    for b in range(2):
        alone = run(w1, W, K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1])
        assert np.allclose(alone, a[b:b + 1], rtol=0, atol=1e-12)
    # one visible key: attn2's output is its V row (softmax of one logit)
    q = np.random.default_rng(3).standard_normal((5, 8, 256))
    kk = np.random.default_rng(4).standard_normal((1, 1, 256))
    vv = np.random.default_rng(5).standard_normal((1, 1, 256))
    o = O.attention(q, kk, vv)
    assert np.allclose(o, np.broadcast_to(vv[0, 0], o.shape), rtol=0, atol=1e-15)
    assert np.array_equal(O.attention(q, kk[:0], vv[:0]), np.zeros_like(q))
