"""Benchmark of the action-expert denoise loop on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A "step" here is one whole denoise call: the time path, N Euler steps of the
layer stack with attention over the resident prefix K/V, and the action
updates, for one batch of synthetic inputs already resident in HBM.  The
headline is the Pi0.5-shaped batch-1 workload (c2): action chunks/s.  The
batched workload (c5, 16 requests, bf16 and fp8), the three-camera (c3),
MolmoBot-shaped (c4) and tiny fp32 (c1) workloads, prefix ingest and
"ingest + denoise" are measured as well.  Rank 0 prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA

# Sources the whole-call kernel is compiled and planned from (its split
# counts are chosen in the runtime); a stored counter reading is reported
# only while their digest is the one it was taken with.
KERNEL_SOURCES = ["ae_persist.hip", "ae_device.h", "ae_kernels.h", "ae_runtime.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "persist_kernel_c2_traffic.txt")

DESCRIPTIONS = {
    "c1": "tiny fp32 expert",
    "c2": "Pi0.5-shaped action expert",
    "c3": "Pi0.5-shaped expert, three camera slots with one masked",
    "c4": "MolmoBot-shaped expert",
    "c5": "Pi0.5-shaped expert, 16 concurrent requests",
    "c5fp8": "Pi0.5-shaped expert, 16 concurrent requests, e4m3 QKV / gate-up / down",
    "c5fp8r": "Pi0.5-shaped expert, 16 concurrent requests, e4m3 QKV / O / gate-up / down with row-wise "
              "scales (per activation row, per weight column)",
    "c4dit": "MolmoBot-shaped expert with the DiT-style block (attn1 over the actions, attn2 over the prefix)",
    "c2fp8r": "Pi0.5-shaped action expert, e4m3 QKV / O / gate-up / down with row-wise scales",
}


def kernel_digest():
    """Digest of the persistent kernel's code: comments and layout are
    stripped first, so only a change to what compiles invalidates a stored
    counter reading."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vla_flow_matching_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
    reading (scaled by a plain copy's reading), or None when absent or taken
    on other kernel sources."""
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_FILE).read().split("\n")
                  if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("digest", "").strip() != kernel_digest() or kv.get("workload", "").strip() != workload:
        return None
    return float(kv["hbm_bytes_per_launch"])


def algorithmic_work(w, n_valid, with_time_path=False):
    """Bytes a denoise call must move and FLOPs it must do (masked / padded
    prefix rows excluded; activations excluded: they stay in L2 / MALL).
    The time path (time MLP + every layer's modulation) depends only on the
    step count and the weights; the library keeps its table across calls, so
    a steady-state call does not include it."""
    D, L, F, A, T, N = w.width, w.n_layers, w.mlp_dim, w.action_dim, w.action_horizon, w.n_steps
    qd, kd = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    layer_params = D * (qd + 2 * kd) + qd * D + 2 * D * F + F * D
    if getattr(w, "block", "joint") == "dit":  # attn2's q2 and o2
        layer_params += 2 * D * qd
    step_params = L * layer_params + 2 * A * D
    t_params = 6 * L * D * D + 2 * D * D + 2 * D * D
    kv_bytes = L * int(np.sum(n_valid)) * 2 * kd * esz
    # e4m3 projections move one byte per weight (their per-column scales are negligible)
    f8_params = 0
    if getattr(w, "proj_dtype", "same") == "fp8":
        f8_params = L * (D * (qd + 2 * kd) + 2 * D * F + F * D + (qd * D if getattr(w, "fp8_o", False) else 0))
    step_bytes = f8_params + (step_params - f8_params) * esz
    bytes_call = N * (step_bytes + kv_bytes) + (t_params * esz if with_time_path else 0)
    B = len(n_valid)
    attn_flops = sum(4 * T * w.n_q_heads * w.head_dim * (int(n) + T) for n in n_valid) * L * N
    flops_call = 2 * B * T * step_params * N + attn_flops + (2 * N * t_params if with_time_path else 0)
    return bytes_call, flops_call


def fp8_flops_split(w, n_valid):
    """(FLOPs of the e4m3 GEMMs: QKV, gate/up, down and, with fp8_o, O; all
    other FLOPs) per call."""
    D, L, F, T, N = w.width, w.n_layers, w.mlp_dim, w.action_horizon, w.n_steps
    qd, kd = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    B = len(n_valid)
    fp8_params = L * (D * (qd + 2 * kd) + 2 * D * F + F * D + (qd * D if getattr(w, "fp8_o", False) else 0))
    f8 = 2 * B * T * fp8_params * N
    _, total = algorithmic_work(w, n_valid)
    return f8, total - f8


def prefix_bytes(w, n_valid):
    """Bytes prefix ingest must move: the visible rows of K and V read once
    and written once into the cache (the mask read and the tables are
    negligible)."""
    esz = 2 if w.dtype == "bf16" else 4
    return 2 * 2 * w.n_layers * int(np.sum(n_valid)) * w.n_kv_heads * w.head_dim * esz


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


class DeviceErrors(RuntimeError):
    pass


def inputs_of(name):
    """Seeded inputs of one workload (c3: the three-camera prefix built from
    the two-camera one, its third slot masked)."""
    from vla_flow_matching_amd import synth

    if name == "c3":
        w2 = synth.workload("c2")
        W = synth.make_weights(synth.workload("c3"))
        K2, V2, m2 = synth.make_prefix(w2)
        K, V, m = synth.insert_camera_slot(synth.workload("c3"), K2, V2, m2, slot=2, garbage="nan")
        return synth.workload("c3"), W, K, V, m, synth.make_noise(w2)
    w = synth.workload(name)
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w, garbage="nan")
    return w, W, K, V, m, synth.make_noise(w)


def run_gpu(name, calls, warmup, prefix_reps=0, exec_path=0):
    """Time `calls` graph replays of one workload's denoise call (events on
    the library's stream around all of them), then the same number with an
    event pair per call (percentiles), then prefix ingest alone and ingest +
    denoise.  exec_path: the library's choice (0) or a forced path (1
    whole-call, 2 per-phase).  Raises DeviceErrors if a whole-call kernel
    wait timed out."""
    import torch

    from vla_flow_matching_amd import binding

    w, W, K, V, m, x0 = inputs_of(name)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    res = {}
    with binding.ActionExpert(binding.make_config(w, exec_path=exec_path)) as ex:
        ex.load_weights(binding.weights_to_device(W, w.dtype))
        del W
        Kt = torch.from_numpy(K).to("cuda", dt)
        Vt = torch.from_numpy(V).to("cuda", dt)
        mt = torch.from_numpy(m).cuda()
        del K, V
        ex.set_prefix_kv(Kt, Vt, mt)
        x = torch.from_numpy(x0).cuda()
        out = torch.empty_like(x)
        for _ in range(warmup):
            ex.denoise(x, w.n_steps, out=out)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        t0, t1 = ev(), ev()
        wall0 = time.perf_counter()
        t0.record(stream)
        for _ in range(calls):
            ex.denoise(x, w.n_steps, out=out)
        t1.record(stream)
        torch.cuda.synchronize()
        res["wall_s"] = time.perf_counter() - wall0
        res["ms"] = t0.elapsed_time(t1) / calls
        # the same calls with an event pair each (latency distribution)
        pairs = [(ev(), ev()) for _ in range(calls)]
        for a, b in pairs:
            a.record(stream)
            ex.denoise(x, w.n_steps, out=out)
            b.record(stream)
        torch.cuda.synchronize()
        lat = [a.elapsed_time(b) for a, b in pairs]
        res["p10"], res["p50"], res["p90"] = pct(lat, 10), pct(lat, 50), pct(lat, 90)
        if prefix_reps:
            pairs = [(ev(), ev()) for _ in range(prefix_reps)]
            for a, b in pairs:
                a.record(stream)
                ex.set_prefix_kv(Kt, Vt, mt)
                b.record(stream)
            torch.cuda.synchronize()
            res["prefix_ms"] = [a.elapsed_time(b) for a, b in pairs]
            pairs = [(ev(), ev()) for _ in range(prefix_reps)]
            for a, b in pairs:
                a.record(stream)
                ex.set_prefix_kv(Kt, Vt, mt)
                ex.denoise(x, w.n_steps, out=out)
                b.record(stream)
            torch.cuda.synchronize()
            res["set_denoise_ms"] = [a.elapsed_time(b) for a, b in pairs]
        if not torch.isfinite(out).all().item():
            raise DeviceErrors(f"{name}: non-finite actions")
        st = ex.stats()
        if st["device_errors"] != 0:
            raise DeviceErrors(f"{name}: {st['device_errors']} whole-call launch(es) timed out; "
                               "their results are invalid")
    res["stats"] = st
    res["w"] = w
    res["n_valid"] = m.sum(axis=1)
    return res


def vendor_gemm_yardstick(name="c5", per_graph=50, replays=10):
    """The vendor library's bf16 products (hipBLASLt through torch.matmul,
    replayed from a graph) on one layer's four product shapes of a workload:
    a reference point for what a general-purpose GEMM reaches at these
    shapes, beside the fused per-phase kernels (whose per-kernel times come
    from the kernel trace).  No part of the denoise path runs here."""
    import torch
    from vla_flow_matching_amd import synth

    w = synth.workload(name)
    M, D, F = w.batch * w.action_horizon, w.width, w.mlp_dim
    qdim, kvdim = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    shapes = {"qkv": (M, D, qdim + 2 * kvdim), "o": (M, qdim, D), "gate_up": (M, D, 2 * F), "down": (M, F, D)}
    out = {"library": "hipBLASLt (torch.matmul, bf16, graph replay)", "rows": M}
    total = 0.0
    for key, (m, k, n) in shapes.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
        c = a @ b
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                c = a @ b
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (per_graph * replays)
        tf = 2.0 * m * k * n / (us * 1e-6) / 1e12
        out[key] = {"m": m, "k": k, "n": n, "us": us, "tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS}
        total += us
        del g, a, b, c
    out["us_per_layer"] = total
    return out


def run_prepare(reps, context_width=2560, state_dim=14):
    """Time ae_prepare_prefix on the MolmoBot-shaped workload: every layer's
    context K/V from per-layer hidden states of a Qwen3-4B-wide context
    (2560) plus the 14-D robot state, once per query."""
    import torch

    from vla_flow_matching_amd import binding, synth

    w = synth.workload("c4", prefix_len=2047)
    W = synth.make_weights(w)
    CW = synth.make_context_weights(w, context_width, state_dim)
    m = np.zeros((1, w.prefix_len), np.uint8)
    m[0, :1600 + 27] = 1
    H, _ = synth.make_context(w, context_width, mask=m)
    state = synth.make_state(w, state_dim)
    cfg = binding.make_config(w, max_prefix_len=2048, context_width=context_width, state_dim=state_dim)
    with binding.ActionExpert(cfg) as ex:
        ex.load_weights({**binding.weights_to_device(W, w.dtype), **binding.weights_to_device(CW, w.dtype)})
        Ht = torch.from_numpy(H).to("cuda", torch.bfloat16)
        mt = torch.from_numpy(m).cuda()
        st = torch.from_numpy(state).cuda()
        x = torch.from_numpy(synth.make_noise(w)).cuda()
        for _ in range(3):
            ex.prepare_prefix(Ht, mt, st)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        pairs = [(ev(), ev()) for _ in range(reps)]
        for a, b in pairs:
            a.record(stream)
            ex.prepare_prefix(Ht, mt, st)
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in pairs]
        pairs = [(ev(), ev()) for _ in range(reps)]
        for a, b in pairs:
            a.record(stream)
            ex.prepare_prefix(Ht, mt, st)
            ex.denoise(x, w.n_steps)
            b.record(stream)
        torch.cuda.synchronize()
        ms2 = [a.elapsed_time(b) for a, b in pairs]
        if ex.stats()["device_errors"]:
            raise DeviceErrors("prepare: a whole-call launch timed out")
    L, P, kd = w.n_layers, w.prefix_len, w.n_kv_heads * w.head_dim
    n = int(m.sum()) + 1
    flops = 2 * L * (P + 1) * context_width * 2 * kd
    byts = 2 * (L * P * context_width + L * context_width * 2 * kd + L * n * 2 * kd)
    p50 = float(np.median(ms))
    return {"workload": f"c4 context preparation: {L} layers, {P} context rows ({n - 1} visible) + the "
                        f"{state_dim}-D state, context width {context_width}, Hkv {w.n_kv_heads} x {w.head_dim}",
            "ms_p50": p50, "ms_p10": pct(ms, 10), "ms_p90": pct(ms, 90),
            "prepare_plus_denoise_ms_p50": float(np.median(ms2)),
            "algorithmic_flops": flops, "algorithmic_bytes": byts,
            "achieved_TFLOPs": flops / (p50 * 1e-3) / 1e12, "achieved_GBps": byts / (p50 * 1e-3) / 1e9}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, budget_s):
    """The oracle as it stands, on this host's cores, over a bounded sample
    of whole denoise calls of the same workload; then on one thread over a
    3-step call (the per-step cost, scaled to the 10-step call)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import ae_oracle as O
    from vla_flow_matching_amd import synth

    w = synth.workload(name)
    W = synth.make_weights(w)
    K, V, m = synth.make_prefix(w)
    x0 = synth.make_noise(w)
    E = O.Expert(W, O.Params.like(w))
    calls, t0 = 0, time.perf_counter()
    while True:
        E.denoise(x0, K, V, m, w.n_steps)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 8:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    with threadpool_limits(1):
        n1 = 3
        t1 = time.perf_counter()
        E.denoise(x0, K, V, m, n1)
        el1 = time.perf_counter() - t1
    call1 = el1 / n1 * w.n_steps
    return {"value": calls * w.batch / el, "unit": "chunks/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{calls} whole {w.name} denoise call(s) ({w.n_steps} steps, batch {w.batch}) "
                      f"in {el:.1f} s, NumPy float64 with {threads} BLAS threads "
                      f"on {os.cpu_count()} host CPUs",
            "cpu_model": cpu_model(),
            "value_1thread": w.batch / call1,
            "sample_1thread": f"one {n1}-step {w.name} call on 1 thread in {el1:.1f} s, scaled to "
                              f"{w.n_steps} steps ({call1:.1f} s per call)"}


def workload_line(name, r, bound):
    w, nv = r["w"], r["n_valid"]
    b, f = algorithmic_work(w, nv)
    ms = r["ms"]
    d = {"workload": f"{name}: {DESCRIPTIONS.get(name, name)}, {w.n_layers} layers, width {w.width}, "
                     f"{w.n_q_heads}/{w.n_kv_heads} heads x {w.head_dim}, MLP {w.mlp_dim}, batch {w.batch}, "
                     f"prefix {w.prefix_len} ({int(nv.sum())} visible), {w.action_horizon}x{w.action_dim} "
                     f"actions, {w.n_steps} steps, {w.dtype}",
         "value": w.batch / (ms * 1e-3), "unit": "chunks/s", "ms_per_call": ms, "us_per_call": ms * 1e3,
         "denoise_steps_per_s": w.n_steps / (ms * 1e-3),
         "latency_ms": {"p10": r["p10"], "p50": r["p50"], "p90": r["p90"]},
         "persistent_calls": r["stats"]["persistent_calls"],
         # the kernels the library chose for this workload (AE_PATH_AUTO)
         "path": "whole-call kernel" if r["stats"]["persistent_calls"] > 0 else "per-phase kernels",
         # launches in the call's graph (the whole-call kernel: a counter fill and itself)
         "kernels_per_call": r["stats"]["graph_nodes"],
         "kernels_per_step": r["stats"]["graph_nodes"] / w.n_steps}
    if bound == "hbm":
        gbs = b / (ms * 1e-3) / 1e9
        d["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": b}
    elif bound == "mfma":
        tf = f / (ms * 1e-3) / 1e12
        d["roofline"] = {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS, "algorithmic_flops_per_call": f}
    elif bound == "mfma-fp8":
        f8 = fp8_flops_split(w, nv)
        t_peak = f8[0] / (FP8_PEAK_TFLOPS * 1e12) + f8[1] / (BF16_PEAK_TFLOPS * 1e12)
        d["roofline"] = {"bound": "mfma (mixed fp8 / bf16 peak)", "achieved": f / (ms * 1e-3) / 1e12,
                         "unit": "TFLOP/s", "peak_time_ms": t_peak * 1e3, "frac": t_peak / (ms * 1e-3),
                         "algorithmic_flops_per_call": f, "fp8_flops": f8[0], "bf16_flops": f8[1]}
    else:
        d["roofline"] = {"bound": "latency", "note": "a few MB per call: neither roofline applies"}
    if "prefix_ms" in r:
        pb = prefix_bytes(w, nv)
        pm = float(np.median(r["prefix_ms"]))
        d["prefix_ingest"] = {"ms_p50": pm, "ms_p10": pct(r["prefix_ms"], 10), "ms_p90": pct(r["prefix_ms"], 90),
                              "algorithmic_bytes": pb, "achieved_GBps": pb / (pm * 1e-3) / 1e9}
        d["set_plus_denoise_ms"] = {"p10": pct(r["set_denoise_ms"], 10), "p50": pct(r["set_denoise_ms"], 50),
                                    "p90": pct(r["set_denoise_ms"], 90)}
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--others", default="c5,c5fp8,c5fp8r,c4,c4dit,c3,c2fp8r,c1",
                    help="further workloads measured after the headline, or 'none'")
    ap.add_argument("--other-calls", type=int, default=0,
                    help="timed calls of each further workload (0: from --steps)")
    ap.add_argument("--no-prepare", action="store_true", help="skip the context-preparation timing")
    ap.add_argument("--no-yardstick", action="store_true",
                    help="skip timing the vendor library's products at c5's shapes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--proc-maps", default="",
                    help="write the process's memory map to this file at the end (to attribute an "
                         "address printed by a crash in a later exit handler, e.g. a profiler's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, run two plain 256 MiB device copies (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the denoise path shards by request with no "
              "exchange between GPUs, so the figure it reports is a single GPU's throughput "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    try:
        r = run_gpu(args.workload, args.steps, args.warmup, prefix_reps=20)
        w, n_valid, ms = r["w"], r["n_valid"], r["ms"]
        bytes_call, flops_call = algorithmic_work(w, n_valid)
        gbs = bytes_call / (ms * 1e-3) / 1e9
        head = workload_line(args.workload, r, "hbm")
        line = {
            "metric": "action chunks/s (10-step denoise) at batch 1; % HBM roofline",
            "value": w.batch / (ms * 1e-3),
            "unit": "chunks/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16" if w.dtype == "bf16" else "f32",
            "data": "synthetic (seeded random-init weights, N(0,1) prefix K/V and noise)",
            "config": {
                "workload": head["workload"],
                "batch": w.batch, "n_steps": w.n_steps, "prefix_len": w.prefix_len,
                "n_valid": [int(v) for v in n_valid],
            },
            "denoise_steps_per_s": w.n_steps / (ms * 1e-3),
            "latency_ms": head["latency_ms"],
            "prefix_ingest": head.get("prefix_ingest"),
            "set_plus_denoise_ms": head.get("set_plus_denoise_ms"),
            "path": head["path"],
            "kernels_per_call": head["kernels_per_call"],
            "roofline": {
                "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS,
                "traffic": stored_traffic(w.name) if r["stats"]["persistent_calls"] > 0 else None,
                "kernel": "persist_kernel: one launch per denoise call (the call's graph also "
                          "holds a 256-int counter fill)" if r["stats"]["persistent_calls"] > 0 else
                          "per-phase kernels (a graph of several launches per layer)",
                "algorithmic_bytes_per_launch": bytes_call,
            },
            "graph": {"captures": r["stats"]["graph_captures"], "replays": r["stats"]["graph_replays"],
                      "hits": r["stats"]["graph_hits"], "misses": r["stats"]["graph_misses"]},
            "wall_s_timed": r["wall_s"],
        }
        others = {}
        bounds = {"c5": "mfma", "c5fp8": "mfma-fp8", "c5fp8r": "mfma-fp8", "c4": "hbm", "c4dit": "hbm", "c3": "hbm",
                  "c2fp8r": "hbm",
                  "c1": "latency", "c2": "hbm"}
        if args.others != "none":
            for name in [s for s in args.others.split(",") if s]:
                heavy = name.startswith("c5")
                calls = max(5, args.steps // 8) if heavy else max(10, args.steps // 2)
                warm, reps = max(2, args.warmup // 4), 5 if heavy else 10
                if args.other_calls > 0:  # a short run (e.g. under a counter profiler)
                    calls, warm, reps = args.other_calls, 1, 1
                ro = run_gpu(name, calls, warm, prefix_reps=reps)
                others[name] = workload_line(name, ro, bounds.get(name, "hbm"))
            for c4 in ("c4", "c4dit"):
                if c4 in others:
                    others[c4]["roofline"]["note"] = (
                        "the MolmoBot-shaped weights (208 MB per step, 236 MB with the DiT block's q2 / o2) "
                        "and the visible K/V (~20 MB) nearly fit in the 256 MB last-level cache, so a call "
                        "can run above the HBM bound (and the library runs it on the per-phase kernels, "
                        "which find a step's weights still cached); reported against 8 TB/s")
        line["workloads"] = others
        if args.others != "none":
            # the same call on the path the library did not choose (the
            # evidence for its choice; a short run)
            def other_path(name, chosen_calls):
                alt = 2 if chosen_calls > 0 else 1
                ro = run_gpu(name, 10, 2, 0, exec_path=alt)
                return {"path": "per-phase kernels" if alt == 2 else "whole-call kernel", "ms_per_call": ro["ms"],
                        "persistent_calls": ro["stats"]["persistent_calls"]}
            line["other_path"] = other_path(args.workload, r["stats"]["persistent_calls"])
            if "c4" in others:
                others["c4"]["other_path"] = other_path("c4", others["c4"]["persistent_calls"])
        if args.others != "none" and not args.no_prepare:
            line["context_preparation"] = run_prepare(20)
        if "c5" in others:
            if not args.no_yardstick:
                others["c5"]["vendor_gemm_yardstick"] = vendor_gemm_yardstick("c5")
            line["secondary"] = others["c5"]
        if "c5fp8" in others:
            line["secondary_fp8"] = others["c5fp8"]
        if "c5fp8r" in others:
            line["secondary_fp8_rowwise"] = others["c5fp8r"]
    except DeviceErrors as e:
        print(f"bench.py: {e}", file=sys.stderr, flush=True)
        sys.exit(3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    line["kernel_digest"] = kernel_digest()
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        import torch

        a = torch.ones(64 << 20, device="cuda")
        b = torch.empty_like(a)
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copy calibration: 2 copies of 268435456 bytes", file=sys.stderr, flush=True)
    if args.proc_maps:
        with open("/proc/self/maps") as src, open(args.proc_maps, "w") as dst:
            dst.write(src.read())


if __name__ == "__main__":
    main()
