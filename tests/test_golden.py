"""Fixtures under tests/golden/, each with its citation, against the oracle
(e4m3 values of the OCP FP8 spec) and the synthetic workloads (token counts
the pages state)."""

import os

import numpy as np

from oracle import ae_oracle as O
from vla_flow_matching_amd import synth

HERE = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(HERE, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            out.append(line.split())
    return out


def test_e4m3_spec_values():
    for bits, val in _rows("e4m3_ocp.txt"):
        v = float(val)
        b = int(bits, 16)
        sign = -1.0 if b & 0x80 else 1.0
        e, f = (b >> 3) & 0xF, b & 0x7
        decoded = sign * (f / 8.0 * 2.0 ** -6 if e == 0 else (1 + f / 8.0) * 2.0 ** (e - 7))
        assert decoded == v
        assert O.e4m3(np.array([v]))[0] == v
    # one spacing above the max normal saturates instead of overflowing
    assert O.e4m3(np.array([480.0]))[0] == 448.0


def test_workloads_follow_page_token_counts():
    g = {k: int(v) for k, v in _rows("pages_workloads.txt")}
    c2, c3, c4 = synth.workload("c2"), synth.workload("c3"), synth.workload("c4")
    assert c2.action_horizon == g["pi05_action_tokens"]
    # two cameras + instruction + actions = 762 tokens; our c2 prefix holds 2x256 + 200 text
    assert c2.prefix_len + c2.action_horizon == g["pi05_two_camera_sequence"]
    assert c3.prefix_len - c2.prefix_len == g["pi05_observed_sequence"] - g["pi05_two_camera_sequence"] + 50
    assert c2.n_layers == g["pi05_decoder_layers"] and c2.n_steps == g["molmobot_flow_steps"]
    assert c4.prefix_len == g["molmobot_pad_len"]
    m = synth.valid_masks(synth.workload("c4", batch=64))
    n_ctx = m.sum(1) - 1  # minus the encoded state row
    assert n_ctx.min() >= g["molmobot_seq_len_min"] and n_ctx.max() <= g["molmobot_seq_len_max"]
    m2 = synth.valid_masks(synth.workload("c2", batch=64))
    assert m2.sum(1).min() >= 520 and m2.sum(1).max() <= 712
    m5 = synth.valid_masks(synth.workload("c5"))
    assert m5.shape == (16, 1024) and m5.sum(1).min() >= 700
