"""Pins of the oracle's camera cross-attention (CPU only).

Video tokens read the time-aligned camera tokens of their segment (fluxbbs
teardown, "Architecture", camera paragraph).  Pinned by the closed form of
radius 0 (one visible key: weight exactly 1, O = that frame's camera value,
lse = its score), the library routine when every camera token is visible
(torch scaled_dot_product_attention in fp64), and a pure-Python loop for
intermediate radii.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _exact_quant import bf16_to_fraction


def _f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("name", ["c1", "m1", "m4"])
def test_radius0_is_own_frame_value(name):
    w = W.config(name)
    d = W.generate(w)
    O, lse = oracle.camera_attention(w, d, 0)
    P = w.current.tokens_per_frame
    V, K, Q = _f64(d["v_cam"]), _f64(d["k_cam"]), _f64(d["q_vid"])
    f = np.arange(w.current.video_len) // P
    assert np.array_equal(O, V[f])
    score = np.einsum("rhd,rhd->hr", Q, K[f]) / math.sqrt(128)
    assert np.max(np.abs(lse - score)) < 1e-12


@pytest.mark.parametrize("name", ["c1", "m1"])
def test_full_radius_is_library_sdpa(name):
    w = W.config(name)
    d = W.generate(w)
    O, _ = oracle.camera_attention(w, d, radius=10 ** 6)
    Q = torch.from_numpy(_f64(d["q_vid"])).permute(1, 0, 2)
    K = torch.from_numpy(_f64(d["k_cam"])).permute(1, 0, 2)
    V = torch.from_numpy(_f64(d["v_cam"])).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).permute(1, 0, 2).numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


def _brute(w, d, radius, rows):
    cur = w.current
    P, F = cur.tokens_per_frame, cur.frames
    out = []
    for r in rows:
        f = r // P
        per_head = []
        for h in range(w.heads):
            q = [float(bf16_to_fraction(int(b))) for b in d["q_vid"][r, h]]
            keys = [g for g in range(F) if abs(g - f) <= radius]
            sc = []
            for g in keys:
                k = [float(bf16_to_fraction(int(b))) for b in d["k_cam"][g, h]]
                sc.append(sum(a * b for a, b in zip(q, k)) / math.sqrt(128))
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            o = [0.0] * 128
            for wgt, g in zip(e, keys):
                v = [float(bf16_to_fraction(int(b))) for b in d["v_cam"][g, h]]
                for i in range(128):
                    o[i] += wgt * v[i]
            per_head.append([x / sum(e) for x in o])
        out.append(per_head)
    return np.asarray(out)


@pytest.mark.parametrize("radius", [1, 2])
def test_brute_force_radius(radius):
    w = W.config("m1")
    d = W.generate(w)
    O, _ = oracle.camera_attention(w, d, radius)
    rows = [0, 7, w.current.video_len // 2, w.current.video_len - 1]
    assert np.max(np.abs(O[rows] - _brute(w, d, radius, rows))) < 1e-12
