"""Pins of the oracle's fp64 masked softmax attention (CPU only).

Pinned by: a pure-Python brute force on tiny inputs; bit-identical outputs
when invisible keys are perturbed (their weight is exactly zero); rows that
sum to one; closed forms (Q = 0 gives the mean of the visible values, a
one-hot value on one source gives that source's attention mass); and the
special case with no history and no tails, which is plain unmasked attention
and is checked against torch's scaled_dot_product_attention in fp64.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from _brute import brute_attention


def _gen(w):
    return W.generate(w)


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future"])
def test_brute_force_c1(name):
    w = W.config(name)
    d = _gen(w)
    rows = list(range(0, 48, 5)) + [47]
    O, lse, rs = oracle.attention(w, d, rows)
    Ob, lseb = brute_attention(w, d, rows)
    assert np.max(np.abs(O - np.asarray(Ob))) < 1e-12
    assert np.max(np.abs(lse - np.asarray(lseb))) < 1e-11


@pytest.mark.parametrize("name", ["m1", "m3", "m4"])
def test_brute_force_medium_rows(name):
    w = W.config(name)
    d = _gen(w)
    nq = w.current.video_len
    rows = [0, nq // 3, nq - 1]
    O, lse, rs = oracle.attention(w, d, rows)
    Ob, lseb = brute_attention(w, d, rows)
    assert np.max(np.abs(O - np.asarray(Ob))) < 1e-12
    assert np.max(np.abs(lse - np.asarray(lseb))) < 1e-11


@st.composite
def tiny(draw):
    nseg = draw(st.integers(1, 3))
    P = draw(st.integers(1, 4))
    segs = []
    for _ in range(nseg):
        F = draw(st.integers(1, 3))
        m = draw(st.integers(0, 2))
        tails = [draw(st.integers(1, 3)) for _ in range(m)]
        wins = []
        for _ in range(m):
            a = draw(st.integers(0, F))
            wins.append((a, draw(st.integers(a, F))))
        segs.append(W.Segment(F, P, draw(st.integers(0, 3)), tails,
                              [x[0] for x in wins], [x[1] for x in wins]))
    S = draw(st.integers(0, nseg - 1))
    return W.Workload("tiny", 1, segs, S, draw(st.one_of(st.none(), st.integers(1, 4))),
                      draw(st.integers(0, 10_000)),
                      kv_dist=draw(st.sampled_from(["normal", "student_t4"])))


@settings(max_examples=12, deadline=None)
@given(tiny())
def test_brute_force_random_layouts(w):
    d = _gen(w)
    O, lse, rs = oracle.attention(w, d)
    Ob, lseb = brute_attention(w, d)
    assert np.max(np.abs(O - np.asarray(Ob))) < 1e-12


def _perturb(d, s, key, rows, rng):
    d2 = {"segments": [dict(x) for x in d["segments"]], "q_vid": d["q_vid"]}
    if "csr" in d:
        d2["csr"] = d["csr"]
    for nm in (key, key.replace("k_", "v_")):
        a = d2["segments"][s][nm].copy()
        a[rows] = W.f32_to_bf16_bits(rng.standard_normal(a[rows].shape, dtype=np.float32) * 5)
        d2["segments"][s][nm] = a
    return d2


def test_invisible_keys_get_exactly_zero_weight():
    rng = np.random.default_rng(7)
    # future segment (c1_future: query segment 2 of 3)
    w = W.config("c1_future")
    d = _gen(w)
    O0 = oracle.attention(w, d)[0]
    for s, key, rows in [(2, "k_txt", slice(None)), (2, "k_vid", slice(None)),
                         (0, "k_txt", slice(16, 32))]:          # earlier segment's tails
        O1 = oracle.attention(w, _perturb(d, s, key, rows, rng))[0]
        assert np.array_equal(O0, O1)
    # evicted frame (W=3 drops global frame 0 = segment 0 frame 0)
    w = W.config("c1_evict")
    d = _gen(w)
    O0 = oracle.attention(w, d)[0]
    O1 = oracle.attention(w, _perturb(d, 0, "k_vid", slice(0, 24), rng))[0]
    assert np.array_equal(O0, O1)
    O2 = oracle.attention(w, _perturb(d, 0, "k_vid", slice(24, 48), rng))[0]
    assert not np.array_equal(O0, O2)                           # frame 1 is kept
    # own tail outside its window: tail 1 ([1,2)) is invisible to frame-0 queries
    w = W.config("c1")
    d = _gen(w)
    rows0 = list(range(24))
    O0 = oracle.attention(w, d, rows0)[0]
    O1 = oracle.attention(w, _perturb(d, 2, "k_txt", slice(24, 32), rng), rows0)[0]
    assert np.array_equal(O0, O1)
    O2 = oracle.attention(w, _perturb(d, 2, "k_txt", slice(16, 24), rng), rows0)[0]
    assert not np.array_equal(O0, O2)


def test_unkept_sparse_tiles_get_zero_weight():
    rng = np.random.default_rng(8)
    w = W.config("m4")
    d = _gen(w)
    csr = d["csr"]
    rows = list(range(0, 128))
    kept = set(csr["col"][csr["row_ptr"][0]:csr["row_ptr"][1]].tolist())
    unkept = [t for t in range(csr["n_qtiles"]) if t not in kept]
    O0 = oracle.attention(w, d, rows)[0]
    t = unkept[0]
    O1 = oracle.attention(w, _perturb(d, 0, "k_vid", slice(t * 128, (t + 1) * 128), rng), rows)[0]
    assert np.array_equal(O0, O1)


@pytest.mark.parametrize("name", ["c1", "m1", "m2", "m3"])
def test_rows_sum_to_one(name):
    w = W.config(name)
    d = _gen(w)
    O, lse, rs = oracle.attention(w, d)
    assert np.max(np.abs(rs - 1.0)) < 1e-12


def test_zero_queries_give_mean_of_visible_values():
    w = W.config("m1")
    d = _gen(w)
    d["q_vid"] = np.zeros_like(d["q_vid"])
    O, lse, rs = oracle.attention(w, d)
    m = oracle.mask(w)
    K, V = oracle.key_values(w, d)
    for r in (0, 77, w.current.video_len - 1):
        vis = np.nonzero(m[r])[0]
        assert np.max(np.abs(O[r] - V[vis].mean(axis=0))) < 1e-12
        assert abs(lse[0, r] - math.log(len(vis))) < 1e-12


def test_one_hot_values_measure_source_mass():
    # V = e0 on the own head's tokens and 0 elsewhere: O[:, 0] is the softmax
    # mass on the own head, O[:, 1:] is exactly zero.
    w = W.config("m1")
    d = _gen(w)
    S = w.query_segment
    h = w.current.head_len
    zero = np.zeros_like
    for s, seg in enumerate(d["segments"]):
        seg["v_txt"] = zero(seg["v_txt"])
        seg["v_vid"] = zero(seg["v_vid"])
    d["segments"][S]["v_txt"][:h, :, 0] = 0x3F80  # bf16 1.0
    O, lse, rs = oracle.attention(w, d)
    K, _ = oracle.key_values(w, d)
    Q = W.bf16_bits_to_f32(d["q_vid"]).astype(np.float64)
    m = oracle.mask(w)
    tab = oracle.token_table(w)
    head_cols = (tab["seg"] == S) & (tab["kind"] == oracle.HEAD)
    for r in (3, 140, w.current.video_len - 1):
        for hh in range(w.heads):
            s = K[:, hh, :] @ Q[r, hh] / math.sqrt(128)
            s[~m[r]] = -np.inf
            p = np.exp(s - s.max())
            p /= p.sum()
            assert abs(O[r, hh, 0] - p[head_cols].sum()) < 1e-12
    assert np.all(O[:, :, 1:] == 0)


def test_no_history_no_tails_equals_library_sdpa():
    seg = W.Segment(3, 40, 25, [], [], [])
    w = W.Workload("plain", 2, [seg], 0, 4, 21)
    d = _gen(w)
    O, lse, rs = oracle.attention(w, d)
    q = torch.from_numpy(W.bf16_bits_to_f32(d["q_vid"]).astype(np.float64)).permute(1, 0, 2)
    k = np.concatenate([d["segments"][0]["k_txt"], d["segments"][0]["k_vid"]])
    v = np.concatenate([d["segments"][0]["v_txt"], d["segments"][0]["v_vid"]])
    k = torch.from_numpy(W.bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)
    v = torch.from_numpy(W.bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


def test_sdpa_per_frame_group_on_gathered_keys():
    # any layout: queries of one latent frame share a mask; SDPA on the gathered
    # visible keys of that frame must give the oracle's rows
    w = W.config("m2")
    d = _gen(w)
    O, lse, rs = oracle.attention(w, d)
    K, V = oracle.key_values(w, d)
    Q = W.bf16_bits_to_f32(d["q_vid"]).astype(np.float64)
    P = w.current.tokens_per_frame
    for f in range(w.current.frames):
        vis = np.nonzero(oracle.mask(w, [f * P])[0])[0]
        rows = slice(f * P, (f + 1) * P)
        q = torch.from_numpy(Q[rows]).permute(1, 0, 2)
        k = torch.from_numpy(K[vis]).permute(1, 0, 2)
        v = torch.from_numpy(V[vis]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).numpy()
        assert np.max(np.abs(O[rows] - ref)) < 1e-12
