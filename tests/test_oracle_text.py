"""Pins of the oracle's text-stream queries (CPU only).

Text queries are the query segment's own head and tail tokens.  Rules
(fluxbbs teardown, "Architecture": segment-causal attention is bidirectional
inside a segment and sees earlier segments only; heads stay visible across
segments, tails only inside their own segment; the sliding window of earlier
video, hyphentech explainer, history row of the configuration table), with
the reading for tails: a tail token sees its own tail only, a head token no
tail.  Pinned by closed-form counts, a rule-by-rule check, the pure-Python
brute force, exact-zero weights under perturbation, and rows summing to one.
"""
import numpy as np
import pytest
from hypothesis import given, settings

import oracle
import workloads as W
from _brute import _tokens, brute_attention, brute_visible_text, text_query_tail
from test_oracle_attn import tiny
from test_oracle_mask import tiny_workload


# hand-derived counts (head query, tail query):
#  c1: 2 x 16 earlier heads + 4 x 24 window video + 16 own head + 48 own video = 192; +8 tail = 200
#  c1_evict (W=3): 24 fewer = 168 / 176
#  c2: 768 + 11,700 = 12,468; +128 = 12,596
#  c3: 3 x 768 + 18 x 880 + 768 + 26,400 = 45,312; +128 = 45,440
#  c4: 6 x 1,280 + 180 x 880 + 768 + 26,400 = 193,248; +128 = 193,376
@pytest.mark.parametrize("name,head_q,tail_q", [("c1", 192, 200), ("c1_evict", 168, 176),
                                                ("c2", 12468, 12596), ("c3", 45312, 45440),
                                                ("c4", 193248, 193376)])
def test_text_visible_counts(name, head_q, tail_q):
    w = W.config(name)
    cur = w.current
    tab = oracle.token_table(w)
    first_tail = cur.head_len
    rows = [0, cur.head_len - 1, first_tail, cur.text_len - 1]
    m = oracle.mask_text(w, rows, tab)
    assert m.sum(axis=1).tolist() == [head_q, head_q, tail_q, tail_q]


def test_text_rule_by_rule_c1():
    for name in ("c1", "c1_evict", "c1_future"):
        w = W.config(name)
        tab = oracle.token_table(w)
        seg, kind, tail, gframe = (tab[k] for k in ("seg", "kind", "tail", "gframe"))
        m = oracle.mask_text(w)
        S = w.query_segment
        cur = w.current
        g0 = sum(s.frames for s in w.segments[:S])
        assert not m[:, seg > S].any()                                   # future: never
        assert not m[:, (seg < S) & (kind == oracle.TAIL)].any()         # earlier tails: never
        assert m[:, (seg < S) & (kind == oracle.HEAD)].all()             # earlier heads: always
        assert m[:, (seg == S) & (kind == oracle.HEAD)].all()            # own head: always
        assert m[:, (seg == S) & (kind == oracle.VIDEO)].all()           # own video: always
        hv = (seg < S) & (kind == oracle.VIDEO)
        inside = gframe >= g0 - w.window
        assert m[:, hv & inside].all() and not m[:, hv & ~inside].any()  # window
        for r in range(cur.text_len):
            qj = text_query_tail(cur, r)
            for j in range(len(cur.action_len)):
                cols = (seg == S) & (kind == oracle.TAIL) & (tail == j)
                assert m[r, cols].all() == (qj == j) and m[r, cols].any() == (qj == j)


@settings(max_examples=150, deadline=None)
@given(tiny_workload())
def test_text_mask_matches_brute_rules(w):
    m = oracle.mask_text(w)
    toks = _tokens(w)
    for r in range(w.current.text_len):
        qj = text_query_tail(w.current, r)
        assert m[r].tolist() == [brute_visible_text(w, t, qj) for t in toks]


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future", "m1"])
def test_text_brute_force(name):
    w = W.config(name)
    d = W.generate(w)
    n = w.current.text_len
    rows = sorted(set([0, 1, n // 2, n - 1]))
    O, lse, rs = oracle.attention(w, d, rows, queries="text")
    Ob, lseb = brute_attention(w, d, rows, queries="text")
    assert np.max(np.abs(O - np.asarray(Ob))) < 1e-12
    assert np.max(np.abs(lse - np.asarray(lseb))) < 1e-11


@settings(max_examples=12, deadline=None)
@given(tiny())
def test_text_brute_force_random_layouts(w):
    if w.current.text_len == 0:
        return
    d = W.generate(w)
    O, lse, rs = oracle.attention(w, d, queries="text")
    Ob, lseb = brute_attention(w, d, queries="text")
    assert np.max(np.abs(O - np.asarray(Ob))) < 1e-12


def _perturb(d, s, key, rows, rng):
    d2 = {"segments": [dict(x) for x in d["segments"]], "q_vid": d["q_vid"], "q_txt": d["q_txt"]}
    for nm in (key, key.replace("k_", "v_")):
        a = d2["segments"][s][nm].copy()
        a[rows] = W.f32_to_bf16_bits(rng.standard_normal(a[rows].shape, dtype=np.float32) * 5)
        d2["segments"][s][nm] = a
    return d2


def test_text_invisible_keys_get_exactly_zero_weight():
    rng = np.random.default_rng(11)
    # c1: own text rows 0..15 head, 16..23 tail 0, 24..31 tail 1
    w = W.config("c1")
    d = W.generate(w)
    att = lambda dd, rows: oracle.attention(w, dd, rows, queries="text")[0]
    head_rows, t0_rows, t1_rows = list(range(16)), list(range(16, 24)), list(range(24, 32))
    O_head, O_t0, O_t1 = att(d, head_rows), att(d, t0_rows), att(d, t1_rows)
    # any own tail is invisible to head queries
    d_t0 = _perturb(d, 2, "k_txt", slice(16, 24), rng)
    d_t1 = _perturb(d, 2, "k_txt", slice(24, 32), rng)
    assert np.array_equal(att(d_t0, head_rows), O_head)
    assert np.array_equal(att(d_t1, head_rows), O_head)
    # another tail is invisible to a tail query; its own tail is not
    assert np.array_equal(att(d_t1, t0_rows), O_t0)
    assert not np.array_equal(att(d_t0, t0_rows), O_t0)
    assert np.array_equal(att(d_t0, t1_rows), O_t1)
    # earlier segments' tails: never
    assert np.array_equal(att(_perturb(d, 0, "k_txt", slice(16, 32), rng), head_rows), O_head)
    # future segment and evicted frames: never
    w = W.config("c1_future")
    d = W.generate(w)
    O0 = oracle.attention(w, d, queries="text")[0]
    O1 = oracle.attention(w, _perturb(d, 2, "k_vid", slice(None), rng), queries="text")[0]
    assert np.array_equal(O0, O1)
    w = W.config("c1_evict")
    d = W.generate(w)
    O0 = oracle.attention(w, d, queries="text")[0]
    assert np.array_equal(O0, oracle.attention(w, _perturb(d, 0, "k_vid", slice(0, 24), rng),
                                               queries="text")[0])
    assert not np.array_equal(O0, oracle.attention(w, _perturb(d, 0, "k_vid", slice(24, 48), rng),
                                                   queries="text")[0])


@pytest.mark.parametrize("name", ["c1", "m1", "m2"])
def test_text_rows_sum_to_one(name):
    w = W.config(name)
    d = W.generate(w)
    O, lse, rs = oracle.attention(w, d, queries="text")
    assert np.max(np.abs(rs - 1.0)) < 1e-12


def test_text_zero_queries_give_mean_of_visible_values():
    w = W.config("c1")
    d = W.generate(w)
    d = dict(d)
    d["q_txt"] = np.zeros_like(d["q_txt"])
    K, V = oracle.key_values(w, d)
    vis = oracle.mask_text(w)
    O = oracle.attention(w, d, queries="text", kv=(K, V))[0]
    for r in (0, 20, 31):
        ref = V[vis[r]].mean(axis=0)
        assert np.max(np.abs(O[r] - ref)) < 1e-12
