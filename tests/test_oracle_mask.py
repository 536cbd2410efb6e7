"""Pins of the oracle's explicit mask (CPU only).

Rules (fluxbbs teardown, "Architecture"; hyphentech explainer, history row of
the configuration table and the warning under it; fluxbbs teardown, fourth
trick, for block sparsity):
  earlier segment: head always, tail never, video iff inside the W-frame window;
  own segment: head always, tail j iff its window holds the query frame, video always;
  later segment: never.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from _brute import _tokens, brute_visible


def closed_form_count(w, frame):
    """Visible keys of a query at local frame `frame` (no block sparsity)."""
    S = w.query_segment
    cur = w.segments[S]
    g0 = sum(s.frames for s in w.segments[:S])
    kept = g0 if w.window is None else min(g0, w.window)
    n = sum(s.head_len for s in w.segments[:S]) + kept * cur.tokens_per_frame
    n += cur.head_len + cur.video_len
    n += sum(a for a, f0, f1 in zip(cur.action_len, cur.action_f0, cur.action_f1) if f0 <= frame < f1)
    return n


# hand-derived counts for the target configurations:
#  c1: 2 earlier heads x 16 + 4 window frames x 24 + own head 16 + one 8-token tail + 48 video = 200
#  c1 with W=3: one history frame fewer (-24) = 176
#  c2: 768 head + one 128-token tail + 30 x 390 video = 12,596
#  c3: 3 x 768 heads + 18 x 880 ring + 768 + 128 + 26,400 = 45,440
#  c4: 6 x 1,280 heads + 180 x 880 history + 768 + 128 + 26,400 = 193,376
@pytest.mark.parametrize("name,count", [("c1", 200), ("c1_evict", 176), ("c2", 12596),
                                        ("c3", 45440), ("c4", 193376)])
def test_visible_counts_target_configs(name, count):
    w = W.config(name)
    P = w.current.tokens_per_frame
    tab = oracle.token_table(w)
    for f in range(w.current.frames):
        m = oracle.mask(w, [f * P, f * P + P - 1], None, tab)
        assert m.sum(axis=1).tolist() == [count, count]
        assert closed_form_count(w, f) == count


@pytest.mark.parametrize("name", ["m1", "m2", "c1_future"])
def test_visible_counts_medium(name):
    w = W.config(name)
    m = oracle.mask(w)
    P = w.current.tokens_per_frame
    for r in range(w.current.video_len):
        assert m[r].sum() == closed_form_count(w, r // P)


def test_rule_by_rule_c1():
    tab_names = ("seg", "kind", "tail", "gframe")
    for name in ("c1", "c1_evict", "c1_future"):
        w = W.config(name)
        tab = oracle.token_table(w)
        seg, kind, tail, gframe = (tab[k] for k in tab_names)
        m = oracle.mask(w)
        S = w.query_segment
        g0 = sum(s.frames for s in w.segments[:S])
        assert not m[:, seg > S].any()                                   # future: never
        assert not m[:, (seg < S) & (kind == oracle.TAIL)].any()         # earlier tails: never
        assert m[:, (seg < S) & (kind == oracle.HEAD)].all()             # earlier heads: always
        assert m[:, (seg == S) & (kind == oracle.HEAD)].all()            # own head: always
        assert m[:, (seg == S) & (kind == oracle.VIDEO)].all()           # own video: always
        hv = (seg < S) & (kind == oracle.VIDEO)
        inside = gframe >= g0 - w.window
        assert m[:, hv & inside].all() and not m[:, hv & ~inside].any()  # window
        P = w.current.tokens_per_frame
        for j in range(2):
            cols = (seg == S) & (kind == oracle.TAIL) & (tail == j)
            for r in range(w.current.video_len):
                assert m[r, cols].all() == (r // P == j)                 # tail j <-> frame j
                assert m[r, cols].any() == (r // P == j)
    # eviction: W=3 drops the oldest history frame (global frame 0) and keeps 1..3
    w = W.config("c1_evict")
    tab = oracle.token_table(w)
    m = oracle.mask(w)
    for g in range(4):
        cols = (tab["kind"] == oracle.VIDEO) & (tab["gframe"] == g)
        assert m[:, cols].all() == (g >= 1)


@st.composite
def tiny_workload(draw):
    nseg = draw(st.integers(1, 4))
    P = draw(st.integers(1, 6))
    segs = []
    for _ in range(nseg):
        F = draw(st.integers(1, 4))
        m = draw(st.integers(0, 3))
        tails = [draw(st.integers(0, 3)) for _ in range(m)]
        wins = []
        for _ in range(m):
            a = draw(st.integers(0, F))
            b = draw(st.integers(a, F))
            wins.append((a, b))
        segs.append(W.Segment(F, P, draw(st.integers(0, 4)), tails,
                              [x[0] for x in wins], [x[1] for x in wins]))
    S = draw(st.integers(0, nseg - 1))
    win = draw(st.one_of(st.none(), st.integers(1, 6)))
    return W.Workload("tiny", 1, segs, S, win, draw(st.integers(0, 1000)))


@settings(max_examples=150, deadline=None)
@given(tiny_workload())
def test_mask_matches_brute_rules(w):
    m = oracle.mask(w)
    toks = _tokens(w)
    P = w.current.tokens_per_frame
    for r in range(w.current.video_len):
        ref = [brute_visible(w, t, r // P, r) for t in toks]
        assert m[r].tolist() == ref


def test_block_sparse_counts_c5():
    w = W.config("c5")
    d = W.generate(w)
    csr = d["csr"]
    rp, col = csr["row_ptr"], csr["col"]
    n_own_tiles = -(-w.current.video_len // W.TILE)
    assert csr["n_qtiles"] == 92 and n_own_tiles == 92
    sizes = [min(W.TILE, w.current.video_len - t * W.TILE) for t in range(n_own_tiles)]
    assert sizes[-1] == 11700 - 91 * 128 == 52
    P = w.current.tokens_per_frame
    tab = oracle.token_table(w)
    rows = [0, 127, 128, 5000, 11699]
    m = oracle.mask(w, rows, csr, tab)
    for i, r in enumerate(rows):
        t = r // 128
        kept = col[rp[t]:rp[t + 1]]
        assert len(kept) == 23 and t in kept                   # 25% of 92, diagonal kept
        assert m[i].sum() == 768 + 128 + sum(sizes[c] for c in kept)


@pytest.mark.parametrize("name", ["m3", "m4"])
def test_block_sparse_matches_brute(name):
    w = W.config(name)
    d = W.generate(w)
    csr = d["csr"]
    toks = _tokens(w)
    P = w.current.tokens_per_frame
    rows = list(range(0, w.current.video_len, 7)) + [w.current.video_len - 1]
    m = oracle.mask(w, rows, csr)
    for i, r in enumerate(rows):
        ref = [brute_visible(w, t, r // P, r, csr) for t in toks]
        assert m[i].tolist() == ref
