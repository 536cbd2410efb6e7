"""Pins of the oracle's effective-FLOP counts (the numerator of every
throughput figure): 4 x 128 multiply-adds per visible (query, key) pair per
head, the pairs counted from the layout by closed forms written from the
segment-causal, action-aware rule ("Hy-Nomas 拆解" teardown, section "架构";
window: same page, "单卡 4090 怎么做到的", second technique), not from the
oracle's masks.

480x832 segment (c2): every video row sees the 768-token head, the one
action tail whose window holds its latent frame (four windows tile the 30
frames) and all 11,700 video tokens: 12,596 keys; a head row sees 768 +
11,700 keys, a tail row also its own 128-token tail.  1280x704 steady state
(c3): plus 3 x 768 earlier heads and the 18-frame window of 880-token frames.
7th 1280x704 segment (c4): plus 6 x 1,280 earlier heads and all 180 earlier
frames.
"""
import numpy as np
import pytest

import oracle
import workloads as W

D = 128


def _video_pairs_closed(w):
    """Visible (video query, key) pairs per head from the layout alone."""
    S, cur = w.query_segment, w.current
    P = cur.tokens_per_frame
    hist_frames = sum(s.frames for s in w.segments[:S])
    kept = hist_frames if w.window is None else min(hist_frames, w.window)
    base = sum(s.head_len for s in w.segments[:S]) + kept * P + cur.head_len + cur.video_len
    total = 0
    for f in range(cur.frames):
        tails = sum(a for a, f0, f1 in zip(cur.action_len, cur.action_f0, cur.action_f1) if f0 <= f < f1)
        total += (base + tails) * P
    return total


def _text_pairs_closed(w):
    S, cur = w.query_segment, w.current
    P = cur.tokens_per_frame
    hist_frames = sum(s.frames for s in w.segments[:S])
    kept = hist_frames if w.window is None else min(hist_frames, w.window)
    base = sum(s.head_len for s in w.segments[:S]) + kept * P + cur.head_len + cur.video_len
    return cur.text_len * base + sum(a * a for a in cur.action_len)


@pytest.mark.parametrize("name,per_row", [("c2", 12596), ("c3", 45440), ("c4", 193376)])
def test_target_config_counts(name, per_row):
    w = W.config(name)
    rows = w.current.video_len
    assert _video_pairs_closed(w) == per_row * rows
    assert oracle.effective_flops(w) == 4.0 * D * per_row * rows * w.heads


def test_c2_numbers():
    w = W.config("c2")
    # 147,373,200 pairs per head; the text queries: 768 head rows x 12,468 +
    # 4 x 128 tail rows x 12,596
    assert oracle.effective_flops(w) == 4.0 * D * 147_373_200 * 16
    assert oracle.effective_flops_text(w) == 4.0 * D * (768 * 12_468 + 512 * 12_596) * 16


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future", "m1", "m2", "m4", "arch", "c3", "c4"])
def test_closed_forms_match(name):
    w = W.config(name)
    assert oracle.effective_flops(w) == 4.0 * D * _video_pairs_closed(w) * w.heads
    assert oracle.effective_flops_text(w) == 4.0 * D * _text_pairs_closed(w) * w.heads


def test_planted_mistakes_are_caught():
    """A count that forgot the tails, the window or the earlier heads differs."""
    w = W.config("c3")
    good = _video_pairs_closed(w)
    no_window = W.Workload(w.name, w.heads, w.segments, w.query_segment, None, w.seed)
    assert _video_pairs_closed(no_window) != good
    assert oracle.effective_flops(no_window) != oracle.effective_flops(w)
    cur = w.current
    untailed = W.Workload(w.name, w.heads, w.segments[:-1] + [W._seg(cur.frames, cur.tokens_per_frame,
                                                                      cur.head_len, [], [])],
                          w.query_segment, w.window, w.seed)
    assert oracle.effective_flops(untailed) != oracle.effective_flops(w)
