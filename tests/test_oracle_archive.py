"""Pins of the oracle's history archive (CPU only).

Which frames leave the GPU window when a segment is appended (hyphentech
explainer, configuration table, history row: earlier history is archived to
CPU; fluxbbs teardown, second trick: an 18-frame window) is pinned against a
frame-by-frame simulation of the window, closed forms for the target
configuration, and conservation: every frame ever stored in the ring is
either still in the window or archived, exactly once, in order.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _simulate(seg_frames, window):
    """Frame-by-frame: the ring stores the last min(F, W) frames of each
    segment and holds the newest W frames it has stored."""
    ring, evicted, g = [], [], 0
    for F in seg_frames:
        stored = list(range(g + F - min(F, window), g + F))
        out = []
        for fr in stored:
            ring.append(fr)
            if len(ring) > window:
                out.append(ring.pop(0))
        evicted.append(out)
        g += F
    return evicted


@pytest.mark.parametrize("seg_frames,window", [([3] * 6, 4), ([30, 30, 30, 30], 18), ([5, 1, 7, 2, 9], 3),
                                               ([2, 2, 2], 10), ([1] * 9, 1), ([4, 12, 3], 5)])
def test_evicted_frames_match_simulation(seg_frames, window):
    sim = _simulate(seg_frames, window)
    fs = 0
    for F, exp in zip(seg_frames, sim):
        g0, g1 = oracle.evicted_frames(fs, F, window)
        got = [g for g in range(g0, g1)]
        # frames stored and evicted by this very append never reach the archive
        # through the ring's front: they are the ones a long segment drops at once
        exp_front = [g for g in exp if g < fs]
        assert got == exp_front
        fs += F


def test_evicted_frames_closed_forms():
    # 1280x704 steady state: W = 18, segments of 30 latent frames
    assert oracle.evicted_frames(0, 30, 18) == (0, 0)        # frames 12..29 stored, 0..11 never
    assert oracle.evicted_frames(30, 30, 18) == (12, 30)     # the whole ring turns over
    assert oracle.evicted_frames(60, 30, 18) == (42, 60)
    # window not yet full: nothing leaves until it is
    assert oracle.evicted_frames(3, 2, 10) == (0, 0)
    assert oracle.evicted_frames(9, 3, 10) == (0, 2)


def test_archive_conservation():
    w = W.config("arch")
    d = W.generate(w)
    k, v, ks, vs = oracle.archive_of(w, d, 6)
    # 18 frames stored, the newest 4 in the window, the other 14 archived in order
    assert k.shape == (14, 16, 2, 128) and ks.shape == (14, 16, 2)
    P = 16
    for g in range(14):
        s, f = divmod(g, 3)
        qk, sk = oracle.quantize(d["segments"][s]["k_vid"][f * P:(f + 1) * P])
        assert np.array_equal(k[g], qk) and np.array_equal(ks[g], sk)
    # before the window fills nothing is archived
    assert oracle.archive_of(w, d, 1)[0].shape[0] == 0
