"""GPU parity on degenerate layouts: one-token frames, empty heads,
zero-length tails, empty and full tail windows, the maximum of 64 action
tails, a one-frame window, a segment longer than the window (only its last
frames reach the ring), a history of heads only, one head.  Every video and
text row is compared with the fp64 oracle, and the DENSE mask bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G


def _seg(F, P, head, tails, wins):
    return W.Segment(F, P, head, list(tails), [a for a, b in wins], [b for a, b in wins])


CASES = {
    # one head, one-token frames, empty first head, zero-length and empty-window tails, W = 1
    "tiny_p1": W.Workload("tiny_p1", 1, [_seg(1, 1, 0, [], []),
                                         _seg(3, 1, 2, [0, 3, 2], [(0, 0), (1, 3), (2, 2)])], 1, 1, 101),
    # 64 one-token tails (the maximum), windows cycling over the frames, no window
    "tails64": W.Workload("tails64", 2, [_seg(5, 7, 0, [1] * 64, [(j % 5, j % 5 + 1) for j in range(64)])],
                          0, None, 102),
    # first segment longer than the window: only its last 2 of 6 frames reach the ring
    "long_first": W.Workload("long_first", 2, [_seg(6, 9, 4, [3], [(0, 6)]),
                                               _seg(2, 9, 3, [2, 2], [(0, 2), (1, 2)])], 1, 2, 103),
    # history of heads only (every earlier frame evicted): W = 1 and a 3-segment history
    "heads_only": W.Workload("heads_only", 3, [_seg(1, 4, 6, [], []), _seg(1, 4, 5, [1], [(0, 1)]),
                                               _seg(1, 4, 0, [], []), _seg(8, 4, 7, [5], [(1, 3)])], 3, 1, 104),
    # large frames, a single frame, Student-t values
    "one_frame": W.Workload("one_frame", 2, [_seg(2, 300, 40, [20], [(0, 1)]), _seg(1, 300, 0, [9], [(0, 1)])],
                            1, 4, 105, kv_dist="student_t4"),
}


def _bar(w, got, ref):
    G.check_bar(got, ref, w.name)


@pytest.mark.parametrize("name", list(CASES))
def test_edge_layout(name):
    print(f"[edge] {name}", flush=True)
    w = CASES[name]
    d = W.generate(w)
    run = G.Run(w, d)
    # mask, video then text rows
    lq, tl = w.current.video_len, w.current.text_len
    cols = G.canonical_columns(w)
    got = run.dense(0, lq + tl)
    ref = np.concatenate([oracle.mask(w)[:, cols], oracle.mask_text(w)[:, cols]]) if tl else \
        oracle.mask(w)[:, cols]
    assert np.array_equal(got, ref)
    # attention, video and text queries in one call
    if tl > 0:
        o, o_txt, lse, lse_txt = run.attn_joint()
        ref_t, ref_lse_t, _ = oracle.attention(w, d, queries="text")
        _bar(w, o_txt.float().cpu().numpy(), ref_t)
        assert np.abs(lse_txt.cpu().numpy() - ref_lse_t).max() <= 1e-2
    else:
        o, lse = run.attn()
    ref_o, ref_lse, _ = oracle.attention(w, d)
    _bar(w, o.float().cpu().numpy(), ref_o)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
    assert run.plan.visible_pairs * 4 * 128 * w.heads == oracle.effective_flops(w)
