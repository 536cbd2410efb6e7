"""GPU parity of the 384-row query tiles (12 waves of 32 rows, three per SIMD,
Q in LDS, the first 8 waves staging the key tiles) where the automatic
choice does not take them: small layouts with masks, ragged tiles, INT8
history, action tails and text queries, with and without forced key splits,
and the 2-head share of the 1280x704 steady state (138 blocks on 256 CUs).
Where the automatic choice does take them (the 480x832 segment, the 1280x704
steady state and its 7th segment) the other attention tests cover them.
Bar: the same as for every tile height, against the fp64 oracle; the video
outputs of a joint call are bitwise those of the video-only call, and a
repeated call gives the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_attention_hn_amd as hn
    import _gpu as G

ROWS = 384


@pytest.mark.parametrize("name,splits,text_splits", [("c1", 0, 0), ("c1_evict", 0, 0), ("c1_future", 0, 0),
                                                     ("m1", 0, 0), ("m2", 0, 0), ("c1", 3, 2),
                                                     ("m1", 5, 1), ("m2", 2, 3), ("m1", 1, 4)])
def test_rows384_small(name, splits, text_splits):
    print(f"[rows384] {name} x{splits} text x{text_splits}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    run = G.Run(w, d, opts=hn.PlanOpts(n_splits=splits, n_splits_text=text_splits, tile_rows=ROWS))
    assert run.plan.c.tile_q == ROWS
    if w.current.text_len > 0:
        o, o_t, lse, lse_t = run.attn_joint()
        ref_t, ref_lse_t, _ = oracle.attention(w, d, queries="text")
        G.check_bar(o_t.float().cpu().numpy(), ref_t, f"{name} text")
        assert np.abs(lse_t.cpu().numpy() - ref_lse_t).max() <= 1e-2
    else:
        o, lse = run.attn()
    ref, ref_lse, _ = oracle.attention(w, d)
    err = G.check_bar(o.float().cpu().numpy(), ref, f"{name} video")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
    print(f"  max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    o2, lse2 = run.attn()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


def test_rows384_head_share():
    # the 2-head share: 69 384-row tiles per head, text queries in the same launch
    print("[rows384] c3_h2", flush=True)
    w = W.config("c3_h2")
    d = W.generate(w)
    run = G.Run(w, d, opts=hn.PlanOpts(tile_rows=ROWS))
    assert run.plan.c.tile_q == ROWS
    o, o_t, lse, lse_t = run.attn_joint()
    rows = G.sample_rows(w.current.video_len)
    ref, ref_lse, _ = oracle.attention(w, d, rows)
    err = G.check_bar(o.float().cpu().numpy()[rows], ref, "c3_h2 video")
    assert np.abs(lse.cpu().numpy()[:, rows] - ref_lse).max() <= 1e-2
    rows_t = G.sample_rows(w.current.text_len, tile=32)
    ref_t, ref_lse_t, _ = oracle.attention(w, d, rows_t, queries="text")
    G.check_bar(o_t.float().cpu().numpy()[rows_t], ref_t, "c3_h2 text")
    assert np.abs(lse_t.cpu().numpy()[:, rows_t] - ref_lse_t).max() <= 1e-2
    print(f"  max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
