"""GPU parity of the text-stream queries (the segment's own head and tail
tokens as queries, in the same hn_seg_attn_fwd call as the video queries).

Mask: the DENSE rows past the video rows must equal the oracle's mask_text
bit for bit.  Attention: the same bar as the video queries (max-abs <= 2e-2
and mean-abs <= 2e-3 on unit-variance inputs; elements with |O_ref| >= 8 may
also carry half a bf16 unit in the last place: tests/_gpu.py).  Adding the text queries must leave the
video outputs bit-identical, and tails a text query cannot see must not
change its output at all.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G

_DATA = {}


def data_of(name):
    if name not in _DATA:
        _DATA[name] = W.generate(W.config(name))
    return _DATA[name]


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future", "m1", "m2", "m3", "m4", "c2", "c3"])
def test_text_dense_mask(name):
    print(f"[text mask] {name}", flush=True)
    w = W.config(name)
    d = data_of(name)
    run = G.Run(w, d)
    lq, tl = w.current.video_len, w.current.text_len
    rows = np.arange(tl) if tl <= 256 else np.unique(np.r_[0:64, tl - 64:tl, w.current.head_len - 1:
                                                          w.current.head_len + 2])
    got = np.concatenate([run.dense(lq + int(r), 1) for r in rows]) if tl > 256 else run.dense(lq, tl)
    ref = oracle.mask_text(w, rows)[:, G.canonical_columns(w)]
    assert np.array_equal(got, ref)
    assert run.plan.visible_pairs_text == int(oracle.mask_text(w).sum())


def _check(w, d, o_txt, lse_txt, rows):
    ref, ref_lse, _ = oracle.attention(w, d, rows, queries="text")
    o = o_txt.float().cpu().numpy()[rows]
    lse = lse_txt.cpu().numpy()[:, rows]
    err = np.abs(o - ref)
    print(f"  text max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
          f"lse max-abs {np.abs(lse - ref_lse).max():.3e}", flush=True)
    G.check_bar(o, ref, f"{w.name} text")
    assert np.abs(lse - ref_lse).max() <= 1e-2
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future", "m1", "m2", "m3", "m4", "c2", "c3",
                                  "c4"])
def test_text_attention(name):
    print(f"[text attn] {name}", flush=True)
    w = W.config(name)
    d = data_of(name)
    run = G.Run(w, d)
    o, o_txt, lse, lse_txt = run.attn_joint()
    tl = w.current.text_len
    if name == "c4":
        rows = G.sample_rows(tl, tile=32)
    else:
        rows = np.arange(tl)
    _check(w, d, o_txt, lse_txt, rows)
    # the video outputs of the joint call are those of the video-only call
    o_only, lse_only = run.attn()
    assert torch.equal(o, o_only) and torch.equal(lse, lse_only)
    if name == "c4":
        _DATA.pop(name)


def test_text_invisible_tails_leave_outputs_unchanged():
    w = W.config("c1")
    d = data_of("c1")
    run = G.Run(w, d)
    _, o_txt, _, _ = run.attn_joint()
    base = o_txt.clone()
    # c1 own text: rows 0..15 head, 16..23 tail 0, 24..31 tail 1
    for rows_pert, unchanged in ((slice(24, 32), slice(0, 24)), (slice(16, 24), np.r_[0:16, 24:32])):
        k = run.k_txt.clone()
        v = run.v_txt.clone()
        k[rows_pert] = torch.randn_like(k[rows_pert]) * 5
        v[rows_pert] = torch.randn_like(v[rows_pert]) * 5
        run.k_txt, run.v_txt = k, v
        _, o2, _, _ = run.attn_joint()
        idx = torch.as_tensor(np.arange(32)[unchanged]).cuda()
        assert torch.equal(o2.index_select(0, idx), base.index_select(0, idx))
        changed = torch.as_tensor(np.arange(32)[rows_pert]).cuda()
        assert not torch.equal(o2.index_select(0, changed), base.index_select(0, changed))
        run.k_txt, run.v_txt = G.dev(d["segments"][2]["k_txt"]), G.dev(d["segments"][2]["v_txt"])
