"""Checkpoint and resume of the cache: it is caller-owned device buffers plus
a plain counter struct, so copying both out and into a fresh cache of the
same shape must resume exactly -- attention and later appends bit-identical
to the cache that was never saved."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_attention_hn_amd as hn
    import _gpu as G


def _append(cache, w, d, s):
    seg = G.layout(s, w.segments[s])
    x = d["segments"][s]
    hn.hn_kv_quant_append(cache, seg, G.dev(x["k_txt"]), G.dev(x["v_txt"]), G.dev(x["k_vid"]),
                          G.dev(x["v_vid"]))


def _attn(cache, w, d):
    S = w.query_segment
    seg = G.layout(S, w.current)
    x = d["segments"][S]
    plan = hn.build_plan(cache, seg)
    o, lse = hn.seg_attn(cache, seg, plan, G.dev(d["q_vid"]), G.dev(x["k_txt"]), G.dev(x["v_txt"]),
                         G.dev(x["k_vid"]), G.dev(x["v_vid"]), with_lse=True)
    torch.cuda.synchronize()
    return o, lse


def test_checkpoint_resume():
    w = W.config("arch")
    d = W.generate(w)
    a = G.new_cache(w)
    for s in range(2):
        _append(a, w, d, s)
    torch.cuda.synchronize()
    state = a.state_dict()
    b = G.new_cache(w)
    b.load_state_dict(state)
    for s in range(2, 3):
        _append(a, w, d, s)
        _append(b, w, d, s)
    oa, la = _attn(a, w, d)
    ob, lb = _attn(b, w, d)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    for n in ("ring_k", "ring_ks", "heads_k", "heads_vs"):
        assert torch.equal(getattr(a, n), getattr(b, n))
    bad = hn.KVCache(w.heads, 16, w.ring_frames + 1, w.head_cap)
    with pytest.raises(ValueError):
        bad.load_state_dict(state)
