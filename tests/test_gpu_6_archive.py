"""GPU tests of the host archive of evicted history and of rewinding.

Six segments of 3 latent frames with a 4-frame window ("arch" layout): the
archive must hold exactly the oracle's INT8 codes and scales of the 14
frames that left the window, in order; rewinding to the state after 3
segments must give a ring window and head store identical to a cache that
only ever appended 3 segments, attention on it identical (bit for bit) to
that cache's and within the bar of the oracle, and appending from there must
continue as if the detour had not happened.
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


def _append(cache, w, d, s, archive=None):
    seg = G.layout(s, w.segments[s])
    x = d["segments"][s]
    if archive is not None:
        hn.hn_kv_archive_evict(cache, seg, archive)
    hn.hn_kv_quant_append(cache, seg, G.dev(x["k_txt"]), G.dev(x["v_txt"]), G.dev(x["k_vid"]),
                          G.dev(x["v_vid"]))


def _archived(ar, n, P):
    """Archive contents of n frames as [frames][P][H][...] (oracle layout)."""
    H = ar.k.shape[0]
    k = ar.k[:, :n * P].numpy().reshape(H, n, P, -1).transpose(1, 2, 0, 3)
    v = ar.v[:, :n * P].numpy().reshape(H, n, P, -1).transpose(1, 2, 0, 3)
    ks = ar.ks[:, :n * P].numpy().reshape(H, n, P).transpose(1, 2, 0)
    vs = ar.vs[:, :n * P].numpy().reshape(H, n, P).transpose(1, 2, 0)
    return k, v, ks, vs


def _window_equal(a, b, fs, W_, P):
    for g in range(fs - min(fs, W_), fs):
        sl = slice((g % W_) * P, (g % W_ + 1) * P)
        for t in ("ring_k", "ring_v", "ring_ks", "ring_vs"):
            if not torch.equal(getattr(a, t)[:, sl], getattr(b, t)[:, sl]):
                return False
    return True


def _attention(cache, w, d):
    S = w.query_segment
    seg = G.layout(S, w.current)
    x = d["segments"][S]
    plan = hn.build_plan(cache, seg)
    o, lse = hn.seg_attn(cache, seg, plan, G.dev(d["q_vid"]), G.dev(x["k_txt"]), G.dev(x["v_txt"]),
                         G.dev(x["k_vid"]), G.dev(x["v_vid"]), with_lse=True)
    torch.cuda.synchronize()
    return o, lse


def test_archive_and_rewind():
    print("[archive] arch", flush=True)
    w = W.config("arch")
    d = W.generate(w)
    P, W_ = 16, w.ring_frames
    cache = G.new_cache(w)
    ar = hn.KVArchive(w.heads, P, 32)
    states = []
    for s in range(6):
        states.append((cache.frames_seen, cache.head_tokens, cache.segments))
        _append(cache, w, d, s, ar)
    torch.cuda.synchronize()
    assert ar.frames == 14 and ar.first_frame == 0
    ref = oracle.archive_of(w, d, 6)
    for got, exp in zip(_archived(ar, 14, P), ref):
        assert np.array_equal(got, exp)

    # rewind to the state after 3 segments (query segment 3 comes next)
    fs3, ht3, sg3 = states[3]
    hn.hn_kv_cache_rewind(cache, ar, fs3, ht3, sg3)
    torch.cuda.synchronize()
    assert (cache.frames_seen, cache.head_tokens, cache.segments) == (fs3, ht3, sg3)
    assert ar.frames == fs3 - min(fs3, W_)
    fresh = G.new_cache(w)
    for s in range(3):
        _append(fresh, w, d, s)
    torch.cuda.synchronize()
    assert _window_equal(cache, fresh, fs3, W_, P)
    assert torch.equal(cache.heads_k[:, :ht3], fresh.heads_k[:, :ht3])
    assert torch.equal(cache.heads_ks[:, :ht3], fresh.heads_ks[:, :ht3])

    o, lse = _attention(cache, w, d)
    o_f, lse_f = _attention(fresh, w, d)
    assert torch.equal(o, o_f) and torch.equal(lse, lse_f)
    ref_o, ref_lse, _ = oracle.attention(w, d)
    err = np.abs(o.float().cpu().numpy() - ref_o)
    print(f"  after rewind: max-abs {err.max():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3

    # continue as if nothing happened: append 3..5 again with eviction
    for s in range(3, 6):
        _append(cache, w, d, s, ar)
    torch.cuda.synchronize()
    assert ar.frames == 14
    for got, exp in zip(_archived(ar, 14, P), ref):
        assert np.array_equal(got, exp)


def test_rewind_to_start_and_refill():
    w = W.config("arch")
    d = W.generate(w)
    P = 16
    cache = G.new_cache(w)
    ar = hn.KVArchive(w.heads, P, 32)
    for s in range(6):
        _append(cache, w, d, s, ar)
    hn.hn_kv_cache_rewind(cache, ar, 0, 0, 0)
    assert ar.frames == 0 and cache.frames_seen == 0
    for s in range(6):
        _append(cache, w, d, s, ar)
    torch.cuda.synchronize()
    for got, exp in zip(_archived(ar, 14, P), oracle.archive_of(w, d, 6)):
        assert np.array_equal(got, exp)
