"""GPU parity over a long rollout: one cache carried through eight segments.

Segments of 3 latent frames (24 tokens each) through a 5-frame window, so
that the ring wraps and evicts frames at every append, with description
heads of varied length and two action tails per segment; after each append
the next segment's video and text queries attend to the cache as it stands
(segment-causal, action-aware attention over INT8 history: "Hy-Nomas 拆解"
teardown, sections "架构" and "单卡 4090 怎么做到的", first and second
techniques), and every row is compared with the oracle at the bar.  The same
cache object is appended to in place, so the ring position, the head-store
offset and the counters of every step come from the library's own state.
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


def _segments():
    segs = []
    for s in range(8):
        head = 9 + 3 * s                      # heads of 9 .. 30 tokens
        tails = [5 + s % 3, 7]
        windows = [(0, 1 + s % 3), (2, 3)]
        segs.append(W._seg(3, 24, head, tails, windows))
    return segs


def test_rollout_eight_segments():
    segs = _segments()
    head_cap = sum(s.head_len for s in segs)
    cache = None
    for S in range(1, 8):
        w = W.Workload("rollout", 2, segs, S, 5, 77, kv_dist="student_t4")
        d = W.generate(w)
        if cache is None:
            cache = hn.KVCache(w.heads, 24, 5, head_cap)
        x = d["segments"][S - 1]
        hn.hn_kv_quant_append(cache, G.layout(S - 1, segs[S - 1]), G.dev(x["k_txt"]), G.dev(x["v_txt"]),
                              G.dev(x["k_vid"]), G.dev(x["v_vid"]))
        assert cache.segments == S and cache.frames_seen == 3 * S
        assert cache.head_tokens == sum(s.head_len for s in segs[:S])
        seg = G.layout(S, segs[S])
        cur = d["segments"][S]
        plan = hn.build_plan(cache, seg)
        o, o_t, lse, lse_t = hn.seg_attn_joint(cache, seg, plan, G.dev(d["q_vid"]), G.dev(d["q_txt"]),
                                               G.dev(cur["k_txt"]), G.dev(cur["v_txt"]),
                                               G.dev(cur["k_vid"]), G.dev(cur["v_vid"]))
        torch.cuda.synchronize()
        ref, ref_lse, _ = oracle.attention(w, d)
        err = G.check_bar(o.float().cpu().numpy(), ref, f"segment {S} video")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
        ref_t, ref_lse_t, _ = oracle.attention(w, d, queries="text")
        err_t = G.check_bar(o_t.float().cpu().numpy(), ref_t, f"segment {S} text")
        assert np.abs(lse_t.cpu().numpy() - ref_lse_t).max() <= 1e-2
        print(f"  segment {S}: max-abs video {err.max():.3e} text {err_t.max():.3e}", flush=True)
