"""GPU parity on 160 seeded random layouts.

Each case draws a segment sequence (1-4 segments of 1-5 latent frames, 1-97
tokens per frame, heads of 0-40 tokens, 0-3 action tails with random
windows, some empty), a history window (or none), 1-4 attention heads,
normal or heavy-tailed keys and values, sometimes a keep list, and the plan
options (tile height, forced key splits for video and text tiles, leading
video tiles left whole).  The
cache is filled through hn_kv_quant_append and the query segment's video
and text queries attend in one call; every row of both outputs and of the
LSE is compared with the oracle at the bar; the DENSE expansion of the plan
and the cache's INT8 codes and scales bit for bit.  The draws come from a fixed
seed, so the cases are the same on every run; each prints its layout first.
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


def _layout(seed):
    rng = np.random.default_rng(1000 + seed)
    n_seg = int(rng.integers(1, 5))
    P = int(rng.choice([1, 7, 24, 50, 97]))
    segs = []
    for _ in range(n_seg):
        F = int(rng.integers(1, 6))
        head = int(rng.integers(0, 41))
        m = int(rng.integers(0, 4))
        tails = [int(rng.integers(0, 30)) for _ in range(m)]
        wins = []
        for _ in range(m):
            a = int(rng.integers(0, F + 1))
            b = int(rng.integers(a, F + 1))
            wins.append((a, b))
        segs.append(W._seg(F, P, head, tails, wins))
    # mostly the last segment, so that most cases carry INT8 history
    S = n_seg - 1 if rng.random() < 0.7 else int(rng.integers(0, n_seg))
    hist = sum(s.frames for s in segs[:S])
    window = None if rng.random() < 0.3 else int(rng.integers(1, max(2, hist + 2)))
    heads = int(rng.integers(1, 5))
    dist = "student_t4" if rng.random() < 0.4 else "normal"
    keep = float(rng.choice([0.25, 0.5])) if rng.random() < 0.3 else None
    w = W.Workload(f"rand{seed}", heads, segs, S, window, 500 + seed, kv_dist=dist, sparse_keep=keep,
                   sparse_seed=(900 + seed) if keep else None)
    # a keep list fixes 128-row query tiles
    rows = int(rng.choice([0, 128] if keep else [0, 128, 256, 384]))
    n_splits = int(rng.choice([0, 1, 2, 3]))
    n_splits_text = int(rng.choice([0, 1, 2]))
    # with a forced split, sometimes the leading video tiles whole (>= the
    # tile count: no split)
    whole = int(rng.integers(0, 3)) if n_splits > 1 else 0
    opts = hn.PlanOpts(n_splits=n_splits, n_splits_text=n_splits_text, tile_rows=rows, whole_tiles=whole)
    return w, opts


@pytest.mark.parametrize("seed", range(160))
def test_random_layout(seed):
    w, opts = _layout(seed)
    cur = w.current
    print(f"[random] seed {seed}: H={w.heads} S={w.query_segment} W={w.window} "
          f"segments={[(s.frames, s.tokens_per_frame, s.head_len, s.action_len, s.action_f0, s.action_f1) for s in w.segments]} "
          f"{w.kv_dist} keep={w.sparse_keep} opts=({opts.n_splits},{opts.n_splits_text},{opts.tile_rows},"
          f"{opts.whole_tiles})",
          flush=True)
    d = W.generate(w)
    run = G.Run(w, d, opts=opts)
    if cur.text_len > 0:
        o, o_t, lse, lse_t = run.attn_joint()
    else:
        o, lse = run.attn()
    if cur.video_len > 0:
        ref, ref_lse, _ = oracle.attention(w, d)
        G.check_bar(o.float().cpu().numpy(), ref, f"seed {seed} video")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
    if cur.text_len > 0:
        ref_t, ref_lse_t, _ = oracle.attention(w, d, queries="text")
        G.check_bar(o_t.float().cpu().numpy(), ref_t, f"seed {seed} text")
        assert np.abs(lse_t.cpu().numpy() - ref_lse_t).max() <= 1e-2
    _check_mask(w, d, run)
    _check_cache(w, d, run.cache)


def _check_mask(w, d, run):
    """DENSE expansion of the plan (video rows, then text rows) bit for bit
    against the oracle's explicit masks in the canonical key order, and the
    plan's pair count against the oracle's."""
    cur = w.current
    csr = d.get("csr") if w.sparse_keep is not None else None
    cols = G.canonical_columns(w)
    ref = oracle.mask(w, None, csr)
    if cur.text_len > 0:
        ref = np.concatenate([ref, oracle.mask_text(w)])
    absent = np.ones(ref.shape[1], bool)
    absent[cols] = False
    assert not ref[:, absent].any()
    got = run.dense(0, cur.video_len + cur.text_len)
    assert np.array_equal(got, ref[:, cols])
    if csr is None:  # a keep-list plan reports -1 (its count depends on the list)
        assert run.plan.visible_pairs * 4 * 128 * w.heads == oracle.effective_flops(w)
    else:
        assert run.plan.visible_pairs == -1
    if cur.text_len > 0:
        assert run.plan.visible_pairs_text * 4 * 128 * w.heads == oracle.effective_flops_text(w)


def _check_cache(w, d, cache):
    """Ring frames in the window and the whole head store, codes and scales,
    bit for bit against the oracle quantizer."""
    S, P, Wf = w.query_segment, w.current.tokens_per_frame, w.ring_frames
    src = [(s, f) for s in range(S) for f in range(w.segments[s].frames)]
    fs = len(src)
    H = w.heads
    for g in range(fs - min(fs, Wf), fs):
        s, f = src[g]
        slot = g % Wf
        for nm, codes, scales in (("k_vid", cache.ring_k, cache.ring_ks), ("v_vid", cache.ring_v, cache.ring_vs)):
            q, sc = oracle.quantize(d["segments"][s][nm][f * P:(f + 1) * P])
            got_q = codes[:, slot * P:(slot + 1) * P].cpu().numpy().transpose(1, 0, 2)
            got_s = scales[:, slot * P:(slot + 1) * P].cpu().numpy().T
            assert np.array_equal(got_q, q) and np.array_equal(got_s.view(np.uint32), sc.view(np.uint32))
    off = 0
    for s in range(S):
        hl = w.segments[s].head_len
        for nm, codes, scales in (("k_txt", cache.heads_k, cache.heads_ks), ("v_txt", cache.heads_v, cache.heads_vs)):
            q, sc = oracle.quantize(d["segments"][s][nm][:hl])
            got_q = codes[:, off:off + hl].cpu().numpy().transpose(1, 0, 2).reshape(hl, H, 128)
            got_s = scales[:, off:off + hl].cpu().numpy().T.reshape(hl, H)
            assert np.array_equal(got_q, q) and np.array_equal(got_s.view(np.uint32), sc.view(np.uint32))
        off += hl
