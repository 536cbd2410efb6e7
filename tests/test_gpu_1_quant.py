"""GPU parity of hn_kv_quant_append against the oracle quantizer: bit-exact
codes and scales, ring slot placement and eviction order, head-store order."""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_attention_hn_amd as hn
    import _gpu as G


def expected_cache(w, data):
    """Expected ring/head-store contents after appending segments 0..S-1."""
    H, P, Wf = w.heads, w.current.tokens_per_frame, w.ring_frames
    ring_q = np.zeros((2, H, Wf * P, 128), dtype=np.int8)
    ring_s = np.zeros((2, H, Wf * P), dtype=np.float32)
    cap = w.head_cap
    head_q = np.zeros((2, H, max(cap, 1), 128), dtype=np.int8)
    head_s = np.zeros((2, H, max(cap, 1)), dtype=np.float32)
    g = 0
    hoff = 0
    for s in range(w.query_segment):
        seg = w.segments[s]
        d = data["segments"][s]
        for t, (kn, vn) in enumerate([("k_txt", "v_txt")]):
            for i, nm in enumerate((kn, vn)):
                q, sc = oracle.quantize(d[nm][:seg.head_len])          # [h][H][D], [h][H]
                head_q[i, :, hoff:hoff + seg.head_len] = q.transpose(1, 0, 2)
                head_s[i, :, hoff:hoff + seg.head_len] = sc.T
        keep = min(seg.frames, Wf)
        for f in range(seg.frames - keep, seg.frames):
            slot = (g + f) % Wf
            for i, nm in enumerate(("k_vid", "v_vid")):
                q, sc = oracle.quantize(d[nm][f * P:(f + 1) * P])
                ring_q[i, :, slot * P:(slot + 1) * P] = q.transpose(1, 0, 2)
                ring_s[i, :, slot * P:(slot + 1) * P] = sc.T
        g += seg.frames
        hoff += seg.head_len
    return ring_q, ring_s, head_q, head_s


def got_cache(cache):
    t = lambda x: x.cpu().numpy()
    return (np.stack([t(cache.ring_k), t(cache.ring_v)]), np.stack([t(cache.ring_ks), t(cache.ring_vs)]),
            np.stack([t(cache.heads_k), t(cache.heads_v)]), np.stack([t(cache.heads_ks), t(cache.heads_vs)]))


@pytest.mark.parametrize("name", ["c1", "c1_evict", "c1_future", "m1", "m2", "m3"])
def test_append_bitexact_and_ring_order(name):
    print(f"[quant] {name}", flush=True)
    w = W.config(name)
    data = W.generate(w)
    cache = G.new_cache(w)
    G.fill_history(w, data, cache)
    torch.cuda.synchronize()
    exp = expected_cache(w, data)
    got = got_cache(cache)
    for e, g_, what in zip(exp, got, ("ring codes", "ring scales", "head codes", "head scales")):
        assert np.array_equal(e.view(np.uint8) if e.dtype == np.int8 else e.view(np.uint32),
                              g_.view(np.uint8) if g_.dtype == np.int8 else g_.view(np.uint32)), what
    assert cache.segments == w.query_segment
    assert cache.frames_seen == sum(s.frames for s in w.segments[:w.query_segment])


def _check_frames_and_heads(w, data, cache, appended, frames):
    """Ring slots of the given global frames and the whole head store after
    segments 0 .. appended-1 were appended, bit for bit against the oracle."""
    P, Wf = w.segments[0].tokens_per_frame, w.ring_frames
    src = []  # (segment, local frame) of every global frame
    for s in range(appended):
        src += [(s, f) for f in range(w.segments[s].frames)]
    fs = len(src)
    for g in frames:
        assert fs - min(fs, Wf) <= g < fs, "frame not in the window"
        s, f = src[g]
        slot = g % Wf
        for nm, codes, scales in (("k_vid", cache.ring_k, cache.ring_ks), ("v_vid", cache.ring_v, cache.ring_vs)):
            q, sc = oracle.quantize(data["segments"][s][nm][f * P:(f + 1) * P])   # [P][H][D], [P][H]
            got_q = codes[:, slot * P:(slot + 1) * P].cpu().numpy().transpose(1, 0, 2)
            got_s = scales[:, slot * P:(slot + 1) * P].cpu().numpy().T
            assert np.array_equal(got_q, q), f"{nm} codes of frame {g}"
            assert np.array_equal(got_s.view(np.uint32), sc.view(np.uint32)), f"{nm} scales of frame {g}"
    hoff = 0
    for s in range(appended):
        hl = w.segments[s].head_len
        for nm, codes, scales in (("k_txt", cache.heads_k, cache.heads_ks), ("v_txt", cache.heads_v, cache.heads_vs)):
            q, sc = oracle.quantize(data["segments"][s][nm][:hl])
            got_q = codes[:, hoff:hoff + hl].cpu().numpy().transpose(1, 0, 2)
            got_s = scales[:, hoff:hoff + hl].cpu().numpy().T
            assert np.array_equal(got_q, q), f"{nm} codes of segment {s}"
            assert np.array_equal(got_s.view(np.uint32), sc.view(np.uint32)), f"{nm} scales of segment {s}"
        hoff += hl
    assert cache.head_tokens == hoff and cache.frames_seen == fs


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_append_bitexact_target_shapes(name):
    """The appends of the five target configurations' shapes: the 480x832
    segment itself (12,468 tokens x 16 heads, no window: every frame checked);
    three 1280x704 segments through the 18-frame window (every kept frame:
    30-frame segments wrap the ring); six 1280x704 segments with 1,280-token
    heads and no window (a spread of 24 of the 180 frames, first and last of
    every segment included).  All heads of the head store are checked."""
    print(f"[quant] {name}", flush=True)
    w = W.config(name)
    data = W.generate(w)
    cache = G.new_cache(w)
    if w.query_segment == 0:
        appended = 1
        seg = w.segments[0]
        d = data["segments"][0]
        hn.hn_kv_quant_append(cache, G.layout(0, seg), G.dev(d["k_txt"]), G.dev(d["v_txt"]),
                              G.dev(d["k_vid"]), G.dev(d["v_vid"]))
    else:
        appended = w.query_segment
        G.fill_history(w, data, cache)
    torch.cuda.synchronize()
    fs = sum(s.frames for s in w.segments[:appended])
    kept = list(range(fs - min(fs, w.ring_frames), fs))
    if len(kept) > 30:
        ends = [g for s in range(appended) for g in (30 * s, 30 * s + 29)]
        kept = sorted(set(ends + kept[::15]))
    _check_frames_and_heads(w, data, cache, appended, kept)


def _append_rows(rows_bits: np.ndarray, H: int = 16):
    """Append rows [n][128] as one segment (F=1, P=n/H tokens, heads inner) and
    return (codes [n][128], scales [n]) read back from the ring."""
    n = rows_bits.shape[0]
    assert n % H == 0
    P = n // H
    cache = hn.KVCache(H, P, 1, 0)
    x = rows_bits.reshape(P, H, 128)
    kv = G.dev(x)
    seg = hn.SegLayout(0, 1, P, 0)
    hn.hn_kv_quant_append(cache, seg, None, None, kv, kv)
    torch.cuda.synchronize()
    q = cache.ring_k.cpu().numpy().transpose(1, 0, 2).reshape(n, 128)
    s = cache.ring_ks.cpu().numpy().T.reshape(n)
    qv = cache.ring_v.cpu().numpy().transpose(1, 0, 2).reshape(n, 128)
    assert np.array_equal(q, qv)
    return q, s


def test_crafted_rows():
    rng = np.random.default_rng(5)
    rows = []
    # exact ties at scale 1 (amax = 127): half-integers round to even
    r = np.zeros(128, np.float32); r[0] = 127
    r[1:64] = np.arange(1, 64) - 0.5
    r[64:127] = -(np.arange(1, 64) - 0.5)
    rows.append(r)
    rows.append(np.zeros(128, np.float32))                         # zero row
    rows.append(np.full(128, 3.0, np.float32))                     # constant row
    rows.append(np.full(128, -2.0 ** -130, np.float32))            # subnormal constant
    for e in (-133, -128, -126, -100, 0, 100, 125, 126):  # |x| < 2^128 stays finite
        rows.append(rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** e))
    r = np.zeros(128, np.float32); r[0] = 1.0; r[1:5] = [-0.5, 0.5, 0.25, 0.75]
    rows.append(r)
    while len(rows) % 16:
        rows.append(rng.standard_normal(128).astype(np.float32))
    bits = W.f32_to_bf16_bits(np.stack(rows))
    q, s = _append_rows(bits)
    qe, se = oracle.quantize(bits)
    assert np.array_equal(q, qe)
    assert np.array_equal(s.view(np.uint32), se.view(np.uint32))


def _sweep_rows(a_lo: int, a_hi: int) -> np.ndarray:
    """Rows covering every bf16 x with |x| <= amax, for amax bit patterns in
    [a_lo, a_hi): each row is [amax, x_1 .. x_127]."""
    rows = []
    for a in range(a_lo, a_hi):
        vals = np.concatenate([np.arange(0, a + 1, dtype=np.uint16),
                               np.arange(0x8000, 0x8000 + a + 1, dtype=np.uint16)])
        vals = np.resize(vals, len(vals) + (-len(vals)) % 127)  # repeat to whole rows
        block = np.empty((len(vals) // 127, 128), dtype=np.uint16)
        block[:, 0] = a
        block[:, 1:] = vals.reshape(-1, 127)
        rows.append(block)
    out = np.concatenate(rows)
    return np.resize(out, (out.shape[0] + (-out.shape[0]) % 16, 128))


def test_exhaustive_element_sweep():
    """q(x, amax) for every finite bf16 pair with |x| <= amax (about 1.07e9
    pairs) plus scale(amax) for every positive finite bf16 amax, bit-exact."""
    t0 = time.time()
    edges = np.unique(np.round(np.sqrt(np.linspace(1, 0x7F80 ** 2, 33))).astype(int))
    total = 0
    for a_lo, a_hi in zip(edges[:-1], edges[1:]):
        bits = _sweep_rows(int(a_lo), int(a_hi))
        q, s = _append_rows(bits)
        qe, se = oracle.quantize(bits)
        bad = np.nonzero(np.any(q != qe, axis=1) | (s.view(np.uint32) != se.view(np.uint32)))[0]
        assert len(bad) == 0, f"amax {hex(int(bits[bad[0], 0]))}: row {bad[0]}"
        total += bits.shape[0] * 127
        print(f"[sweep] amax < {hex(int(a_hi))}: {total:.3e} pairs, {time.time() - t0:.1f}s", flush=True)
    assert total > 1.0e9
