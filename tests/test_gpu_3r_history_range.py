"""GPU parity of the two range guards of the INT8 history's fp16 arithmetic.

hn_seg_attn_fwd computes history tiles in fp16 with power-of-two shifts
(include/hn.h, hn_seg_attn_fwd):
  * a query row holding |Q| >= 2^15 enters the fp16 products as Q * 2^-qs,
    the shift folded back into that row's score scale;
  * a history key or value beyond fp16's reach (|K| > 65,024, |V| > 8.3e6)
    sends its block back to the start, to take every tile in bf16.
Neither occurs with unit-variance inputs, so these tests force them.

Huge queries: Q scaled by 2^k with sm_scale scaled by 2^-k leaves every
score unchanged in exact arithmetic, so the outputs must meet the bar of the
oracle on the unscaled inputs; and two scalings that put every row through
the shift (2^16 and 2^20) must give bit-identical outputs, since the kernel
then sees the same fp16 operands and the same score scale.

Huge key: one history token's key is set to 2^17 on one dimension (zero
elsewhere: its INT8 scale is 131072 / 127 > 512) at several places of the
plan's history tiles (the first tile, a later head tile, ring frames old and
new), so that the restart happens before any step, after an odd and after an
even number of fp16 steps.  The oracle computes the same modified inputs.
Staged in fp16 the planted key would overflow (127 x 1032 > 65,504), so the
outputs meet the bar only if the block restarted in bf16.

Small values: every value (history and current) scaled by 2^-9 scales O by
2^-9 in exact arithmetic and leaves the scores alone, so 2^9 x O must meet
the bar of the oracle on the unscaled inputs.  This holds only if the fp16
staging keeps small scales in fp16's normal range (a value scale of 3e-4 x
2^-7 would be subnormal and lose up to 8% of its bits).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_attention_hn_amd as hn
    import _gpu as G

SM = 1.0 / math.sqrt(128)
BF16_2P17 = 0x4800  # bf16 bits of 2^17


def _scaled(t, k):
    out = (t.float() * 2.0 ** k).to(torch.bfloat16)
    assert torch.equal(out.float(), t.float() * 2.0 ** k)  # exact: powers of two
    return out


def _joint(run, k):
    o, o_t, lse, lse_t = hn.seg_attn_joint(run.cache, run.seg, run.plan, _scaled(run.q, k),
                                           _scaled(run.q_txt, k), run.k_txt, run.v_txt, run.k_vid,
                                           run.v_vid, sm_scale=SM * 2.0 ** -k)
    torch.cuda.synchronize()
    return o, o_t, lse, lse_t


def _check(w, d, o, o_t, lse, lse_t, what):
    ref, ref_lse, _ = oracle.attention(w, d)
    err = G.check_bar(o.float().cpu().numpy(), ref, what + " video")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
    ref_t, ref_lse_t, _ = oracle.attention(w, d, queries="text")
    err_t = G.check_bar(o_t.float().cpu().numpy(), ref_t, what + " text")
    assert np.abs(lse_t.cpu().numpy() - ref_lse_t).max() <= 1e-2
    print(f"  {what}: max-abs video {err.max():.3e} text {err_t.max():.3e}", flush=True)


@pytest.mark.parametrize("rows", ["auto", "128", "384"])
@pytest.mark.parametrize("name", ["c1", "m1", "m2", "m3"])
def test_huge_queries(name, rows):
    print(f"[range] huge queries {name} rows={rows}", flush=True)
    w = W.config(name)
    if rows == "384" and w.sparse_keep is not None:
        pytest.skip("a keep list fixes 128-row query tiles")
    d = W.generate(w)
    opts = None if rows == "auto" else hn.PlanOpts(tile_rows=int(rows))
    run = G.Run(w, d, opts=opts)
    # 2^13: a few rows reach 2^15 (shifted), most do not; 2^16: every row shifted
    for k in (13, 16):
        _check(w, d, *_joint(run, k), f"{name} Q x 2^{k}")
    a = _joint(run, 16)
    b = _joint(run, 20)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _plant_key(d, src, seg, token, dim=5):
    k = d["segments"][seg][src]
    k[token] = 0
    k[token, :, dim] = BF16_2P17


# (source, segment, token): m1's history is segments 0 and 1 (heads of 40 and
# 33 tokens, then ring frames 3 of segment 0 and 0-4 of segment 1, 50 tokens
# each); c1's is two segments of 16-token heads and 2 frames of 24 tokens
PLACES = {
    "m1": [("k_txt", 0, 0), ("k_txt", 1, 30), ("k_vid", 0, 3 * 50 + 10), ("k_vid", 1, 2 * 50 + 7),
           ("k_vid", 1, 5 * 50 - 1)],
    "c1": [("k_txt", 0, 3), ("k_vid", 0, 30), ("k_vid", 1, 47)],
}


@pytest.mark.parametrize("rows", ["auto", "128", "384"])
@pytest.mark.parametrize("name,place", [(n, p) for n, ps in PLACES.items() for p in ps])
def test_huge_history_key_restarts_in_bf16(name, place, rows):
    print(f"[range] huge key {name} {place} rows={rows}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    _plant_key(d, *place)
    # the planted row's INT8 scale is beyond the fp16 staging's range
    q, sc = oracle.quantize(d["segments"][place[1]][place[0]][place[2]:place[2] + 1])
    assert sc.min() > 512 and np.all(q[0, :, 5] == 127)
    opts = None if rows == "auto" else hn.PlanOpts(tile_rows=int(rows))
    run = G.Run(w, d, opts=opts)
    _check(w, d, *_joint(run, 0), f"{name} {place}")


@pytest.mark.parametrize("name", ["m1", "m2", "c3_h2"])
def test_small_values_keep_precision(name):
    print(f"[range] small values {name}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    ref_o, ref_lse, _ = oracle.attention(w, d, G.sample_rows(w.current.video_len)
                                         if w.current.video_len > 4096 else None)
    for seg in d["segments"]:
        for nm in ("v_txt", "v_vid"):
            x = W.bf16_bits_to_f32(seg[nm]) * np.float32(2.0 ** -9)
            seg[nm] = W.f32_to_bf16_bits(x)       # exact: a power of two
    run = G.Run(w, d)
    o, lse = run.attn()
    rows = G.sample_rows(w.current.video_len) if w.current.video_len > 4096 else np.arange(w.current.video_len)
    got = o.float().cpu().numpy()[rows] * 2.0 ** 9
    err = G.check_bar(got, ref_o, f"{name} V x 2^-9")
    assert np.abs(lse.cpu().numpy()[:, rows] - ref_lse).max() <= 1e-2
    print(f"  {name}: max-abs of 2^9 O {err.max():.3e}", flush=True)


@pytest.mark.parametrize("name", ["m1", "m2"])
def test_key_scale_invariance_bitwise(name):
    """Keys scaled by 2^-4 with sm_scale scaled by 2^4 leave every score
    unchanged: the INT8 codes are the same, the scales exactly 2^-4 times
    theirs, fp16(code x fp16(scale)) and the bf16 keys exactly 2^-4 times
    theirs (all in fp16's normal range for unit-variance rows), and the
    products and sums scale exactly.  So the outputs must equal those of the
    unscaled inputs bit for bit."""
    print(f"[range] key scale {name}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    run = G.Run(w, d)
    ref = run.attn_joint()
    for seg in d["segments"]:
        for nm in ("k_txt", "k_vid"):
            seg[nm] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(seg[nm]) * np.float32(2.0 ** -4))
    run2 = G.Run(w, d)
    got = hn.seg_attn_joint(run2.cache, run2.seg, run2.plan, run2.q, run2.q_txt, run2.k_txt, run2.v_txt,
                            run2.k_vid, run2.v_vid, sm_scale=SM * 2.0 ** 4)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["m1", "m2"])
def test_large_values_keep_precision(name):
    """Every value scaled by 2^12 (up to |V| ~ 10^5 on heavy tails, inside the
    fp16 staging's range): 2^-12 O must meet the bar of the oracle on the
    unscaled inputs."""
    print(f"[range] large values {name}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    ref_o, ref_lse, _ = oracle.attention(w, d)
    for seg in d["segments"]:
        for nm in ("v_txt", "v_vid"):
            seg[nm] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(seg[nm]) * np.float32(2.0 ** 12))
    run = G.Run(w, d)
    o, lse = run.attn()
    G.check_bar(o.float().cpu().numpy() * 2.0 ** -12, ref_o, f"{name} V x 2^12")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
