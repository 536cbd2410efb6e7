"""Host-side checks of the C ABI that need no GPU: every function declared in
include/hn.h is exported by libhn.so, and argument validation returns its
status before anything is enqueued (device pointers below are never touched)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import masked_attention_hn_amd as hn  # noqa: E402  (conftest builds the library if needed)

FAKE = 0x10000  # a non-NULL device address; validation never dereferences it


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hn_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "hn_seg_attn_fwd" in names and "hn_kv_quant_append" in names
    lib = ctypes.CDLL(hn.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(hn.EXPORTS) == set(names)


def fake_cache(H=2, P=24, W=4, cap=48, head_dim=128):
    return hn.hn_kv_cache(H, head_dim, P, W, cap, 0, *([FAKE] * 8), 0, 0, 0)


def seg_c(index=0, F=2, P=24, h=16, tails=((8, 0, 1), (8, 1, 2))):
    return hn.SegLayout(index, F, P, h, [t[0] for t in tails], [t[1] for t in tails],
                        [t[2] for t in tails])


def call_append(cache, seg):
    return hn._lib.hn_kv_quant_append(ctypes.byref(cache), ctypes.byref(seg.c), FAKE, FAKE, FAKE,
                                      FAKE, None)


def test_status_strings():
    assert hn.hn_status_string(0) == "ok"
    assert "order" in hn.hn_status_string(hn.HN_ERR_ORDER)


def test_append_validation():
    c = fake_cache()
    assert hn._lib.hn_kv_quant_append(None, ctypes.byref(seg_c().c), FAKE, FAKE, FAKE, FAKE,
                                      None) == hn.HN_ERR_NULL
    assert call_append(fake_cache(head_dim=64), seg_c()) == hn.HN_ERR_UNSUPPORTED
    assert call_append(c, seg_c(index=1)) == hn.HN_ERR_ORDER
    assert "segment index 1" in hn.hn_last_error()
    assert call_append(c, seg_c(P=25)) == hn.HN_ERR_INVALID
    assert call_append(c, seg_c(tails=((8, 1, 3),))) == hn.HN_ERR_INVALID      # window past F
    assert call_append(c, seg_c(tails=((8, 2, 1),))) == hn.HN_ERR_INVALID      # f0 > f1
    assert call_append(c, seg_c(tails=((-1, 0, 1),))) == hn.HN_ERR_INVALID
    assert call_append(c, seg_c(tails=((1, 0, 1),) * 65)) == hn.HN_ERR_UNSUPPORTED
    assert call_append(fake_cache(cap=10), seg_c()) == hn.HN_ERR_CAPACITY
    c.head_tokens = 40
    assert call_append(c, seg_c()) == hn.HN_ERR_CAPACITY
    assert (c.frames_seen, c.head_tokens, c.segments) == (0, 40, 0)   # unchanged
    z = fake_cache()
    z.ring_k = None
    assert call_append(z, seg_c()) == hn.HN_ERR_NULL


def test_append_rejects_2pow31_rows():
    """The quantize/append kernel indexes (token, head) rows in 32 bits: a
    segment with 2^31 or more surviving rows is refused before any launch;
    without a device, one just below the bound gets past that check (and
    fails at the launch instead)."""
    H, P, F = 16, 4096, 32768                    # 16 x 4096 x 32768 = 2^31 rows
    c = fake_cache(H=H, P=P, W=F, cap=0)
    s = hn.SegLayout(0, F, P, 0, [], [], [])
    assert call_append(c, s) == hn.HN_ERR_UNSUPPORTED
    assert "2^31" in hn.hn_last_error()
    assert (c.frames_seen, c.head_tokens, c.segments) == (0, 0, 0)
    if not torch.cuda.is_available():           # the fake pointers must never reach a GPU
        small = hn.SegLayout(0, F - 1, P, 0, [], [], [])
        assert call_append(fake_cache(H=H, P=P, W=F, cap=0), small) == hn.HN_ERR_HIP


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device failure path")
def test_failed_launch_leaves_cache_unchanged():
    c = fake_cache()
    st = call_append(c, seg_c())
    assert st == hn.HN_ERR_HIP
    assert (c.frames_seen, c.head_tokens, c.segments) == (0, 0, 0)


def test_workspace_sizes_and_plan_checks():
    c = fake_cache()
    s = seg_c()
    n = hn._lib.hn_attn_workspace_size(ctypes.byref(c), ctypes.byref(s.c), None, None)
    # counts padded to 256 bytes + (one video + one text query tile) x (4 + 2 tails)
    # spans of 32 bytes, padded to 256 bytes (4 query tiles of 2 heads: no key split)
    assert n == 256 + 512
    assert 256 + 2 * 6 * 32 <= n
    bad = hn.hn_block_sparse(64, 64, 1, 0, FAKE, FAKE)
    assert hn._lib.hn_attn_workspace_size(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(bad), None) == 0
    sp = hn.hn_block_sparse(128, 128, 1, 0, FAKE, FAKE)
    n_sp = hn._lib.hn_attn_workspace_size(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(sp), None)
    assert n_sp == 256 + 2 * (4 + 2 + 0 + 1 + 1) * 32   # already a multiple of 256
    plan = hn.hn_tile_plan()
    build = hn._lib.hn_attn_mask_build
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 0, 0, 0, FAKE, n - 1,
                 ctypes.byref(plan), None) == hn.HN_ERR_WORKSPACE
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 0, 0, 0, FAKE + 4, n,
                 ctypes.byref(plan), None) == hn.HN_ERR_INVALID                # misaligned
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 0, 0, 0, FAKE, n, None,
                 None) == hn.HN_ERR_NULL
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 1, 0, 48, FAKE, 48 * 1000,
                 ctypes.byref(plan), None) == hn.HN_ERR_INVALID                # plan in DENSE
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 1, 40, 41, FAKE, 10 ** 6, None,
                 None) == hn.HN_ERR_INVALID                    # rows past F*P + h + sum(a)
    lk = 0 + 0 + 32 + 48
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 1, 0, 48, FAKE, 48 * lk - 1, None,
                 None) == hn.HN_ERR_WORKSPACE
    assert build(ctypes.byref(c), ctypes.byref(s.c), None, None, 7, 0, 0, FAKE, n,
                 None, None) == hn.HN_ERR_INVALID


def test_attention_rejects_stale_plan():
    c = fake_cache()
    s = seg_c()
    plan = hn.hn_tile_plan(dev=FAKE, tile_q=128, n_qtiles=1, n_text_tiles=1, max_spans=6,
                           n_splits=1, n_splits_text=1, visible_pairs=-1)
    fwd = hn._lib.hn_seg_attn_fwd
    q = [FAKE, None]                # q_vid, q_txt
    kv = [FAKE] * 4                 # k_txt, v_txt, k_vid, v_vid
    out = [FAKE, None, None, None]  # o_vid, o_txt, lse, lse_txt
    call = lambda seg, pl, qq=q, oo=out, scale=0.1: fwd(ctypes.byref(c), ctypes.byref(seg.c), pl,
                                                        *qq, *kv, *oo, scale, None)
    # dense plans come in the heights the kernel has instances for (128, 256
    # and 384): a plan with one of them gets past the staleness check to the
    # scale check
    tiles = [t for t in (64, 128, 192, 256, 384, 512)
             if (setattr(plan, "tile_q", t), call(s, ctypes.byref(plan), scale=float("nan")))[1]
             == hn.HN_ERR_INVALID]
    assert tiles == [128, 256, 384]
    plan.sparse = 1                # a keep-list plan is always 128 rows
    plan.tile_q = 256
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.sparse = 0
    plan.tile_q = tiles[0]
    plan.frames_seen = 24          # built for another cache state
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.frames_seen = 0
    plan.seg_index = 1
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.seg_index = 0
    plan.n_text_tiles = 2          # text tiles of another layout
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.n_text_tiles = 1
    plan.n_splits = 0              # not a plan the builder writes
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.n_splits = 1
    plan.n_splits_text = 17
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.n_splits_text = 1
    # leading whole tiles only with a split, and fewer than the query tiles
    plan.n_whole = 1               # without a split
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.n_splits = 2
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER        # 1 whole of 1 query tile
    plan.n_whole = -1
    assert call(s, ctypes.byref(plan)) == hn.HN_ERR_ORDER
    plan.n_whole = 0
    assert call(s, ctypes.byref(plan), scale=float("nan")) == hn.HN_ERR_INVALID   # a valid split plan
    plan.n_splits = 1
    assert call(s, None) == hn.HN_ERR_NULL
    assert call(s, ctypes.byref(plan), scale=float("nan")) == hn.HN_ERR_INVALID
    assert call(s, ctypes.byref(plan), scale=-0.1) == hn.HN_ERR_INVALID   # positive scales only
    assert call(s, ctypes.byref(plan), scale=0.0) == hn.HN_ERR_INVALID
    # text queries without their output
    assert call(s, ctypes.byref(plan), qq=[FAKE, FAKE]) == hn.HN_ERR_NULL
    s2 = seg_c(index=1)
    assert call(s2, ctypes.byref(plan)) == hn.HN_ERR_ORDER


def test_cache_sizes():
    rb, rsb, hb, hsb = hn.hn_kv_cache_sizes(16, 18, 880, 2304)
    assert rb == 16 * 18 * 880 * 128 and rsb == 16 * 18 * 880 * 4
    assert hb == 16 * 2304 * 128 and hsb == 16 * 2304 * 4
    with pytest.raises(hn.HNError):
        hn.hn_kv_cache_sizes(0, 18, 880, 0)


def ws_size(c, seg, sparse=None, n_splits=0, n_splits_text=0, tile_rows=0, whole_tiles=0):
    """hn_attn_workspace_size with plan options (0 = automatic)."""
    opts = hn.PlanOpts(n_splits, n_splits_text, tile_rows, whole_tiles)
    return hn._lib.hn_attn_workspace_size(ctypes.byref(c), ctypes.byref(seg.c),
                                          ctypes.byref(sparse) if sparse is not None else None,
                                          ctypes.byref(opts))


def test_split_count_forced_and_sized():
    """opts.n_splits forces the key split; the workspace then also holds the
    partial results: H x virtual tiles x tile rows x (128 + 1) floats."""
    c = fake_cache()
    s = seg_c()
    n1 = hn._lib.hn_attn_workspace_size(ctypes.byref(c), ctypes.byref(s.c), None, None)
    assert ws_size(c, s) == n1                 # zeroed options = automatic = NULL options
    n3 = ws_size(c, s, n_splits=3)
    vt = 1 * 3 + 1 * 1                         # video tile x 3 splits + text tile (80 keys: unsplit)
    spans = -(-(256 + vt * 6 * 32) // 256) * 256
    a256 = lambda b: -(-b // 256) * 256
    # partials for the dense plans' query-tile height R (the kernel's choice)
    fits = [R for R in (64, 128, 256, 384, 512)
            if n3 == spans + a256(2 * vt * R * 128 * 4) + a256(2 * vt * R * 4)]
    assert len(fits) == 1 and n3 > n1
    # out-of-range options are an error, not a silent fallback
    assert ws_size(c, s, n_splits=17) == 0 and "split counts" in hn.hn_last_error()
    assert ws_size(c, s, n_splits_text=-1) == 0
    assert ws_size(c, s, tile_rows=64) == 0 and "tile_rows" in hn.hn_last_error()
    # whole_tiles only with a forced split count > 1, and not negative
    assert ws_size(c, s, whole_tiles=1) == 0 and "whole_tiles" in hn.hn_last_error()
    assert ws_size(c, s, n_splits=1, whole_tiles=1) == 0
    assert ws_size(c, s, n_splits=3, whole_tiles=-1) == 0
    sp = hn.hn_block_sparse(128, 128, 1, 0, FAKE, FAKE)
    assert ws_size(c, s, sp, tile_rows=128) > 0
    assert ws_size(c, s, sp, tile_rows=fits[0]) == (0 if fits[0] != 128 else ws_size(c, s, sp))


def test_whole_tiles_sized():
    """With whole_tiles = w the first w video query tiles run whole and the
    others split: w + (n_qtiles - w) x splits video virtual tiles, partial
    results for the split ones and the text tiles (here one text tile);
    w >= n_qtiles means no split at all."""
    c = fake_cache(H=2, P=24, W=4, cap=48)
    s = hn.SegLayout(0, 30, 24, 16, [8, 8], [0, 15], [15, 30])     # 720 video rows, 32 text rows
    a256 = lambda b: -(-b // 256) * 256
    R = 256
    nq = 3
    for w in (0, 1, 2):
        vt = w + (nq - w) * 3 + 1
        n_pvt = vt - w
        spans = a256(a256(vt * 4) + vt * 6 * 32)
        want = spans + a256(2 * n_pvt * R * 128 * 4) + a256(2 * n_pvt * R * 4)
        assert ws_size(c, s, n_splits=3, n_splits_text=1, tile_rows=R, whole_tiles=w) == want
    # every tile whole: the plan of no split
    assert (ws_size(c, s, n_splits=3, n_splits_text=1, tile_rows=R, whole_tiles=nq)
            == ws_size(c, s, n_splits=1, n_splits_text=1, tile_rows=R))


def test_tile_rows_option():
    """tile_rows = 128 gives 128-row tiles to a dense plan (the default is the
    kernel's larger tile); the plan records the height it was built with."""
    c = fake_cache()
    s = hn.SegLayout(0, 30, 24, 16, [8, 8], [0, 15], [15, 30])   # 720 video rows
    n_auto, n_128 = ws_size(c, s), ws_size(c, s, tile_rows=128)
    assert n_auto > 0 and n_128 > 0 and n_auto != n_128


def test_dense_tile_height_follows_the_makespan_estimate():
    """Without a device (256 compute units assumed): a dense plan takes 384-row
    query tiles where their estimated makespan is smaller (the 480x832
    segment: 496 blocks in 2 rounds against 736 in 3; the 1280x704 steady
    state and its 7th segment, split in two either way), and 256-row ones
    where 384-row blocks would leave more CUs idle (the 2-head share: 138
    blocks against 208 in one round) or where the segment has at most 256
    rows; a keep list fixes 128 rows."""

    def heights(H, P, frames, W_, seen):
        c = fake_cache(H=H, P=P, W=W_, cap=1 << 14)
        c.frames_seen = seen
        c.segments = 0
        seg = hn.SegLayout(0, frames, P, 16, [], [], [])
        auto = ws_size(c, seg, n_splits_text=1)
        return [R for R in (128, 256, 384) if ws_size(c, seg, n_splits_text=1, tile_rows=R) == auto]

    assert heights(16, 390, 30, 1, 0) == [384]        # 480x832 segment
    assert heights(16, 880, 30, 18, 18) == [384]      # 1280x704 steady state
    assert heights(16, 880, 30, 210, 180) == [384]    # its 7th segment (no window)
    assert heights(2, 880, 30, 18, 18) == [256]       # 2-head share
    # 240 rows of 1 head over a 24,000-key ring: one tile either way, split
    # (so that the partial results, sized by the height, tell them apart)
    assert heights(1, 120, 2, 200, 200) == [256]
    c = fake_cache(H=16, P=390, W=1)
    seg = hn.SegLayout(0, 30, 390, 16, [], [], [])
    sp = hn.hn_block_sparse(128, 128, 92, 0, FAKE, FAKE)
    assert ws_size(c, seg, sp) == ws_size(c, seg, sp, tile_rows=128) > 0


def test_automatic_split_only_for_small_grids():
    """Without a device (256 compute units assumed) a 16-head grid with short
    key lists (31 query tiles of 384 rows per head) is not split; a 1-head
    layout with 2 query tiles of long key lists is split to about two blocks
    per CU, capped at 16 and at 1024 keys per split."""
    plan_sizes = {}
    for H, P, frames, W_ in ((16, 390, 30, 1), (1, 128, 2, 200)):
        c = fake_cache(H=H, P=P, W=W_)
        c.frames_seen = W_          # a full ring of history
        seg = hn.SegLayout(0, frames, P, 16, [], [], [])
        c.segments = 0
        plan_sizes[H] = ws_size(c, seg, n_splits_text=1)   # video tiles only here
    # 16 heads x 31 tiles (+1 text tile): spans only (no partial results)
    n_vt = 31 + 1
    assert plan_sizes[16] == -(-(-(-n_vt * 4 // 256) * 256 + n_vt * 4 * 32) // 256) * 256
    # 1 head x 1-2 video tiles (+1 text tile): ring 25,600 + 16 + 256 keys -> 16 splits
    a256 = lambda b: -(-b // 256) * 256
    ok = []
    for R in (128, 256):
        n_vt = -(-256 // R) * 16 + 1        # video tiles x 16 splits + the (unsplit) text tile
        spans = a256(a256(n_vt * 4) + n_vt * 4 * 32)
        ok.append(plan_sizes[1] == spans + a256(n_vt * R * 128 * 4) + a256(n_vt * R * 4))
    assert any(ok)


def test_automatic_split_fills_the_last_round():
    """Without a device (256 compute units assumed): a 16-head grid whose last
    round of blocks is partly empty and whose query tiles visit long key
    lists (the 1280x704 steady state: 26,400 queries, 18-frame ring) keeps
    its leading tiles whole for the full rounds and splits the last tiles of
    every head so that their pieces fill the last round; the same grid with
    short key lists (the 480x832 segment), and the 2-head share (one round of
    blocks), are not split.  The automatic workspace size must equal the one
    of the forced choice."""

    def ws(H, P, frames, W_, splits=0, whole=0):
        c = fake_cache(H=H, P=P, W=W_)
        c.frames_seen = W_          # a full ring of history
        c.segments = 0
        seg = hn.SegLayout(0, frames, P, 16, [], [], [])
        return ws_size(c, seg, n_splits=splits, n_splits_text=1, whole_tiles=whole)

    # 1,104 blocks of 384 rows: 4 full rounds and 80 blocks; the last 5 tiles
    # of each head are split three ways (240 pieces for the last round)
    steady = (16, 880, 30, 18)
    assert ws(*steady) == ws(*steady, splits=3, whole=64) != ws(*steady, splits=2)
    assert ws(*steady, splits=2) != ws(*steady, splits=1)
    short = (16, 390, 30, 1)         # 12,106 keys per query tile
    assert ws(*short) == ws(*short, splits=1)
    share = (2, 880, 30, 18)         # 208 blocks: one round either way
    assert ws(*share) == ws(*share, splits=1)


def test_text_split_count_follows_the_round_model():
    """Without a device (256 compute units assumed): the text tiles of a joint
    launch are split so that they fill what the video blocks leave free.  The
    480x832 segment (496 unsplit video blocks of 384 rows: 16 slots free in
    the last round) takes 4; so does the 1280x704 steady state (4 full
    rounds of whole video blocks, then 240 split pieces); short text tiles
    stay whole.  The automatic workspace size must equal the one of the
    forced count."""

    def ws(H, P, frames, W_, text_splits=0, head=768, tails=(128,) * 4):
        c = fake_cache(H=H, P=P, W=W_, cap=4096)
        c.frames_seen = W_ if W_ > 1 else 0   # a full ring of history (none for the first segment)
        c.segments = 0
        seg = hn.SegLayout(0, frames, P, head, list(tails), [0] * len(tails), [frames] * len(tails))
        return ws_size(c, seg, n_splits_text=text_splits)

    first = (16, 390, 30, 1)
    assert ws(*first) == ws(*first, text_splits=4) != ws(*first, text_splits=8)
    steady = (16, 880, 30, 18)
    assert ws(*steady) == ws(*steady, text_splits=4) != ws(*steady, text_splits=8)
    short = (2, 24, 2, 4)
    assert ws(*short, head=16, tails=(8, 8)) == ws(*short, text_splits=1, head=16, tails=(8, 8))


def test_archive_checks():
    """Validation of hn_kv_archive_evict / hn_kv_cache_rewind on the host
    (cases that copy nothing; the copies themselves are GPU tests)."""
    c = fake_cache(H=2, P=24, W=4)
    s = seg_c()                      # 2 frames
    ar = hn.hn_kv_archive(FAKE, FAKE, FAKE, FAKE, 8, 0, 0, 0)
    ev = hn._lib.hn_kv_archive_evict
    rw = hn._lib.hn_kv_cache_rewind
    # nothing leaves a window that is not yet full: OK, archive unchanged
    assert ev(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(ar), None) == hn.HN_OK
    assert ar.frames == 0
    assert ev(ctypes.byref(c), ctypes.byref(s.c), None, None) == hn.HN_ERR_NULL
    bad = hn.hn_kv_archive(FAKE, FAKE, FAKE, FAKE, 8, 0, 0, 9)   # frames > capacity
    assert ev(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(bad), None) == hn.HN_ERR_INVALID
    assert ev(ctypes.byref(c), ctypes.byref(seg_c(index=1).c), ctypes.byref(ar), None) == hn.HN_ERR_ORDER
    # full window (6 frames seen, W = 4): appending 2 frames evicts frames 2, 3
    c.frames_seen, c.segments = 6, 0
    small = hn.hn_kv_archive(FAKE, FAKE, FAKE, FAKE, 1, 0, 0, 0)
    assert ev(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(small), None) == hn.HN_ERR_CAPACITY
    gap = hn.hn_kv_archive(FAKE, FAKE, FAKE, FAKE, 8, 0, 0, 1)    # holds frame 0 only: 1 is missing
    assert ev(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(gap), None) == hn.HN_ERR_ORDER
    assert small.frames == 0 and gap.frames == 1
    # rewind: targets must be earlier states
    c.frames_seen, c.head_tokens, c.segments = 6, 16, 3
    assert rw(ctypes.byref(c), None, 7, 16, 2, None) == hn.HN_ERR_INVALID
    assert rw(ctypes.byref(c), None, 6, 20, 2, None) == hn.HN_ERR_INVALID
    assert rw(ctypes.byref(c), None, 4, 16, 3, None) == hn.HN_ERR_INVALID   # same segments, other frames
    # the window of frames_seen = 2 is frames [0, 2), no longer in the ring
    # (it holds [2, 6)) and not archived
    assert rw(ctypes.byref(c), None, 2, 8, 1, None) == hn.HN_ERR_CAPACITY
    assert (c.frames_seen, c.head_tokens, c.segments) == (6, 16, 3)
    # a target whose window the ring still holds needs no archive
    assert rw(ctypes.byref(c), None, 6, 16, 3, None) == hn.HN_OK
    c.frames_seen, c.segments = 3, 2      # window [0, 3) with W = 4: all in the ring
    assert rw(ctypes.byref(c), None, 2, 8, 1, None) == hn.HN_OK
    assert (c.frames_seen, c.head_tokens, c.segments) == (2, 8, 1)


def test_camera_checks():
    s = seg_c()
    cam = hn._lib.hn_camera_attn_fwd
    args = [FAKE, FAKE, FAKE, FAKE, None]   # q, k_cam, v_cam, o, lse
    assert cam(None, 2, 0, *args, 0.1, None) == hn.HN_ERR_NULL
    assert cam(ctypes.byref(s.c), 0, 0, *args, 0.1, None) == hn.HN_ERR_INVALID
    assert cam(ctypes.byref(s.c), 2, -1, *args, 0.1, None) == hn.HN_ERR_INVALID
    assert cam(ctypes.byref(s.c), 2, 0, *args, float("inf"), None) == hn.HN_ERR_INVALID
    assert cam(ctypes.byref(s.c), 2, 0, FAKE, None, FAKE, FAKE, None, 0.1, None) == hn.HN_ERR_NULL
    # (token, head) rows are numbered in 28 bits: 1,024 frames x 16,384 tokens
    # x 16 heads = 2^28 rows is refused before any launch
    big = hn.SegLayout(0, 1024, 16384, 0, [], [], [])
    assert cam(ctypes.byref(big.c), 16, 0, *args, 0.1, None) == hn.HN_ERR_UNSUPPORTED
    assert "2^28" in hn.hn_last_error()


def test_attention_rejects_sources_over_2gib():
    """Every key/value source is addressed with 32-bit buffer offsets: a video
    source of more than 2 GiB (here 600 frames x 880 tokens x 16 heads x 256 B)
    is refused before anything is enqueued."""
    c = fake_cache(H=16, P=880, W=18, cap=0)
    F, P = 600, 880
    s = hn.SegLayout(0, F, P, 0, [], [], [])
    fwd = hn._lib.hn_seg_attn_fwd
    for rows in (128, 256):
        plan = hn.hn_tile_plan(dev=FAKE, tile_q=rows, n_qtiles=-(-F * P // rows), n_text_tiles=0,
                               max_spans=4, n_splits=1, n_splits_text=1, visible_pairs=-1)
        st = fwd(ctypes.byref(c), ctypes.byref(s.c), ctypes.byref(plan), FAKE, None, None, None,
                 FAKE, FAKE, FAKE, None, None, None, 0.1, None)
        if st != hn.HN_ERR_ORDER:          # the plan height the library uses
            assert st == hn.HN_ERR_UNSUPPORTED
            break
    else:
        raise AssertionError("no plan height accepted")


def test_text_tiles_split_separately():
    """Text query tiles get their own split count: forced to 4 with video tiles
    unsplit, the partial results cover only the text tiles."""
    c = fake_cache()
    s = seg_c()
    n1 = ws_size(c, s)
    n4 = ws_size(c, s, n_splits_text=4)
    a256 = lambda b: -(-b // 256) * 256
    vt = 1 + 4                                 # video tile unsplit + text tile x 4
    spans = a256(a256(vt * 4) + vt * 6 * 32)
    fits = [R for R in (64, 128, 256, 512)
            if n4 == spans + a256(2 * 4 * R * 128 * 4) + a256(2 * 4 * R * 4)]   # 4 text slots per head
    assert len(fits) == 1 and n4 > n1
