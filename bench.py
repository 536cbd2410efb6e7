"""Benchmark of the segment-attention hot path on one MI355X.

One step = one pass of the hot path over one segment of the 480x832 workload
(16 heads x 128 dims, 30 latent frames x 390 tokens = 11,700 video queries,
768-token description head + 4 action tails of 128 tokens, no history):
    hn_attn_mask_build (tile plan) -> hn_seg_attn_fwd -> hn_kv_quant_append.
Inputs are seeded synthetic bf16 N(0,1) tensors already resident in HBM.

value = effective attention FLOPs of the step / step time, where effective
FLOPs count only unmasked (query, key) pairs: 4 * D per pair per head
(Q K^T and P V multiply-adds).  The roofline object reports the attention
kernel alone (HIP events around each launch on its stream) against the bf16
dense MFMA peak; the append object reports the quantize/append kernel's
bytes (776 per (token, head): 512 read, 256 INT8 + 8 scale bytes written)
against 8 TB/s, with rotating buffers so the bytes come from HBM, timed as
launches back to back between one pair of events (each launch's own event
pair is reported beside it).
cpu_baseline times the fp64 CPU oracle on a sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TFLOP/s (unmasked pairs) + % bf16 MFMA peak; KV append GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
APPEND_BYTES_PER_ROW = 2 * 128 * 2 + 2 * 128 + 2 * 4   # 776


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps; the clock ramps over the first ~50 ms of work")
    ap.add_argument("--workload", default="c2", help="c2 (default), c3, c4 or c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="query rows the oracle computes (default: about 10-30 s of CPU work)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the joint, camera and archive measurements (counter runs)")
    ap.add_argument("--splits", type=int, default=0,
                    help="key splits per video query tile (0 = the library's automatic choice)")
    ap.add_argument("--text-splits", type=int, default=0,
                    help="key splits per text query tile (0 = automatic)")
    ap.add_argument("--whole-tiles", type=int, default=0,
                    help="with --splits > 1: leading video query tiles left unsplit (0 = every tile split)")
    ap.add_argument("--tile-rows", type=int, default=0,
                    help="query rows per tile of a plan without keep list: 128, 256 or 384 (0 = automatic)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


KERNEL_SOURCES = ("masked_attention_hn_amd/csrc/attn_fwd.hip", "masked_attention_hn_amd/csrc/hn_internal.h")
COUNTERS = os.path.join(ROOT, "profiles", "seg_attn_fwd_c2_counters.json")


def normalize_source(src):
    """C++ source text with comments removed and whitespace collapsed."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_sources_sha256():
    """SHA-256 of the attention kernel's normalized sources, so that only a
    change of code invalidates stored counters."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            h.update(normalize_source(fh.read()).encode())
    return h.hexdigest()


def counter_traffic(workload):
    """HBM bytes per attention launch from the stored FETCH_SIZE/WRITE_SIZE
    counters, each scaled by what the counter reads for a plain 1 GiB device
    copy; None when the counters were taken on other kernel sources or
    another workload."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as fh:
        c = json.load(fh)
    if c["workload"] != workload or c["kernel_sources_sha256"] != kernel_sources_sha256():
        return None
    gib_kib = float(1 << 20)
    fetch = c["fetch_kib"] * gib_kib / c["copy_1gib_fetch_kib"]
    write = c["write_kib"] * gib_kib / c["copy_1gib_write_kib"]
    return round((fetch + write) * 1024)


def max_engine_clock_mhz():
    """Highest engine clock level the amdgpu driver lists for an AMD card
    (sysfs pp_dpm_sclk), or None where it cannot be read."""
    import glob
    import re
    best = None
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(os.path.join(os.path.dirname(f), "vendor")) as fh:
                if fh.read().strip() != "0x1002":
                    continue
            with open(f) as fh:
                mhz = [int(m) for m in re.findall(r"(\d+)\s*[Mm]hz", fh.read())]
        except OSError:
            continue
        if mhz:
            best = max(mhz) if best is None else max(best, max(mhz))
    return best


def device_info():
    """The GPU the line was measured on, and what its bf16 peak assumes."""
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "max_engine_clock_mhz": max_engine_clock_mhz(),
            "peak_basis": "published MI355X dense bf16 MFMA 2.5 PFLOP/s (256 CUs at 2.4 GHz); HBM 8 TB/s"}


def visible_pairs_text(w):
    """Unmasked (text query, key) pairs per head, from the layout (no oracle):
    every text row sees earlier heads, kept history video, its own head and
    video; a tail row also sees its own tail."""
    S = w.query_segment
    cur = w.current
    g0 = sum(s.frames for s in w.segments[:S])
    kept = g0 if w.window is None else min(g0, w.window)
    base = sum(s.head_len for s in w.segments[:S]) + kept * cur.tokens_per_frame \
        + cur.head_len + cur.video_len
    return cur.text_len * base + sum(a * a for a in cur.action_len)


def visible_pairs(w, csr=None):
    """Unmasked (query, key) pairs per head, from the layout (no oracle)."""
    S = w.query_segment
    cur = w.current
    P = cur.tokens_per_frame
    g0 = sum(s.frames for s in w.segments[:S])
    kept = g0 if w.window is None else min(g0, w.window)
    hist_heads = sum(s.head_len for s in w.segments[:S])
    if csr is None:
        tot = 0
        for f in range(cur.frames):
            n = hist_heads + kept * P + cur.head_len + cur.video_len
            n += sum(a for a, f0, f1 in zip(cur.action_len, cur.action_f0, cur.action_f1) if f0 <= f < f1)
            tot += n * P
        return tot
    # block-sparse: text + kept video tiles
    n_hist_tiles = -(-kept * P // 128)
    def tile_len(c):
        if c < n_hist_tiles:
            return min(128, kept * P - c * 128)
        c -= n_hist_tiles
        return min(128, cur.video_len - c * 128)
    tot = 0
    for r in range(cur.video_len):
        f = r // P
        t = r // 128
        n = hist_heads + cur.head_len
        n += sum(a for a, f0, f1 in zip(cur.action_len, cur.action_f0, cur.action_f1) if f0 <= f < f1)
        cols = csr["col"][csr["row_ptr"][t]:csr["row_ptr"][t + 1]]
        n += sum(tile_len(int(c)) for c in cols)
        tot += n
    return tot


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the method shards by attention head with no exchange inside the path)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not os.path.exists(os.path.join(ROOT, "masked_attention_hn_amd", "libhn.so")):
        import __graft_entry__
        __graft_entry__.build()
    import masked_attention_hn_amd as hn
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 3}))
        return

    w = W.config(args.workload)
    data = W.generate(w)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    def lay(i, s):
        return hn.SegLayout(i, s.frames, s.tokens_per_frame, s.head_len, s.action_len,
                            s.action_f0, s.action_f1)

    cache = hn.KVCache(w.heads, w.current.tokens_per_frame, w.ring_frames, w.head_cap)
    for s in range(w.query_segment):
        x = data["segments"][s]
        hn.hn_kv_quant_append(cache, lay(s, w.segments[s]), to_dev(x["k_txt"]), to_dev(x["v_txt"]),
                              to_dev(x["k_vid"]), to_dev(x["v_vid"]))
    S = w.query_segment
    seg = lay(S, w.current)
    x = data["segments"][S]
    k_txt, v_txt, k_vid, v_vid = (to_dev(x[n]) for n in ("k_txt", "v_txt", "k_vid", "v_vid"))
    q = to_dev(data["q_vid"])
    o = torch.empty_like(q)
    sparse = None
    csr = None
    if w.sparse_keep is not None:
        csr = data["csr"]
        sparse = hn.BlockSparse(torch.from_numpy(csr["row_ptr"]), torch.from_numpy(csr["col"]),
                                csr["n_qtiles"])
    opts = hn.PlanOpts(n_splits=args.splits, n_splits_text=args.text_splits, tile_rows=args.tile_rows,
                       whole_tiles=args.whole_tiles)
    ws = torch.empty(hn.hn_attn_workspace_size(cache, seg, sparse, opts), dtype=torch.uint8, device=dev)
    plan_c = hn.hn_tile_plan()
    plan = hn.Plan(ws, plan_c)
    saved = (cache.c.frames_seen, cache.c.head_tokens, cache.c.segments)
    pairs = visible_pairs(w, csr)
    flops = 4.0 * 128 * pairs * w.heads

    # one call on the cache as the history left it, before any step appends
    # (each step re-appends this segment, which in a full window overwrites
    # the oldest history frames: same work, other data), kept for the CPU
    # leg's parity check
    o_check = torch.empty_like(q)
    hn.hn_attn_mask_build(cache, seg, sparse, hn.HN_MASK_TILE_PLAN, 0, 0, ws, plan_c, opts=opts)
    hn.hn_seg_attn_fwd(cache, seg, plan, q, k_txt, v_txt, k_vid, v_vid, o_check)

    ev_a0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None, timed=False):
        cache.c.frames_seen, cache.c.head_tokens, cache.c.segments = saved
        hn.hn_attn_mask_build(cache, seg, sparse, hn.HN_MASK_TILE_PLAN, 0, 0, ws, plan_c, opts=opts)
        if timed:
            ev_a0[i].record(stream)
        hn.hn_seg_attn_fwd(cache, seg, plan, q, k_txt, v_txt, k_vid, v_vid, o)
        if timed:
            ev_a1[i].record(stream)
        hn.hn_kv_quant_append(cache, seg, k_txt, v_txt, k_vid, v_vid)

    # the engine clock ramps up over the first ~50 ms of sustained work: before
    # the counted warm-up steps, run the same step untimed for 0.25 s of wall
    # time so that a short --warmup still times the steady state (reported as
    # clock_prewarm_steps)
    prewarm = 0
    tp = time.perf_counter()
    while time.perf_counter() - tp < 0.25:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        prewarm += 10
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in zip(ev_a0, ev_a1)]
    attn_avg = sum(attn_ms) / len(attn_ms)
    achieved = flops / (attn_avg * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    if plan_c.visible_pairs >= 0:
        assert plan_c.visible_pairs == pairs, (plan_c.visible_pairs, pairs)

    def time_append(cur, kv, window, heads):
        """Median time of the quantize/append kernel alone on segment shape
        cur (appended as segment 0 into an empty cache with a window of
        `window` frames), rotating input and cache buffers over > 600 MB (more
        than the 256 MB MALL) so that every launch reads and writes HBM."""
        surv = min(cur.frames, window)
        nbytes = (cur.head_len + surv * cur.tokens_per_frame) * heads * APPEND_BYTES_PER_ROW
        n_sets = max(3, math.ceil(600e6 / max(1, nbytes)))
        sets = []
        for r in range(n_sets):
            c = hn.KVCache(heads, cur.tokens_per_frame, window, max(1, cur.head_len))
            sets.append((c, [t.clone() for t in kv]))
        seg0 = lay(0, cur)
        for c, kvs in sets:
            hn.hn_kv_quant_append(c, seg0, *kvs)
            hn.hn_kv_cache_reset(c)
        torch.cuda.synchronize()
        reps = 4 * n_sets
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            c, kvs = sets[i % n_sets]
            hn.hn_kv_cache_reset(c)
            e0[i].record(stream)
            hn.hn_kv_quant_append(c, seg0, *kvs)
            e1[i].record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in zip(e0, e1))[reps // 2]
        # the same launches back to back between one pair of events: each
        # per-launch pair above also times its own recording (~5 us, 7% of a
        # 70 us launch); this figure carries only the gaps between launches
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb0.record(stream)
        for i in range(reps):
            c, kvs = sets[i % n_sets]
            hn.hn_kv_cache_reset(c)
            hn.hn_kv_quant_append(c, seg0, *kvs)
        eb1.record(stream)
        torch.cuda.synchronize()
        ms_b = eb0.elapsed_time(eb1) / reps
        del sets
        gbs = nbytes / (ms_b * 1e-3) / 1e9
        return {
            "kernel": "quant_append_kernel",
            "bound": "hbm",
            "rows": (cur.head_len + surv * cur.tokens_per_frame) * heads,
            "bytes": nbytes,
            "ms_per_launch": round(ms_b, 4),
            "timing": f"{reps} launches back to back over the rotating sets, one event pair",
            "median_ms_own_events": round(ms, 4),
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "rotating_sets": n_sets,
        }

    append = time_append(w.current, (k_txt, v_txt, k_vid, v_vid), w.ring_frames, w.heads)
    append["shape"] = f"this workload's segment ({args.workload})"
    # the 1280x704 segment with no window (30 frames x 880 tokens + 768-token
    # head, 16 heads: 337 MB), seeded N(0,1) bf16 drawn on the device
    big = W.config("c4").current
    if w.heads == 16 and (w.current.frames, w.current.tokens_per_frame, w.current.head_len,
                          w.ring_frames >= big.frames) == (big.frames, big.tokens_per_frame,
                                                           big.head_len, True):
        append_big = dict(append)
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(1280704)
        mk = lambda n: torch.randn((n, 16, 128), generator=g, device=dev).to(torch.bfloat16)
        kv_big = (mk(big.text_len), mk(big.text_len), mk(big.video_len), mk(big.video_len))
        append_big = time_append(big, kv_big, big.frames, 16)
        del kv_big
    append_big["shape"] = "1280x704 segment, no window: (768 + 30 x 880) tokens x 16 heads"

    def time_copy(nbytes):
        """A plain device copy (torch) moving the same bytes (half read, half
        written), rotating buffers over > 600 MB, launches back to back: what
        HBM delivers to a copy of this size, the reference for the append."""
        half = nbytes // 2
        n_sets = max(3, math.ceil(600e6 / nbytes))
        src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        for a, b in zip(src, dst):
            b.copy_(a)
        torch.cuda.synchronize()
        reps = 4 * n_sets
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(reps):
            dst[i % n_sets].copy_(src[i % n_sets])
        c1.record(stream)
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / reps
        return {"bytes": 2 * half, "ms_per_launch": round(ms, 4),
                "achieved": round(2 * half / (ms * 1e-3) / 1e9, 1), "unit": "GB/s"}

    append_big["plain_copy_same_bytes"] = time_copy(append_big["bytes"])

    traffic = counter_traffic(args.workload)

    # camera cross-attention: each video token attends to the camera tokens of
    # its segment within `radius` latent frames of its own.  Radius 0 reduces
    # to a copy of the frame's camera value (one key, weight 1); radius 1 (up
    # to 3 keys) exercises the scores and the softmax.  Rotating query/output
    # sets over 600 MB so the bytes come from HBM.
    camera = None
    k_cam, v_cam = to_dev(data["k_cam"]), to_dev(data["v_cam"])
    cam_rows = w.current.video_len * w.heads
    cam_bytes = cam_rows * (128 * 2 * 2 + 4)
    n_cam = 0 if args.no_extras else max(3, math.ceil(600e6 / cam_bytes))
    cam_sets = [(q.clone(), torch.empty_like(q),
                 torch.empty((w.heads, w.current.video_len), dtype=torch.float32, device=dev))
                for _ in range(n_cam)]

    def time_camera(radius):
        for qq, oo, ll in cam_sets:
            hn.hn_camera_attn_fwd(seg, w.heads, radius, qq, k_cam, v_cam, oo, ll)
        torch.cuda.synchronize()
        reps = 4 * n_cam
        ec0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        ec1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            qq, oo, ll = cam_sets[i % n_cam]
            ec0[i].record(stream)
            hn.hn_camera_attn_fwd(seg, w.heads, radius, qq, k_cam, v_cam, oo, ll)
            ec1[i].record(stream)
        torch.cuda.synchronize()
        med = sorted(a.elapsed_time(b) for a, b in zip(ec0, ec1))[reps // 2]
        # back to back between one event pair (as for the append)
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb0.record(stream)
        for i in range(reps):
            qq, oo, ll = cam_sets[i % n_cam]
            hn.hn_camera_attn_fwd(seg, w.heads, radius, qq, k_cam, v_cam, oo, ll)
        eb1.record(stream)
        torch.cuda.synchronize()
        return eb0.elapsed_time(eb1) / reps, med, reps

    if n_cam:
        cam_ms, cam_med, cam_reps = time_camera(1)
        cam0_ms, cam0_med, _ = time_camera(0)
        camera = {
            "kernel": "camera_attn_kernel",
            "what": "video tokens x heads attending to the camera tokens within 1 latent frame "
                    "of their own (up to 3 keys; O, LSE written)",
            "bound": "hbm",
            "bytes": cam_bytes,
            "ms_per_launch": round(cam_ms, 4),
            "timing": f"{cam_reps} launches back to back over the rotating sets, one event pair",
            "median_ms_own_events": round(cam_med, 4),
            "achieved": round(cam_bytes / (cam_ms * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(cam_bytes / (cam_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "radius0_ms_per_launch": round(cam0_ms, 4),
            "radius0_median_ms_own_events": round(cam0_med, 4),
            "radius0_achieved": round(cam_bytes / (cam0_ms * 1e-3) / 1e9, 1),
        }
    del cam_sets

    # history archive: evict (device -> pinned host) the frames the append of
    # this segment pushes out of the window, append, then rewind (host ->
    # device) to the state before it; repeated, each copy timed on the stream
    archive = None
    if w.window is not None and saved[0] >= w.window and not args.no_extras:
        P = w.current.tokens_per_frame
        ar = hn.KVArchive(w.heads, P, saved[0] + w.current.frames)
        n_ar = 6
        ed = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ar)]
        eh = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ar)]
        for i in range(n_ar):
            cache.c.frames_seen, cache.c.head_tokens, cache.c.segments = saved
            ar.c.frames = 0
            ed[i][0].record(stream)
            hn.hn_kv_archive_evict(cache, seg, ar)
            ed[i][1].record(stream)
            hn.hn_kv_quant_append(cache, seg, k_txt, v_txt, k_vid, v_vid)
            eh[i][0].record(stream)
            hn.hn_kv_cache_rewind(cache, ar, *saved)
            eh[i][1].record(stream)
        torch.cuda.synchronize()
        n_frames = min(w.current.frames, w.window)
        ar_bytes = n_frames * P * w.heads * (2 * 128 + 2 * 4)
        d2h = sorted(a.elapsed_time(b) for a, b in ed)[n_ar // 2]
        h2d = sorted(a.elapsed_time(b) for a, b in eh)[n_ar // 2]
        archive = {
            "what": "history frames leaving the window: device -> pinned host on append, "
                    "host -> device on rewind (median of 6)",
            "frames": n_frames,
            "bytes": ar_bytes,
            "d2h_ms": round(d2h, 4),
            "d2h_GBps": round(ar_bytes / (d2h * 1e-3) / 1e9, 2),
            "h2d_ms": round(h2d, 4),
            "h2d_GBps": round(ar_bytes / (h2d * 1e-3) / 1e9, 2),
        }
        cache.c.frames_seen, cache.c.head_tokens, cache.c.segments = saved

    # the same call with the segment's text queries added (one launch for both)
    joint = None
    if w.current.text_len > 0 and not args.no_extras:
        cache.c.frames_seen, cache.c.head_tokens, cache.c.segments = saved
        hn.hn_attn_mask_build(cache, seg, sparse, hn.HN_MASK_TILE_PLAN, 0, 0, ws, plan_c, opts=opts)
        q_txt = to_dev(data["q_txt"])
        o_txt = torch.empty_like(q_txt)
        pairs_t = visible_pairs_text(w)
        assert plan_c.visible_pairs_text == pairs_t, (plan_c.visible_pairs_text, pairs_t)
        n_j = max(10, args.steps // 4)
        ej0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_j)]
        ej1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_j)]
        for i in range(n_j):
            ej0[i].record(stream)
            hn.hn_seg_attn_fwd(cache, seg, plan, q, k_txt, v_txt, k_vid, v_vid, o,
                               q_txt=q_txt, o_txt=o_txt)
            ej1[i].record(stream)
        torch.cuda.synchronize()
        j_ms = sum(a.elapsed_time(b) for a, b in zip(ej0, ej1)) / n_j
        j_flops = 4.0 * 128 * (pairs + pairs_t) * w.heads
        joint = {
            "what": "video + text-stream queries in one hn_seg_attn_fwd launch",
            "text_queries": w.current.text_len,
            "visible_pairs_text_per_head": pairs_t,
            "effective_flop": j_flops,
            "avg_launch_ms": round(j_ms, 4),
            "achieved": round(j_flops / (j_ms * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s",
            "frac": round(j_flops / (j_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        }

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_prewarm_steps": prewarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": {
                "c2": "480x832 single segment: 16 heads x 128, 30 latent frames x 390 tokens "
                      "= 11,700 video queries, 768-token head + 4 x 128-token action tails, no history",
                "c3": "1280x704 steady state: 26,400 queries, INT8 ring of 18 frames (15,840 tokens) "
                      "+ 3 x 768 cached heads, own 768 + 4 x 128 text",
                "c4": "1280x704 7th segment, no window: 26,400 queries, INT8 history of 158,400 video "
                      "tokens + 6 x 1,280 heads, Student-t keys/values",
                "c5": "480x832 single segment, block-sparse: 25% of video tiles kept per query tile",
            }.get(args.workload, args.workload),
            "name": args.workload,
            "step": "tile plan + attention + INT8 quantize/append",
            "key_splits": args.splits or "automatic",
            "key_splits_text": args.text_splits or "automatic",
            "tile_rows": args.tile_rows or "automatic",
            "whole_tiles": args.whole_tiles if args.splits else "automatic",
            # what the plan of the timed launch took (text splits: of the joint launch)
            "plan": {"tile_rows": plan_c.tile_q, "key_splits": plan_c.n_splits,
                     "whole_tiles": plan_c.n_whole, "key_splits_text": plan_c.n_splits_text},
            "effective_flop_per_step": flops,
            "visible_pairs_per_head": pairs,
        },
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "device": device_info(),
        "roofline": {
            "kernel": "seg_attn_fwd_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(attn_avg, 4),
        },
        "memory": {
            "cache_bytes": sum(t.numel() * t.element_size() for t in (
                cache.ring_k, cache.ring_v, cache.ring_ks, cache.ring_vs,
                cache.heads_k, cache.heads_v, cache.heads_ks, cache.heads_vs)),
            "plan_workspace_bytes": ws.numel(),
            "peak_allocated_bytes": torch.cuda.max_memory_allocated(),
        },
        "joint": joint,
        "archive": archive,
        "camera": camera,
        "append": append,
        "append_1280x704": append_big,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        import oracle
        n_rows = args.cpu_rows or {"c3": 128, "c4": 64, "c3_h2": 1024}.get(args.workload, 11700)
        rows = np.linspace(0, w.current.video_len - 1, min(n_rows, w.current.video_len)).astype(int)
        rows = np.unique(rows)
        tc0 = time.perf_counter()
        ref, _, _ = oracle.attention(w, data, rows)
        tc = time.perf_counter() - tc0
        # the same rows of the GPU output against it (max-abs 2e-2, plus half a
        # bf16 ulp where |O_ref| >= 8; mean-abs 2e-3)
        got = o_check.float().cpu().numpy()[rows]
        err = np.abs(got - ref)
        half_ulp = np.where(np.abs(ref) >= 8.0,
                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8), 0.0)
        parity = {
            "rows": int(len(rows)),
            "max_abs": float(f"{err.max():.4e}"),
            "mean_abs": float(f"{err.mean():.4e}"),
            "within_bar": bool((err <= 2e-2 + half_ulp).all() and err.mean() <= 2e-3),
        }
        if csr is None:
            per_row = pairs / w.current.video_len
            sample_pairs = per_row * len(rows)
        else:
            sample_pairs = pairs * len(rows) / w.current.video_len
        cpu_tflops = 4.0 * 128 * sample_pairs * w.heads / tc / 1e12
        avail = len(os.sched_getaffinity(0))
        threads = 1
        try:
            import threadpoolctl
            blas = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
            if blas:
                threads = max(blas)
        except ImportError:
            pass
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as fh:
                for line in fh:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        out["cpu_baseline"] = {
            "value": round(cpu_tflops, 6),
            "unit": "TFLOP/s",
            "cores": min(threads, avail),
            "kind": "oracle",
            "cpu": cpu_model,
            "cores_available": avail,
            "gpu_parity": parity,
            "sample": f"{len(rows)} of {w.current.video_len} query rows (evenly spaced), all "
                      f"{w.heads} heads, fp64 numpy oracle incl. key preparation; {tc:.1f} s; "
                      "its products run on the BLAS threads, the rest on one thread",
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
