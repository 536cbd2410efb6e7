"""CPU oracle for action-aware segment-causal attention over an INT8 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs
this package; only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP path: it takes its inputs
from the seeded generators in ``workloads`` and computes everything itself,
plainly and slowly, in numpy.

What it computes, and the passages it follows (pages about Tencent's
Hy-Nomas world model):

* quantize(): INT8 storage of keys and values with float scale factors;
  quantization happens only on the storage side and attention runs in
  BF16 (fluxbbs teardown, "How one 4090 does it", first trick; clawpk news,
  "single 4090" section).  The pages give no formula; the reading used is one
  fp32 scale per (token, head) row of 128 values: scale = amax / 127 with an
  IEEE fp32 division, q = round-half-even(x / scale) with a correctly
  rounded fp32 quotient, clamped to [-127, 127]; an all-zero row gets
  scale 0 and q 0.  Dequantized value = q * scale (exact in fp64).

* mask(): the visibility of every token of the whole multi-segment sequence
  for a video query of the query segment, written out as an explicit boolean
  matrix:
    - segment-causal: bidirectional inside a segment, and a segment sees
      only itself and earlier segments (fluxbbs teardown, "Architecture",
      first stage; continued-pretraining stage of "Training");
    - action-aware: each segment's text is a description head, visible
      across segments, plus action tails that are visible only inside their
      own segment and time window (fluxbbs teardown, "Architecture", second
      stage; papers.ananclaw guide, "What it is", method paragraph);
    - sliding window: at most W latent frames of history video are kept
      (fluxbbs teardown, second trick; hyphentech explainer, table row on
      history context); the window limits history only, never the current
      segment (hyphentech explainer, warning under the table);
    - optional block sparsity: later denoising steps keep only 25% of the
      candidate video blocks (fluxbbs teardown, fourth trick).
  Readings where the pages are silent: tail windows are half-open
  [f0, f1) in local latent frames and overlap by OR; the window keeps video
  frames whose global index is >= (first frame of the query segment) - W;
  heads of every earlier segment stay visible.

* mask_text(): the same visibility for the query segment's text-stream
  queries (its head and tail tokens; the MMDiT attends text and video
  jointly).  The segment-causal rule holds for them as stated (own segment
  and earlier ones only, earlier video inside the window); the pages give
  tails' time windows only in terms of video frames, so the reading for
  text queries is: a tail token sees its own tail and no other, a head token
  sees no tail (an action description never reaches the head that later
  segments keep).  Keep lists concern video query tiles only, so text
  queries attend densely.

* evicted_frames() / archive_of(): the single-GPU configuration keeps at most
  W history frames on the GPU and archives earlier history to CPU memory
  (hyphentech explainer, configuration table, history row; fluxbbs teardown,
  second trick for the 18-frame window).  Appending F frames to a cache that
  has seen fs frames keeps the last min(fs + F, W) of all frames; the frames
  that leave the window are the archived ones, oldest first, each stored as
  the same INT8 codes and scales the cache held.

* camera_attention(): each latent frame has one camera token (four frame
  poses folded into a 64-dimensional vector and projected), and in every
  block the video tokens read, by cross-attention, the time-aligned camera
  tokens of their own segment (fluxbbs teardown, "Architecture", camera
  paragraph; papers.ananclaw guide, "What it is": the extrinsics
  cross-attention path).  The projections need trained weights, so the
  camera tokens' keys and values are inputs.  Reading of "time-aligned": a
  video token at latent frame f sees the camera tokens of frames f' of its
  segment with |f' - f| <= radius; radius 0 (its own frame's token only) is
  the pages' statement, larger radii a generalization.

* attention(): plain softmax attention in fp64 per head over the masked
  full sequence: s = (q . k) * sm_scale, masked scores are -inf,
  p = exp(s - max) / sum, o = sum p v.  Keys and values of earlier segments
  are the dequantized INT8 values; the query segment's own keys, values and
  queries are its bf16 values widened to fp64 (quantization is storage-only).

Every function above is pinned outside itself by tests/: hand-derived and
exact-rational quantizer values, closed-form visible-key counts, a pure-Python
brute force, closed forms of attention and a library SDPA special case.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

from workloads import TILE, Workload, bf16_bits_to_f32

HEAD, TAIL, VIDEO = 0, 1, 2


# ---------------------------------------------------------------- quantizer
def quantize(x_bits: np.ndarray):
    """INT8 quantization of bf16 rows (last axis = one (token, head) row).

    Returns (q int8 [..., D], scale float32 [...]).  All arithmetic is IEEE
    float32 as numpy performs it: |x| and max are exact, the two divisions are
    correctly rounded, np.rint rounds half to even.
    """
    x = bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(y), -127, 127)
    q[zero] = 0
    scale = np.where(zero, np.float32(0.0), scale).astype(np.float32)
    return q.astype(np.int8), scale


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return q.astype(np.float64) * scale.astype(np.float64)[..., None]


# ------------------------------------------------------------- token table
def token_table(w: Workload) -> Dict[str, np.ndarray]:
    """Attributes of every token of every segment, in sequence order.

    Within a segment: description head, action tails in order, then video
    frame-major.  gframe is the global latent frame: the frames of all
    earlier segments plus the local frame.  src/row say where the token's
    K and V live in that segment's inputs (0 = text rows, 1 = video rows).
    """
    parts = []
    g = 0
    for s, seg in enumerate(w.segments):
        nt, nv = seg.text_len, seg.video_len
        kind_t = np.full(nt, HEAD, dtype=np.int64)
        tail_t = np.full(nt, -1, dtype=np.int64)
        r = seg.head_len
        for j, a in enumerate(seg.action_len):
            kind_t[r:r + a] = TAIL
            tail_t[r:r + a] = j
            r += a
        lf = np.repeat(np.arange(seg.frames, dtype=np.int64), seg.tokens_per_frame)
        parts.append({
            "seg": np.full(nt + nv, s, dtype=np.int64),
            "kind": np.concatenate([kind_t, np.full(nv, VIDEO, dtype=np.int64)]),
            "tail": np.concatenate([tail_t, np.full(nv, -1, dtype=np.int64)]),
            "lframe": np.concatenate([np.full(nt, -1, dtype=np.int64), lf]),
            "gframe": np.concatenate([np.full(nt, -1, dtype=np.int64), g + lf]),
            "src": np.concatenate([np.zeros(nt, np.int64), np.ones(nv, np.int64)]),
            "row": np.concatenate([np.arange(nt, dtype=np.int64), np.arange(nv, dtype=np.int64)]),
        })
        g += seg.frames
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def _first_frame(w: Workload, s: int) -> int:
    return sum(seg.frames for seg in w.segments[:s])


# ----------------------------------------------------------------- archive
def evicted_frames(frames_seen: int, frames: int, window: int):
    """Global latent frames [g0, g1) that leave a W-frame window when `frames`
    new frames are appended after `frames_seen`: the window held
    [fs - min(fs, W), fs) and holds [fs + F - min(fs + F, W), fs + F) after."""
    kept_before = min(frames_seen, window)
    kept_after = min(frames_seen + frames, window)
    g0 = frames_seen - kept_before
    g1 = max(g0, min(frames_seen, frames_seen + frames - kept_after))
    return g0, g1


def archive_of(w: Workload, data: dict, upto: int):
    """INT8 codes and scales of every history frame evicted while segments
    0 .. upto-1 are appended, in global frame order: (k, v, ks, vs) with
    shapes [frames][P][H][D] int8 and [frames][P][H] float32."""
    P = w.segments[0].tokens_per_frame
    ks, vs, kss, vss = [], [], [], []
    fs = 0
    frames_src = []  # (segment, local frame) of every global frame
    for s in range(upto):
        seg = w.segments[s]
        g0, g1 = evicted_frames(fs, seg.frames, w.ring_frames)
        for g in range(g0, g1):
            sg, f = frames_src[g]
            rows = slice(f * P, (f + 1) * P)
            qk, sk = quantize(data["segments"][sg]["k_vid"][rows])
            qv, sv = quantize(data["segments"][sg]["v_vid"][rows])
            ks.append(qk); vs.append(qv); kss.append(sk); vss.append(sv)
        frames_src += [(s, f) for f in range(seg.frames)]
        fs += seg.frames
    if not ks:
        H, D = w.heads, w.head_dim
        return (np.zeros((0, P, H, D), np.int8), np.zeros((0, P, H, D), np.int8),
                np.zeros((0, P, H), np.float32), np.zeros((0, P, H), np.float32))
    return np.stack(ks), np.stack(vs), np.stack(kss), np.stack(vss)


# -------------------------------------------------------------------- mask
def mask(w: Workload, rows: Optional[Sequence[int]] = None,
         csr: Optional[dict] = None, tab: Optional[dict] = None) -> np.ndarray:
    """Explicit boolean visibility [len(rows)][L] over the full sequence.

    rows index the video queries of the query segment (frame-major).  csr is
    the optional block-sparse keep list (query tiles and video key tiles of
    TILE tokens; video tiles number the kept history video oldest frame first,
    then the query segment's own video).  tab is token_table(w), if already built.
    """
    if tab is None:
        tab = token_table(w)
    S = w.query_segment
    cur = w.current
    P = cur.tokens_per_frame
    nq = cur.video_len
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    fq = rows // P  # local latent frame of each query
    g0 = _first_frame(w, S)

    seg, kind, tail, gframe = tab["seg"], tab["kind"], tab["tail"], tab["gframe"]
    earlier = seg < S
    same = seg == S
    if w.window is None:
        in_window = np.ones_like(earlier)
    else:
        in_window = gframe >= g0 - w.window

    # rules that do not depend on the query row
    col_vis = (earlier & (kind == HEAD)) | (earlier & (kind == VIDEO) & in_window) \
        | (same & (kind == HEAD)) | (same & (kind == VIDEO))
    vis = np.broadcast_to(col_vis, (len(rows), len(seg))).copy()

    # own action tails: visible iff the query's local frame is in [f0, f1)
    f0 = np.asarray(cur.action_f0, dtype=np.int64)
    f1 = np.asarray(cur.action_f1, dtype=np.int64)
    own_tail = same & (kind == TAIL)
    idx = np.nonzero(own_tail)[0]
    if len(idx):
        j = tail[idx]
        ok = (f0[j][None, :] <= fq[:, None]) & (fq[:, None] < f1[j][None, :])
        vis[:, idx] = ok

    if csr is not None:
        # video keys outside the query tile's kept list become invisible
        hist_frames = g0 if w.window is None else min(g0, w.window)
        first_hist = g0 - hist_frames
        vid_tile = np.full(len(seg), -1, dtype=np.int64)
        hv = earlier & (kind == VIDEO) & in_window
        pos = (gframe[hv] - first_hist) * P + (tab["row"][hv] % P)
        vid_tile[hv] = pos // TILE
        n_hist_tiles = -(-hist_frames * P // TILE)
        ov = same & (kind == VIDEO)
        vid_tile[ov] = n_hist_tiles + tab["row"][ov] // TILE
        rp = np.asarray(csr["row_ptr"])
        col = np.asarray(csr["col"])
        qt = rows // TILE
        is_vid = kind == VIDEO
        n_ids = int(max(vid_tile.max(), col.max() if len(col) else 0)) + 2
        for i, t in enumerate(qt):
            kept = np.zeros(n_ids, dtype=bool)
            kept[col[rp[t]:rp[t + 1]]] = True
            keep_col = ~is_vid | ((vid_tile >= 0) & kept[np.maximum(vid_tile, 0)])
            vis[i] &= keep_col
    return vis


def mask_text(w: Workload, rows: Optional[Sequence[int]] = None,
              tab: Optional[dict] = None) -> np.ndarray:
    """Explicit boolean visibility [len(rows)][L] over the full sequence for
    text-stream queries: rows index the query segment's text tokens (head,
    then tails in order)."""
    if tab is None:
        tab = token_table(w)
    S = w.query_segment
    cur = w.current
    rows = np.arange(cur.text_len) if rows is None else np.asarray(rows, dtype=np.int64)
    g0 = _first_frame(w, S)

    # tail index of each query row (-1 for head rows)
    q_tail = np.full(cur.text_len, -1, dtype=np.int64)
    r = cur.head_len
    for j, a in enumerate(cur.action_len):
        q_tail[r:r + a] = j
        r += a
    qj = q_tail[rows]

    seg, kind, tail, gframe = tab["seg"], tab["kind"], tab["tail"], tab["gframe"]
    earlier = seg < S
    same = seg == S
    if w.window is None:
        in_window = np.ones_like(earlier)
    else:
        in_window = gframe >= g0 - w.window
    col_vis = (earlier & (kind == HEAD)) | (earlier & (kind == VIDEO) & in_window) \
        | (same & (kind == HEAD)) | (same & (kind == VIDEO))
    vis = np.broadcast_to(col_vis, (len(rows), len(seg))).copy()
    own_tail = same & (kind == TAIL)
    idx = np.nonzero(own_tail)[0]
    if len(idx):
        vis[:, idx] = (qj[:, None] >= 0) & (qj[:, None] == tail[idx][None, :])
    return vis


# ------------------------------------------------------------------ values
def key_values(w: Workload, data: dict):
    """Keys and values of the whole sequence as fp64 [L][H][D].

    Earlier segments contribute their dequantized INT8 values; the query
    segment and any later segment contribute bf16 values widened to fp64.
    """
    S = w.query_segment
    ks, vs = [], []
    for s, seg in enumerate(w.segments):
        d = data["segments"][s]
        for kname, vname in (("k_txt", "v_txt"), ("k_vid", "v_vid")):
            kb, vb = d[kname], d[vname]
            if s < S:
                ks.append(dequantize(*quantize(kb)))
                vs.append(dequantize(*quantize(vb)))
            else:
                ks.append(bf16_bits_to_f32(kb).astype(np.float64))
                vs.append(bf16_bits_to_f32(vb).astype(np.float64))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


# --------------------------------------------------------------- attention
def attention(w: Workload, data: dict, rows: Optional[Sequence[int]] = None,
              sm_scale: Optional[float] = None, chunk: int = 256,
              kv: Optional[tuple] = None, queries: str = "video"):
    """Masked softmax attention in fp64.

    queries: "video" (rows of Q_vid, mask()) or "text" (rows of Q_txt,
    mask_text()).  Returns (O [nrows][H][D], lse [H][nrows], rowsum
    [H][nrows]); lse is the natural log of sum(exp(s)) over visible keys,
    rowsum the sum of the normalized weights.
    """
    H, D = w.heads, w.head_dim
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if queries not in ("video", "text"):
        raise ValueError(queries)
    K, V = kv if kv is not None else key_values(w, data)
    Q = bf16_bits_to_f32(data["q_vid" if queries == "video" else "q_txt"]).astype(np.float64)
    nq = Q.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), H, D))
    lse = np.zeros((H, len(rows)))
    rsum = np.zeros((H, len(rows)))
    csr = data.get("csr") if w.sparse_keep is not None else None
    Kh = [np.ascontiguousarray(K[:, h, :]) for h in range(H)]
    Vh = [np.ascontiguousarray(V[:, h, :]) for h in range(H)]
    tab = token_table(w)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        vis = mask(w, r, csr, tab) if queries == "video" else mask_text(w, r, tab)
        for h in range(H):
            s = (Q[r, h, :] @ Kh[h].T) * sm_scale
            s = np.where(vis, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=1, keepdims=True)
            p = e / l
            O[c0:c0 + len(r), h, :] = p @ Vh[h]
            lse[h, c0:c0 + len(r)] = m[:, 0] + np.log(l[:, 0])
            rsum[h, c0:c0 + len(r)] = np.sum(p, axis=1)
    return O, lse, rsum


def camera_attention(w: Workload, data: dict, radius: int = 0,
                     sm_scale: Optional[float] = None):
    """Cross-attention of the query segment's video tokens to its camera
    tokens in fp64: query row r (latent frame f = r // P) sees camera tokens
    f' with |f' - f| <= radius.  Returns (O [rows][H][D], lse [H][rows])."""
    cur = w.current
    H, D, P, F = w.heads, w.head_dim, cur.tokens_per_frame, cur.frames
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    Q = bf16_bits_to_f32(data["q_vid"]).astype(np.float64)
    K = bf16_bits_to_f32(data["k_cam"]).astype(np.float64)
    V = bf16_bits_to_f32(data["v_cam"]).astype(np.float64)
    O = np.zeros((cur.video_len, H, D))
    lse = np.zeros((H, cur.video_len))
    for f in range(F):
        lo, hi = max(0, f - radius), min(F, f + radius + 1)
        rows = slice(f * P, (f + 1) * P)
        for h in range(H):
            s = (Q[rows, h, :] @ K[lo:hi, h, :].T) * sm_scale
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=1, keepdims=True)
            O[rows, h, :] = (e / l) @ V[lo:hi, h, :]
            lse[h, rows] = m[:, 0] + np.log(l[:, 0])
    return O, lse


def effective_flops_text(w: Workload) -> float:
    """4 * D * (visible (text query, key) pairs) * H."""
    return 4.0 * w.head_dim * int(mask_text(w).sum()) * w.heads


def effective_flops(w: Workload, data: Optional[dict] = None) -> float:
    """4 * D * (visible (query, key) pairs) * H: the multiply-adds of
    Q K^T and P V over the unmasked pairs only."""
    csr = data.get("csr") if (data is not None and w.sparse_keep is not None) else None
    nq = w.current.video_len
    P = w.current.tokens_per_frame
    total = 0
    tab = token_table(w)
    if csr is None:
        # without block sparsity a query's mask depends only on its latent frame
        for f in range(w.current.frames):
            total += int(mask(w, [f * P], None, tab).sum()) * P
    else:
        for c0 in range(0, nq, 512):
            total += int(mask(w, np.arange(c0, min(nq, c0 + 512)), csr, tab).sum())
    return 4.0 * w.head_dim * total * w.heads
