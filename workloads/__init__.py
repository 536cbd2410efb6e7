"""Seeded synthetic workloads for segment-causal attention over an INT8 KV cache.

This module only describes shapes and draws random inputs.  It holds none of
the method's arithmetic (no quantization, no masking, no attention) so that
both the CPU oracle and the HIP path can take their inputs from it without
sharing any computation.

Shapes follow the pages on Hy-Nomas:
  * 16 heads x 128 head dim of the MMDiT (papers.ananclaw.com guide,
    "What it is": model-card architecture bullet).
  * DCAE-V f32t4c32 latents: 32x spatial compression, so 1280x704 gives a
    40x22 = 880-token latent frame and 480x832 a 15x26 = 390-token frame
    (same bullet list, video decoder / DCAE-V line; inference-size override
    in "Getting started").
  * 30 latent frames per 5-second segment (Diffusers example,
    segment_latent_lengths=[30, 30]; prompt-JSON example with 5 s segments).
  * 768-token description head (text length before annealing, fluxbbs
    teardown, "Training", stage 3), 1,280 after annealing.
  * 18-latent-frame history window (fluxbbs teardown, "How one 4090 does it",
    second trick).

Every tensor is drawn as float32 from numpy's PCG64 generator and rounded to
bfloat16 (round to nearest even); arrays hold the raw bf16 bit patterns as
uint16 in token-major [tokens][heads][head_dim] layout.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

HEAD_DIM = 128
TILE = 128  # query/key tile of the block-sparse tile lists


@dataclasses.dataclass
class Segment:
    """Token layout of one generated segment.

    Text tokens come first: the description head (head_len tokens), then the
    action tails in order.  Tail j holds action_len[j] tokens and belongs to
    the half-open latent-frame window [action_f0[j], action_f1[j]).  Video
    tokens follow, frame-major, tokens_per_frame per latent frame.
    """

    frames: int
    tokens_per_frame: int
    head_len: int
    action_len: List[int]
    action_f0: List[int]
    action_f1: List[int]

    @property
    def text_len(self) -> int:
        return self.head_len + sum(self.action_len)

    @property
    def video_len(self) -> int:
        return self.frames * self.tokens_per_frame


@dataclasses.dataclass
class Workload:
    name: str
    heads: int
    segments: List[Segment]
    query_segment: int  # 0-based index of the segment whose video queries attend
    window: Optional[int]  # history window in latent frames; None = keep all history
    seed: int
    kv_dist: str = "normal"  # "normal" or "student_t4"
    sparse_keep: Optional[float] = None  # fraction of candidate video tiles kept per query tile
    sparse_seed: Optional[int] = None
    head_dim: int = HEAD_DIM

    @property
    def current(self) -> Segment:
        return self.segments[self.query_segment]

    @property
    def history_frames(self) -> int:
        return sum(s.frames for s in self.segments[: self.query_segment])

    @property
    def ring_frames(self) -> int:
        """Ring capacity in latent frames used by the cache (no window: all history)."""
        if self.window is not None:
            return self.window
        return max(1, self.history_frames + self.current.frames)

    @property
    def head_cap(self) -> int:
        return max(1, sum(s.head_len for s in self.segments))


def even_windows(frames: int, m: int):
    """Contiguous tail windows covering frames 0..F-1: boundary j at floor(j*F/m)."""
    b = [(j * frames) // m for j in range(m + 1)]
    return b[:-1], b[1:]


def _seg(frames, p, head, tails, windows=None):
    if windows is None:
        f0, f1 = even_windows(frames, len(tails))
    else:
        f0 = [w[0] for w in windows]
        f1 = [w[1] for w in windows]
    return Segment(frames, p, head, list(tails), list(f0), list(f1))


def config(name: str) -> Workload:
    """The named workloads.  c1..c5 are the five configurations of the target;
    the others are parity cases that span several tiles with ragged ends."""
    if name == "c1":
        s = [_seg(2, 24, 16, [8, 8], [(0, 1), (1, 2)]) for _ in range(3)]
        return Workload("c1", 2, s, 2, 4, 42)
    if name == "c1_evict":
        s = [_seg(2, 24, 16, [8, 8], [(0, 1), (1, 2)]) for _ in range(3)]
        return Workload("c1_evict", 2, s, 2, 3, 42)
    if name == "c1_future":
        s = [_seg(2, 24, 16, [8, 8], [(0, 1), (1, 2)]) for _ in range(3)]
        return Workload("c1_future", 2, s, 1, 4, 42)
    if name == "c2":
        return Workload("c2", 16, [_seg(30, 390, 768, [128] * 4)], 0, None, 1)
    if name == "c3":
        s = [_seg(30, 880, 768, [128] * 4) for _ in range(4)]
        return Workload("c3", 16, s, 3, 18, 3)
    if name == "c4":
        s = [_seg(30, 880, 1280, [128] * 4) for _ in range(6)]
        s.append(_seg(30, 880, 768, [128] * 4))
        return Workload("c4", 16, s, 6, None, 4, kv_dist="student_t4")
    if name == "c5":
        return Workload("c5", 16, [_seg(30, 390, 768, [128] * 4)], 0, None, 1,
                        sparse_keep=0.25, sparse_seed=5)
    # per-GPU share of the 8-way head split at the steady-state shape
    if name == "arch":
        # eviction and rewind: 6 segments of 3 latent frames (4x4 tokens), window 4
        segs = [_seg(3, 16, 8, [4, 4], [(0, 1), (1, 3)]) for _ in range(6)]
        return Workload("arch", 2, segs, 3, 4, 9)
    if name == "c3_h2":
        s = [_seg(30, 880, 768, [128] * 4) for _ in range(4)]
        return Workload("c3_h2", 2, s, 3, 18, 3)
    # medium parity cases: several query/key tiles, ragged tails, overlapping
    # and empty action windows, a wrapped ring
    if name == "m1":
        s = [
            _seg(4, 50, 40, [24, 16], [(0, 2), (2, 4)]),
            _seg(5, 50, 33, [20, 20, 9], [(0, 2), (1, 4), (3, 5)]),
            _seg(5, 50, 40, [24, 30, 7, 12], [(0, 2), (1, 4), (3, 5), (2, 2)]),
        ]
        return Workload("m1", 3, s, 2, 6, 11)
    if name == "m2":
        s = [_seg(3, 97, 61, [13], [(0, 3)]), _seg(4, 97, 70, [40, 41], [(1, 3), (0, 1)]),
             _seg(6, 97, 130, [64, 5, 70], [(0, 6), (5, 6), (1, 2)])]
        return Workload("m2", 4, s, 2, None, 12, kv_dist="student_t4")
    if name == "m3":
        s = [_seg(3, 60, 20, [10, 10]), _seg(4, 60, 25, [12, 12]), _seg(5, 60, 30, [16, 16])]
        return Workload("m3", 2, s, 2, 5, 13, sparse_keep=0.25, sparse_seed=14)
    if name == "m4":
        return Workload("m4", 2, [_seg(7, 37, 19, [200, 3], [(0, 7), (6, 7)])], 0, 2, 15,
                        sparse_keep=0.4, sparse_seed=16)
    raise KeyError(name)


ALL_CONFIGS = ["c1", "c1_evict", "c1_future", "c2", "c3", "c4", "c5", "c3_h2",
               "m1", "m2", "m3", "m4", "arch"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "student_t4":
        # Student-t with 4 degrees of freedom has variance 2; scale to unit variance
        x = (rng.standard_t(4.0, size=shape) * math.sqrt(0.5)).astype(np.float32)
    else:
        raise ValueError(dist)
    return f32_to_bf16_bits(x)


def generate(w: Workload) -> Dict[str, object]:
    """Draw the inputs of a workload.

    Draw order: for every segment in sequence order, K_txt, V_txt, K_vid,
    V_vid (each [tokens][H][D]); then Q_vid of the query segment, then its
    Q_txt (text-stream queries: head and tail tokens), then the keys and
    values of its camera tokens K_cam, V_cam ([frames][H][D], one token per
    latent frame).  Queries and camera tokens are always N(0,1); keys and
    values follow w.kv_dist.
    """
    rng = np.random.default_rng(w.seed)
    H, D = w.heads, w.head_dim
    segs = []
    for s in w.segments:
        segs.append({
            "k_txt": _draw(rng, (s.text_len, H, D), w.kv_dist),
            "v_txt": _draw(rng, (s.text_len, H, D), w.kv_dist),
            "k_vid": _draw(rng, (s.video_len, H, D), w.kv_dist),
            "v_vid": _draw(rng, (s.video_len, H, D), w.kv_dist),
        })
    q = _draw(rng, (w.current.video_len, H, D), "normal")
    qt = _draw(rng, (w.current.text_len, H, D), "normal")
    kc = _draw(rng, (w.current.frames, H, D), "normal")
    vc = _draw(rng, (w.current.frames, H, D), "normal")
    out = {"segments": segs, "q_vid": q, "q_txt": qt, "k_cam": kc, "v_cam": vc}
    if w.sparse_keep is not None:
        out["csr"] = block_sparse_csr(w)
    return out


def video_tile_counts(w: Workload):
    """(history-video tiles, own-video tiles) of TILE keys each, ragged last tiles.

    History video is the part of earlier segments' video that the window keeps:
    the last min(history frames, window) latent frames.
    """
    hist_frames = w.history_frames
    if w.window is not None:
        hist_frames = min(hist_frames, w.window)
    P = w.current.tokens_per_frame
    n_hist = -(-hist_frames * P // TILE)
    n_own = -(-w.current.video_len // TILE)
    return n_hist, n_own


def block_sparse_csr(w: Workload):
    """Seeded block-sparse keep list: for every query tile keep ceil(keep*n)
    of the n candidate video tiles, always including the diagonal own-video
    tile (same index as the query tile); the others are drawn uniformly
    without replacement.  Columns are sorted; ids number history-video tiles
    first, then own-video tiles."""
    n_hist, n_own = video_tile_counts(w)
    n = n_hist + n_own
    n_qt = -(-w.current.video_len // TILE)
    k = min(n, math.ceil(w.sparse_keep * n))
    rng = np.random.default_rng(w.sparse_seed)
    row_ptr = [0]
    cols = []
    for t in range(n_qt):
        diag = n_hist + t
        others = np.array([c for c in range(n) if c != diag], dtype=np.int64)
        pick = rng.choice(others, size=k - 1, replace=False) if k > 1 else np.zeros(0, np.int64)
        row = sorted([diag] + [int(c) for c in pick])
        cols.extend(row)
        row_ptr.append(len(cols))
    return {"tile_q": TILE, "tile_k": TILE, "n_qtiles": n_qt,
            "row_ptr": np.array(row_ptr, dtype=np.int32),
            "col": np.array(cols, dtype=np.int32)}
