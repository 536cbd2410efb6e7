"""Python binding of libhn.so: segment-causal, action-aware attention over an
INT8 sliding-window KV cache on an AMD MI355X (gfx950).

This module only marshals arguments: every step of the computation runs in
the library's HIP kernels.  torch supplies device memory and streams.  The
library must be built (``masked_attention_hn_amd._build``); importing this
package without it raises ImportError, and there is no fallback path.

The exported functions carry the C names:
    hn_kv_quant_append, hn_attn_mask_build, hn_seg_attn_fwd,
    hn_attn_workspace_size, hn_kv_cache_sizes, hn_kv_cache_reset,
    hn_kv_archive_evict, hn_kv_cache_rewind, hn_camera_attn_fwd,
    hn_seg_attn_fwd_noalloc, hn_status_string, hn_last_error
plus small helpers (KVCache, KVArchive, SegLayout, BlockSparse, PlanOpts,
build_plan, dense_mask, seg_attn, seg_attn_joint) that own the buffers those
calls need.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhn.so")

HEAD_DIM = 128
MAX_ACTIONS = 64
TILE = 128

HN_OK, HN_ERR_NULL, HN_ERR_INVALID, HN_ERR_UNSUPPORTED = 0, 1, 2, 3
HN_ERR_CAPACITY, HN_ERR_WORKSPACE, HN_ERR_ORDER, HN_ERR_HIP = 4, 5, 6, 7
HN_MASK_TILE_PLAN, HN_MASK_DENSE = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run masked_attention_hn_amd/_build.py "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)

_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


class hn_seg_layout(ctypes.Structure):
    _fields_ = [("index", ctypes.c_int32), ("frames", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("head_len", ctypes.c_int32),
                ("num_actions", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("action_len", _i32p), ("action_f0", _i32p), ("action_f1", _i32p)]


class hn_kv_cache(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("head_cap_tokens", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("ring_k", _vp), ("ring_v", _vp), ("ring_ks", _vp), ("ring_vs", _vp),
                ("heads_k", _vp), ("heads_v", _vp), ("heads_ks", _vp), ("heads_vs", _vp),
                ("frames_seen", ctypes.c_int64), ("head_tokens", ctypes.c_int32),
                ("segments", ctypes.c_int32)]


class hn_block_sparse(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("n_qtiles", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("row_ptr", _vp), ("col", _vp)]


class hn_plan_opts(ctypes.Structure):
    _fields_ = [("n_splits", ctypes.c_int32), ("n_splits_text", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("whole_tiles", ctypes.c_int32)]


class hn_tile_plan(ctypes.Structure):
    _fields_ = [("dev", _vp), ("tile_q", ctypes.c_int32), ("n_qtiles", ctypes.c_int32),
                ("n_text_tiles", ctypes.c_int32), ("max_spans", ctypes.c_int32),
                ("seg_index", ctypes.c_int32), ("head_tokens", ctypes.c_int32),
                ("frames_seen", ctypes.c_int64), ("sparse", ctypes.c_int32),
                ("n_splits", ctypes.c_int32), ("visible_pairs", ctypes.c_int64),
                ("visible_pairs_text", ctypes.c_int64), ("n_splits_text", ctypes.c_int32),
                ("n_whole", ctypes.c_int32)]


class hn_kv_archive(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("ks", _vp), ("vs", _vp),
                ("cap_frames", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("first_frame", ctypes.c_int64), ("frames", ctypes.c_int64)]


_S = ctypes.c_int
_lib.hn_status_string.argtypes = [_S]
_lib.hn_status_string.restype = ctypes.c_char_p
_lib.hn_last_error.argtypes = []
_lib.hn_last_error.restype = ctypes.c_char_p
_lib.hn_kv_cache_sizes.argtypes = [ctypes.c_int32] * 4 + [ctypes.POINTER(ctypes.c_size_t)] * 4
_lib.hn_kv_cache_sizes.restype = _S
_lib.hn_kv_cache_reset.argtypes = [ctypes.POINTER(hn_kv_cache)]
_lib.hn_kv_cache_reset.restype = _S
_lib.hn_kv_quant_append.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                    _vp, _vp, _vp, _vp, _vp]
_lib.hn_kv_quant_append.restype = _S
_lib.hn_attn_workspace_size.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                        ctypes.POINTER(hn_block_sparse), ctypes.POINTER(hn_plan_opts)]
_lib.hn_attn_workspace_size.restype = ctypes.c_size_t
_lib.hn_attn_mask_build.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                    ctypes.POINTER(hn_block_sparse), ctypes.POINTER(hn_plan_opts),
                                    _S, ctypes.c_int32,
                                    ctypes.c_int32, _vp, ctypes.c_size_t,
                                    ctypes.POINTER(hn_tile_plan), _vp]
_lib.hn_attn_mask_build.restype = _S
_lib.hn_seg_attn_fwd.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                 ctypes.POINTER(hn_tile_plan),
                                 _vp, _vp,            # q_vid, q_txt
                                 _vp, _vp, _vp, _vp,  # k_txt, v_txt, k_vid, v_vid
                                 _vp, _vp, _vp, _vp,  # o_vid, o_txt, lse, lse_txt
                                 ctypes.c_float, _vp]
_lib.hn_seg_attn_fwd.restype = _S

_lib.hn_seg_attn_fwd_noalloc.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                         ctypes.POINTER(hn_block_sparse),
                                         _vp, _vp,            # q_vid, q_txt
                                         _vp, _vp, _vp, _vp,  # k_txt, v_txt, k_vid, v_vid
                                         _vp, _vp, _vp, _vp,  # o_vid, o_txt, lse, lse_txt
                                         ctypes.c_float, _vp]
_lib.hn_seg_attn_fwd_noalloc.restype = _S
NOALLOC_PLAN_BYTES = 4 << 20

_lib.hn_kv_archive_evict.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_seg_layout),
                                     ctypes.POINTER(hn_kv_archive), _vp]
_lib.hn_kv_archive_evict.restype = _S
_lib.hn_kv_cache_rewind.argtypes = [ctypes.POINTER(hn_kv_cache), ctypes.POINTER(hn_kv_archive),
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp]
_lib.hn_kv_cache_rewind.restype = _S

_lib.hn_camera_attn_fwd.argtypes = [ctypes.POINTER(hn_seg_layout), ctypes.c_int32, ctypes.c_int32,
                                    _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp]
_lib.hn_camera_attn_fwd.restype = _S

EXPORTS = ["hn_status_string", "hn_last_error", "hn_kv_cache_sizes", "hn_kv_cache_reset",
           "hn_kv_quant_append", "hn_attn_workspace_size", "hn_attn_mask_build", "hn_seg_attn_fwd",
           "hn_kv_archive_evict", "hn_kv_cache_rewind", "hn_camera_attn_fwd", "hn_seg_attn_fwd_noalloc"]


class HNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{hn_status_string(status)} ({status}): {msg}")
        self.status = status


def hn_status_string(s: int) -> str:
    return _lib.hn_status_string(s).decode()


def hn_last_error() -> str:
    return _lib.hn_last_error().decode()


def _check(st: int):
    if st != HN_OK:
        raise HNError(st, hn_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class SegLayout:
    """Layout of one segment: description head, action tails with latent-frame
    windows [f0, f1), then frames x tokens_per_frame video tokens."""

    def __init__(self, index: int, frames: int, tokens_per_frame: int, head_len: int,
                 action_len: Sequence[int] = (), action_f0: Sequence[int] = (),
                 action_f1: Sequence[int] = ()):
        m = len(action_len)
        if not (len(action_f0) == len(action_f1) == m):
            raise ValueError("action arrays differ in length")
        self._len = (ctypes.c_int32 * max(m, 1))(*action_len)
        self._f0 = (ctypes.c_int32 * max(m, 1))(*action_f0)
        self._f1 = (ctypes.c_int32 * max(m, 1))(*action_f1)
        self.c = hn_seg_layout(index, frames, tokens_per_frame, head_len, m, 0,
                               ctypes.cast(self._len, _i32p), ctypes.cast(self._f0, _i32p),
                               ctypes.cast(self._f1, _i32p))

    @property
    def text_len(self) -> int:
        return self.c.head_len + sum(self._len[i] for i in range(self.c.num_actions))

    @property
    def video_len(self) -> int:
        return self.c.frames * self.c.tokens_per_frame


def hn_kv_cache_sizes(num_heads: int, window_frames: int, tokens_per_frame: int, head_cap: int):
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(_lib.hn_kv_cache_sizes(num_heads, window_frames, tokens_per_frame, head_cap,
                                  *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


class KVCache:
    """Device buffers of the INT8 cache (allocated here with torch) plus the
    library's counter struct."""

    def __init__(self, num_heads: int, tokens_per_frame: int, window_frames: int,
                 head_cap_tokens: int, device="cuda"):
        rb, rsb, hb, hsb = hn_kv_cache_sizes(num_heads, window_frames, tokens_per_frame,
                                             head_cap_tokens)
        H, W, P, C = num_heads, window_frames, tokens_per_frame, head_cap_tokens
        self.ring_k = torch.zeros((H, W * P, HEAD_DIM), dtype=torch.int8, device=device)
        self.ring_v = torch.zeros_like(self.ring_k)
        self.ring_ks = torch.zeros((H, W * P), dtype=torch.float32, device=device)
        self.ring_vs = torch.zeros_like(self.ring_ks)
        self.heads_k = torch.zeros((H, max(C, 1), HEAD_DIM), dtype=torch.int8, device=device)
        self.heads_v = torch.zeros_like(self.heads_k)
        self.heads_ks = torch.zeros((H, max(C, 1)), dtype=torch.float32, device=device)
        self.heads_vs = torch.zeros_like(self.heads_ks)
        assert self.ring_k.numel() == rb and self.ring_ks.numel() * 4 == rsb
        self.c = hn_kv_cache(H, HEAD_DIM, P, W, C, 0,
                             self.ring_k.data_ptr(), self.ring_v.data_ptr(),
                             self.ring_ks.data_ptr(), self.ring_vs.data_ptr(),
                             self.heads_k.data_ptr(), self.heads_v.data_ptr(),
                             self.heads_ks.data_ptr(), self.heads_vs.data_ptr(), 0, 0, 0)

    def state_dict(self) -> dict:
        """Checkpoint of the cache: its buffers copied to host memory plus the
        counters (the cache is caller-owned buffers and a plain struct)."""
        names = ("ring_k", "ring_v", "ring_ks", "ring_vs", "heads_k", "heads_v", "heads_ks", "heads_vs")
        out = {n: getattr(self, n).cpu() for n in names}
        out["counters"] = (self.c.frames_seen, self.c.head_tokens, self.c.segments)
        return out

    def load_state_dict(self, state: dict):
        """Restore a checkpoint taken from a cache of the same shape."""
        for n, t in state.items():
            if n == "counters":
                continue
            dst = getattr(self, n)
            if dst.shape != t.shape or dst.dtype != t.dtype:
                raise ValueError(f"checkpoint {n} has shape {tuple(t.shape)}, cache {tuple(dst.shape)}")
            dst.copy_(t)
        self.c.frames_seen, self.c.head_tokens, self.c.segments = state["counters"]

    @property
    def frames_seen(self) -> int:
        return self.c.frames_seen

    @property
    def head_tokens(self) -> int:
        return self.c.head_tokens

    @property
    def segments(self) -> int:
        return self.c.segments


class KVArchive:
    """Pinned host buffers of the history archive (allocated here with torch,
    pin_memory=True) plus the library's counter struct."""

    def __init__(self, num_heads: int, tokens_per_frame: int, cap_frames: int):
        H, P, C = num_heads, tokens_per_frame, cap_frames
        self.k = torch.zeros((H, max(C, 1) * P, HEAD_DIM), dtype=torch.int8, pin_memory=True)
        self.v = torch.zeros_like(self.k, pin_memory=True)
        self.ks = torch.zeros((H, max(C, 1) * P), dtype=torch.float32, pin_memory=True)
        self.vs = torch.zeros_like(self.ks, pin_memory=True)
        self.c = hn_kv_archive(self.k.data_ptr(), self.v.data_ptr(), self.ks.data_ptr(),
                               self.vs.data_ptr(), C, 0, 0, 0)

    @property
    def frames(self) -> int:
        return self.c.frames

    @property
    def first_frame(self) -> int:
        return self.c.first_frame


def hn_kv_archive_evict(cache: KVCache, seg: SegLayout, archive: KVArchive, stream=None):
    _check(_lib.hn_kv_archive_evict(ctypes.byref(cache.c), ctypes.byref(seg.c),
                                    ctypes.byref(archive.c), _stream(stream)))


def hn_kv_cache_rewind(cache: KVCache, archive: Optional[KVArchive], frames_seen: int,
                       head_tokens: int, segments: int, stream=None):
    _check(_lib.hn_kv_cache_rewind(ctypes.byref(cache.c),
                                   ctypes.byref(archive.c) if archive is not None else None,
                                   int(frames_seen), int(head_tokens), int(segments),
                                   _stream(stream)))


def hn_kv_cache_reset(cache: KVCache):
    _check(_lib.hn_kv_cache_reset(ctypes.byref(cache.c)))


def hn_kv_quant_append(cache: KVCache, seg: SegLayout, k_txt, v_txt, k_vid, v_vid, stream=None):
    _check(_lib.hn_kv_quant_append(ctypes.byref(cache.c), ctypes.byref(seg.c), _ptr(k_txt),
                                   _ptr(v_txt), _ptr(k_vid), _ptr(v_vid), _stream(stream)))


class BlockSparse:
    """Keep list of video tiles per query tile (CSR, device memory)."""

    def __init__(self, row_ptr: torch.Tensor, col: torch.Tensor, n_qtiles: int):
        self.row_ptr = row_ptr.to(device="cuda", dtype=torch.int32).contiguous()
        self.col = col.to(device="cuda", dtype=torch.int32).contiguous()
        if self.col.numel() == 0:
            self.col = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.c = hn_block_sparse(TILE, TILE, n_qtiles, 0, self.row_ptr.data_ptr(),
                                 self.col.data_ptr())


def _sp(sparse: Optional[BlockSparse]):
    return ctypes.byref(sparse.c) if sparse is not None else None


def PlanOpts(n_splits: int = 0, n_splits_text: int = 0, tile_rows: int = 0,
             whole_tiles: int = 0) -> hn_plan_opts:
    """Plan choices for hn_attn_mask_build / hn_attn_workspace_size (0 = automatic;
    whole_tiles: with n_splits > 1, the leading video query tiles left unsplit)."""
    return hn_plan_opts(n_splits, n_splits_text, tile_rows, whole_tiles)


def _op(opts: Optional[hn_plan_opts]):
    return ctypes.byref(opts) if opts is not None else None


def hn_attn_workspace_size(cache: KVCache, seg: SegLayout, sparse: Optional[BlockSparse] = None,
                           opts: Optional[hn_plan_opts] = None) -> int:
    n = _lib.hn_attn_workspace_size(ctypes.byref(cache.c), ctypes.byref(seg.c), _sp(sparse), _op(opts))
    if n == 0:
        raise HNError(HN_ERR_INVALID, hn_last_error())
    return n


def hn_attn_mask_build(cache: KVCache, seg: SegLayout, sparse: Optional[BlockSparse], mode: int,
                       row0: int, nrows: int, out: torch.Tensor, plan: Optional[hn_tile_plan],
                       stream=None, opts: Optional[hn_plan_opts] = None):
    _check(_lib.hn_attn_mask_build(ctypes.byref(cache.c), ctypes.byref(seg.c), _sp(sparse), _op(opts),
                                   mode, row0, nrows, _ptr(out), out.numel() * out.element_size(),
                                   ctypes.byref(plan) if plan is not None else None,
                                   _stream(stream)))


class Plan:
    """A tile plan plus the workspace tensor that holds it."""

    def __init__(self, workspace: torch.Tensor, c: hn_tile_plan):
        self.workspace = workspace
        self.c = c

    @property
    def visible_pairs(self) -> int:
        return self.c.visible_pairs

    @property
    def visible_pairs_text(self) -> int:
        return self.c.visible_pairs_text


def build_plan(cache: KVCache, seg: SegLayout, sparse: Optional[BlockSparse] = None,
               workspace: Optional[torch.Tensor] = None, stream=None,
               opts: Optional[hn_plan_opts] = None) -> Plan:
    n = hn_attn_workspace_size(cache, seg, sparse, opts)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device="cuda")
    c = hn_tile_plan()
    hn_attn_mask_build(cache, seg, sparse, HN_MASK_TILE_PLAN, 0, 0, workspace, c, stream, opts)
    return Plan(workspace, c)


def dense_mask(cache: KVCache, seg: SegLayout, sparse: Optional[BlockSparse] = None,
               row0: int = 0, nrows: Optional[int] = None, stream=None,
               opts: Optional[hn_plan_opts] = None) -> torch.Tensor:
    """Rows [0, video_len) are the video queries, [video_len, video_len + text_len)
    the text queries."""
    nrows = seg.video_len - row0 if nrows is None else nrows
    kept = min(cache.frames_seen, cache.c.window_frames)
    lk = cache.head_tokens + kept * cache.c.tokens_per_frame + seg.text_len + seg.video_len
    out = torch.empty((max(nrows, 1), lk), dtype=torch.uint8, device="cuda")
    hn_attn_mask_build(cache, seg, sparse, HN_MASK_DENSE, row0, nrows, out, None, stream, opts)
    return out[:nrows]


def hn_seg_attn_fwd(cache: KVCache, seg: SegLayout, plan: Plan, q_vid, k_txt, v_txt, k_vid, v_vid,
                    o_vid: torch.Tensor, lse: Optional[torch.Tensor] = None,
                    sm_scale: Optional[float] = None, stream=None, q_txt=None,
                    o_txt: Optional[torch.Tensor] = None, lse_txt: Optional[torch.Tensor] = None):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(_lib.hn_seg_attn_fwd(ctypes.byref(cache.c), ctypes.byref(seg.c), ctypes.byref(plan.c),
                                _ptr(q_vid), _ptr(q_txt), _ptr(k_txt), _ptr(v_txt), _ptr(k_vid),
                                _ptr(v_vid), _ptr(o_vid), _ptr(o_txt), _ptr(lse), _ptr(lse_txt),
                                float(sm_scale), _stream(stream)))


def seg_attn(cache: KVCache, seg: SegLayout, plan: Plan, q_vid, k_txt, v_txt, k_vid, v_vid,
             with_lse: bool = False, sm_scale: Optional[float] = None, stream=None):
    """Allocate the outputs and run hn_seg_attn_fwd."""
    o = torch.empty_like(q_vid)
    lse = None
    if with_lse:
        lse = torch.empty((cache.c.num_heads, seg.video_len), dtype=torch.float32, device="cuda")
    hn_seg_attn_fwd(cache, seg, plan, q_vid, k_txt, v_txt, k_vid, v_vid, o, lse, sm_scale, stream)
    return (o, lse) if with_lse else o


def seg_attn_joint(cache: KVCache, seg: SegLayout, plan: Plan, q_vid, q_txt, k_txt, v_txt, k_vid,
                   v_vid, sm_scale: Optional[float] = None, stream=None):
    """Video and text queries in one hn_seg_attn_fwd call; returns
    (o_vid, o_txt, lse_vid, lse_txt)."""
    H = cache.c.num_heads
    o = torch.empty_like(q_vid)
    o_txt = torch.empty_like(q_txt)
    lse = torch.empty((H, seg.video_len), dtype=torch.float32, device="cuda")
    lse_txt = torch.empty((H, seg.text_len), dtype=torch.float32, device="cuda")
    hn_seg_attn_fwd(cache, seg, plan, q_vid, k_txt, v_txt, k_vid, v_vid, o, lse, sm_scale, stream,
                    q_txt=q_txt, o_txt=o_txt, lse_txt=lse_txt)
    return o, o_txt, lse, lse_txt


def hn_seg_attn_fwd_noalloc(cache: KVCache, seg: SegLayout, sparse: Optional[BlockSparse], q_vid, k_txt,
                            v_txt, k_vid, v_vid, o_vid: torch.Tensor, lse: Optional[torch.Tensor] = None,
                            sm_scale: Optional[float] = None, stream=None, q_txt=None,
                            o_txt: Optional[torch.Tensor] = None, lse_txt: Optional[torch.Tensor] = None):
    """Plan and attention in one call, with the plan in the library's own
    device buffer (no workspace; for callers that cannot allocate)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(_lib.hn_seg_attn_fwd_noalloc(ctypes.byref(cache.c), ctypes.byref(seg.c), _sp(sparse),
                                        _ptr(q_vid), _ptr(q_txt), _ptr(k_txt), _ptr(v_txt), _ptr(k_vid),
                                        _ptr(v_vid), _ptr(o_vid), _ptr(o_txt), _ptr(lse), _ptr(lse_txt),
                                        float(sm_scale), _stream(stream)))


def hn_camera_attn_fwd(seg: SegLayout, num_heads: int, radius: int, q_vid, k_cam, v_cam,
                       o_vid: torch.Tensor, lse: Optional[torch.Tensor] = None,
                       sm_scale: Optional[float] = None, stream=None):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(_lib.hn_camera_attn_fwd(ctypes.byref(seg.c), int(num_heads), int(radius), _ptr(q_vid),
                                   _ptr(k_cam), _ptr(v_cam), _ptr(o_vid), _ptr(lse), float(sm_scale),
                                   _stream(stream)))


def camera_attn(seg: SegLayout, num_heads: int, q_vid, k_cam, v_cam, radius: int = 0,
                sm_scale: Optional[float] = None, stream=None):
    """Allocate the outputs and run hn_camera_attn_fwd; returns (o, lse)."""
    o = torch.empty_like(q_vid)
    lse = torch.empty((num_heads, seg.video_len), dtype=torch.float32, device=q_vid.device)
    hn_camera_attn_fwd(seg, num_heads, radius, q_vid, k_cam, v_cam, o, lse, sm_scale, stream)
    return o, lse
