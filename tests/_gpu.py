"""Helpers that drive the HIP library through its C ABI for the GPU tests."""
import numpy as np
import torch

import masked_attention_hn_amd as hn
import oracle
import workloads as W


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def layout(index: int, seg: W.Segment) -> hn.SegLayout:
    return hn.SegLayout(index, seg.frames, seg.tokens_per_frame, seg.head_len,
                        seg.action_len, seg.action_f0, seg.action_f1)


def new_cache(w: W.Workload) -> hn.KVCache:
    return hn.KVCache(w.heads, w.current.tokens_per_frame, w.ring_frames, w.head_cap)


def fill_history(w: W.Workload, data: dict, cache: hn.KVCache):
    for s in range(w.query_segment):
        d = data["segments"][s]
        hn.hn_kv_quant_append(cache, layout(s, w.segments[s]), dev(d["k_txt"]), dev(d["v_txt"]),
                              dev(d["k_vid"]), dev(d["v_vid"]))


def sparse_of(w: W.Workload, data: dict):
    if w.sparse_keep is None:
        return None
    csr = data["csr"]
    return hn.BlockSparse(torch.from_numpy(csr["row_ptr"]), torch.from_numpy(csr["col"]),
                          csr["n_qtiles"])


class Run:
    """Cache filled with the history of a workload, a plan for the query segment,
    and the query segment's inputs on the GPU."""

    def __init__(self, w: W.Workload, data: dict, use_sparse: bool = True, opts=None):
        self.w = w
        self.opts = opts
        self.data = data
        self.cache = new_cache(w)
        fill_history(w, data, self.cache)
        S = w.query_segment
        self.seg = layout(S, w.current)
        d = data["segments"][S]
        self.k_txt, self.v_txt = dev(d["k_txt"]), dev(d["v_txt"])
        self.k_vid, self.v_vid = dev(d["k_vid"]), dev(d["v_vid"])
        self.q = dev(data["q_vid"])
        self.q_txt = dev(data["q_txt"]) if w.current.text_len > 0 else None
        self.sparse = sparse_of(w, data) if use_sparse else None
        self.plan = hn.build_plan(self.cache, self.seg, self.sparse, opts=opts)

    def attn(self, with_lse=True):
        out = hn.seg_attn(self.cache, self.seg, self.plan, self.q, self.k_txt, self.v_txt,
                          self.k_vid, self.v_vid, with_lse=with_lse)
        torch.cuda.synchronize()
        return out

    def attn_joint(self):
        """(o_vid, o_txt, lse_vid, lse_txt) of one call with both query sets."""
        out = hn.seg_attn_joint(self.cache, self.seg, self.plan, self.q, self.q_txt, self.k_txt,
                                self.v_txt, self.k_vid, self.v_vid)
        torch.cuda.synchronize()
        return out

    def dense(self, row0=0, nrows=None):
        m = hn.dense_mask(self.cache, self.seg, self.sparse, row0, nrows, opts=self.opts)
        torch.cuda.synchronize()
        return m.cpu().numpy().astype(bool)


def canonical_columns(w: W.Workload) -> np.ndarray:
    """Full-sequence indices of the keys present in the cache state plus the
    query segment, in the library's canonical DENSE order."""
    tab = oracle.token_table(w)
    S = w.query_segment
    g0 = sum(s.frames for s in w.segments[:S])
    seg, kind, gframe = tab["seg"], tab["kind"], tab["gframe"]
    heads = np.nonzero((seg < S) & (kind == oracle.HEAD))[0]
    vid = (seg < S) & (kind == oracle.VIDEO)
    if w.window is not None:
        vid &= gframe >= g0 - w.window
    own = np.nonzero(seg == S)[0]
    return np.concatenate([heads, np.nonzero(vid)[0], own])


def sample_rows(nq: int, tile: int = 128) -> np.ndarray:
    """The first and last row of every `tile`-row query tile (so at least two
    rows of every 128- and 256-row tile, both edges of each) plus the row in
    the middle of each tile; deterministic."""
    starts = np.arange(0, nq, tile)
    ends = np.minimum(starts + tile, nq) - 1
    mids = (starts + ends) // 2
    return np.unique(np.concatenate([starts, ends, mids]))


# Parity bar of the attention outputs against the fp64 oracle: max-abs 2e-2
# and mean-abs 2e-3.  Where |O_ref| >= 8 the bf16 output alone may be off by
# half a unit in its last place (2^-5 = 0.031 at 8, more above), which no
# bf16 result can avoid, so those elements may also carry that half unit.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of bf16 (8 significant bits) at |x|."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float64).tiny)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def tolerance(ref: np.ndarray) -> np.ndarray:
    return MAX_ABS + np.where(np.abs(ref) >= 8.0, half_ulp_bf16(ref), 0.0)


def check_bar(got: np.ndarray, ref: np.ndarray, what: str = "") -> np.ndarray:
    """Assert the parity bar elementwise; returns |got - ref|."""
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bad = err > tolerance(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - tolerance(ref)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements above the bar; worst at {i}: "
                             f"|err| {err[i]:.4e}, |O_ref| {abs(ref[i]):.4f}")
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    return err
