"""hn_seg_attn_fwd_noalloc: the plan and the attention in one call, with the
plan in the library's own static device buffer (for callers that cannot
allocate).  Its plans never split keys, so its outputs must equal, bit for
bit, those of hn_attn_mask_build + hn_seg_attn_fwd with an unsplit plan.
Calls in a row share the buffer: a larger plan, then a smaller one (whose
slots the first call's leftovers surround), then a keep-list plan."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W

import masked_attention_hn_amd as hn

FAKE = 0x10000  # a non-NULL device address; host validation never dereferences it


def test_oversized_plan_rejected_before_any_device_work():
    """A keep-list plan over 1375 query tiles needs ~60 MB of spans, beyond
    the 4 MiB buffer: refused on the host (no device is touched)."""
    H, F, P = 1, 200, 880
    c = hn.hn_kv_cache(H, 128, P, 4, 16, 0, *([FAKE] * 8), 0, 0, 0)
    seg = hn.SegLayout(0, F, P, 0, [], [], [])
    nqt = -(-F * P // 128)
    sp = hn.hn_block_sparse(128, 128, nqt, 0, FAKE, FAKE)
    st = hn._lib.hn_seg_attn_fwd_noalloc(ctypes.byref(c), ctypes.byref(seg.c), ctypes.byref(sp),
                                         FAKE, None, None, None, FAKE, FAKE, FAKE, None, None, None,
                                         0.1, None)
    assert st == hn.HN_ERR_WORKSPACE
    assert "no-allocation" in hn.hn_last_error()
    # argument errors come back the same way as from hn_seg_attn_fwd
    st = hn._lib.hn_seg_attn_fwd_noalloc(ctypes.byref(c), ctypes.byref(hn.SegLayout(1, 2, P, 0).c), None,
                                         FAKE, None, None, None, FAKE, FAKE, FAKE, None, None, None,
                                         0.1, None)
    assert st == hn.HN_ERR_ORDER


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_equals_the_workspace_entry_point():
    import _gpu as G
    for name in ("c3_h2", "m2", "m4"):
        print(f"[noalloc] {name}", flush=True)
        w = W.config(name)
        d = W.generate(w)
        run = G.Run(w, d, opts=hn.PlanOpts(n_splits=1, n_splits_text=1))
        o_ref, o_txt_ref, lse_ref, lse_txt_ref = run.attn_joint()
        o, o_txt = torch.empty_like(run.q), torch.empty_like(run.q_txt)
        lse, lse_txt = torch.empty_like(lse_ref), torch.empty_like(lse_txt_ref)
        st = hn._lib.hn_seg_attn_fwd_noalloc(
            ctypes.byref(run.cache.c), ctypes.byref(run.seg.c),
            ctypes.byref(run.sparse.c) if run.sparse is not None else None,
            run.q.data_ptr(), run.q_txt.data_ptr(), run.k_txt.data_ptr(), run.v_txt.data_ptr(),
            run.k_vid.data_ptr(), run.v_vid.data_ptr(), o.data_ptr(), o_txt.data_ptr(),
            lse.data_ptr(), lse_txt.data_ptr(), ctypes.c_float(1.0 / np.sqrt(128.0)),
            torch.cuda.current_stream().cuda_stream)
        assert st == hn.HN_OK, hn.hn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(o_txt.view(torch.int16), o_txt_ref.view(torch.int16))
        assert torch.equal(lse, lse_ref) and torch.equal(lse_txt, lse_txt_ref)
        if w.current.video_len <= 4096:
            ref, _, _ = oracle.attention(w, d)
            G.check_bar(o.float().cpu().numpy(), ref, name)
