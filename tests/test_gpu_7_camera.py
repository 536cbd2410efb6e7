"""GPU parity of the camera cross-attention (video tokens read the
time-aligned camera tokens of their segment).

Radius 0 (the pages' time alignment) has one visible key of weight exactly 1,
so the output must equal the frame's camera value bit for bit; wider radii
are held to the attention bar (max-abs 2e-2, mean-abs 2e-3) against the
fp64 oracle, and lse to 1e-2.
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


@pytest.mark.parametrize("name,radius", [("c1", 0), ("m1", 0), ("m1", 1), ("m4", 2), ("m2", 100),
                                         ("c2", 0), ("c2", 3), ("c3", 1)])
def test_camera_attention(name, radius):
    print(f"[camera] {name} r={radius}", flush=True)
    w = W.config(name)
    d = W.generate(w)
    seg = G.layout(w.query_segment, w.current)
    o, lse = hn.camera_attn(seg, w.heads, G.dev(d["q_vid"]), G.dev(d["k_cam"]), G.dev(d["v_cam"]),
                            radius=radius)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    nq = w.current.video_len
    rows = np.arange(nq) if nq <= 4096 else G.sample_rows(nq, tile=16)
    if radius == 0:
        P = w.current.tokens_per_frame
        v = W.bf16_bits_to_f32(d["v_cam"])
        assert np.array_equal(got, v[np.arange(nq) // P])
    ref, ref_lse = oracle.camera_attention(w, d, radius)
    err = np.abs(got[rows] - ref[rows])
    print(f"  max-abs {err.max():.3e} lse {np.abs(lse.cpu().numpy() - ref_lse).max():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
