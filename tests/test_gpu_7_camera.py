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


def _edge_workloads():
    """Degenerate camera layouts: a one-frame segment (every radius sees one
    camera token, the rest of a chunk masked), one-token frames of one head,
    five frames of 7 tokens, eight frames of 4 tokens."""
    seg = lambda F, P: W.Segment(F, P, 0, [], [], [])
    return {
        "cam_one_frame": W.Workload("cam_one_frame", 2, [seg(1, 300)], 0, None, 201),
        "cam_p1": W.Workload("cam_p1", 1, [seg(3, 1)], 0, None, 202),
        "cam_f5": W.Workload("cam_f5", 2, [seg(5, 7)], 0, None, 203),
        "cam_f8": W.Workload("cam_f8", 3, [seg(8, 4)], 0, None, 204),
    }


# radii 0, 1 and 2+ take chunks of 1, 3 and 4 camera tokens; radius 5 on 8
# frames spans up to 3 chunks, and a radius beyond the segment sees all of it
@pytest.mark.parametrize("name,radius", [("cam_one_frame", 0), ("cam_one_frame", 1), ("cam_one_frame", 2),
                                         ("cam_p1", 1), ("cam_p1", 2), ("cam_f5", 1), ("cam_f5", 2),
                                         ("cam_f8", 3), ("cam_f8", 5), ("cam_f8", 40)])
def test_camera_edge_layouts(name, radius):
    print(f"[camera edge] {name} r={radius}", flush=True)
    w = _edge_workloads()[name]
    d = W.generate(w)
    seg = G.layout(0, w.current)
    o, lse = hn.camera_attn(seg, w.heads, G.dev(d["q_vid"]), G.dev(d["k_cam"]), G.dev(d["v_cam"]),
                            radius=radius)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ref, ref_lse = oracle.camera_attention(w, d, radius)
    if radius == 0 or w.current.frames == 1:
        # one visible camera token: weight exactly 1
        P = w.current.tokens_per_frame
        v = W.bf16_bits_to_f32(d["v_cam"])
        assert np.array_equal(got, v[np.arange(w.current.video_len) // P])
    err = np.abs(got - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2
