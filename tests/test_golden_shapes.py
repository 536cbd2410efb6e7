"""The workload shapes against the facts the pages state (tests/golden/page_shapes.json).

Every configuration of the benchmark and the parity tests is built from a few
stated facts: 16 heads of 128 dimensions, a DCAE-V latent with 32x spatial and
4x temporal compression, 30-latent-frame (5 s at 24 fps) segments at
1280x704, an 18-frame history window and 768/1280-token description heads.
These tests derive the workload numbers from the fixture and compare them
with the workload module and the oracle's token table."""
import json
import os

import oracle
import workloads as W

HERE = os.path.dirname(__file__)
F = {k: v["value"] for k, v in json.load(open(os.path.join(HERE, "golden", "page_shapes.json")))["facts"].items()}


def test_fixture_is_self_consistent():
    ex = F["diffusers_example"]
    # 240 frames at 4x temporal compression = the two 30-frame segments of the example
    assert ex["num_frames"] // F["temporal_compression"] == sum(ex["segment_latent_lengths"])
    # a 5 s segment at 24 fps is 30 latent frames
    assert F["segment_seconds"] * ex["fps"] // F["temporal_compression"] == ex["segment_latent_lengths"][0]
    assert F["num_heads"] % F["heads_per_gpu_in_8way_split"] == 0


def tokens_per_frame(width, height):
    s = F["spatial_compression"]
    return (width // s) * (height // s)


def test_tokens_per_latent_frame():
    ex = F["diffusers_example"]
    assert tokens_per_frame(ex["width"], ex["height"]) == 880          # 40 x 22
    assert tokens_per_frame(832, 480) == 390                            # 26 x 15
    for name in ("c3", "c4", "c3_h2"):
        assert W.config(name).current.tokens_per_frame == 880
    for name in ("c2", "c5"):
        assert W.config(name).current.tokens_per_frame == 390


def test_heads_frames_window_and_text_lengths():
    seg_frames = F["diffusers_example"]["segment_latent_lengths"][0]
    for name in ("c2", "c3", "c4", "c5"):
        w = W.config(name)
        assert w.heads == F["num_heads"] and w.head_dim == F["head_dim"]
        assert all(s.frames == seg_frames for s in w.segments)
    assert W.config("c3_h2").heads == F["heads_per_gpu_in_8way_split"]
    assert W.config("c3").window == F["history_window_latent_frames"]
    assert W.config("c3").current.head_len == F["text_len_before_annealing"]
    c4 = W.config("c4")
    assert all(s.head_len == F["text_len_after_annealing"] for s in c4.segments[:-1])
    assert c4.current.head_len == F["text_len_before_annealing"]


def test_history_and_query_counts_of_the_steady_state():
    """c3: 26,400 queries; the window keeps 18 x 880 = 15,840 history video
    tokens, and the oracle's token table of the whole sequence agrees."""
    w = W.config("c3")
    assert w.current.video_len == 30 * 880 == 26400
    tab = oracle.token_table(w)
    S = w.query_segment
    g0 = sum(s.frames for s in w.segments[:S])
    hist = (tab["seg"] < S) & (tab["kind"] == oracle.VIDEO) & (tab["gframe"] >= g0 - w.window)
    assert int(hist.sum()) == F["history_window_latent_frames"] * 880 == 15840
