"""Planted mistakes in the oracle must fail its pins.

Each case patches one plausible error into the oracle (on the CPU only) and
runs a pin from the other oracle test modules, expecting it to fail.
"""
import numpy as np
import pytest

import oracle
import workloads as W
import test_oracle_attn as TA
import test_oracle_mask as TM
import test_oracle_quant as TQ

_real_quantize = oracle.quantize
_real_mask = oracle.mask


def _quant_half_away(x_bits):
    x = W.bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127)).astype(np.float32)
    y = x / np.where(amax == 0, np.float32(1), scale)[..., None]
    q = np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -127, 127)
    return q.astype(np.int8), np.where(amax == 0, np.float32(0), scale).astype(np.float32)


def _quant_reciprocal(x_bits):
    x = W.bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127)).astype(np.float32)
    inv = (np.float32(127) / np.where(amax == 0, np.float32(1), amax)).astype(np.float32)
    q = np.clip(np.rint((x * inv[..., None]).astype(np.float32)), -127, 127)
    return q.astype(np.int8), np.where(amax == 0, np.float32(0), scale).astype(np.float32)


def _quant_scale_128(x_bits):
    x = W.bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(128)).astype(np.float32)
    q = np.clip(np.rint(x / np.where(amax == 0, np.float32(1), scale)[..., None]), -127, 127)
    return q.astype(np.int8), np.where(amax == 0, np.float32(0), scale).astype(np.float32)


@pytest.mark.parametrize("bad,pin", [
    (_quant_half_away, TQ.test_worked_example_scale_one_ties_to_even),
    (_quant_reciprocal, TQ.test_matches_exact_rational_random_rows),
    (_quant_scale_128, TQ.test_invariants_random),
])
def test_quantizer_mutations_are_caught(monkeypatch, bad, pin):
    monkeypatch.setattr(oracle, "quantize", bad)
    with pytest.raises(AssertionError):
        pin()


def _mask_with(post):
    def m(w, rows=None, csr=None, tab=None):
        vis = _real_mask(w, rows, csr, tab)
        tab = oracle.token_table(w) if tab is None else tab
        return post(w, vis, tab, rows)
    return m


def _earlier_tails_visible(w, vis, tab, rows):
    vis[:, (tab["seg"] < w.query_segment) & (tab["kind"] == oracle.TAIL)] = True
    return vis


def _window_off_by_one(w, vis, tab, rows):
    if w.window is None:
        return vis
    S = w.query_segment
    g0 = sum(s.frames for s in w.segments[:S])
    cols = (tab["seg"] < S) & (tab["kind"] == oracle.VIDEO) & (tab["gframe"] == g0 - w.window - 1)
    vis[:, cols] = True
    return vis


def _future_visible(w, vis, tab, rows):
    vis[:, tab["seg"] > w.query_segment] = True
    return vis


def _own_tails_always(w, vis, tab, rows):
    vis[:, (tab["seg"] == w.query_segment) & (tab["kind"] == oracle.TAIL)] = True
    return vis


@pytest.mark.parametrize("post,pin,arg", [
    (_earlier_tails_visible, TM.test_visible_counts_target_configs, ("c3", 45440)),
    (_window_off_by_one, TM.test_visible_counts_target_configs, ("c1_evict", 176)),
    (_future_visible, TM.test_visible_counts_medium, ("c1_future",)),
    (_own_tails_always, TM.test_visible_counts_target_configs, ("c2", 12596)),
])
def test_mask_mutations_are_caught(monkeypatch, post, pin, arg):
    monkeypatch.setattr(oracle, "mask", _mask_with(post))
    with pytest.raises(AssertionError):
        pin(*arg)


def test_attention_missing_scale_is_caught(monkeypatch):
    real = oracle.attention

    def bad(w, d, rows=None, sm_scale=None, chunk=256, kv=None):
        return real(w, d, rows, sm_scale=1.0, chunk=chunk, kv=kv)
    monkeypatch.setattr(oracle, "attention", bad)
    with pytest.raises(AssertionError):
        TA.test_brute_force_c1("c1")


def test_attention_head_mixup_is_caught(monkeypatch):
    real_kv = oracle.key_values

    def bad_kv(w, d):
        K, V = real_kv(w, d)
        return K, V[:, ::-1, :].copy()   # values of the wrong head
    monkeypatch.setattr(oracle, "key_values", bad_kv)
    with pytest.raises(AssertionError):
        TA.test_brute_force_c1("c1")


def test_attention_unquantized_history_is_caught(monkeypatch):
    # history must be the dequantized INT8 values, not the bf16 originals
    monkeypatch.setattr(oracle, "dequantize", lambda q, s: q.astype(np.float64) * 0 + 1e-3)
    with pytest.raises(AssertionError):
        TA.test_brute_force_c1("c1")


# ---- text-stream queries: plausible mistakes in mask_text are caught by its pins
import test_oracle_text as TT  # noqa: E402

_real_mask_text = oracle.mask_text


def _text_mask_with(post):
    def m(w, rows=None, tab=None):
        vis = _real_mask_text(w, rows, tab)
        tab = oracle.token_table(w) if tab is None else tab
        return post(w, vis, tab)
    return m


def _text_all_own_tails(w, vis, tab):
    vis[:, (tab["seg"] == w.query_segment) & (tab["kind"] == oracle.TAIL)] = True
    return vis


def _text_no_history_video(w, vis, tab):
    vis[:, (tab["seg"] < w.query_segment) & (tab["kind"] == oracle.VIDEO)] = False
    return vis


def _text_no_own_tail(w, vis, tab):
    vis[:, (tab["seg"] == w.query_segment) & (tab["kind"] == oracle.TAIL)] = False
    return vis


@pytest.mark.parametrize("post,pin,arg", [
    (_text_all_own_tails, TT.test_text_visible_counts, ("c2", 12468, 12596)),
    (_text_no_history_video, TT.test_text_visible_counts, ("c3", 45312, 45440)),
    (_text_no_own_tail, TT.test_text_visible_counts, ("c1", 192, 200)),
])
def test_text_mask_mutations_are_caught(monkeypatch, post, pin, arg):
    monkeypatch.setattr(oracle, "mask_text", _text_mask_with(post))
    with pytest.raises(AssertionError):
        pin(*arg)
