"""Pins of the oracle's INT8 row quantizer (CPU only).

The pages say keys and values are stored as INT8 with float scale factors and
computed in BF16 (fluxbbs teardown, "How one 4090 does it", first trick).
The exact formula is a reading: per (token, head) row, scale = fp32(amax/127),
q = round-half-even(fp32(x/scale)) clamped to +-127, zero row -> 0.
"""
import struct

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, bf16_bits_to_f32
from _exact_quant import quantize_row_exact, bf16_to_fraction, round_to_f32, f32_bits


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _row(vals, D=128):
    v = list(vals) + [0.0] * (D - len(vals))
    return _bits(v)[None, :]


def test_worked_example_scale_one_ties_to_even():
    # amax = 127 gives scale = 127/127 = 1 exactly, so x/scale = x and every
    # half-integer is an exact tie: round-half-even sends 0.5->0, 1.5->2,
    # 2.5->2, 62.5->62 (round-half-away would give 1, 2, 3, 63).
    q, s = oracle.quantize(_row([127.0, 62.5, -62.5, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]))
    assert s[0] == np.float32(1.0)
    assert list(q[0, :10]) == [127, 62, -62, 0, 2, 2, 0, -2, -2, 4]
    assert np.all(q[0, 10:] == 0)


def test_worked_example_unit_amax():
    # amax = 1: scale = fp32(1/127) = 0x3C010204 (0.0078740157...), slightly
    # below 1/127, so 0.5/scale = 63.50000023... whose fp32 rounding is 63.5
    # exactly -> 64 (even); 0.25/scale -> 31.75 -> 32; 0.75/scale -> 95.25 -> 95;
    # 1/scale -> 127.0000004 -> 127.
    q, s = oracle.quantize(_row([1.0, -0.5, 0.5, 0.25, 0.75]))
    assert struct.unpack("<I", struct.pack("<f", float(s[0])))[0] == 0x3C010204
    assert list(q[0, :5]) == [127, -64, 64, 32, 95]


def test_zero_row():
    q, s = oracle.quantize(np.zeros((3, 128), dtype=np.uint16))
    assert np.all(q == 0) and np.all(s == 0)
    # negative zero is a zero row too
    q, s = oracle.quantize(np.full((1, 128), 0x8000, dtype=np.uint16))
    assert np.all(q == 0) and np.all(s == 0)


def _check_exact(rows):
    q, s = oracle.quantize(rows)
    for i in range(rows.shape[0]):
        qe, se = quantize_row_exact([int(b) for b in rows[i]])
        assert f32_bits(se) == struct.unpack("<I", struct.pack("<f", float(s[i])))[0], i
        assert list(q[i]) == qe, i


def test_matches_exact_rational_random_rows():
    rng = np.random.default_rng(0)
    rows = f32_to_bf16_bits(rng.standard_normal((300, 128), dtype=np.float32))
    _check_exact(rows)


def test_matches_exact_rational_extreme_scales():
    rng = np.random.default_rng(1)
    rows = []
    # subnormal and tiny amax (scale becomes subnormal), huge amax, mixed
    for e in (-133, -130, -126, -120, -60, 0, 60, 120, 126):
        x = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** e)
        rows.append(f32_to_bf16_bits(x))
    # smallest bf16 subnormals as amax
    for amax_bits in (0x0001, 0x0002, 0x0003, 0x007F, 0x0080, 0x7F7F, 0x7F00):
        r = rng.integers(0, amax_bits + 1, 128).astype(np.uint16)
        r[rng.integers(0, 128)] = amax_bits
        r[rng.random(128) < 0.5] |= 0x8000
        rows.append(r)
    _check_exact(np.stack(rows))


def test_scale_for_every_positive_bf16_amax():
    # scale(amax) over all positive finite bf16 values, against exact rationals
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    rows = np.zeros((len(amax), 128), dtype=np.uint16)
    rows[:, 0] = amax
    q, s = oracle.quantize(rows)
    got = s.view(np.uint32)
    for i in range(len(amax)):
        se = round_to_f32(bf16_to_fraction(int(amax[i])) / 127)
        assert got[i] == f32_bits(se), hex(int(amax[i]))
    assert np.all(q[:, 0] == 127)


def test_invariants_random():
    rng = np.random.default_rng(2)
    rows = f32_to_bf16_bits(rng.standard_normal((200_000, 128), dtype=np.float32))
    q, s = oracle.quantize(rows)
    x = bf16_bits_to_f32(rows).astype(np.float64)
    # every non-zero row reaches the full code range
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    # sign is kept or the code is zero
    sx, sq = np.sign(x), np.sign(q)
    assert np.all((sq == 0) | (sq == sx))
    # reconstruction error: rounding (1/2) plus the fp32 quotient error
    err = np.abs(x - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16))
    assert q.min() >= -127


def test_power_of_two_equivariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2000, 128), dtype=np.float32)
    q0, s0 = oracle.quantize(f32_to_bf16_bits(x))
    for k in (-20, -3, 1, 7, 40):
        qk, sk = oracle.quantize(f32_to_bf16_bits(x * np.float32(2.0 ** k)))
        assert np.array_equal(q0, qk)
        assert np.array_equal(sk, (s0 * np.float32(2.0 ** k)).astype(np.float32))
