"""Pins of the oracle's FP4 (OCP E2M1) quantization in the FP8 groupings.

Independent of the oracle's code: the E2M1 code table written from the format's definition, a nearest-value
search in exact rational arithmetic over every rounding midpoint and its fp32 neighbours, hand-worked groups
(values and nibble order), invariants and the error bound.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def e2m1_value(code):
    """OCP E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal."""
    sign = -1 if code & 8 else 1
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return sign * mag


def nearest_code(v: float) -> int:
    """Nearest E2M1 code by exact search, ties to the even code, saturating; the sign kept (also for 0)."""
    a = abs(Fraction(v))
    best = min(range(8), key=lambda c: (abs(e2m1_value(c) - a), c & 1))
    return best | (8 if np.signbit(v) else 0)


def bf16(values):
    v = np.asarray(values, np.float32)
    assert np.all(v.view(np.uint32) & 0xFFFF == 0)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def test_decode_table(olib):
    vals = oracle.e2m1_decode(np.arange(16), lib=olib)
    assert [float(e2m1_value(c)) for c in range(16)] == list(vals)
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_encoder_against_exact_nearest_search(olib):
    """Every rounding midpoint between neighbouring magnitudes, each with its two fp32 neighbours, the code
    values themselves, values past 6, and both signs."""
    mags = [float(e2m1_value(c)) for c in range(8)]
    pts = set()
    for lo, hi in zip(mags, mags[1:]):
        mid = np.float32((lo + hi) / 2)
        pts |= {float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(10)))}
    pts |= set(mags) | {6.5, 7.0, 100.0, 1e30, 1e-30, 0.1, 2.2, 4.9999}
    v = np.array(sorted(pts), np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e2m1_encode(v, lib=olib)
    want = np.array([nearest_code(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, want)


def test_round_trip_of_every_code(olib):
    vals = np.array([float(e2m1_value(c)) for c in range(16)], np.float32)
    vals[8] = -0.0    # code 8 is negative zero
    assert np.array_equal(oracle.e2m1_encode(vals, lib=olib), np.arange(16, dtype=np.uint8))


def test_hand_worked_activation_group(olib):
    """amax 6 makes the scale exactly 1; the codes then follow the table: 6 -> 7, 3 -> 5, -1.5 -> 0xB,
    0.25 (a tie) -> 0, 0.75 (a tie) -> 2 (1.0), 5 (a tie) -> 6 (4.0), -0 -> 8; element 2i is the low nibble."""
    g = np.zeros(128, np.float32)
    g[:8] = [6.0, 3.0, -1.5, 0.25, 0.75, 5.0, -0.0, 2.5]
    q, s = oracle.quant_act_fp4_1x128(bf16(g[None, :]), lib=olib)
    assert q.shape == (1, 64) and s[0, 0] == np.float32(1.0)
    assert list(q[0, :4]) == [0x7 | (0x5 << 4), 0xB | (0x0 << 4), 0x2 | (0x6 << 4), 0x8 | (0x4 << 4)]


def test_amax_encodes_to_six_and_negation_flips_sign_bits(olib):
    rng = np.random.default_rng(71)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oracle.quant_act_fp4_1x128(xb, lib=olib)
    qn, sn = oracle.quant_act_fp4_1x128(xb ^ 0x8000, lib=olib)
    assert np.array_equal(s, sn) and np.array_equal(qn, q ^ 0x88)
    lo, hi = q & 0xF, q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(8, 512)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).reshape(8, 4, 128)
    arg = np.abs(xf).argmax(axis=2)
    for m in range(8):
        for kb in range(4):
            assert codes[m, kb * 128 + arg[m, kb]] & 7 == 7


def test_error_bound_and_weight_blocks(olib):
    """|dec(q) s - x| is at most half the spacing at |x|/s (1 below 6, 0.5 below 4, 0.25 below 2) times s,
    for activation groups and for 128x128 weight blocks with their own scales."""
    rng = np.random.default_rng(72)
    w = (rng.standard_normal((256, 384)).astype(np.float32) *
         np.kron(np.exp2(rng.integers(-6, 7, size=(2, 3))), np.ones((128, 128))).astype(np.float32))
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, s = oracle.quant_w_fp4_128x128(wb, lib=olib)
    assert q.shape == (256, 192) and s.shape == (2, 3)
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(256, 384)
    dec = oracle.e2m1_decode(codes, lib=olib) * np.kron(s.astype(np.float64), np.ones((128, 128)))
    for nb in range(2):
        for kb in range(3):
            blk = wf[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert s[nb, kb] == np.float32(np.float32(np.abs(blk).max()) / np.float32(6.0))
    r = np.abs(wf) / np.kron(s.astype(np.float64), np.ones((128, 128)))
    half = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0)) * np.kron(s.astype(np.float64), np.ones((128, 128)))
    assert np.all(np.abs(dec - wf) <= half * (1 + 1e-6))


def test_rejects_ragged_groups(olib):
    with pytest.raises(ValueError):
        oracle.quant_act_fp4_1x128(np.zeros((2, 100), np.uint16), lib=olib)
    with pytest.raises(ValueError):
        oracle.quant_w_fp4_128x128(np.zeros((100, 128), np.uint16), lib=olib)
