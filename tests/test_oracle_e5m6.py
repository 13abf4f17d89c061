"""Pins of the oracle's E5M6 activation quantization (sign, 5 exponent bits with bias 15, 6 mantissa bits;
1x128 groups, scale = fl32(amax / 65024), nearest even, saturating; two 12-bit codes per 3 bytes).

Independent of the oracle's code: numpy's IEEE half precision (an E5M10 format with the same bias, so a
12-bit code shifted left by 4 is the half-precision pattern of the same value), an exact nearest-value search
in rational arithmetic, brute force over every half-precision value, hand-worked groups and byte layout,
invariants and the error bound.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

FINITE = np.array([c for c in range(0x1000) if ((c >> 6) & 31) != 31], np.uint16)


def bf16(values):
    v = np.asarray(values, np.float32)
    assert np.all(v.view(np.uint32) & 0xFFFF == 0)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def as_half(codes):
    return (np.asarray(codes, np.uint16) << 4).astype(np.uint16).view(np.float16).astype(np.float64)


def test_decode_equals_half_precision_with_four_zero_bits(olib):
    got = oracle.e5m6_decode(FINITE, lib=olib)
    assert np.array_equal(got, as_half(FINITE))
    assert got[FINITE == 0x7BF][0] == 65024.0 and got[FINITE == 1][0] == 2.0 ** -20
    assert got[FINITE == 0x40][0] == 2.0 ** -14
    special = oracle.e5m6_decode(np.array([0x7C0, 0xFC0, 0x7C1], np.uint16), lib=olib)
    assert special[0] == np.inf and special[1] == -np.inf and np.isnan(special[2])


def nearest(v: float) -> int:
    """Nearest finite E5M6 code by exact search over all magnitudes, ties to the even code, sign kept."""
    a = abs(Fraction(v))
    mags = [Fraction(float(x)) for x in as_half(np.arange(0x7C0, dtype=np.uint16))]
    if a >= mags[-1]:
        c = 0x7BF
    else:
        lo = max(i for i, m in enumerate(mags) if m <= a)
        dl, du = a - mags[lo], mags[lo + 1] - a
        c = lo + 1 if (du < dl or (du == dl and (lo + 1) % 2 == 0)) else lo
    return c | (0x800 if np.signbit(v) else 0)


def test_encoder_against_exact_search_on_midpoints(olib):
    """Every rounding midpoint in sampled binades (subnormal, normal, the top) with its two fp32 neighbours,
    values past the largest, and both signs."""
    mags = as_half(np.arange(0x7C0, dtype=np.uint16))
    pick = list(range(0, 70)) + list(range(0x3B0, 0x3D0)) + list(range(0x780, 0x7BF))
    pts = set()
    for i in pick:
        mid = np.float32((mags[i] + mags[i + 1]) / 2)
        pts |= {float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9)))}
    pts |= {65280.0, 65279.0, 70000.0, 1e30, 1e-30, 2.0 ** -21, 0.0}
    v = np.array(sorted(pts), np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e5m6_encode(v, lib=olib)
    want = np.array([nearest(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, want)


def test_encoder_on_every_half_precision_value(olib):
    """Every finite half-precision value: brute-force nearest E5M6 magnitude by float64 distances (exact here:
    both sides are short binary fractions), ties to the even code."""
    h = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mags = as_half(np.arange(0x7C0, dtype=np.uint16))
    a = h.astype(np.float64)
    hi = np.searchsorted(mags, a, side="left").clip(0, len(mags) - 1)
    lo = (hi - 1).clip(0)
    dlo, dhi = np.abs(a - mags[lo]), np.abs(mags[hi] - a)
    want = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    want = np.where(a >= mags[-1], 0x7BF, want).astype(np.uint16)
    assert np.array_equal(oracle.e5m6_encode(h, lib=olib), want)
    assert np.array_equal(oracle.e5m6_encode(-h, lib=olib), want | 0x800)


def test_hand_worked_group_and_byte_layout(olib):
    """amax 65024 makes the scale exactly 1.  Codes by hand: 65024 -> 0x7BF, 1 -> 0x3C0, -2.5 -> 0xC10,
    1 + 2^-7 (a tie) -> 0x3C0, 1 + 3 * 2^-7 (a tie) -> 0x3C2, 2^-20 -> 0x001, 2^-21 (a tie) -> 0, -0 -> 0x800.
    Pairs pack as c0[7:0], c0[11:8] | c1[3:0] << 4, c1[11:4]."""
    g = np.zeros(128, np.float32)
    g[:8] = [65024.0, 1.0, -2.5, 1 + 2 ** -7, 1 + 3 * 2 ** -7, 2.0 ** -20, 2.0 ** -21, -0.0]
    q, s = oracle.quant_act_e5m6_1x128(bf16(g[None, :]), lib=olib)
    assert q.shape == (1, 192) and s[0, 0] == np.float32(1.0)
    assert list(q[0, :12]) == [0xBF, 0x07, 0x3C, 0x10, 0x0C, 0x3C, 0xC2, 0x13, 0x00, 0x00, 0x00, 0x80]
    assert np.all(q[0, 12:] == 0)


def test_amax_encodes_to_the_largest_code_and_negation_flips_sign_bits(olib):
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((8, 512)) * np.exp2(rng.integers(-30, 30, size=(8, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oracle.quant_act_e5m6_1x128(xb, lib=olib)
    qn, sn = oracle.quant_act_e5m6_1x128(xb ^ 0x8000, lib=olib)
    assert np.array_equal(s, sn)
    c, cn = oracle.e5m6_unpack(q), oracle.e5m6_unpack(qn)
    assert np.array_equal(cn, c ^ 0x800)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).reshape(8, 4, 128)
    arg = np.abs(xf).argmax(axis=2)
    for m in range(8):
        for kb in range(4):
            assert c[m, kb * 128 + arg[m, kb]] & 0x7FF == 0x7BF


def test_error_bound_and_scales(olib):
    """s = fl32(amax / 65024) per group, and |dec(q) s - x| is at most half an E5M6 spacing (2^-7 of the
    binade, 2^-21 below 2^-14) times s."""
    rng = np.random.default_rng(82)
    x = (rng.standard_normal((16, 1024)) * np.exp2(rng.integers(-20, 20, size=(16, 8)).repeat(128, axis=1)))
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    q, s = oracle.quant_act_e5m6_1x128(xb, lib=olib)
    amax = np.abs(xf).reshape(16, 8, 128).max(axis=2)
    assert np.array_equal(s.T, (amax / np.float32(65024.0)).astype(np.float32))
    sc = np.repeat(s.T.astype(np.float64), 128, axis=1)
    dec = as_half(oracle.e5m6_unpack(q) & 0x7FF) * np.where(oracle.e5m6_unpack(q) & 0x800, -1.0, 1.0) * sc
    r = np.abs(xf.astype(np.float64)) / sc
    half = np.where(r < 2.0 ** -14, 2.0 ** -21, np.exp2(np.floor(np.log2(np.maximum(r, 2.0 ** -14))) - 7)) * sc
    assert np.all(np.abs(dec - xf) <= half * (1 + 1e-6))


def test_rejects_ragged_groups(olib):
    with pytest.raises(ValueError):
        oracle.quant_act_e5m6_1x128(np.zeros((2, 100), np.uint16), lib=olib)
