"""Pins of the oracle's FP8 -> BF16 weight conversion (w = bf16(fl32(dec(q) * s)) per 128x128 block).

Independent of the oracle's code: the expected values come from exact rational arithmetic (Python's
fractions), from the OCP E4M3 closed form, and from numpy's float32 multiply.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def e4m3_value(code):
    """OCP E4M3 value of a finite code, from the format's definition (exact)."""
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)      # m/8 * 2^-6
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def bf16_value(bits):
    """Exact value of a finite bf16 bit pattern."""
    f = np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def nearest_bf16_ties_even(x: Fraction, negative: bool = False) -> int:
    """bf16 bit pattern nearest to the exact value x (ties to even), found by search over neighbours.
    `negative` gives the sign of a zero x (rationals have no -0)."""
    if x == 0:
        return 0x8000 if negative else 0x0000
    f = np.float32(float(x))                      # within an ulp of x; bf16 neighbours lie around it
    u = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    cands = [(u + d) & 0xFFFF for d in (-2, -1, 0, 1, 2)]
    cands = [c for c in cands if (c & 0x7F80) != 0x7F80]   # finite only
    best = min(cands, key=lambda c: (abs(bf16_value(c) - x), c & 1))
    return best


def fl32(x: Fraction) -> Fraction:
    """Exact value of x rounded to float32 (x needs at most 53 significant bits here)."""
    return Fraction(float(np.float32(float(x))))


FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def one_block(olib, code, scale):
    q = np.full((128, 128), code, np.uint8)
    s = np.array([[scale]], np.float32)
    return oracle.dequant_w_128x128(q, s, lib=olib)[0, 0]


def test_every_code_times_sampled_scales_is_rounded_exactly(olib):
    """All 254 finite codes x 64 random fp32 scales: fl32 of the exact product, then nearest bf16."""
    g = np.random.default_rng(0)
    scales = np.concatenate([np.exp2(g.uniform(-30, 10, 60)).astype(np.float32), np.float32([1, 2.5, 1e-4, 3e-9])])
    for s in scales:
        codes = np.zeros((128, 256), np.uint8)
        codes[0, :254] = FINITE
        w = oracle.dequant_w_128x128(codes, np.array([[s, s]], np.float32), lib=olib)
        for i, c in enumerate(FINITE):
            expected = nearest_bf16_ties_even(fl32(e4m3_value(c) * Fraction(float(s))), bool(c & 0x80))
            assert int(w[0, i]) == expected, (hex(c), float(s))


def test_matches_numpy_float32_multiply_then_bf16(olib):
    """Second route to the same value: numpy's float32 product, rounded to bf16 by exact search."""
    g = np.random.default_rng(1)
    codes = g.choice(FINITE, size=(256, 384)).astype(np.uint8)
    s = (np.exp2(g.uniform(-20, 4, (2, 3)))).astype(np.float32)
    w = oracle.dequant_w_128x128(codes, s, lib=olib)
    lut = np.array([float(e4m3_value(c)) if c in FINITE else 0.0 for c in range(256)], np.float32)
    for _ in range(2000):
        n, k = g.integers(0, 256), g.integers(0, 384)
        p = lut[codes[n, k]] * s[n // 128, k // 128]          # numpy float32 multiply (IEEE, RNE)
        assert int(w[n, k]) == nearest_bf16_ties_even(Fraction(float(p)), bool(codes[n, k] & 0x80))


def test_unit_code_returns_the_scale_and_powers_of_two_are_exact(olib):
    assert one_block(olib, 0x38, np.float32(0.0078125)) == 0x3C00            # 1.0 * 2^-7
    for c in FINITE:
        for k in (-12, 0, 7):                                          # dec(q) * 2^k is exact in bf16
            v = e4m3_value(c) * Fraction(2) ** k
            assert bf16_value(one_block(olib, c, np.float32(2.0 ** k))) == v, (hex(c), k)


def test_zero_scale_and_zero_code_give_signed_zeros(olib):
    assert one_block(olib, 0x00, np.float32(3.0)) == 0x0000
    assert one_block(olib, 0x80, np.float32(3.0)) == 0x8000
    assert one_block(olib, 0x45, np.float32(0.0)) == 0x0000
    assert one_block(olib, 0xC5, np.float32(0.0)) == 0x8000


def test_double_rounding_follows_the_fp32_route(olib):
    """Where rounding the exact product straight to bf16 differs from rounding it to fp32 first, the
    oracle takes the fp32 route (the reading).  Such products are built on purpose: code 0x3C (1.5) times
    fp32 scales next to (bf16 midpoint) / 1.5, so that the product lies a fraction of an fp32 ulp from a
    bf16 midpoint."""
    seen = 0
    for j in range(64):
        t = 1 + Fraction(2 * j + 1, 256)                       # a bf16 rounding midpoint in [1, 2)
        s0 = np.float32(float(t / Fraction(3, 2)))
        for d in range(-3, 4):
            s = np.float32(s0)
            for _ in range(abs(d)):
                s = np.nextafter(s, np.float32(np.inf if d > 0 else -np.inf), dtype=np.float32)
            for c in (0x3C, 0xBC):
                exact = e4m3_value(c) * Fraction(float(s))
                via32 = nearest_bf16_ties_even(fl32(exact), bool(c & 0x80))
                if via32 != nearest_bf16_ties_even(exact, bool(c & 0x80)):
                    seen += 1
                    assert one_block(olib, c, s) == via32, (hex(c), float(s))
    assert seen >= 8


def test_each_block_uses_its_own_scale(olib):
    """Unit codes everywhere and a distinct power-of-two scale per block: the output is the scale grid
    expanded, which a transposed or shifted scale index would break."""
    N, K = 384, 512
    s = np.exp2(np.arange(12, dtype=np.float32).reshape(3, 4) - 6).astype(np.float32)
    w = oracle.dequant_w_128x128(np.full((N, K), 0x38, np.uint8), s, lib=olib)
    f = (w.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f, np.kron(s, np.ones((128, 128), np.float32)))


def test_rejects_nan_codes_and_ragged_shapes(olib):
    with pytest.raises(ValueError):
        oracle.dequant_w_128x128(np.full((128, 128), 0x7F, np.uint8), np.ones((1, 1), np.float32), lib=olib)
    with pytest.raises((RuntimeError, AssertionError, ValueError)):
        oracle.dequant_w_128x128(np.zeros((100, 128), np.uint8), np.ones((1, 1), np.float32), lib=olib)
