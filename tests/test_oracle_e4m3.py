"""Pins for the oracle's OCP E4M3 codec (decode table and encoder).

The format is OCP 8-bit floating point E4M3 (the "FN" variant: no infinities, S.1111.111 is NaN).
Pins: the closed-form values the OCP definition fixes, torch's independent float8_e4m3fn codec, a
brute-force nearest-value search, and code-point round trips.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(values_f32):
    # torch's conversion rounds to nearest-even; values above 464 become NaN there, so callers keep |v| <= 448.
    return torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_closed_form_points(olib):
    d = oracle.e4m3_decode(np.arange(256), lib=olib)
    assert d[0x7E] == 448.0            # largest finite value S.1111.110
    assert d[0xFE] == -448.0
    assert d[0x08] == 2.0 ** -6        # smallest normal
    assert d[0x01] == 2.0 ** -9        # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9    # largest subnormal
    assert d[0x38] == 1.0              # exponent field 7 = bias
    assert d[0x3F] == 1.875
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])


def test_decode_matches_torch_and_is_monotone(olib):
    d = oracle.e4m3_decode(np.arange(256), lib=olib)
    t = torch_decode(np.arange(256))
    assert np.array_equal(np.isnan(d), np.isnan(t))
    fin = ~np.isnan(d)
    assert np.array_equal(d[fin], t[fin])
    pos = d[:127]
    assert np.all(np.diff(pos) > 0)                           # codes 0..126 strictly increasing
    assert np.array_equal(d[128:255], -pos)                   # sign bit negates


def test_roundtrip_all_finite_codes(olib):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes, lib=olib).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals, lib=olib), codes)


def brute_force_encode(v):
    """Nearest finite E4M3 magnitude by exhaustive search, ties to the even code, saturating at 448.
    Magnitudes come from torch's codec; distances are exact in float64 for |v| >= 2^-12, and below
    that every value is nearest to 0."""
    mags = torch_decode(np.arange(127))
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer the even code; a tie has exactly two neighbours, one of them even
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def all_finite_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("amax", [448.0, 1.0, 3.5, 0.02, 7.25e-3, 65504.0, 2.0 ** -100, 1.0e30])
def test_encoder_vs_brute_force_all_bf16_quotients(olib, amax):
    """Every finite bf16 x with |x| <= amax divided by fl32(amax/448): the encoder equals the exhaustive
    nearest-value search and torch's codec."""
    x = all_finite_bf16_as_f32()
    amax32 = np.float32(torch.tensor(amax, dtype=torch.bfloat16).float().item())
    x = x[np.abs(x) <= amax32]
    s = amax32 / np.float32(448.0)
    q = (x / s).astype(np.float32)
    enc = oracle.e4m3_encode(q, lib=olib)
    for lo in range(0, len(q), 8192):
        sl = slice(lo, lo + 8192)
        assert np.array_equal(enc[sl], brute_force_encode(q[sl]))
    assert np.array_equal(enc, torch_encode(np.clip(q, -448, 448)))


def test_encoder_vs_torch_sampled_fp32_range(olib):
    """fp32 patterns over [0, 448] with stride 97, plus every rounding midpoint and its fp32 neighbours."""
    pat = np.arange(0, 0x43E00001, 97, dtype=np.uint32)
    mags = torch_decode(np.arange(127))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    mb = mids.view(np.uint32)
    around = np.concatenate([mb - 2, mb - 1, mb, mb + 1, mb + 2, np.array([0x43E00000], np.uint32)])
    v = np.concatenate([pat, around]).view(np.float32)
    for sign in (1.0, -1.0):
        vv = (v * np.float32(sign)).astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(vv, lib=olib), torch_encode(vv))


def test_encoder_saturates_above_448(olib):
    v = np.array([448.0, 448.00003, 463.99997, 464.0, 1000.0, 3.0e38], dtype=np.float32)
    assert list(oracle.e4m3_encode(v, lib=olib)) == [0x7E] * 6
    assert list(oracle.e4m3_encode(-v, lib=olib)) == [0xFE] * 6


def test_encoder_signed_zero_and_underflow(olib):
    v = np.array([0.0, -0.0, 1e-45, -1e-45, 2.0 ** -11, -(2.0 ** -11)], dtype=np.float32)
    assert list(oracle.e4m3_encode(v, lib=olib)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
