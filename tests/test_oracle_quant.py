"""Pins for the oracle's 1x128 activation and 128x128 weight quantizers.

Grouping: 1x128 tiles for activations, 128x128 blocks for weights (page "The Definitive Information
To Deepseek", the passage referring to Figure 7 (a)).  Scale reading: fl32(amax/448).
Pins: hand-worked groups (tests/golden/hand_cases.json), and invariants the definition fixes:
the amax element always encodes to +-448, negating the input flips only the sign bits, scaling the
input by 2^j scales the scale by 2^j and keeps the codes, and the dequantization error bound of a
3-bit-mantissa format.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def f32_bits_to_float(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def val(v):
    return np.float32(-0.0) if v == "-0.0" else np.float32(v)


def to_bf16_bits_exact(values):
    """Bits of float32 values that are exactly bf16 (the fixtures only use such values)."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "fixture value is not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("case", load_golden()["act_groups"], ids=lambda c: c["name"])
def test_hand_worked_activation_groups(olib, case):
    vals = [val(v) for v in case["values"]]
    row = np.zeros(128, dtype=np.float32)
    row[: len(vals)] = vals
    # the group sits at K-block 1 of a 2x256 activation; the other groups are all zero
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 128:] = row
    q, s = oracle.quant_act_1x128(to_bf16_bits_exact(x), lib=olib)
    assert s.shape == (2, 2)
    assert s[1, 1].view(np.uint32) == np.uint32(int(case["scale_bits"], 16))
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    want = [int(c, 16) for c in case["codes"]] + [int(case["rest_code"], 16)] * (128 - len(vals))
    assert list(q[1, 128:]) == want
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)


@pytest.mark.parametrize("case", load_golden()["weight_blocks"], ids=lambda c: c["name"])
def test_hand_worked_weight_block(olib, case):
    w = np.zeros((256, 384), dtype=np.float32)     # 2 x 3 blocks; the case sits in block (1, 2)
    for i, j, v in case["entries"]:
        w[128 + i, 256 + j] = v
    q, s = oracle.quant_w_128x128(to_bf16_bits_exact(w), lib=olib)
    assert s.shape == (2, 3)
    assert s[1, 2].view(np.uint32) == np.uint32(int(case["scale_bits"], 16))
    assert np.count_nonzero(s) == 1
    expect = np.full((256, 384), int(case["rest_code"], 16), dtype=np.uint8)
    for i, j, c in case["codes"]:
        expect[128 + i, 256 + j] = int(c, 16)
    assert np.array_equal(q, expect)


def random_acts(seed, M, K, spread=True):
    g = np.random.default_rng(seed)
    a = g.standard_normal((M, K)).astype(np.float32)
    if spread:  # per-group magnitudes over many binades, including tiny groups
        a *= np.exp2(g.integers(-30, 30, size=(M, K // 128))).repeat(128, axis=1).astype(np.float32)
    return wl.bf16_bits(a)


def test_amax_element_encodes_to_448(olib):
    x = random_acts(1, 64, 1024)
    q, s = oracle.quant_act_1x128(x, lib=olib)
    f = wl.bf16_to_f32(x).reshape(64, 8, 128)
    idx = np.abs(f).argmax(axis=2)
    qq = q.reshape(64, 8, 128)
    picked = np.take_along_axis(qq, idx[..., None], axis=2)[..., 0]
    sign = np.take_along_axis(f, idx[..., None], axis=2)[..., 0] < 0
    assert np.all(picked == np.where(sign, 0xFE, 0x7E))
    w = random_acts(2, 256, 256)
    qw, sw = oracle.quant_w_128x128(w, lib=olib)
    fw = wl.bf16_to_f32(w).reshape(2, 128, 2, 128).transpose(0, 2, 1, 3).reshape(2, 2, -1)
    qb = qw.reshape(2, 128, 2, 128).transpose(0, 2, 1, 3).reshape(2, 2, -1)
    i = np.abs(fw).argmax(axis=2)
    assert np.all((np.take_along_axis(qb, i[..., None], 2)[..., 0] & 0x7F) == 0x7E)


def test_negation_flips_sign_bits_only(olib):
    x = random_acts(3, 32, 512)
    q, s = oracle.quant_act_1x128(x, lib=olib)
    qn, sn = oracle.quant_act_1x128(x ^ np.uint16(0x8000), lib=olib)
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ np.uint8(0x80))


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 25])
def test_power_of_two_scaling(olib, j):
    x = random_acts(4, 32, 512, spread=False)       # magnitudes near 1: 2^j stays in the normal range
    q, s = oracle.quant_act_1x128(x, lib=olib)
    xs = wl.bf16_bits(wl.bf16_to_f32(x) * np.float32(2.0 ** j))  # exact: only the exponent moves
    q2, s2 = oracle.quant_act_1x128(xs, lib=olib)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_dequant_error_bound(olib):
    """|dec(q)*s - x| <= 2^-4 |x| (normal E4M3 range: 3 mantissa bits) or <= 2^-10 s (subnormal range),
    up to the two fp32 roundings (scale and quotient)."""
    x = random_acts(5, 64, 2048)
    q, s = oracle.quant_act_1x128(x, lib=olib)
    f = wl.bf16_to_f32(x).astype(np.float64)
    deq = oracle.e4m3_decode(q, lib=olib) * np.repeat(s.T.astype(np.float64), 128, axis=1)
    err = np.abs(deq - f)
    sc = np.repeat(s.T.astype(np.float64), 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(f), 2.0 ** -10 * sc) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_weight_blocks_use_their_own_scale(olib):
    """Each 128x128 block's scale depends only on that block (indexing of s_w [N/128, K/128])."""
    g = np.random.default_rng(6)
    w = g.standard_normal((384, 256)).astype(np.float32)
    mult = np.array([[1, 2.0 ** 5], [2.0 ** -7, 4], [2.0 ** 11, 2.0 ** -2]], dtype=np.float32)
    w *= np.kron(mult, np.ones((128, 128), np.float32))
    bits = wl.bf16_bits(w)
    q, s = oracle.quant_w_128x128(bits, lib=olib)
    f = np.abs(wl.bf16_to_f32(bits))
    for nb in range(3):
        for kb in range(2):
            amax = f[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].max()
            assert s[nb, kb] == amax / np.float32(448.0)


def test_expert_stack_equals_per_expert(olib):
    g = np.random.default_rng(7)
    w = wl.bf16_bits(g.standard_normal((3, 256, 128)).astype(np.float32))
    q, s = oracle.quant_w_128x128(w, lib=olib)
    for e in range(3):
        qe, se = oracle.quant_w_128x128(w[e], lib=olib)
        assert np.array_equal(q[e], qe) and np.array_equal(s[e], se)


def test_rejects_partial_groups_and_nonfinite(olib):
    with pytest.raises(ValueError):
        oracle.quant_act_1x128(np.zeros((2, 100), np.uint16), lib=olib)
    with pytest.raises(ValueError):
        oracle.quant_w_128x128(np.zeros((100, 128), np.uint16), lib=olib)
    x = np.zeros((1, 128), np.uint16)
    x[0, 5] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.quant_act_1x128(x, lib=olib)
