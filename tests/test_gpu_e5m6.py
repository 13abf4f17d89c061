"""GPU parity of the 1x128 E5M6 activation quantization with the oracle, bit-exact: every bf16 value up to
65024 in groups whose scale is exactly 1 (so every E5M6 rounding midpoint and the subnormal range occur as
they are), groups spanning a wide dynamic range, ragged shapes with zero and subnormal groups, and the up
projection's activation."""
import numpy as np
import pytest

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, every_amax_groups, host, say

pytestmark = pytest.mark.gpu


def check(xb, what):
    M, K = xb.shape
    say(f"e5m6: {what} M={M} K={K}")
    q, s = fq.fp8q_quant_act_e5m6_1x128(bf16_dev(xb))
    oq, os_ = oracle.quant_act_e5m6_1x128(xb)
    gq = host(q)
    bad = np.argwhere(gq != oq)
    if bad.size:
        r, b = bad[0]
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at row {r} byte {b}: gpu {gq[r, b]:#04x} "
                             f"oracle {oq[r, b]:#04x}; codes gpu {oracle.e5m6_unpack(gq[r:r+1])[0, (b // 3) * 2:(b // 3) * 2 + 2]} "
                             f"oracle {oracle.e5m6_unpack(oq[r:r+1])[0, (b // 3) * 2:(b // 3) * 2 + 2]}")
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32)), what


def test_every_bf16_value_at_scale_one():
    """Each 128-group starts with 65024 (scale exactly 1), followed by 127 consecutive bf16 patterns of
    magnitude <= 65024, positive and negative: every E5M6 value and midpoint, subnormals included."""
    mags = np.arange(0, 0x4780, dtype=np.uint16)                     # +0 .. 65024 (0x477E) and a little past
    mags = mags[(mags.astype(np.uint32) << 16).view(np.float32) <= 65024.0]
    vals = np.concatenate([mags, mags | 0x8000])
    n = (len(vals) + 127 * 8 - 1) // (127 * 8) * (127 * 8)          # whole rows of 8 groups
    vals = np.concatenate([vals, np.zeros(n - len(vals), np.uint16)]).reshape(-1, 127)
    head = np.full((vals.shape[0], 1), wl.bf16_bits(np.array([65024.0], np.float32))[0], np.uint16)
    x = np.concatenate([head, vals], axis=1).reshape(-1, 1024)
    check(x, "every bf16 value at scale 1")


def test_every_amax():
    """One group per positive finite bf16 amax: every scale fl32(amax / 65024) the quantizer can form."""
    check(every_amax_groups(84), "every bf16 amax")


@pytest.mark.parametrize("M,K", [(37, 640), (1, 128), (16, 512), (300, 1152)])
def test_ragged_wide_range_and_special(M, K):
    rng = np.random.default_rng([61, M, K])
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-40, 40, size=(M, K)))   # spans > 2^30 in a group
    xb = wl.bf16_bits(np.clip(x, -3e38, 3e38).astype(np.float32))
    if M > 3:
        xb[0, :128] = 0
        xb[1, :128] = 0x8000
        xb[2] = rng.integers(0, 0x80, K).astype(np.uint16) | (rng.integers(0, 2, K) << 15).astype(np.uint16)
    check(xb, "ragged")


def test_up_projection_activation():
    check(wl.dense_up()["a"], "up projection activation")
