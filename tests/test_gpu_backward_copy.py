"""GPU parity of the one-pass forward + backward FP8 copies of a Linear input with the oracle, bit-exact:
the forward copy is the 1x128 quantization of x, the backward copy that of x^T (per channel, 128 tokens)."""
import numpy as np
import pytest

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, every_amax_groups, host, say

pytestmark = pytest.mark.gpu


def check(xb, what):
    q, s, qt, st = fq.fp8q_quant_act_dual(bf16_dev(xb))
    oq, os_ = oracle.quant_act_1x128(xb)
    oqt, ost = oracle.quant_act_backward_copy(xb)
    assert np.array_equal(host(q), oq), f"{what}: forward codes"
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32)), f"{what}: forward scales"
    got = host(qt)
    bad = np.argwhere(got != oqt)
    assert bad.size == 0, f"{what}: {len(bad)} backward codes differ, first at {tuple(bad[0])}"
    assert np.array_equal(host(st).view(np.uint32), ost.view(np.uint32)), f"{what}: backward scales"


def test_up_projection_input():
    d = wl.dense_up(N=128)
    say(f"dual quant: up input {d['a'].shape}")
    check(d["a"], "up input")


@pytest.mark.parametrize("M,K", [(128, 128), (384, 640), (1024, 256)])
def test_scaled_channels_and_special_values(M, K):
    """Channels scaled over 2^-20 .. 2^20, some all-zero channels and tokens (scale 0, signed zero codes),
    negative zeros, subnormals and values that round to 448."""
    g = np.random.default_rng([61, M, K])
    x = g.standard_normal((M, K)).astype(np.float32) * np.exp2(g.integers(-20, 21, size=(1, K))).astype(np.float32)
    x[:, g.choice(K, 3, replace=False)] = 0.0
    x[g.choice(M, 2, replace=False), :] = -0.0
    xb = wl.bf16_bits(x)
    sub = g.random((M, K)) < 0.01
    xb[sub] = g.integers(1, 0x80, sub.sum()).astype(np.uint16) | (g.integers(0, 2, sub.sum()) << 15).astype(np.uint16)
    say(f"dual quant: M={M} K={K}")
    check(xb, f"{M}x{K}")


def test_every_amax_for_both_copies():
    """Every positive finite bf16 amax as the maximum of a channel's 128 tokens (the backward copy's groups: the
    groups of every_amax_groups laid out as columns), which also gives the forward groups (one token, 128
    channels) maxima all over the range."""
    cols = every_amax_groups(85).reshape(-1, 128)        # one 128-element group per row
    n = (len(cols) + 127) // 128 * 128                    # whole K-blocks of channels
    cols = np.concatenate([cols, np.zeros((n - len(cols), 128), np.uint16)])
    xb = np.ascontiguousarray(cols.T)                     # [128 tokens, n channels]
    say(f"dual quant: every amax as a channel maximum, {xb.shape}")
    check(xb, "every amax")
