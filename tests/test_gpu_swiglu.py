"""GPU parity of the fused SwiGLU + 1x128 quantization with the oracle, bit-exact: the intermediate
h = bf16(SiLU(x) * y) over every finite gate and every up significand, then codes and scales of the fused
kernel on the down projection's shape, ragged shapes, special values, and one [M, 2K] gate/up tensor."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, host, say

pytestmark = pytest.mark.gpu


def grid(y_exponent, x_max_exponent=126):
    """Every finite bf16 x with |x| < 2^x_max_exponent against every y = +-(1 + m/128) 2^y_exponent (every
    subnormal y for y_exponent None), as an [M, 1024] matrix pair (padded with zeros)."""
    xs = np.arange(65536, dtype=np.uint16)
    xs = xs[((xs >> 7) & 0xFF) < x_max_exponent + 127]
    pos = np.arange(1, 0x80, dtype=np.uint16) if y_exponent is None else \
        (np.arange(0, 0x80, dtype=np.uint16) | ((y_exponent + 127) << 7)).astype(np.uint16)
    ys = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    X, Y = np.repeat(xs, len(ys)), np.tile(ys, len(xs))
    n = (len(X) + 1023) // 1024 * 1024
    X = np.concatenate([X, np.zeros(n - len(X), np.uint16)]).reshape(-1, 1024)
    Y = np.concatenate([Y, np.zeros(n - len(Y), np.uint16)]).reshape(-1, 1024)
    return X, Y


def expect_same(got, want, what, x=None, y=None):
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        extra = f" x={x[i]:#06x} y={y[i]:#06x}" if x is not None else ""
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu {got[i]:#06x} oracle "
                             f"{want[i]:#06x}{extra}")


@pytest.mark.parametrize("y_exp,x_max", [(0, 126), (-60, 126), (-126, 126), (None, 126), (60, 66)])
def test_intermediate_over_every_gate(y_exp, x_max):
    X, Y = grid(y_exp, x_max)
    say(f"swiglu h: all gates x y significands at 2^{y_exp}: {X.size} pairs")
    h = host(fq.fp8q_swiglu_bf16(bf16_dev(X), bf16_dev(Y))).view(np.uint16)
    expect_same(h, oracle.swiglu_bf16(X, Y), f"h at 2^{y_exp}", X, Y)


def special_values(rng, M, K):
    """N(0,1) gates and ups with zeros, signed zeros, large and tiny gates and subnormal ups mixed in."""
    x = wl.bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * 3)
    y = wl.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    specials = wl.bf16_bits(np.array([0.0, -0.0, 48.0, -48.0, 100.0, -100.0, 2.0 ** -133, -2.0 ** -133,
                                      2.0 ** -60, 17.0, -88.0, 1e10], np.float32))
    m = rng.random((M, K)) < 0.05
    x[m] = specials[rng.integers(0, len(specials), m.sum())]
    m = rng.random((M, K)) < 0.02
    y[m] = rng.integers(0, 0x80, m.sum()).astype(np.uint16) | (rng.integers(0, 2, m.sum()) << 15).astype(np.uint16)
    return x, y


@pytest.mark.parametrize("M,K", [(37, 640), (1, 128), (16, 512), (300, 1152)])
def test_fused_ragged_and_special(M, K):
    rng = np.random.default_rng([41, M, K])
    x, y = special_values(rng, M, K)
    say(f"swiglu quant: M={M} K={K}")
    q, s = fq.fp8q_swiglu_quant_act_1x128(bf16_dev(x), bf16_dev(y))
    oq, os_ = oracle.swiglu_quant_1x128(x, y)
    expect_same(host(q), oq, "codes")
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


def test_fused_down_projection_shape():
    """The down projection's activation: gate and up [4096, 18432] ~N(0,1)."""
    d = wl.dense_down(N=128)
    say(f"swiglu quant: down shape {d['x'].shape}")
    q, s = fq.fp8q_swiglu_quant_act_1x128(bf16_dev(d["x"]), bf16_dev(d["y"]))
    oq, os_ = oracle.swiglu_quant_1x128(d["x"], d["y"])
    expect_same(host(q), oq, "codes")
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


def test_one_gate_up_tensor_and_consistency_with_h():
    """x and y as the two halves of one [M, 2K] tensor give the same result as separate tensors, and the
    fused result equals the 1x128 quantization of the written-out intermediate."""
    rng = np.random.default_rng(42)
    M, K = 96, 1024
    x, y = special_values(rng, M, K)
    both = bf16_dev(np.concatenate([x, y], axis=1))
    q1, s1 = fq.fp8q_swiglu_quant_act_1x128(both)
    q2, s2 = fq.fp8q_swiglu_quant_act_1x128(bf16_dev(x), bf16_dev(y))
    h = fq.fp8q_swiglu_bf16(both[:, :K], both[:, K:])
    q3, s3 = fq.fp8q_quant_act_1x128(h)
    for q, s in ((q2, s2), (q3, s3)):
        assert torch.equal(q1, q) and torch.equal(s1.view(torch.int32), s.view(torch.int32))
    oq, os_ = oracle.swiglu_quant_1x128(x, y)
    expect_same(host(q1), oq, "codes")
