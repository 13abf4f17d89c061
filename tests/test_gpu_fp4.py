"""GPU parity of the FP4 (OCP E2M1) quantizers with the oracle, bit-exact: 1x128 activations and 128x128
weights, on the up projection's shapes, ragged token counts and special values (ties, zeros, subnormals)."""
import numpy as np
import pytest

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, every_amax_groups, host, say

pytestmark = pytest.mark.gpu


def same(got_q, got_s, want_q, want_s, what):
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {tuple(bad[0])}: " \
                          f"{got_q[tuple(bad[0])]:#04x} vs {want_q[tuple(bad[0])]:#04x}"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), f"{what}: scales"


def tricky(rng, rows, cols):
    """N(0,1) data with groups whose amax is 6 * 2^k, so quotients land exactly on E2M1 midpoints (ties),
    plus zeros, negative zeros and subnormals."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, -0.0], np.float32)
    m = rng.random((rows, cols)) < 0.3
    x[m] = mids[rng.integers(0, len(mids), m.sum())] * np.where(rng.random(m.sum()) < 0.5, -1, 1)
    for g in range(cols // 128):
        x[:, g * 128] = 6.0 * (2.0 ** (g % 5 - 2))      # amax 6 * 2^k: scale 2^k, quotients exact
    xb = wl.bf16_bits(x)
    sub = rng.random((rows, cols)) < 0.01
    xb[sub] = rng.integers(1, 0x80, sub.sum()).astype(np.uint16)
    return xb


def test_activations_up_input():
    d = wl.dense_up(N=128)
    say(f"fp4 act: up input {d['a'].shape}")
    q, s = fq.fp8q_quant_act_fp4_1x128(bf16_dev(d["a"]))
    same(host(q), host(s), *oracle.quant_act_fp4_1x128(d["a"]), "up input")


def test_activations_every_amax():
    """One group per positive finite bf16 amax: every scale fl32(amax / 6) the activation quantizer can form."""
    xb = every_amax_groups(83)
    say(f"fp4 act: every bf16 amax, {xb.shape}")
    q, s = fq.fp8q_quant_act_fp4_1x128(bf16_dev(xb))
    same(host(q), host(s), *oracle.quant_act_fp4_1x128(xb), "every amax")


@pytest.mark.parametrize("M,K", [(37, 640), (1, 128), (300, 1024)])
def test_activations_ties_and_special_values(M, K):
    xb = tricky(np.random.default_rng([81, M, K]), M, K)
    say(f"fp4 act: M={M} K={K}")
    q, s = fq.fp8q_quant_act_fp4_1x128(bf16_dev(xb))
    same(host(q), host(s), *oracle.quant_act_fp4_1x128(xb), f"{M}x{K}")


def test_weights_up_projection():
    d = wl.dense_up(M=1)
    w = d["w"][:2048]
    say(f"fp4 w: {w.shape}")
    q, s = fq.fp8q_quant_w_fp4_128x128(bf16_dev(w))
    same(host(q), host(s), *oracle.quant_w_fp4_128x128(w), "up W rows 0..2047")


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640)])
def test_weights_ties_and_special_values(N, K):
    wb = tricky(np.random.default_rng([82, N, K]), N, K)
    say(f"fp4 w: N={N} K={K}")
    q, s = fq.fp8q_quant_w_fp4_128x128(bf16_dev(wb))
    same(host(q), host(s), *oracle.quant_w_fp4_128x128(wb), f"{N}x{K}")
