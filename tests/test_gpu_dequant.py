"""GPU parity of the FP8 -> BF16 weight conversion (128x128 block scales) with the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import require_gpu, say, u8_dev, f32_dev, host

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def run(q, s):
    w = fq.fp8q_dequant_w_128x128(u8_dev(q), f32_dev(s))
    torch.cuda.synchronize()
    return host(w).view(np.uint16)


def expect_equal(q, s, what):
    got = run(q, s)
    ref = oracle.dequant_w_128x128(q, s)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: gpu {got[tuple(bad[0])]:#06x} oracle {ref[tuple(bad[0])]:#06x} (code {q[tuple(bad[0])]:#04x})"


def test_every_code_with_many_scales():
    """All 254 finite codes in every row, 48 x 3 blocks with scales from 2^-40 to 2^20 (fp32 subnormal
    products included), and zero-scale blocks."""
    require_gpu()
    g = np.random.default_rng(0)
    N, K = 128 * 48, 384
    q = np.resize(FINITE, (N, K)).astype(np.uint8)
    q = q[:, g.permutation(K)]
    s = np.exp2(g.uniform(-40, 20, (48, 3))).astype(np.float32)
    s[5, 1] = 0.0
    s[7, 0] = np.float32(2.0 ** -130)   # a subnormal scale
    say("dequant: every code x 144 blocks of scales")
    expect_equal(q, s, "codes x scales")


@pytest.mark.parametrize("N,K", [(128, 128), (256, 640), (1152, 4224)])
def test_random_shapes(N, K):
    require_gpu()
    g = np.random.default_rng(N + K)
    q = g.choice(FINITE, size=(N, K)).astype(np.uint8)
    s = (g.uniform(1e-4, 1e-2, (N // 128, K // 128))).astype(np.float32)
    say(f"dequant: random {N}x{K}")
    expect_equal(q, s, f"{N}x{K}")


def test_roundtrip_of_the_weight_quantizer():
    """Quantize a bf16 weight with the library, convert back: every element matches the oracle's
    conversion of the oracle's codes, and is within half a code step of the input."""
    require_gpu()
    d = wl.WORKLOADS["tiny"]()
    wb = d["w"]
    q, s = fq.fp8q_quant_w_128x128(torch.from_numpy(np.ascontiguousarray(wb).view(np.int16)).cuda().view(torch.bfloat16))
    w = host(fq.fp8q_dequant_w_128x128(q, s)).view(np.uint16)
    oq, os_ = oracle.quant_w_128x128(wb)
    assert np.array_equal(w, oracle.dequant_w_128x128(oq, os_))


def test_up_projection_weight_full_size():
    """The up-projection weight (18432 x 7168), converted in full and compared element by element."""
    require_gpu()
    g = np.random.default_rng(7)
    N, K = 18432, 7168
    q = g.choice(FINITE, size=(N, K)).astype(np.uint8)
    s = (g.uniform(1e-4, 1e-2, (N // 128, K // 128))).astype(np.float32)
    say("dequant: 18432 x 7168 in full")
    expect_equal(q, s, "18432x7168")


def test_expert_stack_shape():
    require_gpu()
    g = np.random.default_rng(3)
    q = g.choice(FINITE, size=(3, 256, 512)).astype(np.uint8)
    s = (g.uniform(1e-3, 1.0, (3, 2, 4))).astype(np.float32)
    got = host(fq.fp8q_dequant_w_128x128(u8_dev(q), f32_dev(s))).view(np.uint16)
    assert got.shape == (3, 256, 512)
    assert np.array_equal(got, oracle.dequant_w_128x128(q, s))
