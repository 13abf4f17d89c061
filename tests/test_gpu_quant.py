"""GPU parity of the 1x128 activation and 128x128 weight quantizers: codes and scales must equal the
oracle's bit for bit (through the C ABI, on seeded inputs)."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_act(bits):
    q, s = fq.fp8q_quant_act_1x128(bf16_dev(bits))
    return host(q), host(s)


def gpu_w(bits):
    q, s = fq.fp8q_quant_w_128x128(bf16_dev(bits))
    return host(q), host(s)


def assert_same(gq, gs, oq, os_, what):
    assert gs.shape == os_.shape and gq.shape == oq.shape
    sb, ob = gs.view(np.uint32), os_.view(np.uint32)
    if not np.array_equal(sb, ob):
        i = np.argwhere(sb != ob)[0]
        raise AssertionError(f"{what}: scale mismatch at {tuple(i)}: gpu {gs[tuple(i)]!r} oracle {os_[tuple(i)]!r}")
    if not np.array_equal(gq, oq):
        i = np.argwhere(gq != oq)[0]
        raise AssertionError(f"{what}: code mismatch at {tuple(i)}: gpu 0x{gq[tuple(i)]:02X} oracle 0x{oq[tuple(i)]:02X}"
                             f" ({(gq != oq).sum()} mismatches)")


def spread_bits(seed, rows, cols, group_rows):
    """N(0,1) data with per-group magnitudes spread over 2^-40 .. 2^40, some all-zero groups, and signed zeros."""
    g = np.random.default_rng(seed)
    a = g.standard_normal((rows, cols)).astype(np.float32)
    gr, gc = -(-rows // group_rows), cols // 128
    e = g.integers(-40, 41, size=(gr, gc)).astype(np.float32)
    a *= np.kron(np.exp2(e), np.ones((group_rows, 128), np.float32))[:rows]
    zero = g.random((gr, gc)) < 0.05
    a *= np.kron(~zero, np.ones((group_rows, 128), np.float32))[:rows].astype(np.float32)
    a[g.random((rows, cols)) < 0.01] = -0.0
    return wl.bf16_bits(a)


# ------------------------------------------------------------------ activations

def test_act_tiny_workload():
    d = wl.tiny()
    say("act quant: tiny workload A [128, 512]")
    assert_same(*gpu_act(d["a"]), *oracle.quant_act_1x128(d["a"]), "tiny")


@pytest.mark.parametrize("M,K", [(1, 128), (15, 256), (16, 128), (17, 384), (100, 512), (1000, 1024), (333, 7168),
                                 (64, 18432)])
def test_act_shapes(M, K):
    bits = spread_bits(M * 131 + K, M, K, 1)
    say(f"act quant: M={M} K={K}")
    assert_same(*gpu_act(bits), *oracle.quant_act_1x128(bits), f"act {M}x{K}")


def positive_finite_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint16)  # every positive finite bf16 pattern (denormals included)
    return b


def test_act_every_amax_value():
    """One group per positive finite bf16 amax (32639 groups): the amax at a random position with a random
    sign, the other 127 elements random bf16 patterns of magnitude <= amax with random signs."""
    g = np.random.default_rng(12345)
    amax = positive_finite_bf16()
    n = len(amax)
    lim = amax.astype(np.int64)
    rest = (g.random((n, 127)) * (lim[:, None] + 1)).astype(np.int64)  # magnitudes 0..amax pattern
    rest = np.minimum(rest, lim[:, None]).astype(np.uint16)
    rest |= (g.random((n, 127)) < 0.5).astype(np.uint16) << 15
    rows = np.concatenate([amax[:, None] | ((g.random((n, 1)) < 0.5).astype(np.uint16) << 15), rest], axis=1)
    perm = np.argsort(g.random((n, 128)), axis=1)
    rows = np.take_along_axis(rows, perm, axis=1)
    # pack 8 groups per token row: M = ceil(n / 8), K = 1024
    pad = (-n) % 8
    rows = np.concatenate([rows, np.zeros((pad, 128), np.uint16)])
    bits = rows.reshape(-1, 1024)
    say(f"act quant: every bf16 amax, {bits.shape}")
    assert_same(*gpu_act(bits), *oracle.quant_act_1x128(bits), "every-amax")


AMAX_SET = [0x0001, 0x0080, 0x00FF, 0x0101, 0x1234, 0x3000, 0x3C00, 0x3F80, 0x3FC0, 0x4060, 0x40E0, 0x4180, 0x41E0,
            0x43E0, 0x4500, 0x4B00, 0x5F00, 0x7000, 0x7F7F, 0x3A5C, 0x3B71, 0x3E99, 0x422A, 0x2D55]


@pytest.mark.parametrize("amax_bits", AMAX_SET, ids=lambda b: f"0x{b:04X}")
def test_act_every_x_for_amax(amax_bits):
    """Every finite bf16 x with |x| <= amax, both signs, quantized in groups that all contain amax."""
    mags = np.arange(0, amax_bits + 1, dtype=np.uint16)
    xs = np.concatenate([mags, mags | np.uint16(0x8000)])
    per = 127
    pad = (-len(xs)) % per
    xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, per)
    rows = np.concatenate([np.full((xs.shape[0], 1), amax_bits, np.uint16), xs], axis=1)
    bits = rows.reshape(-1, 128)
    say(f"act quant: all x for amax 0x{amax_bits:04X}: {bits.shape[0]} groups")
    assert_same(*gpu_act(bits), *oracle.quant_act_1x128(bits), f"amax 0x{amax_bits:04X}")


@pytest.mark.parametrize("name", ["up", "down", "decode"])
def test_act_full_workloads(name):
    d = {"up": lambda: wl.dense_up(N=128), "down": lambda: wl.dense_down(N=128),
         "decode": lambda: wl.decode(N=128)}[name]()
    if name == "down":   # A = bf16(SiLU(x) * y), from the oracle
        d["a"] = oracle.swiglu_bf16(d["x"], d["y"])
    say(f"act quant: {name} A {d['a'].shape}")
    assert_same(*gpu_act(d["a"]), *oracle.quant_act_1x128(d["a"]), name)


def test_act_moe_padded_tokens():
    """The 1x128 quantizer on the MoE layer's expert-sorted, 128-padded bf16 rows (layout from the oracle's
    routing); empty rows must give code 0 and scale 0."""
    d = wl.moe(with_weights=False)
    r = oracle.moe_route_topk(d["logits"], d["topk"])
    a = np.zeros((r.M, d["K"]), np.uint16)
    a[r.row_token >= 0] = d["tokens"][r.row_token[r.row_token >= 0]]
    say(f"act quant: moe padded tokens {a.shape}")
    q, s = gpu_act(a)
    oq, os_ = oracle.quant_act_1x128(a)
    assert_same(q, s, oq, os_, "moe tokens")
    pad = r.row_token < 0
    assert np.all(q[pad] == 0) and np.all(s[:, pad] == 0)


def test_act_outputs_untouched_beyond_M():
    bits = spread_bits(5, 17, 256, 1)
    x = bf16_dev(bits)
    q = torch.full((32, 256), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((2, 17), 7.0, dtype=torch.float32, device="cuda")
    fq.fp8q_quant_act_1x128(x, q=q[:17], s=s)
    qh = host(q)
    assert np.all(qh[17:] == 0xAB)
    oq, os_ = oracle.quant_act_1x128(bits)
    assert_same(qh[:17], host(s), oq, os_, "tail")


# ------------------------------------------------------------------ weights

def test_w_tiny_workload():
    d = wl.tiny()
    say("w quant: tiny workload W [256, 512]")
    assert_same(*gpu_w(d["w"]), *oracle.quant_w_128x128(d["w"]), "tiny W")


@pytest.mark.parametrize("N,K", [(128, 128), (384, 256), (256, 1024), (1024, 384)])
def test_w_shapes(N, K):
    bits = spread_bits(N + 7 * K, N, K, 128)
    say(f"w quant: N={N} K={K}")
    assert_same(*gpu_w(bits), *oracle.quant_w_128x128(bits), f"w {N}x{K}")


def test_w_every_amax_magnitude_class():
    """128x128 blocks whose amax runs over 256 bf16 values spread across the whole exponent range."""
    g = np.random.default_rng(77)
    amaxes = np.linspace(1, 0x7F7F, 256).astype(np.uint16)
    blocks = []
    for a in amaxes:
        lim = int(a)
        blk = (g.random((128, 128)) * (lim + 1)).astype(np.int64)
        blk = np.minimum(blk, lim).astype(np.uint16)
        blk |= (g.random((128, 128)) < 0.5).astype(np.uint16) << 15
        blk[g.integers(128), g.integers(128)] = a
        blocks.append(blk)
    bits = np.concatenate(blocks, axis=0)  # [256*128, 128]
    say(f"w quant: 256 amax classes {bits.shape}")
    assert_same(*gpu_w(bits), *oracle.quant_w_128x128(bits), "w amax classes")


@pytest.mark.parametrize("name", ["up", "down"])
def test_w_full_workloads(name):
    d = {"up": lambda: wl.dense_up(M=1), "down": lambda: wl.dense_down(M=1)}[name]()
    say(f"w quant: {name} W {d['w'].shape}")
    assert_same(*gpu_w(d["w"]), *oracle.quant_w_128x128(d["w"]), name + " W")


def test_w_moe_expert_stack():
    d = wl.moe(T=256)
    say(f"w quant: moe expert stack {d['w'].shape}")
    q, s = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    oq, os_ = oracle.quant_w_128x128(d["w"])
    assert s.shape == (64, 16, 56)
    assert_same(host(q), host(s), oq, os_, "moe W")
