"""GPU parity at the largest sizes: operands and outputs beyond 4 GiB, so that every kernel's byte offsets
pass 2^32 (and its 32-bit buffer offsets must stay relative to a tile or row base).  Inputs are drawn on
the device from seeded torch generators (random bf16 values, or random finite E4M3 codes and scales); the
oracle sees host copies of the sampled rows, blocks or columns, which include the rows on both sides of
each 2^32-byte boundary.  The GEMMs also run at the largest K they accept (2^23), where a tile's 32-bit
offsets come closest to their limit."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
from gpu_util import assert_gemm_within_bound, gemm_out_to_f64, host, say

pytestmark = pytest.mark.gpu

K = 7168
BIG = 600064                    # rows: BIG * K > 2^32 codes, and 2 BIG * K > 2^32 bytes of bf16 well before the end
GiB4 = 2 ** 32


def boundary_rows(row_bytes, n):
    """Rows 0 and n-1, the rows on both sides of each 2^32-byte boundary of rows of `row_bytes` bytes, and a
    few seeded others."""
    rows = {0, 1, n - 2, n - 1}
    b = GiB4
    while b < n * row_bytes:
        r = b // row_bytes
        rows |= {r - 1, r, r + 1}
        b += GiB4
    rows |= set(np.random.default_rng(n).integers(0, n, 6).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n))


def bf16_matrix(rows, seed, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((rows, K), device="cuda", generator=g, dtype=torch.float32)
    x.mul_(scale)
    return x.to(torch.bfloat16)


def e4m3_codes(rows, seed):
    """Random finite E4M3 codes (0x7F and 0xFF, the NaNs, left out)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    r = torch.randint(0, 254, (rows, K), device="cuda", generator=g, dtype=torch.int16)
    return (r + (r >= 127).to(torch.int16)).to(torch.uint8)


def scales(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.rand(shape, device="cuda", generator=g) * 1e-2 + 1e-4


@pytest.fixture(autouse=True)
def free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_act_quant_past_4gib():
    x = bf16_matrix(BIG, 101)
    say(f"large: act quant [{BIG}, {K}] ({x.numel() * 2 / 2**30:.1f} GiB in, {x.numel() / 2**30:.1f} GiB codes)")
    q, s = fq.fp8q_quant_act_1x128(x)
    rows = np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K, BIG))
    ri = torch.from_numpy(rows).cuda()
    oq, os_ = oracle.quant_act_1x128(host(x[ri]))
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[:, ri]).view(np.uint32), os_.view(np.uint32))


def test_weight_quant_past_4gib():
    w = bf16_matrix(BIG, 102, 0.02)
    say(f"large: weight quant [{BIG}, {K}]")
    q, s = fq.fp8q_quant_w_128x128(w)
    blocks = np.unique(np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K, BIG)) // 128)
    for nb in blocks:
        r = slice(128 * nb, 128 * nb + 128)
        oq, os_ = oracle.quant_w_128x128(host(w[r]))
        assert np.array_equal(host(q[r]), oq), f"block {nb}"
        assert np.array_equal(host(s[nb:nb + 1]).view(np.uint32), os_.view(np.uint32)), f"block {nb}"


def test_per_channel_quant_past_4gib():
    w = bf16_matrix(BIG, 103, 0.02)
    say(f"large: per-channel quant [{BIG}, {K}]")
    q, s = fq.fp8q_quant_w_per_channel(w)
    rows = np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K, BIG))
    ri = torch.from_numpy(rows).cuda()
    oq, os_ = oracle.quant_w_per_channel(host(w[ri]))
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[ri]).view(np.uint32), os_.view(np.uint32))


def test_dequant_past_4gib():
    q = e4m3_codes(BIG, 104)
    s = scales((BIG // 128, K // 128), 105)
    say(f"large: dequant [{BIG}, {K}] -> {q.numel() * 2 / 2**30:.1f} GiB bf16")
    w = fq.fp8q_dequant_w_128x128(q, s)
    blocks = np.unique(np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K, BIG)) // 128)
    for nb in blocks:
        r = slice(128 * nb, 128 * nb + 128)
        ow = oracle.dequant_w_128x128(host(q[r]), host(s[nb:nb + 1]))
        assert np.array_equal(host(w[r]), ow), f"block {nb}"


@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_gemm_activation_past_4gib(out):
    """A [600064, 7168] codes (4.0 GiB) x W [256, 7168]: rows on both sides of the 2^32-byte boundary."""
    N = 256
    qa, sa = e4m3_codes(BIG, 106), scales((K // 128, BIG), 107)
    qw, sw = e4m3_codes(N, 108), scales((N // 128, K // 128), 109)
    say(f"large: gemm A [{BIG}, {K}] x W [{N}, {K}] -> {out}")
    c = fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=out)
    rows = boundary_rows(K, BIG)
    ri = torch.from_numpy(rows).cuda()
    C, B = oracle.gemm_blockscaled(host(qa[ri]), host(sa[:, ri]), host(qw), host(sw))
    ratio = assert_gemm_within_bound(gemm_out_to_f64(c[ri]), C, B, out == torch.bfloat16, "A past 4 GiB")
    say(f"  max err/bound {ratio:.3g}")


@pytest.mark.parametrize("M", [512, 256, 64])
def test_gemm_weight_past_4gib(M):
    """W [600064, 7168] codes (4.0 GiB) with M = 512 (large-M kernel), M = 256 (mid-size-M kernel) and M = 64
    (small-M kernel): the 128-row weight blocks on both sides of the 2^32-byte boundary and the last one."""
    qa, sa = e4m3_codes(M, 110), scales((K // 128, M), 111)
    qw, sw = e4m3_codes(BIG, 112), scales((BIG // 128, K // 128), 113)
    say(f"large: gemm A [{M}, {K}] x W [{BIG}, {K}]")
    c = fq.fp8q_gemm_blockscaled(qa, sa, qw, sw)
    blocks = np.unique(boundary_rows(K, BIG) // 128)
    ha, hs = host(qa), host(sa)
    for nb in blocks:
        r = slice(128 * nb, 128 * nb + 128)
        C, B = oracle.gemm_blockscaled(ha, hs, host(qw[r]), host(sw[nb:nb + 1]))
        assert_gemm_within_bound(gemm_out_to_f64(c[:, r].contiguous()), C, B, True, f"W block {nb}")


def test_swiglu_quant_past_4gib():
    """Gate and up as the halves of one bf16 [300032, 14336] tensor (8.0 GiB): rows past 2^32 bytes."""
    M = 300032
    both = bf16_matrix(2 * M, 114).view(M, 2 * K)
    say(f"large: swiglu quant [{M}, {2 * K}]")
    q, s = fq.fp8q_swiglu_quant_act_1x128(both)
    rows = boundary_rows(4 * K, M)
    ri = torch.from_numpy(rows).cuda()
    hb = host(both[ri])
    oq, os_ = oracle.swiglu_quant_1x128(hb[:, :K], hb[:, K:])
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[:, ri]).view(np.uint32), os_.view(np.uint32))


def test_dual_copies_past_4gib():
    """x [600064, 7168]: its backward copy x^T [7168, 600064] (4.0 GiB) on the 128-token blocks on both sides
    of the 2^32-byte boundaries, and the forward copy's rows."""
    x = bf16_matrix(BIG, 115)
    say(f"large: dual copies [{BIG}, {K}]")
    q, s, qt, st = fq.fp8q_quant_act_dual(x)
    rows = np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K, BIG))
    ri = torch.from_numpy(rows).cuda()
    oq, os_ = oracle.quant_act_1x128(host(x[ri]))
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[:, ri]).view(np.uint32), os_.view(np.uint32))
    # qt[k, m] sits at byte k * BIG + m: the channels on both sides of each 2^32 boundary, in a few blocks
    for mb in np.unique(rows // 128):
        r = slice(128 * mb, 128 * mb + 128)
        oqt, ost = oracle.quant_act_backward_copy(host(x[r]))
        assert np.array_equal(host(qt[:, r].contiguous()), oqt), f"token block {mb}"
        assert np.array_equal(host(st[mb:mb + 1]).view(np.uint32), ost.view(np.uint32)), f"token block {mb}"


def test_fp4_quant_past_4gib():
    """FP4 in the 1x128 and 128x128 groups over a bf16 input of 8.0 GiB (codes: 2.0 GiB)."""
    x = bf16_matrix(BIG, 116)
    say(f"large: fp4 quant [{BIG}, {K}]")
    q, s = fq.fp8q_quant_act_fp4_1x128(x)
    rows = np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K // 2, BIG))
    ri = torch.from_numpy(rows).cuda()
    oq, os_ = oracle.quant_act_fp4_1x128(host(x[ri]))
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[:, ri]).view(np.uint32), os_.view(np.uint32))
    del q, s
    q, s = fq.fp8q_quant_w_fp4_128x128(x)
    for nb in np.unique(rows // 128):
        r = slice(128 * nb, 128 * nb + 128)
        oq, os_ = oracle.quant_w_fp4_128x128(host(x[r]))
        assert np.array_equal(host(q[r]), oq), f"block {nb}"
        assert np.array_equal(host(s[nb:nb + 1]).view(np.uint32), os_.view(np.uint32)), f"block {nb}"


def test_e5m6_quant_past_4gib():
    """E5M6 codes of [600064, 7168] (6.0 GiB of packed codes): rows on both sides of every 2^32-byte boundary
    of the input and of the codes."""
    x = bf16_matrix(BIG, 117)
    say(f"large: e5m6 quant [{BIG}, {K}]")
    q, s = fq.fp8q_quant_act_e5m6_1x128(x)
    rows = np.union1d(boundary_rows(2 * K, BIG), boundary_rows(K // 2 * 3, BIG))
    ri = torch.from_numpy(rows).cuda()
    oq, os_ = oracle.quant_act_e5m6_1x128(host(x[ri]))
    assert np.array_equal(host(q[ri]), oq)
    assert np.array_equal(host(s[:, ri]).view(np.uint32), os_.view(np.uint32))


KMAX = 2 ** 23                  # the largest K the GEMMs accept: a 256-row tile then spans 2^31 bytes


def codes_k(rows, k, seed):
    """Random finite E4M3 codes [rows, k] (the NaN codes left out)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    r = torch.randint(0, 254, (rows, k), device="cuda", generator=g, dtype=torch.int16)
    return (r + (r >= 127).to(torch.int16)).to(torch.uint8)


# the large-M kernel (a whole and a partial M tile), the mid-size-M kernel (256 and 128 token rows), small-M
@pytest.mark.parametrize("M", [300, 256, 100, 64])
def test_gemm_at_the_largest_k(M):
    """K = 2^23 (65,536 K-blocks): the last row of a 256-row tile starts 255 * 2^23 bytes into it, so the
    per-lane buffer offsets reach 2^31 - 16.  Sampled rows (both ends of each M tile) x sampled columns of
    both 128-row weight blocks.  (Summing 65,536 promoted partials in fp32 has a worst-case rounding error
    of about 4e-3 B, above the bound; random signs keep the actual error far below it.)"""
    N = 256
    qa, sa = codes_k(M, KMAX, 120), scales((KMAX // 128, M), 121)
    qw, sw = codes_k(N, KMAX, 122), scales((N // 128, KMAX // 128), 123)
    say(f"large: gemm A [{M}, 2^23] x W [{N}, 2^23]")
    c = fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=torch.float32)
    rows = np.array(sorted({0, 1, min(255, M - 1), M - 1} | ({256, 257} if M > 256 else set())))
    cols = np.array([0, 5, 127, 128, 200, 255])
    ri = torch.from_numpy(rows).cuda()
    ha, hs = host(qa[ri]), host(sa[:, ri])
    del qa, sa
    C, B = oracle.gemm_blockscaled(ha, hs, host(qw), host(sw), cols=cols)
    got = gemm_out_to_f64(c[ri][:, torch.from_numpy(cols).cuda()])
    ratio = assert_gemm_within_bound(got, C, B, False, f"K = 2^23, M = {M}")
    say(f"  max err/bound {ratio:.3g}")
