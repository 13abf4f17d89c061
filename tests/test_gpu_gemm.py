"""GPU parity of the block-scaled FP8 GEMM (dense, grouped, small-M) against the oracle.

Bound (per output element): |gpu - C| <= 1e-3 * B + 1e-6, with C the exact dequantized product and
B = sum_k |a_deq| |w_deq|.  fp32 outputs are held to that literal bound; bf16 outputs may carry their
own final rounding on top (2^-8 of the magnitude).  Quantized operands come from the GPU quantizers for
the GPU side and from the oracle's quantizers for the oracle side (they are bit-identical, as
test_gpu_quant checks), so each test runs the whole path end to end.
"""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import (assert_gemm_within_bound, bf16_dev, f32_dev, gemm_out_to_f64, host, literal_bound_ratio,
                      require_gpu, say, u8_dev)

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_path(a_bits, w_bits, out):
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(a_bits))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(w_bits))
    return fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=DT[out])


def oracle_path(a_bits, w_bits, rows=None, cols=None):
    qa, sa = oracle.quant_act_1x128(a_bits)
    qw, sw = oracle.quant_w_128x128(w_bits)
    return oracle.gemm_blockscaled(qa, sa, qw, sw, rows=rows, cols=cols)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_tiny_workload_all_elements(out):
    d = wl.tiny()
    say(f"gemm: tiny 128x256x512 out={out}")
    c = gemm_out_to_f64(gpu_path(d["a"], d["w"], out))
    C, B = oracle_path(d["a"], d["w"])
    r = assert_gemm_within_bound(c, C, B, out == "bf16", "tiny")
    say(f"  max err/bound {r:.3g}; literal-bound ratio {literal_bound_ratio(c, C, B):.3g}")


SHAPES = [(1, 128, 128), (7, 256, 384), (129, 384, 512), (300, 640, 1024), (257, 256, 2048), (64, 1024, 896),
          (1000, 128, 256), (33, 512, 1152), (64, 128, 2176), (65, 384, 640), (128, 256, 1280), (511, 896, 384)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_shapes_all_elements(M, N, K, out):
    g = np.random.default_rng(M + 3 * N + 7 * K)
    a = g.standard_normal((M, K)).astype(np.float32)
    a[:, g.choice(K, size=max(1, K // 100), replace=False)] *= 30.0
    a *= np.exp2(g.integers(-6, 7, size=(M, 1))).astype(np.float32)       # per-token magnitude spread
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= np.kron(np.exp2(g.integers(-4, 5, size=(N // 128, K // 128))), np.ones((128, 128))).astype(np.float32)
    ab, wb = wl.bf16_bits(a), wl.bf16_bits(w)
    say(f"gemm: M={M} N={N} K={K} out={out}")
    c = gemm_out_to_f64(gpu_path(ab, wb, out))
    C, B = oracle_path(ab, wb)
    assert_gemm_within_bound(c, C, B, out == "bf16", f"{M}x{N}x{K}")


# N -> the small-M kernel's slice (8 * ceil(N / 2048) rows, at most 80) and so its subtile count NSUB:
# 4352 -> 24 rows (NSUB 2), 6144 -> 24 (2), 8320 -> 40 (3), 10240 -> 40 (3), 12416 -> 56 (4), 16384 -> 64 (4)
@pytest.mark.parametrize("M,N,out", [(64, 4352, "bf16"), (17, 6144, "f32"), (64, 8320, "f32"), (40, 10240, "bf16"),
                                     (64, 12416, "bf16"), (1, 16384, "f32")])
def test_small_m_slice_widths(M, N, out):
    """Every subtile count of the small-M kernel, including slices that end in half a subtile."""
    K = 384
    g = np.random.default_rng([61, M, N])
    ab = wl.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wb = wl.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    say(f"gemm small-M: M={M} N={N} K={K} {out}")
    c = gemm_out_to_f64(gpu_path(ab, wb, out))
    C, B = oracle_path(ab, wb)
    assert_gemm_within_bound(c, C, B, out == "bf16", f"small-M {M}x{N}")


def test_lossless_case_matches_float64_matmul():
    """Inputs that quantize exactly (e4m3 values times one power of two per group, each group holding
    +-448 * 2^k): the GPU result must match numpy's float64 product of the bf16 inputs within the bound."""
    g = np.random.default_rng(5)
    M, N, K = 200, 384, 640
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)

    def build(rows, group_rows):
        v = torch.from_numpy(finite[g.integers(0, len(finite), size=(rows, K))]).view(
            torch.float8_e4m3fn).double().numpy()
        k = g.integers(-5, 6, size=(rows // group_rows, K // 128))
        for i in range(rows // group_rows):
            for j in range(K // 128):
                v[i * group_rows + g.integers(group_rows), j * 128 + g.integers(128)] = 448.0
        return v * np.exp2(np.kron(k, np.ones((group_rows, 128))))

    a, w = build(M, 1), build(N, 128)
    ab, wb = wl.bf16_bits(a.astype(np.float32)), wl.bf16_bits(w.astype(np.float32))
    c = gemm_out_to_f64(gpu_path(ab, wb, "f32"))
    ref = a @ w.T
    refB = np.abs(a) @ np.abs(w).T
    ratio = assert_gemm_within_bound(c, ref, refB, False, "lossless")
    # The FP8 MFMA sums its 128 products at about 2^-13 relative precision (not full fp32), which is why
    # each 128-element partial is promoted into the fp32 accumulator; the bound leaves ample margin.
    say(f"  lossless: max err/bound {ratio:.3g}, max |err|/B {np.max(np.abs(c - ref) / refB):.3g}")


def extreme_scale_operands(M, N, K, seed):
    """Codes below 1/16 in magnitude (so a 128-deep partial sum stays under 1/2) with scales that put s_a*s_w
    near both ends of the fp32 range: K-block 1 at up to 2^127 (just below the fp32 maximum), K-block 2 in
    the fp32 subnormals (about 2^-142), K-block 3 mixed (2^60 * 2^-100), the rest near 1."""
    g = np.random.default_rng(seed)
    small = np.array([c | sgn for c in range(0x18) for sgn in (0, 0x80)], np.uint8)
    qa = small[g.integers(0, len(small), (M, K))]
    qw = small[g.integers(0, len(small), (N, K))]
    sa = g.uniform(1, 2, (K // 128, M)).astype(np.float32)
    sw = g.uniform(1, 2, (N // 128, K // 128)).astype(np.float32)
    sa[1] *= np.float32(2.0 ** 62)
    sw[:, 1] *= np.float32(2.0 ** 63)
    sa[2] *= np.float32(2.0 ** -70)
    sw[:, 2] *= np.float32(2.0 ** -72)
    sa[3] *= np.float32(2.0 ** 60)
    sw[:, 3] *= np.float32(2.0 ** -100)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M", [300, 64])   # the large-M and the small-M kernel
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_scales_near_the_ends_of_the_fp32_range(M, out):
    """The promotion forms s_a * s_w in fp32; with products up to 2^127 and down into the subnormals (and
    outputs that stay finite) the result meets the bound like any other."""
    N, K = 256, 512
    qa, sa, qw, sw = extreme_scale_operands(M, N, K, 77)
    c = fq.fp8q_gemm_blockscaled(u8_dev(qa), f32_dev(sa), u8_dev(qw), f32_dev(sw), out_dtype=DT[out])
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw)
    got = gemm_out_to_f64(c)
    assert np.all(np.isfinite(got)) and np.max(np.abs(C)) > 2.0 ** 115
    ratio = assert_gemm_within_bound(got, C, B, out == "bf16", f"extreme scales M={M}")
    say(f"  extreme scales M={M} {out}: max |C| 2^{np.log2(np.max(np.abs(C))):.1f}, max err/bound {ratio:.3g}")


def test_grouped_scales_near_the_ends_of_the_fp32_range():
    """The same operands through the grouped kernel: two experts of 128 and 256 rows."""
    N, K = 256, 512
    qa, sa, qw0, sw0 = extreme_scale_operands(384, N, K, 78)
    _, _, qw1, sw1 = extreme_scale_operands(8, N, K, 79)
    qw, sw = np.stack([qw0, qw1]), np.stack([sw0, sw1])
    off = np.array([0, 128, 384], np.int32)
    c = fq.fp8q_grouped_gemm_blockscaled(u8_dev(qa), f32_dev(sa), u8_dev(qw), f32_dev(sw),
                                         torch.from_numpy(off).cuda(), out_dtype=torch.float32)
    C, B = oracle.grouped_gemm_blockscaled(qa, sa, qw, sw, off)
    got = gemm_out_to_f64(c)
    assert np.all(np.isfinite(got))
    assert_gemm_within_bound(got, C, B, False, "grouped extreme scales")


def test_deterministic():
    d = wl.tiny()
    c1 = host(gpu_path(d["a"], d["w"], "f32"))
    c2 = host(gpu_path(d["a"], d["w"], "f32"))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_repeat_calls_give_the_same_bits():
    """The small-M kernel (partial sums of 8 waves added in wave order), the mid-size-M kernel (its stage ring,
    128 and 256 token rows), the grouped kernel and its gather-fused form give bit-identical outputs on
    repeated calls, as the dense kernel does."""
    g = np.random.default_rng(9)
    K, N = 1024, 2048
    q = g.integers(0, 254, size=(300, K)).astype(np.uint8)
    q[q >= 0x7F] += 1                                      # finite codes only
    s = g.uniform(1e-4, 1e-2, size=(K // 128, 300)).astype(np.float32)
    w = wl.bf16_bits((g.standard_normal((4 * N, K)) * 0.02).astype(np.float32))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(w).view(4, N, K))
    qd, sd = u8_dev(q), f32_dev(s)
    small = [host(fq.fp8q_gemm_blockscaled(qd[:48], sd[:, :48].contiguous(), qw[0], sw[0])) for _ in range(3)]
    mid = [host(fq.fp8q_gemm_blockscaled(qd[:m], sd[:, :m].contiguous(), qw[1], sw[1], out_dtype=torch.float32))
           for m in (100, 100, 100, 200, 200, 200)]
    off = torch.tensor([0, 128, 128, 256, 256], dtype=torch.int32, device="cuda")
    grouped = [host(fq.fp8q_grouped_gemm_blockscaled(qd[:256], sd[:, :256].contiguous(), qw, sw, off))
               for _ in range(3)]
    rt = torch.from_numpy(g.integers(-1, 300, size=256).astype(np.int32)).cuda()
    gathered = [host(fq.fp8q_grouped_gemm_blockscaled_gather(qd, sd, rt, qw, sw, off, out_dtype=torch.float32))
                for _ in range(3)]
    for runs in (small, mid[:3], mid[3:], grouped, gathered):
        for r in runs[1:]:
            assert np.array_equal(r.view(np.uint8), runs[0].view(np.uint8))


def test_output_untouched_beyond_M():
    d = wl.tiny()
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(d["a"][:100]))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    c = torch.full((128, 256), 3.0, dtype=torch.float32, device="cuda")
    fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=torch.float32, c=c[:100])
    assert np.all(host(c)[100:] == 3.0)


def sample_rows(M, n, seed):
    g = np.random.default_rng(seed)
    rows = set([0, M - 1, M // 2]) | set(g.choice(M, size=min(M, n), replace=False).tolist())
    return np.array(sorted(rows))


# Whole 256-row x 256-column output blocks checked element by element at full K: (first row, first column).
# Up (N = 18432) runs 256 x 256 tiles over columns [0, 16384) and 256 x 128 tiles over the rest; down
# (N = 7168) 256 x 256 tiles over [0, 4096) and 256 x 192 tiles over the rest, so the blocks below cover a
# main tile, a block straddling the last main and first tail column, and the last tail tiles.
WHOLE_TILES = {"up": [(1792, 8192), (3840, 16256), (0, 18176)],
               "down": [(2048, 1024), (1792, 3968), (3840, 6912)]}


@pytest.mark.parametrize("name,out", [("up", "bf16"), ("up", "f32"), ("down", "bf16"), ("down", "f32")])
def test_full_size_dense_sampled(name, out):
    """Full-size FFN projections: every output column of sampled rows, every row of sampled columns, and whole
    256 x 256 output blocks (every element of a tile at full K).  bf16 outputs also report the literal
    bound's ratio (without the allowance for their own final rounding)."""
    d = wl.dense_up() if name == "up" else wl.dense_down()
    if name == "down":   # A = bf16(SiLU(x) * y), from the oracle
        d["a"] = oracle.swiglu_bf16(d["x"], d["y"])
    say(f"gemm: full {name} {d['M']}x{d['N']}x{d['K']} out={out}")
    c = gemm_out_to_f64(gpu_path(d["a"], d["w"], out))
    rows = sample_rows(d["M"], 16, 1)
    cols = sample_rows(d["N"], 8, 2)
    qa, sa = oracle.quant_act_1x128(d["a"])
    qw, sw = oracle.quant_w_128x128(d["w"])
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, rows=rows)
    r1 = assert_gemm_within_bound(c[rows], C, B, out == "bf16", f"{name} rows")
    lit = [literal_bound_ratio(c[rows], C, B)]
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, cols=cols)
    r2 = assert_gemm_within_bound(c[:, cols], C, B, out == "bf16", f"{name} cols")
    lit.append(literal_bound_ratio(c[:, cols], C, B))
    r3 = 0.0
    for m0, n0 in WHOLE_TILES[name]:
        tr, tc = np.arange(m0, m0 + 256), np.arange(n0, n0 + 256)
        C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, rows=tr, cols=tc)
        got = c[m0:m0 + 256, n0:n0 + 256]
        r3 = max(r3, assert_gemm_within_bound(got, C, B, out == "bf16", f"{name} block ({m0}, {n0})"))
        lit.append(literal_bound_ratio(got, C, B))
    say(f"  max err/bound rows {r1:.3g} cols {r2:.3g} whole blocks {r3:.3g}; literal-bound ratio {max(lit):.3g}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_small_m_full_size(out):
    """Decode shape (M = 64) with pre-quantized weights; every output element is checked."""
    d = wl.decode()
    say(f"gemm: decode 64x18432x7168 out={out}")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(d["a"]))
    c = gemm_out_to_f64(fq.fp8q_gemm_blockscaled(qa, sa, u8_dev(d["wq"]), f32_dev(d["sw"]), out_dtype=DT[out]))
    oqa, osa = oracle.quant_act_1x128(d["a"])
    C, B = oracle.gemm_blockscaled(oqa, osa, d["wq"], d["sw"])
    r = assert_gemm_within_bound(c, C, B, out == "bf16", "decode")
    say(f"  max err/bound {r:.3g}; literal-bound ratio {literal_bound_ratio(c, C, B):.3g}")


# N -> slice rows as for the small-M kernel; the mid-size-M kernel (64 < M <= 256) takes every token row in one
# workgroup (128 or 256 of them): 256 -> 8 rows (NSUB 1), 4352 -> 24 (2), 8320 -> 40 (3), 12416 -> 56 (4),
# 18432 -> 72 (5).  K = 128, 256 and 384 leave fewer K-blocks than the copies run ahead.
@pytest.mark.parametrize("M,N,K,out", [(65, 256, 384, "f32"), (128, 4352, 384, "bf16"), (96, 8320, 128, "f32"),
                                       (100, 12416, 384, "bf16"), (127, 18432, 640, "f32"), (128, 18432, 256, "bf16"),
                                       (129, 256, 128, "bf16"), (256, 4352, 640, "f32"), (200, 8320, 256, "bf16"),
                                       (255, 12416, 384, "f32"), (192, 18432, 512, "bf16")])
def test_mid_m_slice_widths(M, N, K, out):
    """Every subtile count of the mid-size-M kernel for both token-row counts, ragged token counts and short
    K."""
    g = np.random.default_rng([67, M, N, K])
    a = g.standard_normal((M, K)).astype(np.float32)
    a *= np.exp2(g.integers(-6, 7, size=(M, 1))).astype(np.float32)
    ab = wl.bf16_bits(a)
    wb = wl.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    say(f"gemm: mid-size M={M} N={N} K={K} out={out}")
    c = gemm_out_to_f64(gpu_path(ab, wb, out))
    C, B = oracle_path(ab, wb)
    assert_gemm_within_bound(c, C, B, out == "bf16", f"mid-size {M}x{N}x{K}")


@pytest.mark.parametrize("M,out", [(128, "f32"), (96, "bf16"), (256, "bf16"), (160, "f32")])
def test_mid_m_full_size(M, out):
    """M tokens against the decode workload's pre-quantized 18432 x 7168 weight; every output element is
    checked."""
    d = wl.decode()
    g = np.random.default_rng([68, M])
    ab = wl.bf16_bits(g.standard_normal((M, 7168)).astype(np.float32))
    say(f"gemm: mid-size {M}x18432x7168 out={out}")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    c = gemm_out_to_f64(fq.fp8q_gemm_blockscaled(qa, sa, u8_dev(d["wq"]), f32_dev(d["sw"]), out_dtype=DT[out]))
    oqa, osa = oracle.quant_act_1x128(ab)
    C, B = oracle.gemm_blockscaled(oqa, osa, d["wq"], d["sw"])
    r = assert_gemm_within_bound(c, C, B, out == "bf16", "mid-size full")
    say(f"  max err/bound {r:.3g}; literal-bound ratio {literal_bound_ratio(c, C, B):.3g}")


# ------------------------------------------------------------------ grouped (MoE)

def grouped_case(seed, counts, N, K):
    """Segments of the given routed-row counts, padded to 128 with zero rows."""
    g = np.random.default_rng(seed)
    E = len(counts)
    padded = [((c + 127) // 128) * 128 for c in counts]
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    M = int(off[-1])
    a = np.zeros((M, K), np.float32)
    for e, cnt in enumerate(counts):
        a[off[e]:off[e] + cnt] = g.standard_normal((cnt, K))
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    return wl.bf16_bits(a), wl.bf16_bits(w), off


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_grouped_skewed_with_empty_expert(out):
    counts = [300, 0, 1, 128, 129, 700]
    ab, wb, off = grouped_case(21, counts, 256, 512)
    say(f"grouped gemm: counts {counts} out={out}")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(wb))
    c = gemm_out_to_f64(fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).cuda(),
                                                         out_dtype=DT[out]))
    oqa, osa = oracle.quant_act_1x128(ab)
    oqw, osw = oracle.quant_w_128x128(wb)
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, off)
    assert_gemm_within_bound(c, C, B, out == "bf16", "grouped")
    for e, cnt in enumerate(counts):                       # padding rows are exactly zero
        assert np.all(c[off[e] + cnt:off[e + 1]] == 0.0)


@pytest.mark.parametrize("E", [130, 256])
def test_grouped_more_than_64_experts(E):
    """A tile's expert is found by a prefix sum over the offsets, 64 experts per pass: with 130 and 256
    experts (DeepSeek-V3 routes over 256) the tiles of experts in every pass, the empty experts between them
    and a partial last pass must all land on the right weights."""
    g = np.random.default_rng(E)
    counts = g.integers(0, 300, size=E)
    counts[g.random(E) < 0.4] = 0                           # many empty experts
    counts[[0, 63, 64, 127, 128, E - 1]] = [5, 260, 128, 1, 257, 40]
    ab, wb, off = grouped_case(31, counts.tolist(), 128, 256)
    say(f"grouped gemm: E={E} experts, {int(off[-1])} rows")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(wb))
    c = gemm_out_to_f64(fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).cuda(),
                                                         out_dtype=torch.float32))
    oqa, osa = oracle.quant_act_1x128(ab)
    oqw, osw = oracle.quant_w_128x128(wb)
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, off)
    assert_gemm_within_bound(c, C, B, False, f"grouped, {E} experts")
    for e, cnt in enumerate(counts):                       # padding rows are exactly zero
        assert np.all(c[off[e] + cnt:off[e + 1]] == 0.0)


def test_grouped_offsets_outside_the_rules():
    """Offsets that break the layout rules (the header's promise for them): segments that end before
    M_total leave the rows after them untouched, and a last offset past M_total is cut at M_total."""
    K, N, M = 512, 256, 1024
    g = np.random.default_rng(5)
    ab = wl.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wb = wl.bf16_bits((g.standard_normal((2, N, K)) * 0.02).astype(np.float32))
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(wb))
    oqa, osa = oracle.quant_act_1x128(ab)
    oqw, osw = oracle.quant_w_128x128(wb)
    # segments [0, 384) and [384, 640) of a 1024-row buffer: rows 640.. keep the sentinel
    say("grouped gemm: segments ending at 640 of 1024 rows")
    off = np.array([0, 384, 640], np.int32)
    c = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).cuda(), out_dtype=torch.float32, c=c)
    ch = gemm_out_to_f64(c)
    assert np.all(ch[640:] == 7.0)
    C, B = oracle.grouped_gemm_blockscaled(oqa[:640], osa[:, :640], oqw, osw, off)
    assert_gemm_within_bound(ch[:640], C, B, False, "short segments")
    # a last offset of 2048 for a 1024-row buffer: expert 1 covers rows [256, 1024)
    say("grouped gemm: last offset 2048 for 1024 rows")
    off = np.array([0, 256, 2048], np.int32)
    c = fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).cuda(), out_dtype=torch.float32)
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, np.array([0, 256, M], np.int32))
    assert_gemm_within_bound(gemm_out_to_f64(c), C, B, False, "offset past M_total")


@pytest.mark.parametrize("offs", [[0, 1, 2, 3, 300, 301, 384, 512], list(range(0, 129, 2))],
                         ids=["7_experts_ragged", "64_experts_of_2_rows"])
def test_grouped_segments_of_any_length(offs):
    """Offsets that never decrease but are not multiples of 128 rows: each segment's rows are cut into its own
    tiles (one or two rows can be a whole tile), so there can be more tiles than M_total / 256 + E / 2; every
    row must still be computed with its own expert (the oracle takes any non-decreasing offsets), by the
    grouped GEMM and by its gather form (identity row map, bit-identical)."""
    off = np.array(offs, np.int32)
    E, M = len(off) - 1, int(off[-1])
    K, N = 256, 256
    g = np.random.default_rng(len(offs))
    ab = wl.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wb = wl.bf16_bits((g.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    say(f"grouped gemm: {E} segments of {np.diff(off).min()}..{np.diff(off).max()} rows, M_total={M}")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(wb))
    od = torch.from_numpy(off).cuda()
    c1 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, od, out_dtype=torch.float32, c=c1)
    c2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled_gather(qa, sa, torch.arange(M, dtype=torch.int32, device="cuda"), qw, sw, od,
                                            out_dtype=torch.float32, c=c2)
    oqa, osa = oracle.quant_act_1x128(ab)
    oqw, osw = oracle.quant_w_128x128(wb)
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, off)
    assert_gemm_within_bound(gemm_out_to_f64(c1), C, B, False, "segments of any length")
    assert np.array_equal(host(c1).view(np.uint32), host(c2).view(np.uint32))


def test_grouped_gather_with_offsets_outside_the_rules():
    """The gather-reading grouped GEMM under the same broken offsets (short, past M_total, decreasing), with
    the identity row map over 1024 token rows: bit-identical to the grouped GEMM on the same rows, including
    the rows each leaves untouched."""
    K, N, M = 512, 256, 1024
    g = np.random.default_rng(6)
    ab = wl.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wb = wl.bf16_bits((g.standard_normal((2, N, K)) * 0.02).astype(np.float32))
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(ab))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(wb))
    rt = torch.arange(M, dtype=torch.int32, device="cuda")
    for offs in ([0, 384, 640], [0, 256, 2048], [0, 512, 256], [0, 0, 0]):
        say(f"grouped gemm, gather form: offsets {offs}")
        off = torch.tensor(offs, dtype=torch.int32, device="cuda")
        c1 = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
        c2 = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
        fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, off, out_dtype=torch.float32, c=c1)
        fq.fp8q_grouped_gemm_blockscaled_gather(qa, sa, rt, qw, sw, off, out_dtype=torch.float32, c=c2)
        assert np.array_equal(host(c1).view(np.uint32), host(c2).view(np.uint32)), offs


def test_grouped_full_moe_sampled():
    """The full MoE layer: 8192 tokens, top-8 of 64 experts, expert weights [2048, 7168]; sampled rows
    from every expert segment (first, last routed row and a random one), all 2048 columns."""
    d = wl.moe()
    r = oracle.moe_route_topk(d["logits"], d["topk"])       # the expert-sorted layout, from the oracle
    a = np.zeros((r.M, d["K"]), np.uint16)
    a[r.row_token >= 0] = d["tokens"][r.row_token[r.row_token >= 0]]
    d["a"] = a
    say(f"grouped gemm: full moe M_total={r.M} (counts {r.counts.min()}..{r.counts.max()})")
    qa, sa = fq.fp8q_quant_act_1x128(bf16_dev(d["a"]))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    c = gemm_out_to_f64(fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(r.offsets).cuda()))
    g = np.random.default_rng(3)
    rows = []
    for e in range(d["E"]):
        lo, cnt = int(r.offsets[e]), int(r.counts[e])
        if cnt:
            rows += [lo, lo + cnt - 1, lo + int(g.integers(cnt))]
    rows = np.array(sorted(set(rows)))
    oqa, osa = oracle.quant_act_1x128(d["a"])
    oqw, osw = oracle.quant_w_128x128(d["w"])
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, r.offsets, rows=rows)
    ratio = assert_gemm_within_bound(c[rows], C, B, True, "moe")
    pad = r.row_token < 0
    assert np.all(c[pad] == 0.0)
    say(f"  max err/bound {ratio:.3g}")


@pytest.mark.parametrize("M,N,K", [(1280, 2048, 256), (4352, 1024, 256), (768, 4096, 384), (8960, 2816, 128)],
                         ids=["5x8_tiles", "17x4_tiles", "3x16_tiles", "35x11_tiles"])
def test_tile_grids_that_are_not_whole_supergroups(M, N, K):
    """Every output of grids whose tile counts are not multiples of 16 (partial 16 x 16 supergroups in M, in
    N or both): the tile order must still cover each tile once."""
    g = np.random.default_rng(M * 7 + N)
    a = g.standard_normal((M, K)).astype(np.float32)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    ab, wb = wl.bf16_bits(a), wl.bf16_bits(w)
    say(f"gemm tile grid: M={M} N={N} K={K}")
    c = gemm_out_to_f64(gpu_path(ab, wb, "f32"))
    qa, sa = oracle.quant_act_1x128(ab)
    qw, sw = oracle.quant_w_128x128(wb)
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw)
    assert_gemm_within_bound(c, C, B, False, f"{M}x{N}")


@pytest.mark.parametrize("M,N,K", [(2304, 7168, 256), (2048, 7168, 256), (300, 640, 1024), (4096, 7168, 256),
                                   (1024, 18432, 256)],
                         ids=["w256", "w224", "w192", "w256+tail192", "w192+tail128"])
def test_large_m_tile_widths(M, N, K):
    """Shapes for which the large-M kernel's launch plan takes each of its tile widths: 256, 224 and 192
    weight rows alone, and 256 (192) wide tiles over the leading columns followed by 192 (128) wide tiles over
    the rest, starting at column 4096 (12288).  The narrower widths have waves whose weight rows straddle a
    128-row scale block, and the tail tiles start at columns that are not multiples of 128 rows' blocks of
    the main width."""
    g = np.random.default_rng(M + N)
    a = g.standard_normal((M, K)).astype(np.float32)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= np.kron(np.exp2(g.integers(-3, 4, size=(N // 128, K // 128))), np.ones((128, 128))).astype(np.float32)
    ab, wb = wl.bf16_bits(a), wl.bf16_bits(w)
    say(f"gemm tile widths: M={M} N={N} K={K}")
    c = gemm_out_to_f64(gpu_path(ab, wb, "f32"))
    qa, sa = oracle.quant_act_1x128(ab)
    qw, sw = oracle.quant_w_128x128(wb)
    rows = sample_rows(M, 12, 5)
    cols = np.unique(np.concatenate([sample_rows(N, 24, 6), np.arange(0, N, 32)]))  # every 32nd column too
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, rows=rows)
    assert_gemm_within_bound(c[rows], C, B, False, f"{M}x{N} rows")
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, cols=cols)
    assert_gemm_within_bound(c[:, cols], C, B, False, f"{M}x{N} cols")
