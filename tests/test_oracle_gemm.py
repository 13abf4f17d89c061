"""Pins for the oracle's block-scaled GEMM (dense and grouped).

Definition (page "The Definitive Information To Deepseek": the GEMMs take FP8 inputs and produce
BF16/FP32 outputs; partial sums are promoted with the per-block scales): C = A_deq @ W_deq^T where
each element is its E4M3 value times its 1x128 (activation) or 128x128 (weight) group scale.
Pins: a hand-worked product (tests/golden/hand_cases.json); a lossless special case whose result is
numpy's float64 matmul of the bf16 inputs; exact rational sums (fractions.Fraction) on tiny shapes;
and padded rows of the grouped GEMM being exactly zero.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def e4m3_values_torch(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lossless_matrix(g, rows, cols, group_rows, exps):
    """Values e4m3 * 2^k per group (group = group_rows x 128 tile), each group holding +-448 * 2^k, so
    quantization with scale amax/448 = 2^k is exact.  Returns float64 values (exactly bf16)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    codes = finite[g.integers(0, len(finite), size=(rows, cols))]
    v = e4m3_values_torch(codes)
    v[g.random((rows, cols)) < 0.1] = 0.0
    gr, gc = rows // group_rows, cols // 128
    k = g.integers(exps[0], exps[1] + 1, size=(gr, gc))
    for i in range(gr):
        for j in range(gc):
            r = i * group_rows + g.integers(0, group_rows)
            c = j * 128 + g.integers(0, 128)
            v[r, c] = 448.0 if g.random() < 0.5 else -448.0
    return v * np.exp2(np.kron(k, np.ones((group_rows, 128)))), k


def bits_of(v):
    b = wl.bf16_bits(v.astype(np.float32))
    assert np.array_equal(wl.bf16_to_f32(b).astype(np.float64), v), "construction must be bf16-exact"
    return b


def test_hand_worked_gemm(olib):
    case = json.load(open(GOLDEN))["gemm"][0]
    a = np.zeros((case["M"], case["K"]), np.float32)
    w = np.zeros((case["N"], case["K"]), np.float32)
    for i, j, v in case["a_entries"]:
        a[i, j] = v
    for i, j, v in case["w_entries"]:
        w[i, j] = v
    qa, sa = oracle.quant_act_1x128(wl.bf16_bits(a), lib=olib)
    qw, sw = oracle.quant_w_128x128(wl.bf16_bits(w), lib=olib)
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, lib=olib)
    want = np.full((case["M"], case["N"]), case["rest_c"])
    for i, j, v in case["c_entries"]:
        want[i, j] = v
    assert np.array_equal(C, want)
    assert np.array_equal(B, np.abs(want))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 256, 384), (130, 384, 512)])
def test_lossless_case_equals_float64_matmul(olib, M, N, K):
    g = np.random.default_rng(M * 7 + N + K)
    a, ka = lossless_matrix(g, M, K, 1, (-8, 8))
    w, kw = lossless_matrix(g, N, K, 128, (-8, 8))
    qa, sa = oracle.quant_act_1x128(bits_of(a), lib=olib)
    qw, sw = oracle.quant_w_128x128(bits_of(w), lib=olib)
    assert np.array_equal(sa, np.exp2(ka.T).astype(np.float32))      # s_a[kb, m] = 2^k(m, kb)
    assert np.array_equal(sw, np.exp2(kw).astype(np.float32))        # s_w[nb, kb]
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, lib=olib)
    ref = a @ w.T
    refB = np.abs(a) @ np.abs(w).T
    assert np.all(np.abs(C - ref) <= 1e-12 * refB + 1e-300)
    assert np.allclose(B, refB, rtol=1e-12, atol=0)


@pytest.mark.parametrize("M,K", [(1, 128), (2, 256), (3, 128)])
def test_exact_rational_brute_force(olib, M, K):
    N = 256
    g = np.random.default_rng(100 + M + K)
    a = g.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    w = g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    a[:, ::17] *= np.float32(40.0)
    qa, sa = oracle.quant_act_1x128(wl.bf16_bits(a), lib=olib)
    qw, sw = oracle.quant_w_128x128(wl.bf16_bits(w), lib=olib)
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, lib=olib)
    va = [[Fraction(float(x)) for x in row] for row in e4m3_values_torch(qa)]
    vw = [[Fraction(float(x)) for x in row] for row in e4m3_values_torch(qw)]
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            absum = Fraction(0)
            for k in range(K):
                t = va[m][k] * Fraction(float(sa[k // 128, m])) * vw[n][k] * Fraction(float(sw[n // 128, k // 128]))
                exact += t
                absum += abs(t)
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(1, 10 ** 12) * absum
            assert abs(Fraction(B[m, n]) - absum) <= Fraction(1, 10 ** 12) * absum


def test_row_and_column_selection(olib):
    g = np.random.default_rng(9)
    qa, sa = oracle.quant_act_1x128(wl.bf16_bits(g.standard_normal((50, 256)).astype(np.float32)), lib=olib)
    qw, sw = oracle.quant_w_128x128(wl.bf16_bits(g.standard_normal((384, 256)).astype(np.float32)), lib=olib)
    C, B = oracle.gemm_blockscaled(qa, sa, qw, sw, lib=olib)
    Cr, Br = oracle.gemm_blockscaled(qa, sa, qw, sw, rows=[49, 0, 17], lib=olib)
    Cc, Bc = oracle.gemm_blockscaled(qa, sa, qw, sw, cols=[383, 128, 5], lib=olib)
    assert np.array_equal(Cr, C[[49, 0, 17]]) and np.array_equal(Br, B[[49, 0, 17]])
    assert np.array_equal(Cc, C[:, [383, 128, 5]]) and np.array_equal(Bc, B[:, [383, 128, 5]])


def test_grouped_lossless_and_padding(olib):
    """Three experts with segments of 256, 0 and 128 rows; padded rows are all-zero and give exactly 0."""
    g = np.random.default_rng(11)
    E, N, K = 3, 256, 256
    offsets = np.array([0, 256, 256, 384], np.int32)
    a, _ = lossless_matrix(g, 384, K, 1, (-6, 6))
    a[200:256] = 0.0        # padding rows of expert 0
    a[300:384] = 0.0        # padding rows of expert 2
    ws = [lossless_matrix(g, N, K, 128, (-6, 6))[0] for _ in range(E)]
    qa, sa = oracle.quant_act_1x128(bits_of(a), lib=olib)
    qw, sw = oracle.quant_w_128x128(np.stack([bits_of(w) for w in ws]), lib=olib)
    C, B = oracle.grouped_gemm_blockscaled(qa, sa, qw, sw, offsets, lib=olib)
    ref = np.concatenate([a[0:256] @ ws[0].T, a[256:384] @ ws[2].T])
    refB = np.concatenate([np.abs(a[0:256]) @ np.abs(ws[0]).T, np.abs(a[256:384]) @ np.abs(ws[2]).T])
    assert np.all(np.abs(C - ref) <= 1e-12 * refB + 1e-300)
    assert np.all(C[200:256] == 0) and np.all(C[300:384] == 0)
    assert np.all(B[200:256] == 0)


def test_grouped_rejects_bad_offsets(olib):
    qa = np.zeros((256, 128), np.uint8)
    sa = np.zeros((1, 256), np.float32)
    qw = np.zeros((2, 128, 128), np.uint8)
    sw = np.zeros((2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_blockscaled(qa, sa, qw, sw, np.array([0, 200, 128], np.int32), lib=olib)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_blockscaled(qa, sa, qw, sw, np.array([0, 128, 200], np.int32), lib=olib)
