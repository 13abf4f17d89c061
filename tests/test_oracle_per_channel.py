"""Pins of the oracle's per-channel FP8 weights (one scale per output channel over the whole row).
Independent of the oracle's code: scales and quotients recomputed in numpy float32 with the pinned E4M3
encoder, a hand-worked row, and the relation to the 1x128 quantizer when K is 128."""
import numpy as np

import oracle


def test_hand_worked_row(olib):
    """A row whose amax is 896 = 448 * 2: scale 2, and the codes worked by hand from the E4M3 layout
    (sign, 4 exponent bits with bias 7, 3 mantissa bits): 448 -> 0x7E, -1.5 -> 0xBC, 0.25 -> 0x28, -0 -> 0x80,
    and a second row of zeros with scale 0 and codes 0."""
    rows = np.zeros((2, 256), np.float32)
    rows[0, :4] = [896.0, -3.0, 0.5, -0.0]
    wb = (rows.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oracle.quant_w_per_channel(wb, lib=olib)
    assert s[0] == np.float32(2.0) and s[1] == np.float32(0.0)
    assert list(q[0, :4]) == [0x7E, 0xBC, 0x28, 0x80]
    assert np.all(q[0, 4:] == 0) and np.all(q[1] == 0)


def test_matches_rowwise_numpy(olib):
    g = np.random.default_rng(91)
    N, K = 64, 1000                      # K need not be a multiple of 128 in this mode
    w = (g.standard_normal((N, K)) * np.exp2(g.integers(-10, 11, size=(N, 1)))).astype(np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    wf = (wb.astype(np.uint32) << 16).view(np.float32)
    q, s = oracle.quant_w_per_channel(wb, lib=olib)
    want_s = (np.abs(wf).max(axis=1) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s, want_s)
    quot = (wf / want_s[:, None]).astype(np.float32)
    assert np.array_equal(q, oracle.e4m3_encode(quot, lib=olib))


def test_equals_one_group_per_row_when_k_is_128(olib):
    g = np.random.default_rng(92)
    wb = (g.standard_normal((32, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s = oracle.quant_w_per_channel(wb, lib=olib)
    qa, sa = oracle.quant_act_1x128(wb, lib=olib)
    assert np.array_equal(q, qa) and np.array_equal(s, sa[0])
