"""Pins of the oracle's backward-pass copy of a Linear input (the 1x128 quantization of x^T: per channel, per
128 tokens).  Independent of the oracle's code: scales and quotients recomputed column by column in numpy
float32, with the encoder the E4M3 pins already fix, and a hand-worked layout."""
import numpy as np

import oracle


def bf16(a):
    a = np.asarray(a, np.float32)
    assert np.all(a.view(np.uint32) & 0xFFFF == 0)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def test_hand_worked_layout(olib):
    """x[m, k] = 2^(m % 8) * (1 + k/128) over 256 tokens and 128 channels (exact in bf16): every channel's
    amax over a 128-token block is 128 * (1 + k/128) at m % 8 = 7, so s_t = that / 448 and the codes of
    a channel run through 448 * 2^(m%8 - 7), i.e. 3.5, 7, 14, ..., 448, whatever the channel."""
    m = np.arange(256)[:, None]
    k = np.arange(128)[None, :]
    x = (2.0 ** (m % 8)) * (1.0 + k / 128.0)
    q_t, s_t = oracle.quant_act_backward_copy(bf16(x), lib=olib)
    assert q_t.shape == (128, 256) and s_t.shape == (2, 128)
    want_s = (np.float32(128.0) * (np.float32(1.0) + np.arange(128, dtype=np.float32) / np.float32(128.0))
              / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s_t[0], want_s) and np.array_equal(s_t[1], want_s)
    codes = oracle.e4m3_encode(np.float32(448.0) * np.float32(2.0) ** (np.arange(8, dtype=np.float32) - 7), lib=olib)
    for c in (0, 1, 77, 127):
        got = q_t[c].reshape(32, 8)
        # a quotient within an ulp of 448 * 2^j encodes to the code of 448 * 2^j
        assert np.all(got == codes[None, :]), (c, got[0], codes)


def test_matches_columnwise_numpy(olib):
    """Per channel and 128-token block: s = fl32(max |x| / 448), q = E4M3(fl32(x / s)), computed here with
    numpy float32 and the pinned encoder; rows of q_t are channels."""
    g = np.random.default_rng(51)
    M, K = 384, 256
    x = g.standard_normal((M, K)).astype(np.float32) * np.exp2(g.integers(-4, 5, size=(1, K))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    q_t, s_t = oracle.quant_act_backward_copy(xb, lib=olib)
    for mb in range(M // 128):
        blk = xf[mb * 128:(mb + 1) * 128]                       # [128 tokens, K channels]
        s = (np.abs(blk).max(axis=0) / np.float32(448.0)).astype(np.float32)
        assert np.array_equal(s_t[mb], s)
        quot = (blk / s[None, :]).astype(np.float32)           # fl32(x / s)
        want = oracle.e4m3_encode(quot.T.copy(), lib=olib)      # channels as rows
        assert np.array_equal(q_t[:, mb * 128:(mb + 1) * 128], want)


def test_rows_must_fill_token_blocks(olib):
    import pytest
    with pytest.raises(ValueError):
        oracle.quant_act_backward_copy(np.zeros((100, 128), np.uint16), lib=olib)
