"""Seeded generators: determinism, shapes, and the structure of the MoE routing."""
import numpy as np

import workloads as wl


def test_tiny_is_deterministic_and_shaped():
    a = wl.tiny()
    b = wl.tiny()
    assert a["a"].shape == (128, 512) and a["w"].shape == (256, 512)
    assert np.array_equal(a["a"], b["a"]) and np.array_equal(a["w"], b["w"])
    f = wl.bf16_to_f32(a["a"])
    col_rms = np.sqrt((f.astype(np.float64) ** 2).mean(axis=0))
    # the 4 outlier channels (x50) dominate the column RMS
    assert set(np.argsort(col_rms)[-4:]) == set(a["outlier_channels"].tolist())


def test_bf16_rounding_is_rne():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = wl.bf16_bits(x)
    assert list(wl.bf16_to_f32(b)) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]


def test_routing_structure():
    g = np.random.default_rng(0)
    logits = g.standard_normal((1000, 16)).astype(np.float32)
    r = wl.route_topk(logits, 4, pad=128)
    assert r.counts.sum() == 4000
    seg = np.diff(r.offsets.astype(np.int64))
    assert np.all(seg % 128 == 0) and np.all(seg >= r.counts) and np.all(seg - r.counts < 128)
    for e in range(16):
        rows = r.row_token[r.offsets[e]:r.offsets[e + 1]]
        toks = rows[rows >= 0]
        assert len(toks) == r.counts[e] and np.all(np.diff(toks) > 0)       # ascending tokens
        assert np.all(rows[len(toks):] == -1)                                 # padding at the end
        top = np.argsort(-logits[toks], axis=1, kind="stable")[:, :4]
        assert np.all((top == e).any(axis=1))                                 # e is in each token's top-4


def test_routing_empty_expert_and_ties():
    logits = np.zeros((10, 4), np.float32)
    logits[:, 3] = -1.0                       # expert 3 never chosen; ties among 0..2 go to lower index
    r = wl.route_topk(logits, 2, pad=128)
    assert list(r.counts) == [10, 10, 0, 0]
    assert list(r.offsets) == [0, 128, 256, 256, 256]


def test_decode_prequantized_weights_are_finite_codes():
    d = wl.decode(M=2, N=256, K=256)
    assert not np.any((d["wq"] & 0x7F) == 0x7F)
    assert d["sw"].shape == (2, 2) and d["sw"].min() >= 1e-4 and d["sw"].max() <= 1e-2


def test_gather_rows_pads_with_zeros():
    t = np.arange(12, dtype=np.uint16).reshape(3, 4)
    out = wl.gather_rows(t, np.array([2, -1, 0]))
    assert np.array_equal(out, np.array([[8, 9, 10, 11], [0, 0, 0, 0], [0, 1, 2, 3]], np.uint16))
