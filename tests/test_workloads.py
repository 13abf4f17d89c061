"""Seeded generators: determinism and shapes."""
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


def test_moe_inputs_are_deterministic_and_shaped():
    a = wl.moe(T=64, with_weights=False)
    b = wl.moe(T=64, with_weights=False)
    assert a["tokens"].shape == (64, 7168) and a["logits"].shape == (64, 64) and a["logits"].dtype == np.float32
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["logits"], b["logits"])
    assert "routing" not in a      # choosing experts is a step of the method, not of the generator


def test_decode_prequantized_weights_are_finite_codes():
    d = wl.decode(M=2, N=256, K=256)
    assert not np.any((d["wq"] & 0x7F) == 0x7F)
    assert d["sw"].shape == (2, 2) and d["sw"].min() >= 1e-4 and d["sw"].max() <= 1e-2
