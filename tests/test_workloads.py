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


def test_up_recipe_and_the_inputs_that_share_it():
    """The up projection's recipe (72 outlier channels x20 among N(0,1), W ~ N(0, 0.02)), and the f4
    workloads draw exactly the same bytes from the same seed."""
    d = wl.dense_up(M=256, N=256, K=7168)
    assert len(d["outlier_channels"]) == 72
    f = wl.bf16_to_f32(d["a"]).astype(np.float64)
    col_rms = np.sqrt((f ** 2).mean(axis=0))
    assert set(np.argsort(col_rms)[-72:]) == set(d["outlier_channels"].tolist())
    normal = np.setdiff1d(np.arange(7168), d["outlier_channels"])
    assert abs(f[:, normal].std() - 1.0) < 0.01 and abs(f[:, d["outlier_channels"]].std() - 20.0) < 0.5
    w = wl.bf16_to_f32(d["w"]).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.0005 and abs(w.mean()) < 0.0005
    assert np.array_equal(wl.dual(M=256, K=7168)["a"], d["a"])
    assert np.array_equal(wl.e5m6(M=256, K=7168)["a"], d["a"])
    assert np.array_equal(wl.per_channel(N=256, K=7168)["w"], d["w"])
    f4 = wl.fp4(M=256, N=256, K=7168)
    assert np.array_equal(f4["a"], d["a"]) and np.array_equal(f4["w"], d["w"])


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
