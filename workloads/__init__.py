"""Seeded synthetic inputs for the FP8 Linear hot path.

This module is shared by the tests, the benchmark and the smoke check; it feeds
the CPU oracle and the HIP library the same host bytes.  It holds none of the
method's arithmetic (no amax, no scale, no FP8 encoding, no GEMM, no routing): it
only draws random numbers and rounds them to bf16 as input data.  For the MoE
case it supplies tokens, router logits and expert weights; choosing each
token's experts and laying the tokens out per expert are steps of the method.

Generator: numpy PCG64 seeded with ``[workload_seed, tensor_id]``.  Normal draws
are float32, scaled in float32, then rounded to bf16 (round-to-nearest-even,
done by torch's CPU dtype conversion).  bf16 tensors are returned as ``uint16``
bit patterns.

Workloads (shapes from DeepSeek-V3's published configuration: hidden size 7168,
dense FFN width 18432, MoE experts of width 2048; the MoE routing shape, 8K
tokens with top-8 experts, follows the DeepEP V2 test setting on the
deepinsightai.io page):

  tiny    A [128, 512] ~ N(0,1), 4 channels x50; W [256, 512] ~ N(0, 0.02)       seed 0
  up      A [4096, 7168] ~ N(0,1), 72 (1%) channels x20; W [18432, 7168]         seed 1
  down    gate x, up y bf16 [4096, 18432] ~ N(0,1) (A = bf16(SiLU(x) * y) is the
          method's fused SwiGLU step); W [7168, 18432] ~ N(0, 0.02)               seed 2
  moe     8192 tokens x 7168 ~ N(0,1); router logits [8192, 64] ~ N(0,1) (routed
          top-8, segments padded to 128 rows); W [64][2048, 7168] ~ N(0, 0.02)   seed 3
  decode  A [64, 7168] ~ N(0,1); W pre-quantized: E4M3 codes uniform over the 254
          finite codes, 128x128 fp32 scales ~ U(1e-4, 1e-2)                        seed 4
"""
from __future__ import annotations


import numpy as np

SEEDS = {"tiny": 0, "up": 1, "down": 2, "moe": 3, "decode": 4, "dequant": 5}

# tensor ids inside one workload's seed
T_A, T_W, T_OUTLIER, T_X, T_Y, T_LOGITS, T_WQ, T_SW = 0, 1, 2, 3, 4, 5, 6, 7


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, tensor_id]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 data to bf16 (RNE) and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed, tid, shape, sigma=1.0, chunk_rows=None):
    """bf16 N(0, sigma^2) of the given shape; drawn in row chunks to bound float32 temporaries."""
    g = rng(seed, tid)
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1])
    rows = flat.shape[0]
    step = chunk_rows or max(1, (1 << 26) // shape[-1])
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        v = g.standard_normal((r1 - r0, shape[-1]), dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        flat[r0:r1] = bf16_bits(v)
    return out


def activations_with_outliers(seed, M, K, n_outliers, factor, tid_a=T_A, tid_o=T_OUTLIER):
    """A ~ N(0,1) float32 with ``n_outliers`` channels (chosen without replacement) multiplied by
    ``factor`` before the bf16 rounding.  Returns (bits [M, K], outlier channel indices)."""
    g = rng(seed, tid_a)
    a = g.standard_normal((M, K), dtype=np.float32)
    ch = np.sort(rng(seed, tid_o).choice(K, size=n_outliers, replace=False)) if n_outliers else np.zeros(0, np.int64)
    if n_outliers:
        a[:, ch] *= np.float32(factor)
    return bf16_bits(a), ch


def gate_up(seed, M, K):
    """The FFN's gate x and up projection y in bf16, x, y ~ N(0,1), independent streams.  Their SwiGLU,
    bf16(SiLU(x) * y), is the down projection's input; computing it is a step of the method."""
    return normal_bf16(seed, T_X, (M, K)), normal_bf16(seed, T_Y, (M, K))


def finite_e4m3_codes(seed, tid, shape):
    """Codes drawn uniformly from the 254 finite OCP E4M3 codes (0x7F and 0xFF excluded)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    idx = rng(seed, tid).integers(0, len(finite), size=shape, dtype=np.int64)
    return finite[idx]


def uniform_f32(seed, tid, shape, lo, hi):
    return rng(seed, tid).uniform(lo, hi, size=shape).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def tiny():
    s = SEEDS["tiny"]
    a, ch = activations_with_outliers(s, 128, 512, 4, 50.0)
    w = normal_bf16(s, T_W, (256, 512), 0.02)
    return {"name": "tiny", "a": a, "w": w, "outlier_channels": ch, "M": 128, "N": 256, "K": 512}


def dense_up(M=4096, N=18432, K=7168):
    s = SEEDS["up"]
    n_out = int(round(0.01 * K))
    a, ch = activations_with_outliers(s, M, K, n_out, 20.0)
    w = normal_bf16(s, T_W, (N, K), 0.02)
    return {"name": "up", "a": a, "w": w, "outlier_channels": ch, "M": M, "N": N, "K": K}


def dense_down(M=4096, N=7168, K=18432):
    s = SEEDS["down"]
    x, y = gate_up(s, M, K)
    w = normal_bf16(s, T_W, (N, K), 0.02)
    return {"name": "down", "x": x, "y": y, "w": w, "M": M, "N": N, "K": K}


def moe(T=8192, K=7168, E=64, k=8, N=2048, with_weights=True):
    s = SEEDS["moe"]
    tokens = normal_bf16(s, T_A, (T, K))
    logits = rng(s, T_LOGITS).standard_normal((T, E), dtype=np.float32)
    d = {"name": "moe", "tokens": tokens, "logits": logits, "M": None, "N": N, "K": K, "E": E, "T": T, "topk": k}
    if with_weights:
        d["w"] = normal_bf16(s, T_W, (E, N, K), 0.02)
    return d


def decode(M=64, N=18432, K=7168):
    s = SEEDS["decode"]
    a = normal_bf16(s, T_A, (M, K))
    wq = finite_e4m3_codes(s, T_WQ, (N, K))
    sw = uniform_f32(s, T_SW, (N // 128, K // 128), 1e-4, 1e-2)
    return {"name": "decode", "a": a, "wq": wq, "sw": sw, "M": M, "N": N, "K": K}


def dequant(N=18432, K=7168):
    """FP8 weights of the up-projection's shape with 128x128 scales, to be converted to BF16: codes uniform
    over the 254 finite E4M3 codes, scales ~U(1e-4, 1e-2) (the decode workload's recipe)."""
    s = SEEDS["dequant"]
    wq = finite_e4m3_codes(s, T_WQ, (N, K))
    sw = uniform_f32(s, T_SW, (N // 128, K // 128), 1e-4, 1e-2)
    return {"name": "dequant", "wq": wq, "sw": sw, "M": 0, "N": N, "K": K}


def dual(M=4096, K=7168):
    """The up projection's input (same recipe and seed as the up workload's A), for the one-pass forward and
    backward FP8 copies."""
    s = SEEDS["up"]
    a, ch = activations_with_outliers(s, M, K, int(round(0.01 * K)), 20.0)
    return {"name": "dual", "a": a, "outlier_channels": ch, "M": M, "N": 0, "K": K}


def fp4(M=4096, N=18432, K=7168):
    """The up projection's activation and weight (same recipes and seed as the up workload), for FP4."""
    d = dense_up(M, N, K)
    d["name"] = "fp4"
    return d


def e5m6(M=4096, K=7168):
    """The up projection's input (same recipe and seed as the up workload's A), for E5M6."""
    d = dual(M, K)
    d["name"] = "e5m6"
    return d


def per_channel(N=18432, K=7168):
    """The up projection's weight (same recipe and seed as the up workload), for per-channel FP8."""
    w = normal_bf16(SEEDS["up"], T_W, (N, K), 0.02)
    return {"name": "per_channel", "w": w, "M": 0, "N": N, "K": K}


WORKLOADS = {"tiny": tiny, "up": dense_up, "down": dense_down, "moe": moe, "decode": decode, "dequant": dequant,
             "dual": dual, "fp4": fp4, "per_channel": per_channel, "e5m6": e5m6}
