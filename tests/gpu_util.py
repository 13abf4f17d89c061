"""Helpers shared by the GPU parity tests: host <-> device marshalling and the GEMM error bound."""
import sys

import numpy as np
import torch

import fine_grained_quantization_amd as fq


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (run them with -m gpu on an MI355X)")
    fq.load_library()  # raises if the HIP library is missing: there is no fallback


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_out_to_f64(t: torch.Tensor) -> np.ndarray:
    h = host(t)
    return bf16_bits_to_f64(h) if t.dtype == torch.bfloat16 else h.astype(np.float64)


def assert_gemm_within_bound(gpu: np.ndarray, C: np.ndarray, B: np.ndarray, bf16_out: bool, what: str = ""):
    """|gpu - C| <= 1e-3 * B + 1e-6 per element (B = sum |a_deq| |w_deq|); a bf16 output may in addition
    carry its own final rounding, at most 2^-8 of the larger magnitude."""
    err = np.abs(gpu - C)
    tol = 1e-3 * B + 1e-6
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.maximum(np.abs(gpu), np.abs(C))
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of bound; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} oracle={C[tuple(i)]!r} bound={tol[tuple(i)]!r}")
    return float(np.max(err / tol)) if err.size else 0.0


def literal_bound_ratio(gpu: np.ndarray, C: np.ndarray, B: np.ndarray) -> float:
    """max |gpu - C| / (1e-3 B + 1e-6): the literal bound, reported for bf16 outputs too."""
    return float(np.max(np.abs(gpu - C) / (1e-3 * B + 1e-6))) if gpu.size else 0.0


def every_amax_groups(seed, limit=0x7F80):
    """One 128-element group per positive finite bf16 amax pattern below `limit` (denormals included): the amax
    at a random position with a random sign, the other 127 elements random bf16 patterns of magnitude <= amax
    with random signs.  Returns the groups as rows of 8 groups ([ceil(n / 8), 1024] bf16 bits, zero-padded)."""
    g = np.random.default_rng(seed)
    amax = np.arange(1, limit, dtype=np.uint16)
    n = len(amax)
    lim = amax.astype(np.int64)
    rest = np.minimum((g.random((n, 127)) * (lim[:, None] + 1)).astype(np.int64), lim[:, None]).astype(np.uint16)
    rest |= (g.random((n, 127)) < 0.5).astype(np.uint16) << 15
    rows = np.concatenate([amax[:, None] | ((g.random((n, 1)) < 0.5).astype(np.uint16) << 15), rest], axis=1)
    rows = np.take_along_axis(rows, np.argsort(g.random((n, 128)), axis=1), axis=1)
    rows = np.concatenate([rows, np.zeros(((-n) % 8, 128), np.uint16)])
    return rows.reshape(-1, 1024)
