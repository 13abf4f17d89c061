"""CPU oracle for fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
calls it, and it never calls the HIP library; the two share no code.

The arithmetic lives in ``fp8q_oracle.c`` (plain C, fp32 steps exactly as IEEE
binary32, the GEMM in double).  This module only compiles that file with gcc,
loads it with ctypes and marshals numpy arrays.  Every function states which
part of the method it follows; the citations are in the C file's header.

Array conventions (numpy, C-contiguous):
  * bf16 tensors are ``uint16`` bit patterns;
  * FP8 tensors are ``uint8`` OCP E4M3 codes;
  * activation scales ``s_a`` have shape ``[K/128, M]`` (K-block-major);
  * weight scales ``s_w`` have shape ``[N/128, K/128]`` (per expert for MoE).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_fp8q.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc.  Returns the path of the shared library."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building first if needed) the oracle library and declare its C signatures."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or _LIB_PATH
        if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
            build(out=p)
        lib = ctypes.CDLL(p)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode_array.argtypes = [P, I64, P]
        lib.oracle_e4m3_encode_array.restype = None
        lib.oracle_quant_act_1x128.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_act_1x128.restype = ctypes.c_int
        lib.oracle_quant_w_128x128.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_w_128x128.restype = ctypes.c_int
        lib.oracle_gemm_blockscaled.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P, P]
        lib.oracle_gemm_blockscaled.restype = ctypes.c_int
        lib.oracle_grouped_gemm_blockscaled.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, P, I64, P, P]
        lib.oracle_grouped_gemm_blockscaled.restype = ctypes.c_int
        lib.oracle_dequant_w_128x128.argtypes = [P, P, I64, I64, P]
        lib.oracle_dequant_w_128x128.restype = ctypes.c_int
        lib.oracle_moe_route_topk.argtypes = [P, I64, I64, I64, I64, P, P, P, P, I64]
        lib.oracle_moe_route_topk.restype = ctypes.c_int
        lib.oracle_moe_gather_fp8.argtypes = [P, P, I64, I64, P, I64, P, P]
        lib.oracle_moe_gather_fp8.restype = ctypes.c_int
        lib.oracle_swiglu_bf16.argtypes = [P, P, I64, P, P]
        lib.oracle_swiglu_bf16.restype = ctypes.c_int
        lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_decode.restype = ctypes.c_double
        lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        lib.oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_e2m1_encode_array.argtypes = [P, I64, P]
        lib.oracle_e2m1_encode_array.restype = None
        lib.oracle_quant_act_fp4_1x128.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_act_fp4_1x128.restype = ctypes.c_int
        lib.oracle_quant_w_fp4_128x128.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_w_fp4_128x128.restype = ctypes.c_int
        lib.oracle_quant_w_per_channel.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_w_per_channel.restype = ctypes.c_int
        lib.oracle_e5m6_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_e5m6_decode.restype = ctypes.c_double
        lib.oracle_e5m6_encode_array.argtypes = [P, I64, P]
        lib.oracle_e5m6_encode_array.restype = None
        lib.oracle_quant_act_e5m6_1x128.argtypes = [P, I64, I64, P, P]
        lib.oracle_quant_act_e5m6_1x128.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def num_threads(lib=None) -> int:
    """Threads the oracle's OpenMP loops use."""
    return int((lib or load()).oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc == -1:
        raise ValueError(f"{what}: bad shape or index")
    if rc == -2:
        raise ValueError(f"{what}: non-finite input (finite input is a precondition)")
    if rc == -3:
        raise ValueError(f"{what}: the output has fewer rows than the layout needs")
    if rc != 0:
        raise RuntimeError(f"{what}: status {rc}")


# ---------------------------------------------------------------------------
# OCP E4M3 code <-> value
# ---------------------------------------------------------------------------

def e4m3_decode(codes, lib=None) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    lib = lib or load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(values, lib=None) -> np.ndarray:
    """E4M3 code of each fp32 value: nearest, ties to even, saturating at 448."""
    lib = lib or load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------

def quant_act_1x128(x_bits, lib=None):
    """1x128 activation quantization of bf16 ``x [M, K]``.

    Returns ``(q uint8 [M, K], s_a float32 [K/128, M])``.
    """
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((K // 128, M), dtype=np.float32)
    _check(lib.oracle_quant_act_1x128(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant_act_1x128")
    return q, s


def quant_act_backward_copy(x_bits, lib=None):
    """The FP8 copy of a Linear input that the backward pass contracts over tokens (the weight gradient
    dW = dY^T X; page "The Definitive Information To Deepseek", the passage on caching the Linear's input in
    FP8 for backward).  Reading: the 1x128 quantization of x^T, i.e. one scale per channel and 128 tokens,
    from the same bf16 x as the forward copy.  ``x [M, K]`` with M a multiple of 128 ->
    ``(q_t uint8 [K, M], s_t float32 [M/128, K])``: q_t[k, m] = E4M3(fl32(x[m, k] / s_t[m/128, k]))."""
    x = _c(x_bits, np.uint16)
    if x.shape[0] % 128:
        raise ValueError("quant_act_backward_copy: M must be a multiple of 128")
    return quant_act_1x128(np.ascontiguousarray(x.T), lib=lib)


def quant_w_128x128(w_bits, lib=None):
    """128x128 weight quantization of bf16 ``w [N, K]`` (or ``[E, N, K]``, one block grid per expert).

    Returns ``(q uint8, s_w float32 [N/128, K/128])`` (``[E, N/128, K/128]`` for 3-D input).
    """
    lib = lib or load()
    w = _c(w_bits, np.uint16)
    lead = w.shape[:-2]
    N, K = w.shape[-2:]
    rows = int(np.prod(lead, dtype=np.int64)) * N if lead else N
    q = np.empty(w.shape, dtype=np.uint8)
    s = np.empty(lead + (N // 128, K // 128), dtype=np.float32)
    # An [E, N, K] stack with N % 128 == 0 is the same block grid as one [E*N, K] matrix.
    _check(lib.oracle_quant_w_128x128(_ptr(w), rows, K, _ptr(q), _ptr(s)), "quant_w_128x128")
    return q, s


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _elements(M, N, rows, cols):
    if rows is None and cols is None:
        ms = np.repeat(np.arange(M, dtype=np.int64), N)
        ns = np.tile(np.arange(N, dtype=np.int64), M)
        return ms, ns, (M, N)
    if rows is not None and cols is None:
        rows = np.asarray(rows, dtype=np.int64)
        return np.repeat(rows, N), np.tile(np.arange(N, dtype=np.int64), len(rows)), (len(rows), N)
    if rows is None:
        cols = np.asarray(cols, dtype=np.int64)
        return np.repeat(np.arange(M, dtype=np.int64), len(cols)), np.tile(cols, M), (M, len(cols))
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    return np.repeat(rows, len(cols)), np.tile(cols, len(rows)), (len(rows), len(cols))


def gemm_blockscaled(qa, sa, qw, sw, rows=None, cols=None, lib=None):
    """Dequantized GEMM ``C = A_deq @ W_deq^T`` in float64, with the error scale ``B = |A_deq| @ |W_deq|^T``.

    ``rows``/``cols`` select a sub-grid of output elements (all rows / all columns when None).
    Returns ``(C, B)`` as float64 arrays of shape ``[len(rows) or M, len(cols) or N]``.
    """
    lib = lib or load()
    qa = _c(qa, np.uint8)
    qw = _c(qw, np.uint8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape == (N, K) and sa.shape == (K // 128, M) and sw.shape == (N // 128, K // 128)
    ms, ns, shape = _elements(M, N, rows, cols)
    C = np.empty(ms.shape, dtype=np.float64)
    B = np.empty(ms.shape, dtype=np.float64)
    _check(lib.oracle_gemm_blockscaled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, _ptr(ms), _ptr(ns),
                                       len(ms), _ptr(C), _ptr(B)), "gemm_blockscaled")
    return C.reshape(shape), B.reshape(shape)


def grouped_gemm_blockscaled(qa, sa, qw, sw, offsets, rows=None, cols=None, lib=None):
    """Grouped (MoE) dequantized GEMM: rows ``[off[e], off[e+1])`` of A use expert ``e``.

    ``qw [E, N, K]``, ``sw [E, N/128, K/128]``, ``offsets int32 [E+1]``.  Returns ``(C, B)`` like
    :func:`gemm_blockscaled`.
    """
    lib = lib or load()
    qa = _c(qa, np.uint8)
    qw = _c(qw, np.uint8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    off = _c(offsets, np.int32)
    M, K = qa.shape
    E, N, K2 = qw.shape
    assert K2 == K and sa.shape == (K // 128, M) and sw.shape == (E, N // 128, K // 128) and off.shape == (E + 1,)
    ms, ns, shape = _elements(M, N, rows, cols)
    C = np.empty(ms.shape, dtype=np.float64)
    B = np.empty(ms.shape, dtype=np.float64)
    _check(lib.oracle_grouped_gemm_blockscaled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(off), E, M, N, K,
                                               _ptr(ms), _ptr(ns), len(ms), _ptr(C), _ptr(B)),
           "grouped_gemm_blockscaled")
    return C.reshape(shape), B.reshape(shape)


def dequant_w_128x128(q, s, lib=None):
    """FP8 -> BF16 weight conversion with 128x128 block scales: ``w = bf16(fl32(dec(q) * s))``.

    ``q`` uint8 codes ``[N, K]`` (or ``[E, N, K]``), ``s`` fp32 ``[N/128, K/128]`` (``[E, N/128, K/128]``).
    Returns bf16 bit patterns (uint16) of ``q``'s shape.
    """
    lib = lib or load()
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    K = q.shape[-1]
    N = int(np.prod(q.shape[:-1]))
    assert s.size == (N // 128) * (K // 128)
    w = np.empty(q.shape, dtype=np.uint16)
    _check(lib.oracle_dequant_w_128x128(_ptr(q), _ptr(s), N, K, _ptr(w)), "dequant_w_128x128")
    return w


# ---------------------------------------------------------------------------
# MoE routing and the FP8 row gather
# ---------------------------------------------------------------------------

class Routing:
    """Result of :func:`moe_route_topk`.

    ``topk_idx`` int32 ``[T, k]``: token t's experts by decreasing logit (ties: lower index first).
    ``offsets`` int32 ``[E+1]``: expert e owns rows ``offsets[e] .. offsets[e+1]`` (multiples of ``pad``).
    ``row_of`` int32 ``[T, k]``: the row carrying token t's j-th expert.
    ``row_token`` int32 ``[rows]``: the token a row carries, -1 for empty rows and rows past ``offsets[E]``.
    """

    def __init__(self, topk_idx, offsets, row_of, row_token):
        self.topk_idx, self.offsets, self.row_of, self.row_token = topk_idx, offsets, row_of, row_token

    @property
    def counts(self):
        return np.bincount(self.topk_idx.ravel(), minlength=len(self.offsets) - 1).astype(np.int64)

    @property
    def M(self):
        """Rows of the layout (``offsets[E]``)."""
        return int(self.offsets[-1])


def moe_route_capacity(T: int, E: int, k: int, pad: int = 128) -> int:
    """Rows enough for any routing of T tokens to k of E experts: T*k plus pad-1 per expert, rounded up
    to a multiple of pad."""
    return ((T * k + E * (pad - 1)) + pad - 1) // pad * pad


def moe_route_topk(logits, k: int, pad: int = 128, rows: int | None = None, lib=None) -> Routing:
    """Top-k gating and the expert-sorted layout (readings in ``fp8q_oracle.c``).  ``logits`` fp32
    ``[T, E]``; ``rows`` is the length of ``row_token`` (default: exactly ``offsets[E]``)."""
    lib = lib or load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    cap = moe_route_capacity(T, E, k, pad) if rows is None else rows
    topk_idx = np.empty((T, k), dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    row_of = np.empty((T, k), dtype=np.int32)
    row_token = np.empty(cap, dtype=np.int32)
    _check(lib.oracle_moe_route_topk(_ptr(logits), T, E, k, pad, _ptr(topk_idx), _ptr(offsets), _ptr(row_of),
                                     _ptr(row_token), cap), "moe_route_topk")
    if rows is None:
        row_token = row_token[: int(offsets[-1])].copy()
    return Routing(topk_idx, offsets, row_of, row_token)


def moe_gather_fp8(q, s, row_token, lib=None):
    """Expert-sorted FP8 rows: ``qa[r] = q[row_token[r]]`` and ``sa[:, r] = s[:, row_token[r]]``, zero codes
    and scale 0 where ``row_token[r] == -1``.  ``q`` uint8 ``[T, K]``, ``s`` fp32 ``[K/128, T]``.
    Returns ``(qa [rows, K], sa [K/128, rows])``."""
    lib = lib or load()
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    row_token = _c(row_token, np.int32)
    T, K = q.shape
    rows = len(row_token)
    qa = np.empty((rows, K), dtype=np.uint8)
    sa = np.empty((K // 128, rows), dtype=np.float32)
    _check(lib.oracle_moe_gather_fp8(_ptr(q), _ptr(s), T, K, _ptr(row_token), rows, _ptr(qa), _ptr(sa)),
           "moe_gather_fp8")
    return qa, sa


# ---------------------------------------------------------------------------
# Fused SwiGLU + 1x128 quantization
# ---------------------------------------------------------------------------

def _bf16_exact(bits: int):
    from decimal import Decimal
    return Decimal(float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]))


def swiglu_exact_bf16(xb: int, yb: int) -> int:
    """bf16(SiLU(x) * y) for one pair of bf16 bit patterns, from 80-digit decimal arithmetic (exp correctly
    rounded at that precision): the settlement of the values the C evaluation flags as too close to a
    rounding midpoint to decide in double."""
    from decimal import Decimal, localcontext, ROUND_FLOOR
    with localcontext() as ctx:
        ctx.prec = 80
        x, y = _bf16_exact(xb), _bf16_exact(yb)
        # the same value in a form whose exponential cannot overflow
        v = x * y / (1 + (-x).exp()) if x >= 0 else x * y * x.exp() / (1 + x.exp())
        neg = (v < 0) or (v == 0 and ((xb ^ yb) & 0x8000))
        a = abs(v)
        if a == 0:
            return 0x8000 if neg else 0
        ex = int(float(a).hex().split("p")[1]) if float(a) != 0 else -1000
        # the binade of a (its double is within 1e-60 relative; a power of two is itself a bf16 value)
        while Decimal(2) ** ex > a:
            ex -= 1
        while Decimal(2) ** (ex + 1) <= a:
            ex += 1
        ex = max(ex, -126)
        ulp = Decimal(2) ** (ex - 7)
        q = a / ulp
        fl = q.to_integral_value(rounding=ROUND_FLOOR)
        rem = q - fl
        if abs(rem - Decimal("0.5")) <= Decimal(10) ** -60:
            # Not decided at 80 digits: only possible when e^-x vanished next to 1 (x huge) and x*y is the
            # midpoint itself; the true value x*y / (1 + e^-x) then lies just inside it (towards zero).
            assert x > 0 and abs(x * y) == (fl + Decimal("0.5")) * ulp, "an undecided value SiLU cannot give"
        elif rem > Decimal("0.5"):
            fl += 1
        r = float(fl * ulp)
    bits = int(np.array([r], dtype=np.float32).view(np.uint32)[0]) >> 16
    return bits | (0x8000 if neg else 0)


def swiglu_bf16(x_bits, y_bits, lib=None, return_flags=False):
    """h = bf16(SiLU(x) * y) elementwise (the exact value rounded once to nearest even), bf16 in and out as
    uint16 bit patterns of one shape.  Values the C evaluation cannot decide in double are settled by
    :func:`swiglu_exact_bf16`."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    y = _c(y_bits, np.uint16)
    assert x.shape == y.shape
    h = np.empty(x.shape, dtype=np.uint16)
    amb = np.zeros(x.shape, dtype=np.uint8)
    _check(lib.oracle_swiglu_bf16(_ptr(x), _ptr(y), x.size, _ptr(h), _ptr(amb)), "swiglu_bf16")
    flat = np.flatnonzero(amb)
    hf = h.reshape(-1)
    for i in flat:
        hf[i] = swiglu_exact_bf16(int(x.reshape(-1)[i]), int(y.reshape(-1)[i]))
    return (h, amb.astype(bool)) if return_flags else h


def swiglu_quant_1x128(x_bits, y_bits, lib=None):
    """Fused SwiGLU + 1x128 quantization: ``quant_act_1x128(swiglu_bf16(x, y))``.  ``x`` (gate) and ``y``
    (up) bf16 ``[M, K]`` -> ``(q uint8 [M, K], s float32 [K/128, M])``."""
    lib = lib or load()
    return quant_act_1x128(swiglu_bf16(x_bits, y_bits, lib=lib), lib=lib)


# ---------------------------------------------------------------------------
# FP4 (OCP E2M1) quantization in the FP8 groupings
# ---------------------------------------------------------------------------

def e2m1_decode(codes, lib=None) -> np.ndarray:
    """Values of 4-bit E2M1 codes (0..15)."""
    lib = lib or load()
    c = np.asarray(codes, np.uint8)
    return np.array([lib.oracle_e2m1_decode(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def e2m1_encode(values, lib=None) -> np.ndarray:
    """Nearest E2M1 codes (ties to the even code, saturating at +-6) of float32 values."""
    lib = lib or load()
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib.oracle_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def quant_act_fp4_1x128(x_bits, lib=None):
    """1x128 FP4 activation quantization: ``x [M, K]`` bf16 -> ``(q uint8 [M, K/2], s float32 [K/128, M])``,
    two codes a byte (element 2i in the low nibble), scale = fl32(amax / 6)."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K // 2), dtype=np.uint8)
    s = np.empty((K // 128, M), dtype=np.float32)
    _check(lib.oracle_quant_act_fp4_1x128(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant_act_fp4_1x128")
    return q, s


def quant_w_fp4_128x128(w_bits, lib=None):
    """128x128 FP4 weight quantization: ``w [N, K]`` bf16 -> ``(q uint8 [N, K/2], s float32 [N/128, K/128])``."""
    lib = lib or load()
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N // 128, K // 128), dtype=np.float32)
    _check(lib.oracle_quant_w_fp4_128x128(_ptr(w), N, K, _ptr(q), _ptr(s)), "quant_w_fp4_128x128")
    return q, s


def quant_w_per_channel(w_bits, lib=None):
    """Per-channel FP8 weights: one scale per output channel (row of ``w [N, K]``) over all K ->
    ``(q uint8 [N, K], s float32 [N])``."""
    lib = lib or load()
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(N, dtype=np.float32)
    _check(lib.oracle_quant_w_per_channel(_ptr(w), N, K, _ptr(q), _ptr(s)), "quant_w_per_channel")
    return q, s


def e5m6_decode(codes, lib=None) -> np.ndarray:
    """Values of 12-bit E5M6 codes (sign bit 11, exponent bits 10..6 with bias 15, mantissa bits 5..0)."""
    lib = lib or load()
    c = np.asarray(codes, np.uint16)
    return np.array([lib.oracle_e5m6_decode(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def e5m6_encode(values, lib=None) -> np.ndarray:
    """Nearest E5M6 codes (ties to the even code, saturating at +-65024) of float32 values."""
    lib = lib or load()
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_e5m6_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e5m6_unpack(q) -> np.ndarray:
    """12-bit codes [M, K] from packed rows [M, 3K/2] (little-endian bit stream, element j at bits 12j..)."""
    b = np.asarray(q, np.uint16).reshape(q.shape[0], -1, 3)
    c0 = b[..., 0] | ((b[..., 1] & 0xF) << 8)
    c1 = (b[..., 1] >> 4) | (b[..., 2] << 4)
    return np.stack([c0, c1], axis=-1).reshape(q.shape[0], -1).astype(np.uint16)


def quant_act_e5m6_1x128(x_bits, lib=None):
    """1x128 E5M6 activation quantization: ``x [M, K]`` bf16 -> ``(q uint8 [M, 3K/2], s float32 [K/128, M])``,
    scale = fl32(amax / 65024), two 12-bit codes per 3 bytes."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K // 2 * 3), dtype=np.uint8)
    s = np.empty((K // 128, M), dtype=np.float32)
    _check(lib.oracle_quant_act_e5m6_1x128(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant_act_e5m6_1x128")
    return q, s
