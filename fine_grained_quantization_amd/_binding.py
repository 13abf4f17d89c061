"""ctypes binding of ``libfp8q.so`` (the C ABI declared in ``include/fp8q.h``).

Argument marshalling only: every step runs in the HIP library.  torch provides device memory and the
current stream; outputs are allocated with torch when the caller does not pass them.  If the library
is not built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

OUT_BF16 = 0
OUT_F32 = 1

_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfp8q.so and declare the C signatures.  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"fp8q HIP library not found at {path}; build it with "
                               "`python -m fine_grained_quantization_amd.build`")
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.fp8q_quant_act_1x128.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_quant_w_128x128.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_swiglu_quant_act_1x128.argtypes = [P, P, I64, I64, I64, P, P, P]
        lib.fp8q_swiglu_bf16.argtypes = [P, P, I64, I64, I64, P, P]
        lib.fp8q_quant_act_dual.argtypes = [P, I64, I64, P, P, P, P, P]
        lib.fp8q_quant_act_fp4_1x128.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_quant_w_fp4_128x128.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_quant_w_per_channel.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_quant_act_e5m6_1x128.argtypes = [P, I64, I64, P, P, P]
        lib.fp8q_gemm_blockscaled.argtypes = [P, P, P, P, P, I, I64, I64, I64, P]
        lib.fp8q_grouped_gemm_blockscaled.argtypes = [P, P, P, P, P, I, P, I64, I64, I64, I64, P]
        lib.fp8q_dequant_w_128x128.argtypes = [P, P, I64, I64, P, P]
        lib.fp8q_grouped_gemm_blockscaled_gather.argtypes = [P, P, I64, P, P, P, P, I, P, I64, I64, I64, I64, P]
        lib.fp8q_moe_route_topk.argtypes = [P, I64, I64, I64, P, P, P, P, I64, P, I64, P]
        lib.fp8q_moe_gather_fp8.argtypes = [P, P, I64, I64, I64, P, P, P, I64, I64, P, P, P]
        lib.fp8q_moe_route_topk_noalloc.argtypes = [P, I64, I64, I64, P, P, P, P, I64, P]
        for f in (lib.fp8q_quant_act_1x128, lib.fp8q_quant_w_128x128, lib.fp8q_swiglu_quant_act_1x128,
                  lib.fp8q_swiglu_bf16, lib.fp8q_quant_act_dual, lib.fp8q_quant_act_fp4_1x128,
                  lib.fp8q_quant_w_fp4_128x128, lib.fp8q_quant_w_per_channel, lib.fp8q_quant_act_e5m6_1x128,
                  lib.fp8q_gemm_blockscaled,
                  lib.fp8q_grouped_gemm_blockscaled, lib.fp8q_grouped_gemm_blockscaled_gather,
                  lib.fp8q_dequant_w_128x128, lib.fp8q_moe_route_topk, lib.fp8q_moe_route_topk_noalloc,
                  lib.fp8q_moe_gather_fp8):
            f.restype = ctypes.c_int
        lib.fp8q_moe_route_capacity.argtypes = [I64, I64, I64]
        lib.fp8q_moe_route_capacity.restype = I64
        lib.fp8q_moe_route_workspace_bytes.argtypes = [I64, I64]
        lib.fp8q_moe_route_workspace_bytes.restype = I64
        lib.fp8q_status_string.argtypes = [I]
        lib.fp8q_status_string.restype = ctypes.c_char_p
        lib.fp8q_version.argtypes = []
        lib.fp8q_version.restype = ctypes.c_int
        if path == LIB_PATH:
            _lib = lib
        return lib


def status_string(rc: int) -> str:
    return load_library().fp8q_status_string(rc).decode()


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name}: {status_string(rc)}")


# The current stream's handle without building a Stream object (that costs ~3 us a call, a third of a
# call's host time); torch.cuda.current_stream() where this accessor does not exist.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream):
    if stream is None and _RAW_STREAM is not None:
        return ctypes.c_void_p(_RAW_STREAM(torch.cuda.current_device()))
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t: torch.Tensor, name: str, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() not in (ndim if isinstance(ndim, tuple) else (ndim,)):
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.uint8, torch.float8_e4m3fn)


def fp8q_quant_act_1x128(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                         stream=None):
    """1x128 activation quantization.  ``x`` bf16 [M, K] -> ``(q uint8 [M, K], s float32 [K/128, M])``."""
    _need(x, "x", _BF16, 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(q, "q", _FP8)
    _need(s, "s", (torch.float32,))
    if q.numel() != M * K or s.numel() != (K // 128) * M:
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_act_1x128(_ptr(x), M, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_act_1x128")
    return q, s


def fp8q_quant_act_fp4_1x128(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                             stream=None):
    """1x128 FP4 (E2M1) activation quantization.  ``x`` bf16 [M, K] -> ``(q uint8 [M, K/2], s float32
    [K/128, M])``, two codes a byte (element 2i in the low nibble)."""
    _need(x, "x", _BF16, 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(q, "q", (torch.uint8,))
    _need(s, "s", (torch.float32,))
    if q.numel() != M * (K // 2) or s.numel() != (K // 128) * M:
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_act_fp4_1x128(_ptr(x), M, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_act_fp4_1x128")
    return q, s


def fp8q_quant_w_fp4_128x128(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                             stream=None):
    """128x128 FP4 (E2M1) weight quantization.  ``w`` bf16 [N, K] -> ``(q uint8 [N, K/2], s float32
    [N/128, K/128])``."""
    _need(w, "w", _BF16, 2)
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    _need(q, "q", (torch.uint8,))
    _need(s, "s", (torch.float32,))
    if q.numel() != N * (K // 2) or s.numel() != (N // 128) * (K // 128):
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_w_fp4_128x128(_ptr(w), N, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_w_fp4_128x128")
    return q, s


def fp8q_quant_act_e5m6_1x128(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                              stream=None):
    """1x128 E5M6 activation quantization.  ``x`` bf16 [M, K] -> ``(q uint8 [M, 3K/2], s float32 [K/128, M])``,
    two 12-bit codes per 3 bytes (element j at bits 12j of its row)."""
    _need(x, "x", _BF16, 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K // 2 * 3), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(q, "q", (torch.uint8,))
    _need(s, "s", (torch.float32,))
    if q.numel() != M * (K // 2 * 3) or s.numel() != M * (K // 128):
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_act_e5m6_1x128(_ptr(x), M, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_act_e5m6_1x128")
    return q, s


def fp8q_quant_w_per_channel(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                             stream=None):
    """Per-channel FP8 weight quantization, one scale per output channel.  ``w`` bf16 [N, K] (K a multiple of
    8) -> ``(q uint8 [N, K], s float32 [N])``."""
    _need(w, "w", _BF16, 2)
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((N,), dtype=torch.float32, device=w.device)
    _need(q, "q", (torch.uint8,))
    _need(s, "s", (torch.float32,))
    if q.numel() != N * K or s.numel() != N:
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_w_per_channel(_ptr(w), N, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_w_per_channel")
    return q, s


def fp8q_quant_act_dual(x: torch.Tensor, q=None, s=None, qt=None, st=None, stream=None):
    """Forward and backward FP8 copies of a Linear input in one pass.  ``x`` bf16 [M, K] (M, K multiples of
    128) -> ``(q uint8 [M, K], s float32 [K/128, M], qt uint8 [K, M], st float32 [M/128, K])``: the 1x128
    quantization of x and of x^T (per channel, per 128 tokens).  Outputs not given are allocated."""
    _need(x, "x", _BF16, 2)
    M, K = x.shape
    dev = x.device
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((K // 128, M), dtype=torch.float32, device=dev) if s is None else s
    qt = torch.empty((K, M), dtype=torch.uint8, device=dev) if qt is None else qt
    st = torch.empty((M // 128, K), dtype=torch.float32, device=dev) if st is None else st
    for t, name, dt, n in ((q, "q", torch.uint8, M * K), (s, "s", torch.float32, (K // 128) * M),
                           (qt, "qt", torch.uint8, M * K), (st, "st", torch.float32, (M // 128) * K)):
        _need(t, name, (dt,))
        if t.numel() != n:
            raise ValueError(f"{name} has the wrong size")
    _check(load_library().fp8q_quant_act_dual(_ptr(x), M, K, _ptr(q), _ptr(s), _ptr(qt), _ptr(st),
                                              _stream_ptr(stream)), "fp8q_quant_act_dual")
    return q, s, qt, st


def fp8q_swiglu_quant_act_1x128(x: torch.Tensor, y: torch.Tensor | None = None, q: torch.Tensor | None = None,
                                s: torch.Tensor | None = None, stream=None):
    """Fused SwiGLU + 1x128 quantization of h = bf16(SiLU(x) * y).  Either ``x`` (gate) and ``y`` (up) bf16
    [M, K] with equal row strides (views are fine), or ``x`` alone as one [M, 2K] tensor whose halves are the
    gate and the up projection -> ``(q uint8 [M, K], s float32 [K/128, M])``."""
    _need_rows(x, "x")
    if y is None:
        M, K2 = x.shape
        if K2 % 2:
            raise ValueError("a fused gate/up tensor needs an even number of columns")
        K = K2 // 2
        ld = x.stride(0)
        y = x[:, K:]
        x = x[:, :K]
    else:
        _need_rows(y, "y")
        if y.shape != x.shape or y.stride(0) != x.stride(0):
            raise ValueError("x and y must have the same shape and row stride")
        M, K = x.shape
        ld = x.stride(0)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(q, "q", _FP8)
    _need(s, "s", (torch.float32,))
    if q.numel() != M * K or s.numel() != (K // 128) * M:
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_swiglu_quant_act_1x128(_ptr(x), _ptr(y), ld, M, K, _ptr(q), _ptr(s),
                                                      _stream_ptr(stream)), "fp8q_swiglu_quant_act_1x128")
    return q, s


def fp8q_swiglu_bf16(x: torch.Tensor, y: torch.Tensor, h: torch.Tensor | None = None, stream=None):
    """h = bf16(SiLU(x) * y) written out (the intermediate the fused quantizer keeps in registers).  ``x``,
    ``y`` bf16 [M, K] with equal row strides -> ``h`` bf16 [M, K]."""
    _need_rows(x, "x")
    _need_rows(y, "y")
    if y.shape != x.shape or y.stride(0) != x.stride(0):
        raise ValueError("x and y must have the same shape and row stride")
    M, K = x.shape
    if h is None:
        h = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    _need(h, "h", _BF16)
    if h.numel() != M * K:
        raise ValueError("h has the wrong size")
    _check(load_library().fp8q_swiglu_bf16(_ptr(x), _ptr(y), x.stride(0), M, K, _ptr(h), _stream_ptr(stream)),
           "fp8q_swiglu_bf16")
    return h


def _need_rows(t, name):
    """A bf16 [M, K] device view whose rows are contiguous (any row stride)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype not in _BF16 or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D bf16 device tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")


def fp8q_quant_w_128x128(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                         stream=None):
    """128x128 weight quantization.  ``w`` bf16 [N, K] (or an expert stack [E, N, K]) ->
    ``(q uint8, s float32 [N/128, K/128])`` (``[E, N/128, K/128]`` for a stack)."""
    _need(w, "w", _BF16, (2, 3))
    lead = tuple(w.shape[:-2])
    N, K = w.shape[-2:]
    rows = N * (lead[0] if lead else 1)
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty(lead + (N // 128, K // 128), dtype=torch.float32, device=w.device)
    _need(q, "q", _FP8)
    _need(s, "s", (torch.float32,))
    if q.numel() != w.numel() or s.numel() != (rows // 128) * (K // 128):
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_quant_w_128x128(_ptr(w), rows, K, _ptr(q), _ptr(s), _stream_ptr(stream)),
           "fp8q_quant_w_128x128")
    return q, s


def fp8q_dequant_w_128x128(q: torch.Tensor, s: torch.Tensor, w: torch.Tensor | None = None, stream=None):
    """FP8 -> BF16 weight conversion with 128x128 block scales.  ``q`` E4M3 codes [N, K] (or an expert stack
    [E, N, K]), ``s`` float32 [N/128, K/128] (``[E, N/128, K/128]``) -> ``w`` bf16 of ``q``'s shape."""
    _need(q, "q", _FP8, (2, 3))
    _need(s, "s", (torch.float32,))
    K = q.shape[-1]
    rows = q.numel() // K if K else 0
    if s.numel() != (rows // 128) * (K // 128):
        raise ValueError("s has the wrong size")
    if w is None:
        w = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(w, "w", _BF16)
    if w.numel() != q.numel():
        raise ValueError("w has the wrong size")
    _check(load_library().fp8q_dequant_w_128x128(_ptr(q), _ptr(s), rows, K, _ptr(w), _stream_ptr(stream)),
           "fp8q_dequant_w_128x128")
    return w


def _out_code(out_dtype):
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    if out_dtype == torch.float32:
        return OUT_F32
    raise ValueError(f"out_dtype must be torch.bfloat16 or torch.float32, got {out_dtype}")


def fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=torch.bfloat16, c=None, stream=None):
    """Block-scaled FP8 GEMM ``C = A W^T``.  ``qa`` [M, K], ``sa`` [K/128, M], ``qw`` [N, K],
    ``sw`` [N/128, K/128] -> ``c`` [M, N] in ``out_dtype`` (bf16 or fp32)."""
    _need(qa, "qa", _FP8, 2)
    _need(qw, "qw", _FP8, 2)
    _need(sa, "sa", (torch.float32,))
    _need(sw, "sw", (torch.float32,))
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape[1] != K or sa.numel() != (K // 128) * M or sw.numel() != (N // 128) * (K // 128):
        raise ValueError("inconsistent GEMM operand shapes")
    code = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _need(c, "c", (out_dtype,))
    if c.numel() != M * N:
        raise ValueError("c has the wrong size")
    _check(load_library().fp8q_gemm_blockscaled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(c), code, M, N, K,
                                                _stream_ptr(stream)), "fp8q_gemm_blockscaled")
    return c


def fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, offsets, out_dtype=torch.bfloat16, c=None, stream=None):
    """Grouped (MoE) block-scaled FP8 GEMM.  ``qa`` [M_total, K], ``sa`` [K/128, M_total], ``qw`` [E, N, K],
    ``sw`` [E, N/128, K/128], ``offsets`` int32 device [E+1] -> ``c`` [M_total, N]."""
    _need(qa, "qa", _FP8, 2)
    _need(qw, "qw", _FP8, 3)
    _need(sa, "sa", (torch.float32,))
    _need(sw, "sw", (torch.float32,))
    _need(offsets, "offsets", (torch.int32,), 1)
    M, K = qa.shape
    E, N, K2 = qw.shape
    if K2 != K or sa.numel() != (K // 128) * M or sw.numel() != E * (N // 128) * (K // 128) or \
            offsets.numel() != E + 1:
        raise ValueError("inconsistent grouped GEMM operand shapes")
    code = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _need(c, "c", (out_dtype,))
    if c.numel() != M * N:
        raise ValueError("c has the wrong size")
    _check(load_library().fp8q_grouped_gemm_blockscaled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(c), code,
                                                        _ptr(offsets), E, M, N, K, _stream_ptr(stream)),
           "fp8q_grouped_gemm_blockscaled")
    return c


def fp8q_grouped_gemm_blockscaled_gather(q, s, row_token, qw, sw, offsets, out_dtype=torch.bfloat16, c=None,
                                         stream=None):
    """Grouped GEMM reading each row's token through ``row_token`` (the FP8 dispatch folded into the GEMM).
    ``q`` [T, K] token codes, ``s`` [K/128, T] token scales, ``row_token`` int32 device [M_total] (-1: empty
    row), ``qw`` [E, N, K], ``sw`` [E, N/128, K/128], ``offsets`` int32 device [E+1] -> ``c`` [M_total, N]."""
    _need(q, "q", _FP8, 2)
    _need(qw, "qw", _FP8, 3)
    _need(s, "s", (torch.float32,))
    _need(sw, "sw", (torch.float32,))
    _need(row_token, "row_token", (torch.int32,), 1)
    _need(offsets, "offsets", (torch.int32,), 1)
    T, K = q.shape
    E, N, K2 = qw.shape
    M = row_token.numel()
    if K2 != K or s.numel() != (K // 128) * T or sw.numel() != E * (N // 128) * (K // 128) or \
            offsets.numel() != E + 1:
        raise ValueError("inconsistent grouped GEMM operand shapes")
    code = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=qw.device)
    _need(c, "c", (out_dtype,))
    if c.numel() != M * N:
        raise ValueError("c has the wrong size")
    _check(load_library().fp8q_grouped_gemm_blockscaled_gather(
        _ptr(q), _ptr(s), T, _ptr(row_token), _ptr(qw), _ptr(sw), _ptr(c), code, _ptr(offsets), E, M, N, K,
        _stream_ptr(stream)), "fp8q_grouped_gemm_blockscaled_gather")
    return c


def fp8q_moe_route_capacity(T: int, E: int, k: int) -> int:
    """Rows any routing of T tokens to k of E experts fits in (T*k + 127*E, rounded up to 128)."""
    n = load_library().fp8q_moe_route_capacity(T, E, k)
    if n < 0:
        raise ValueError(f"invalid routing sizes T={T} E={E} k={k}")
    return n


def fp8q_moe_route_topk(logits, k: int, rows: int | None = None, workspace=None, out=None, stream=None):
    """Top-k gating and the expert-sorted, 128-padded layout.  ``logits`` float32 [T, E] ->
    ``(topk_idx int32 [T, k], offsets int32 [E+1], row_of int32 [T, k], row_token int32 [rows])``.
    ``rows`` defaults to :func:`fp8q_moe_route_capacity`; ``workspace`` (any device tensor of at least
    ``fp8q_moe_route_workspace_bytes(T, E)`` bytes) and ``out`` (the four outputs) are allocated when
    not given."""
    _need(logits, "logits", (torch.float32,), 2)
    T, E = logits.shape
    lib = load_library()
    cap = fp8q_moe_route_capacity(T, E, k)
    rows = cap if rows is None else rows
    wbytes = lib.fp8q_moe_route_workspace_bytes(T, E)
    if wbytes < 0:
        raise ValueError(f"invalid routing sizes T={T} E={E}")
    if workspace is None:
        workspace = torch.empty(max(wbytes, 4), dtype=torch.uint8, device=logits.device)
    if out is None:
        dev = logits.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty(rows, dtype=torch.int32, device=dev))
    topk_idx, offsets, row_of, row_token = out
    for t, n, size in ((topk_idx, "topk_idx", T * k), (offsets, "offsets", E + 1), (row_of, "row_of", T * k),
                       (row_token, "row_token", rows)):
        _need(t, n, (torch.int32,))
        if t.numel() != size:
            raise ValueError(f"{n} has {t.numel()} elements; expected {size}")
    if not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    _check(lib.fp8q_moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(offsets), _ptr(row_of),
                                   _ptr(row_token), rows, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "fp8q_moe_route_topk")
    return topk_idx, offsets, row_of, row_token


def fp8q_moe_route_topk_noalloc(logits, k: int, rows: int | None = None, out=None, stream=None):
    """:func:`fp8q_moe_route_topk` through the entry point that allocates nothing: its workspace is the
    library's fixed per-GPU array (calls that overlap on one GPU race).  ``out`` (the four outputs) is
    allocated here when not given; the C call itself allocates nothing."""
    _need(logits, "logits", (torch.float32,), 2)
    T, E = logits.shape
    lib = load_library()
    cap = fp8q_moe_route_capacity(T, E, k)
    rows = cap if rows is None else rows
    if out is None:
        dev = logits.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty(rows, dtype=torch.int32, device=dev))
    topk_idx, offsets, row_of, row_token = out
    for t, n, size in ((topk_idx, "topk_idx", T * k), (offsets, "offsets", E + 1), (row_of, "row_of", T * k),
                       (row_token, "row_token", rows)):
        _need(t, n, (torch.int32,))
        if t.numel() != size:
            raise ValueError(f"{n} has {t.numel()} elements; expected {size}")
    _check(lib.fp8q_moe_route_topk_noalloc(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(offsets), _ptr(row_of),
                                           _ptr(row_token), rows, _stream_ptr(stream)),
           "fp8q_moe_route_topk_noalloc")
    return topk_idx, offsets, row_of, row_token


def fp8q_moe_gather_fp8(q, s, row_of, row_token, offsets, qa=None, sa=None, stream=None):
    """Expert-sorted FP8 rows for the grouped GEMM.  ``q`` E4M3 [T, K] and ``s`` float32 [K/128, T] (the
    quantized tokens), ``row_of`` int32 [T, k], ``row_token`` int32 [rows] and ``offsets`` int32 [E+1] (one
    :func:`fp8q_moe_route_topk` call) -> ``(qa uint8 [rows, K], sa float32 [K/128, rows])``; rows from
    ``offsets[E]`` on are left as they were."""
    _need(q, "q", _FP8, 2)
    _need(s, "s", (torch.float32,))
    _need(row_of, "row_of", (torch.int32,), 2)
    _need(row_token, "row_token", (torch.int32,), 1)
    _need(offsets, "offsets", (torch.int32,), 1)
    T, K = q.shape
    if row_of.shape[0] != T:
        raise ValueError("row_of must have one row per token")
    k = row_of.shape[1]
    rows = row_token.numel()
    E = offsets.numel() - 1
    if s.numel() != (K // 128) * T:
        raise ValueError("s has the wrong size")
    if qa is None:
        qa = torch.empty((rows, K), dtype=torch.uint8, device=q.device)
    if sa is None:
        sa = torch.empty((K // 128, rows), dtype=torch.float32, device=q.device)
    _need(qa, "qa", _FP8)
    _need(sa, "sa", (torch.float32,))
    if qa.numel() != rows * K or sa.numel() != (K // 128) * rows:
        raise ValueError("output tensors have the wrong size")
    _check(load_library().fp8q_moe_gather_fp8(_ptr(q), _ptr(s), T, K, k, _ptr(row_of), _ptr(row_token),
                                              _ptr(offsets), E, rows, _ptr(qa), _ptr(sa), _stream_ptr(stream)),
           "fp8q_moe_gather_fp8")
    return qa, sa
