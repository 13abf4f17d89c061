"""The C-ABI library loads, exports every entry point that include/fp8q.h declares, and rejects bad
arguments before touching a device.  No kernel is launched here (CPU-only)."""
import ctypes
import os
import re

import pytest

import fine_grained_quantization_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return fq.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char \*)\s*(fp8q_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8q_quant_act_1x128", "fp8q_quant_w_128x128", "fp8q_gemm_blockscaled",
              "fp8q_grouped_gemm_blockscaled", "fp8q_dequant_w_128x128", "fp8q_moe_route_capacity",
              "fp8q_moe_route_workspace_bytes", "fp8q_moe_route_topk", "fp8q_moe_gather_fp8",
              "fp8q_swiglu_quant_act_1x128", "fp8q_swiglu_bf16", "fp8q_quant_act_dual",
              "fp8q_quant_act_fp4_1x128", "fp8q_quant_w_fp4_128x128", "fp8q_quant_w_per_channel",
              "fp8q_quant_act_e5m6_1x128", "fp8q_grouped_gemm_blockscaled_gather", "fp8q_moe_route_topk_noalloc",
              "fp8q_status_string", "fp8q_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in fp8q.h but not exported"


def test_library_contains_gfx950_code():
    blob = open(fq.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings(lib):
    assert lib.fp8q_version() >= 100
    for code in range(0, -9, -1):
        assert lib.fp8q_status_string(code).decode().startswith("FP8Q_")
    assert b"unknown" in lib.fp8q_status_string(42)


A = ctypes.c_void_p(4096)      # aligned dummy addresses: never dereferenced, every call below fails validation
B = ctypes.c_void_p(8192)
MIS = ctypes.c_void_p(4098)


def test_argument_validation_without_device(lib):
    # shape errors come first
    assert lib.fp8q_quant_act_1x128(A, 4, 100, B, B, None) == -2
    assert lib.fp8q_quant_act_1x128(A, -1, 128, B, B, None) == -2
    assert lib.fp8q_quant_w_128x128(A, 100, 128, B, B, None) == -2
    assert lib.fp8q_gemm_blockscaled(A, A, A, A, B, 0, 4, 100, 128, None) == -2
    assert lib.fp8q_gemm_blockscaled(A, A, A, A, B, 0, 4, 128, 64, None) == -2
    assert lib.fp8q_gemm_blockscaled(A, A, A, A, B, 0, 4, 128, (1 << 23) + 128, None) == -2
    assert lib.fp8q_grouped_gemm_blockscaled(A, A, A, A, B, 0, A, 0, 128, 128, 128, None) == -2
    assert lib.fp8q_grouped_gemm_blockscaled(A, A, A, A, B, 0, A, 2, 100, 128, 128, None) == -2
    # dtype
    assert lib.fp8q_gemm_blockscaled(A, A, A, A, B, 7, 4, 128, 128, None) == -4
    # empty problems succeed without work
    assert lib.fp8q_quant_act_1x128(None, 0, 128, None, None, None) == 0
    assert lib.fp8q_gemm_blockscaled(None, None, None, None, None, 0, 0, 128, 128, None) == 0
    # null and alignment
    assert lib.fp8q_quant_act_1x128(None, 4, 128, B, B, None) == -1
    assert lib.fp8q_quant_w_128x128(A, 128, 128, None, B, None) == -1
    assert lib.fp8q_gemm_blockscaled(A, A, A, None, B, 1, 4, 128, 128, None) == -1
    assert lib.fp8q_grouped_gemm_blockscaled(A, A, A, A, B, 0, None, 2, 128, 128, 128, None) == -1
    assert lib.fp8q_quant_act_1x128(MIS, 4, 128, B, B, None) == -3
    # dequantization
    assert lib.fp8q_dequant_w_128x128(A, B, 100, 128, B, None) == -2
    assert lib.fp8q_dequant_w_128x128(A, B, 128, 64, B, None) == -2
    assert lib.fp8q_dequant_w_128x128(None, None, 0, 128, None, None) == 0
    assert lib.fp8q_dequant_w_128x128(A, None, 128, 128, B, None) == -1
    assert lib.fp8q_dequant_w_128x128(A, B, 128, 128, MIS, None) == -3
    assert lib.fp8q_gemm_blockscaled(A, A, A, A, MIS, 0, 4, 128, 128, None) == -3
    # FP4 in the FP8 groupings
    assert lib.fp8q_quant_act_fp4_1x128(A, 4, 100, B, B, None) == -2
    assert lib.fp8q_quant_w_fp4_128x128(A, 100, 128, B, B, None) == -2
    assert lib.fp8q_quant_act_fp4_1x128(None, 0, 128, None, None, None) == 0
    assert lib.fp8q_quant_act_fp4_1x128(A, 4, 128, None, B, None) == -1
    assert lib.fp8q_quant_w_fp4_128x128(A, 128, 128, MIS, B, None) == -3
    # grouped GEMM reading token rows through row_token
    gg = lib.fp8q_grouped_gemm_blockscaled_gather
    assert gg(A, A, 4, B, A, A, A, 0, B, 2, 100, 128, 128, None) == -2          # M_total not a multiple of 128
    assert gg(A, A, -1, B, A, A, A, 0, B, 2, 128, 128, 128, None) == -2         # negative T
    assert gg(A, A, 1 << 30, B, A, A, A, 0, B, 2, 128, 128, 128, None) == -2    # T * K past 2^31
    assert gg(A, A, 4, B, A, A, A, 0, B, 2, 0, 128, 128, None) == 0             # no rows
    assert gg(A, A, 4, None, A, A, A, 0, B, 2, 128, 128, 128, None) == -1       # no row map
    assert gg(A, A, 4, B, A, A, A, 7, B, 2, 128, 128, 128, None) == -4          # bad out dtype
    # E5M6 activations
    assert lib.fp8q_quant_act_e5m6_1x128(A, 4, 100, B, B, None) == -2
    assert lib.fp8q_quant_act_e5m6_1x128(None, 0, 128, None, None, None) == 0
    assert lib.fp8q_quant_act_e5m6_1x128(A, 4, 128, None, B, None) == -1
    assert lib.fp8q_quant_act_e5m6_1x128(A, 4, 128, B, MIS, None) == -3
    # per-channel weights: any K that is a multiple of 8
    assert lib.fp8q_quant_w_per_channel(A, 4, 100, B, B, None) == -2
    assert lib.fp8q_quant_w_per_channel(A, -1, 128, B, B, None) == -2
    assert lib.fp8q_quant_w_per_channel(None, 0, 128, None, None, None) == 0
    assert lib.fp8q_quant_w_per_channel(A, 4, 1000, B, None, None) == -1
    assert lib.fp8q_quant_w_per_channel(A, 4, 1000, MIS, B, None) == -3
    # forward and backward copies in one pass: M and K multiples of 128
    dual = lib.fp8q_quant_act_dual
    dual.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5
    assert dual(A, 100, 128, B, B, B, B, None) == -2
    assert dual(A, 128, 100, B, B, B, B, None) == -2
    assert dual(None, 0, 128, None, None, None, None, None) == 0
    assert dual(A, 128, 128, B, B, None, B, None) == -1
    assert dual(A, 128, 128, B, B, MIS, B, None) == -3
    # fused SwiGLU + quantization, and the intermediate alone
    sq, sw = lib.fp8q_swiglu_quant_act_1x128, lib.fp8q_swiglu_bf16
    sq.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 3
    sw.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2
    assert sq(A, B, 100, 4, 100, B, B, None) == -2          # K not a multiple of 128
    assert sq(A, B, 100, 4, 128, B, B, None) == -2          # ld < K
    assert sq(A, B, 260, 4, 256, B, B, None) == -2          # ld not a multiple of 8
    assert sq(None, None, 256, 0, 256, None, None, None) == 0
    assert sq(A, None, 256, 4, 256, B, B, None) == -1
    assert sq(A, MIS, 256, 4, 256, B, B, None) == -3
    assert sw(A, B, 12, 4, 12, B, None) == -2                # K not a multiple of 8
    assert sw(A, B, 16, 4, 16, None, None) == -1
    assert sw(MIS, B, 16, 4, 16, B, None) == -3


def test_moe_routing_sizes_and_validation(lib):
    import oracle
    lib.fp8q_moe_route_capacity.restype = ctypes.c_int64
    lib.fp8q_moe_route_capacity.argtypes = [ctypes.c_int64] * 3
    lib.fp8q_moe_route_workspace_bytes.restype = ctypes.c_int64
    lib.fp8q_moe_route_workspace_bytes.argtypes = [ctypes.c_int64] * 2
    I = ctypes.c_int64
    for T, E, k in ((8192, 64, 8), (0, 1, 1), (5, 256, 8), (1000, 1024, 16)):
        assert lib.fp8q_moe_route_capacity(T, E, k) == oracle.moe_route_capacity(T, E, k)
        assert lib.fp8q_moe_route_workspace_bytes(T, E) == 4 * E * ((T + 63) // 64)
    for T, E, k in ((-1, 8, 2), (8, 0, 1), (8, 1025, 2), (8, 8, 9), (8, 32, 17), (8, 8, 0)):
        assert lib.fp8q_moe_route_capacity(T, E, k) == -1
    cap = lib.fp8q_moe_route_capacity(100, 8, 2)
    route = lib.fp8q_moe_route_topk
    route.argtypes = [ctypes.c_void_p, I, I, I, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      I, ctypes.c_void_p, I, ctypes.c_void_p]
    assert route(A, 100, 8, 9, A, A, A, A, cap, A, 4096, None) == -2            # k > E
    assert route(A, 100, 8, 2, A, A, A, A, cap - 1, A, 4096, None) == -2        # rows below the capacity
    assert route(A, 100, 8, 2, A, None, A, A, cap, A, 4096, None) == -1
    assert route(A, 100, 8, 2, A, A, A, A, cap, None, 4096, None) == -1
    assert route(MIS, 100, 8, 2, A, A, A, A, cap, A, 4096, None) == -3
    assert route(A, 100, 8, 2, A, A, A, A, cap, A, 4 * 8 * 2 - 1, None) == -8    # workspace too small
    na = lib.fp8q_moe_route_topk_noalloc
    na.argtypes = [ctypes.c_void_p, I, I, I, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, I,
                   ctypes.c_void_p]
    assert na(A, 100, 8, 9, A, A, A, A, cap, None) == -2                           # k > E
    assert na(A, 100, 8, 2, A, A, A, A, cap - 1, None) == -2                       # rows below the capacity
    assert na(A, 100, 8, 2, A, None, A, A, cap, None) == -1
    assert na(MIS, 100, 8, 2, A, A, A, A, cap, None) == -3
    big_t = 65536 + 64                                                             # 4 * 1024 * 1025 bytes > 4 MiB
    assert na(A, big_t, 1024, 2, A, A, A, A, lib.fp8q_moe_route_capacity(big_t, 1024, 2), None) == -8
    gather = lib.fp8q_moe_gather_fp8
    gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, I, I, I, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       I, I, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert gather(A, A, 4, 100, 2, A, A, A, 8, 512, B, B, None) == -2                 # K not a multiple of 128
    assert gather(A, A, 4, 128, 2, A, A, A, 0, 512, B, B, None) == -2                 # E < 1
    assert gather(A, A, 4, 128, 0, A, A, A, 8, 512, B, B, None) == -2                 # k < 1
    assert gather(None, None, 4, 128, 2, None, None, None, 8, 0, None, None, None) == 0   # no rows
    assert gather(None, A, 4, 128, 2, A, A, A, 8, 512, B, B, None) == -1
    assert gather(A, A, 4, 128, 2, None, A, A, 8, 512, B, B, None) == -1              # row_of
    assert gather(A, A, 4, 128, 2, A, A, A, 8, 512, MIS, B, None) == -3


def test_valid_call_without_gpu_reports_no_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.fp8q_quant_act_1x128(A, 4, 128, B, B, None) in (-5, -6)
