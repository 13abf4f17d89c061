"""Fine-grained FP8 quantization and block-scaled FP8 GEMM for AMD Instinct MI355X (gfx950).

The compute lives in ``libfp8q.so`` (hand-written HIP kernels behind the C ABI of ``include/fp8q.h``);
this package is its Python binding.  Entry points (same names as the C functions):

  fp8q_quant_act_1x128(x)                      bf16 [M, K] -> (E4M3 [M, K], fp32 scales [K/128, M])
  fp8q_quant_act_dual(x)                       bf16 [M, K] -> the 1x128 copies of x and of x^T (backward)
  fp8q_quant_act_fp4_1x128(x), fp8q_quant_w_fp4_128x128(w)   FP4 (E2M1) in the same groups, two codes a byte
  fp8q_quant_act_e5m6_1x128(x)                 bf16 [M, K] -> 12-bit E5M6 codes, two per 3 bytes, 1x128 scales
  fp8q_quant_w_128x128(w)                      bf16 [N, K] -> (E4M3 [N, K], fp32 scales [N/128, K/128])
  fp8q_quant_w_per_channel(w)                  bf16 [N, K] -> (E4M3 [N, K], one fp32 scale per output channel [N])
  fp8q_swiglu_quant_act_1x128(x, y)            bf16 gate, up [M, K] -> 1x128 quantization of bf16(SiLU(x) * y)
  fp8q_swiglu_bf16(x, y)                       the bf16 intermediate SiLU(x) * y alone
  fp8q_gemm_blockscaled(qa, sa, qw, sw)        -> C = A W^T, bf16 or fp32 [M, N]
  fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, offsets)   MoE experts, one segment of rows each
  fp8q_grouped_gemm_blockscaled_gather(q, s, row_token, qw, sw, offsets)   the same, reading token rows directly
  fp8q_dequant_w_128x128(q, s)                 E4M3 [N, K] + fp32 [N/128, K/128] -> bf16 [N, K]
  fp8q_moe_route_topk(logits, k)               top-k experts and the expert-sorted, 128-padded row layout
  fp8q_moe_gather_fp8(q, s, row_of, row_token, offsets)   quantized token rows in that layout (FP8 dispatch)
"""
from ._binding import (  # noqa: F401
    OUT_BF16,
    OUT_F32,
    LIB_PATH,
    fp8q_dequant_w_128x128,
    fp8q_gemm_blockscaled,
    fp8q_grouped_gemm_blockscaled,
    fp8q_grouped_gemm_blockscaled_gather,
    fp8q_moe_gather_fp8,
    fp8q_moe_route_capacity,
    fp8q_moe_route_topk,
    fp8q_moe_route_topk_noalloc,
    fp8q_quant_act_1x128,
    fp8q_quant_act_dual,
    fp8q_quant_act_e5m6_1x128,
    fp8q_quant_act_fp4_1x128,
    fp8q_quant_w_128x128,
    fp8q_quant_w_fp4_128x128,
    fp8q_quant_w_per_channel,
    fp8q_swiglu_bf16,
    fp8q_swiglu_quant_act_1x128,
    load_library,
    status_string,
)
