"""Empty inputs through the binding and the C ABI on the GPU: zero tokens or zero rows give empty outputs and
no error, for every quantizer, the GEMMs and the dequantization."""
import pytest
import torch

import fine_grained_quantization_amd as fq

pytestmark = pytest.mark.gpu


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def test_quantizers_with_no_rows():
    for fn, width in ((fq.fp8q_quant_act_1x128, 512), (fq.fp8q_quant_act_fp4_1x128, 256),
                      (fq.fp8q_quant_act_e5m6_1x128, 768)):
        q, s = fn(bf16(0, 512))
        assert q.shape == (0, width) and s.shape == (4, 0)
    q, s = fq.fp8q_quant_w_128x128(bf16(0, 512))
    assert q.shape == (0, 512) and s.numel() == 0
    q, s = fq.fp8q_quant_w_per_channel(bf16(0, 512))
    assert q.shape == (0, 512) and s.shape == (0,)
    q, s = fq.fp8q_swiglu_quant_act_1x128(bf16(0, 512), bf16(0, 512))
    assert q.shape == (0, 512) and s.shape == (4, 0)
    q, s, qt, st = fq.fp8q_quant_act_dual(bf16(0, 512))
    assert q.shape == (0, 512) and qt.shape == (512, 0) and st.shape == (0, 512)
    torch.cuda.synchronize()


def test_gemms_and_dequant_with_no_rows():
    qw = torch.zeros((256, 512), dtype=torch.uint8, device="cuda")
    sw = torch.ones((2, 4), dtype=torch.float32, device="cuda")
    qa = torch.zeros((0, 512), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    for out in (torch.bfloat16, torch.float32):
        c = fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=out)
        assert c.shape == (0, 256) and c.dtype == out
    off = torch.zeros(3, dtype=torch.int32, device="cuda")
    c = fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw.view(2, 128, 512), sw.view(2, 1, 4), off)
    assert c.shape == (0, 128)
    w = fq.fp8q_dequant_w_128x128(torch.zeros((0, 512), dtype=torch.uint8, device="cuda"),
                                  torch.zeros((0, 4), dtype=torch.float32, device="cuda"))
    assert w.shape == (0, 512)
    torch.cuda.synchronize()
