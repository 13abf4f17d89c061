"""Every call runs on the stream it is given.  The input is still being written on a side stream (about a
millisecond of queued work) when the quantizers and the GEMM are called on that stream, so a launch that
went to any other stream would read the stale input; the results must equal those of the same calls made
after everything has finished.  Streams are created at the default priority."""
import pytest
import torch

import fine_grained_quantization_amd as fq
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def slow_write(dst, src, times=12):
    """dst = src, written `times` times over (exact copies), all queued on the current stream."""
    dst.zero_()
    for _ in range(times):
        dst.copy_(src)


def test_calls_follow_their_stream():
    M, N, K = 8192, 2048, 8192     # a 128 MB bf16 input, so the queued writes take a while
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    src = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    torch.cuda.synchronize()
    # reference: every input complete before the calls
    qa0, sa0 = fq.fp8q_quant_act_1x128(src)
    qw0, sw0 = fq.fp8q_quant_w_128x128(w)
    c0 = fq.fp8q_gemm_blockscaled(qa0, sa0, qw0, sw0)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    x = torch.zeros_like(src)
    qa, sa = torch.empty_like(qa0), torch.empty_like(sa0)
    c = torch.empty_like(c0)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        slow_write(x, src)
    # passed explicitly, from outside the stream context
    fq.fp8q_quant_act_1x128(x, qa, sa, stream=side)
    with torch.cuda.stream(side):              # taken from the current stream
        qw, sw = fq.fp8q_quant_w_128x128(w)
        fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, c=c)
    side.synchronize()
    say("streams: side-stream results vs. reference")
    assert torch.equal(x.view(torch.int16), src.view(torch.int16))
    assert torch.equal(qa, qa0) and torch.equal(sa.view(torch.int32), sa0.view(torch.int32))
    assert torch.equal(qw, qw0) and torch.equal(sw.view(torch.int32), sw0.view(torch.int32))
    assert torch.equal(c.view(torch.int16), c0.view(torch.int16))


def test_benchmark_moe_step_on_two_streams_matches_one_stream():
    """The benchmark's MoE step runs the token quantization and the routing on a second stream beside the
    weight quantization, and the GEMM waits for both.  Several steps back to back (a step's token
    quantization must not overwrite tokens the previous step's GEMM still reads) give, bit for bit, the
    outputs of the same calls made one after another on one stream."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    wk = bench.Workload("moe")
    assert wk.side is not None
    say("moe step on two streams, 4 steps back to back")
    # the GEMM leaves the rows past the routing layout untouched, so both runs start from the same contents
    wk.c.fill_(float("nan"))
    for _ in range(4):
        wk.step()
    torch.cuda.synchronize()
    outs = [t.clone() for t in (wk.qt, wk.st, *wk.route_out, wk.qw, wk.sw, wk.c)]
    # the same kernels in order on the current stream alone
    for t in (wk.qt, wk.qw, *wk.route_out):
        t.zero_()
    wk.st.zero_()
    wk.sw.zero_()
    wk.c.fill_(float("nan"))
    for _, fn, _ in wk.kernels:
        fn()
    torch.cuda.synchronize()
    refs = (wk.qt, wk.st, *wk.route_out, wk.qw, wk.sw, wk.c)
    for i, (a, b) in enumerate(zip(outs, refs)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"output {i} differs"
