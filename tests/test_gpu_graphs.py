"""HIP graph capture of the library's calls.  Each step the benchmark times, at a small size, is captured once
into a graph (torch.cuda.CUDAGraph) and replayed several times: the dense step (quantize A, quantize W, GEMM),
the decode step (quantize 64 tokens, small-M GEMM), the same at 96 and 200 tokens (mid-size-M GEMM) and the
MoE step (token quantization and routing on a second stream beside the weight quantization, then the grouped
GEMM reading the routed token rows).  Between replays
the inputs are rewritten by eager work and every output is overwritten with a sentinel, then the stream is
synchronized; each replay's outputs must equal those of the same calls made eagerly on the same inputs.  The
library records no memset, allocation or synchronization, so a graph holds its kernel launches only."""
import pytest
import torch

import fine_grained_quantization_amd as fq
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bf(shape, g, scale=1.0):
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def capture(step):
    """Run `step` once on a side stream (as torch asks before capturing), then capture it into a graph."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        step()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


def check_replays(what, graph, step, refill, outputs):
    """`refill()` rewrites the inputs (eager work); the outputs are set to a sentinel before the replay and
    before the eager run, so an output the replay failed to write cannot match."""
    for r in range(REPLAYS):
        refill()
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs]
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outputs)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: replay {r}, output {i}"
        say(f"graphs: {what} replay {r} matches the eager calls")


def test_dense_step_in_a_graph():
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    M, N, K = 512, 1024, 1024
    x, w = bf((M, K), g), bf((N, K), g, 0.02)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8q_quant_act_1x128(x, qa, sa)
        fq.fp8q_quant_w_128x128(w, qw, sw)
        fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, c=c)

    def refill():
        x.copy_(bf((M, K), g))
        w.copy_(bf((N, K), g, 0.02))

    check_replays("dense step", capture(step), step, refill, [qa, sa, qw, sw, c])


def test_decode_step_in_a_graph():
    g = torch.Generator(device="cuda")
    g.manual_seed(22)
    M, N, K = 64, 2048, 1024
    x = bf((M, K), g)
    qw, sw = fq.fp8q_quant_w_128x128(bf((N, K), g, 0.02))
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        fq.fp8q_quant_act_1x128(x, qa, sa)
        fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, out_dtype=torch.float32, c=c)

    check_replays("decode step", capture(step), step, lambda: x.copy_(bf((M, K), g)), [qa, sa, c])


@pytest.mark.parametrize("M", [96, 200])
def test_mid_size_step_in_a_graph(M):
    """The decode step at 96 and 200 tokens (the mid-size-M kernel, 128 and 256 token rows per workgroup)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(23 + M)
    N, K = 2048, 1024
    x = bf((M, K), g)
    qw, sw = fq.fp8q_quant_w_128x128(bf((N, K), g, 0.02))
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8q_quant_act_1x128(x, qa, sa)
        fq.fp8q_gemm_blockscaled(qa, sa, qw, sw, c=c)

    check_replays(f"mid-size step, M = {M}", capture(step), step, lambda: x.copy_(bf((M, K), g)), [qa, sa, c])


def test_moe_step_on_two_streams_in_a_graph():
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    T, E, k, N, K = 512, 8, 2, 256, 512
    tokens, w = bf((T, K), g), bf((E, N, K), g, 0.02)
    logits = torch.randn((T, E), device="cuda", generator=g)
    rows = fq.fp8q_moe_route_capacity(T, E, k)
    route = (torch.empty((T, k), dtype=torch.int32, device="cuda"), torch.empty(E + 1, dtype=torch.int32, device="cuda"),
             torch.empty((T, k), dtype=torch.int32, device="cuda"), torch.empty(rows, dtype=torch.int32, device="cuda"))
    ws = torch.empty(fq.load_library().fp8q_moe_route_workspace_bytes(T, E), dtype=torch.uint8, device="cuda")
    qt = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    st = torch.empty((K // 128, T), dtype=torch.float32, device="cuda")
    qw = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    c = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()

    def step():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            fq.fp8q_quant_act_1x128(tokens, qt, st)
            fq.fp8q_moe_route_topk(logits, k, workspace=ws, out=route)
        fq.fp8q_quant_w_128x128(w, qw, sw)
        main.wait_stream(side)
        fq.fp8q_grouped_gemm_blockscaled_gather(qt, st, route[3], qw, sw, route[1], c=c)

    def refill():
        tokens.copy_(bf((T, K), g))
        w.copy_(bf((E, N, K), g, 0.02))
        logits.copy_(torch.randn((T, E), device="cuda", generator=g))

    check_replays("MoE step", capture(step), step, refill, [qt, st, *route, qw, sw, c])
