"""The routing entry point that allocates nothing (its workspace is the library's fixed per-GPU array) against
the routing entry point that takes a caller's workspace: bit-identical outputs (integer work), on two calls in a
row, the second with a smaller input, so that the first call's leftovers in the shared array cannot leak into
the second.  Calls past the array's size are refused before any launch."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
from gpu_util import f32_dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _logits(T, E, seed, ties=False):
    g = np.random.default_rng([41, seed])
    if ties:
        vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
        return vals[g.integers(0, len(vals), size=(T, E))]
    return g.standard_normal((T, E), dtype=np.float32)


def _both(lg, k):
    T, E = lg.shape
    rows = fq.fp8q_moe_route_capacity(T, E, k)
    d = f32_dev(lg)
    outs = []
    for fn in ("noalloc", "workspace"):
        out = tuple(torch.full(shape, -7, dtype=torch.int32, device="cuda")
                    for shape in ((T, k), (E + 1,), (T, k), (rows,)))
        if fn == "noalloc":
            fq.fp8q_moe_route_topk_noalloc(d, k, out=out)
        else:
            ws = torch.full((max(fq.load_library().fp8q_moe_route_workspace_bytes(T, E), 4),), 0x5A,
                            dtype=torch.uint8, device="cuda")
            fq.fp8q_moe_route_topk(d, k, workspace=ws, out=out)
        outs.append([host(t) for t in out])
    return outs


@pytest.mark.parametrize("first,second", [((8192, 64, 8, False), (1000, 256, 8, False)),
                                          ((65536, 1024, 2, True), (777, 64, 8, True))],
                         ids=["moe_layer_then_smaller", "largest_then_tie_heavy"])
def test_noalloc_routing_matches_the_workspace_entry_point(first, second):
    for i, (T, E, k, ties) in enumerate((first, second)):
        say(f"no-alloc routing, call {i + 1}: T={T} E={E} k={k} ties={ties}")
        a, b = _both(_logits(T, E, T + E, ties), k)
        for name, x, y in zip(("topk_idx", "offsets", "row_of", "row_token"), a, b):
            assert np.array_equal(x, y), f"call {i + 1}: {name} differs"


def test_noalloc_routing_refuses_calls_past_the_array():
    T, E, k = 65536 + 64, 1024, 2
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        fq.fp8q_moe_route_topk_noalloc(lg, k)
