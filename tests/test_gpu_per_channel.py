"""GPU parity of the per-channel FP8 weight quantization (one scale per output channel over the whole row)
with the oracle, bit-exact: ragged row counts and lengths, rows longer than the part a workgroup keeps in
registers (8192 elements, 16384 for longer rows; the rest is read twice), special values, the up
projection's full weight, and the K = 128 case against the 1x128 quantizer."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import bf16_dev, host, say

pytestmark = pytest.mark.gpu


def rows_of(rng, N, K):
    """N(0,1) rows at scales 2^-20..2^10, with zero rows, one-element rows, signed zeros, subnormal bf16 and
    the row maximum placed anywhere (also past the first 8192 elements)."""
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-20, 11, size=(N, 1)))).astype(np.float32)
    b = wl.bf16_bits(w)
    if N > 2 and K:
        b[0] = 0
        b[1] = 0x8000
        b[2] = 0
        b[2, rng.integers(K)] = 0xC2F0                      # a single -120
    m = rng.random((N, K)) < 0.01
    b[m] = rng.integers(0, 0x80, m.sum()).astype(np.uint16) | (rng.integers(0, 2, m.sum()) << 15).astype(np.uint16)
    if N > 3 and K:
        b[3:, rng.integers(K)] = 0x4780                     # 65536: every later row's maximum
    return b


def check(wb, what):
    N, K = wb.shape
    say(f"per-channel: {what} N={N} K={K}")
    q = torch.full((N, K), 0xCD, dtype=torch.uint8, device="cuda")
    s = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    fq.fp8q_quant_w_per_channel(bf16_dev(wb), q=q, s=s)
    oq, os_ = oracle.quant_w_per_channel(wb)
    gq, gs = host(q), host(s)
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), what


@pytest.mark.parametrize("N,K", [(37, 1000), (1, 8), (5, 8192), (6, 8200), (130, 24576), (300, 7168),
                                 (4, 0), (3, 136), (9, 16384), (7, 16392)])
def test_matches_oracle(N, K):
    check(rows_of(np.random.default_rng([51, N, K]), N, K), "ragged")


def test_row_maximum_in_the_twice_read_tail():
    """Rows longer than the part a workgroup keeps in registers (16384 elements): the maximum in the chunks that
    are read twice (the last element, or the first chunk past the registers), or in the registers."""
    wb = rows_of(np.random.default_rng(53), 8, 20480)
    wb[3, -1] = 0x4800            # 131072, the row's maximum, in its last element
    wb[4, 16384] = 0xC800         # -131072, the first element past the registers
    wb[5, 16383] = 0x4800         # the last element held in registers
    check(wb, "maximum in the tail")


def test_up_projection_weight():
    check(wl.per_channel()["w"], "up projection weight")


def test_down_projection_weight():
    """The down projection's weight [7168, 18432] (the down workload's recipe and seed): rows past 16384
    elements, so each workgroup keeps 8 chunks a lane in registers and reads the rest twice."""
    check(wl.normal_bf16(wl.SEEDS["down"], wl.T_W, (7168, 18432), 0.02), "down projection weight")


def test_k128_equals_the_1x128_quantizer():
    wb = rows_of(np.random.default_rng(52), 64, 128)
    q1, s1 = fq.fp8q_quant_w_per_channel(bf16_dev(wb))
    q2, s2 = fq.fp8q_quant_act_1x128(bf16_dev(wb))
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32).reshape(-1))
