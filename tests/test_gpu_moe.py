"""GPU parity of the MoE routing (top-k gating and the expert-sorted, 128-padded layout) and of the FP8 row
gather with the oracle: bit-exact, since both are integer and byte work.  Then the whole dispatch path at the
MoE layer's size (quantize tokens, route, gather, grouped GEMM) against the oracle."""
import numpy as np
import pytest
import torch

import fine_grained_quantization_amd as fq
import oracle
import workloads as wl
from gpu_util import (assert_gemm_within_bound, bf16_bits_to_f64, bf16_dev, f32_dev, gemm_out_to_f64, host,
                      literal_bound_ratio, say, u8_dev)

pytestmark = pytest.mark.gpu


def gpu_route(logits, k, rows):
    """Routes on the GPU with every output and the workspace pre-filled with garbage."""
    T, E = logits.shape
    ws_bytes = fq.load_library().fp8q_moe_route_workspace_bytes(T, E)
    ws = torch.full((max(ws_bytes, 4),), 0xA5, dtype=torch.uint8, device="cuda")
    out = tuple(torch.full(shape, -7, dtype=torch.int32, device="cuda")
                for shape in ((T, k), (E + 1,), (T, k), (rows,)))
    fq.fp8q_moe_route_topk(f32_dev(logits), k, rows=rows, workspace=ws, out=out)
    return [host(t) for t in out]


def check_route(logits, k, what, rows=None):
    T, E = logits.shape
    rows = oracle.moe_route_capacity(T, E, k) if rows is None else rows
    say(f"route: {what} T={T} E={E} k={k} rows={rows}")
    got = gpu_route(logits, k, rows)
    r = oracle.moe_route_topk(logits, k, rows=rows)
    for name, g, o in zip(("topk_idx", "offsets", "row_of", "row_token"), got,
                          (r.topk_idx, r.offsets, r.row_of, r.row_token)):
        bad = np.argwhere(g != o)
        assert bad.size == 0, f"{what}: {name} differs at {len(bad)} places, first {tuple(bad[0])}"
    return r


def logits_of(kind, T, E, seed):
    g = np.random.default_rng([21, seed])
    if kind == "ties":       # five values including both zeros: most rows hold ties
        vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
        return vals[g.integers(0, len(vals), size=(T, E))]
    x = g.standard_normal((T, E), dtype=np.float32)
    if kind == "skew":       # experts 0 and 1 win for most tokens; most others are empty
        x[: (T * 2) // 3, :2] += 10.0
    return x


def test_route_moe_layer_logits():
    d = wl.moe(with_weights=False)
    r = check_route(d["logits"], d["topk"], "moe layer")
    say(f"  rows used {r.M}, counts {r.counts.min()}..{r.counts.max()}")


@pytest.mark.parametrize("T,E,k,kind", [
    (1000, 256, 8, "normal"),    # 256 routed experts, top-8
    (777, 64, 8, "ties"),        # ragged last chunk, tie-heavy
    (300, 64, 8, "skew"),        # empty experts and 2-segment skew
    (1, 4, 2, "normal"),
    (0, 8, 2, "normal"),         # no tokens: offsets 0, every row empty
    (65, 16, 16, "ties"),        # k = 16 (the 16-entry list), k = E
    (129, 33, 9, "normal"),      # odd E, k = 9
    (130, 1024, 3, "normal"),    # the largest E
    (100, 64, 1, "ties"),        # k = 1
])
def test_route_matches_oracle(T, E, k, kind):
    check_route(logits_of(kind, T, E, T + E + k), k, f"{kind}")


def test_route_rows_past_capacity_are_empty_and_calls_repeat():
    lg = logits_of("normal", 500, 64, 5)
    cap = oracle.moe_route_capacity(500, 64, 8)
    check_route(lg, 8, "rows past capacity", rows=cap + 300)
    a = gpu_route(lg, 8, cap)
    b = gpu_route(lg, 8, cap)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("T,K,E,k", [(1000, 512, 64, 8), (5, 128, 4, 2), (0, 256, 8, 2), (300, 7168, 64, 8)])
def test_gather_matches_oracle(T, K, E, k):
    """Random codes and scales, the oracle's layout; rows at or past offsets[E] must keep their contents."""
    g = np.random.default_rng([22, T, K])
    q = g.integers(0, 256, size=(T, K), dtype=np.uint8)
    s = g.uniform(1e-4, 1.0, size=(K // 128, T)).astype(np.float32)
    cap = oracle.moe_route_capacity(T, E, k)
    r = oracle.moe_route_topk(logits_of("normal", T, E, 3), k, rows=cap)
    say(f"gather: T={T} K={K} E={E} k={k} rows {r.M} of {cap}")
    qa = torch.full((cap, K), 0xCD, dtype=torch.uint8, device="cuda")
    sa = torch.full((K // 128, cap), -3.0, dtype=torch.float32, device="cuda")
    row_of = torch.from_numpy(r.row_of.reshape(T, k)).cuda()
    fq.fp8q_moe_gather_fp8(u8_dev(q), f32_dev(s), row_of, torch.from_numpy(r.row_token).cuda(),
                           torch.from_numpy(r.offsets).cuda(), qa, sa)
    gq, gs = host(qa), host(sa)
    oq, os_ = oracle.moe_gather_fp8(q, s, r.row_token)
    used = r.M
    assert np.array_equal(gq[:used], oq[:used])
    assert np.array_equal(gs[:, :used].view(np.uint32), os_[:, :used].view(np.uint32))
    assert np.all(gq[used:] == 0xCD) and np.all(gs[:, used:] == -3.0)


def test_full_dispatch_path_of_the_moe_layer():
    """8192 tokens x 7168 quantized, routed top-8 of 64 and gathered on the GPU (bit-exact with the oracle's
    quantizer, routing and gather), then the grouped GEMM over the routing capacity: sampled rows of every
    expert segment within the GEMM bound, padding rows exactly 0, rows past the layout untouched."""
    d = wl.moe()
    T, E, k, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
    cap = fq.fp8q_moe_route_capacity(T, E, k)
    say(f"moe dispatch: T={T} E={E} k={k} K={K}, capacity {cap} rows")
    qt, st = fq.fp8q_quant_act_1x128(bf16_dev(d["tokens"]))
    topk_idx, off, row_of, row_token = fq.fp8q_moe_route_topk(f32_dev(d["logits"]), k)
    qa, sa = fq.fp8q_moe_gather_fp8(qt, st, row_of, row_token, off)
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    c = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, off, c=c)

    oqt, ost = oracle.quant_act_1x128(d["tokens"])
    r = oracle.moe_route_topk(d["logits"], k, rows=cap)
    assert np.array_equal(host(topk_idx), r.topk_idx) and np.array_equal(host(off), r.offsets)
    assert np.array_equal(host(row_of), r.row_of) and np.array_equal(host(row_token), r.row_token)
    used = r.M
    oqa, osa = oracle.moe_gather_fp8(oqt, ost, r.row_token[:used])
    assert np.array_equal(host(qa)[:used], oqa)
    assert np.array_equal(host(sa)[:, :used].view(np.uint32), osa.view(np.uint32))
    say(f"  quantize + route + gather bit-exact over {used} rows")

    oqw, osw = oracle.quant_w_128x128(d["w"])
    g = np.random.default_rng(4)
    counts = r.counts
    rows = []
    for e in range(E):
        lo, cnt = int(r.offsets[e]), int(counts[e])
        if cnt:
            rows += [lo, lo + cnt - 1, lo + int(g.integers(cnt))]
    rows = np.array(sorted(set(rows)))
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, r.offsets, rows=rows)
    ch = gemm_out_to_f64(c)
    ratio = assert_gemm_within_bound(ch[rows], C, B, True, "moe dispatch")
    empty = np.nonzero(r.row_token[:used] < 0)[0]
    assert np.all(ch[empty] == 0.0)
    assert np.all(np.isnan(ch[used:]))
    say(f"  grouped GEMM max err/bound {ratio:.3g}")


def fused_and_separate(q, s, logits, k, qw, sw, out, rows=None):
    """The grouped GEMM on gathered rows, and the gather-fused grouped GEMM on the token rows, both into
    buffers pre-filled with NaN; returns (separate, fused, routing)."""
    T, K = q.shape
    E = logits.shape[1]
    cap = oracle.moe_route_capacity(T, E, k) if rows is None else rows
    r = oracle.moe_route_topk(logits, k, rows=cap)
    N = qw.shape[1]
    off = torch.from_numpy(r.offsets).cuda()
    rt = torch.from_numpy(r.row_token).cuda()
    qd, sd = u8_dev(q), f32_dev(s)
    qa = torch.zeros((cap, K), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((K // 128, cap), dtype=torch.float32, device="cuda")
    fq.fp8q_moe_gather_fp8(qd, sd, torch.from_numpy(r.row_of.reshape(T, k)).cuda(), rt, off, qa, sa)
    c1 = torch.full((cap, N), float("nan"), dtype=out, device="cuda")
    c2 = torch.full((cap, N), float("nan"), dtype=out, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled(qa, sa, qw, sw, off, out_dtype=out, c=c1)
    fq.fp8q_grouped_gemm_blockscaled_gather(qd, sd, rt, qw, sw, off, out_dtype=out, c=c2)
    return host(c1), host(c2), r


def same_bits(a, b):
    return np.array_equal(a.view(np.uint16 if a.dtype == np.uint16 else np.uint32),
                          b.view(np.uint16 if b.dtype == np.uint16 else np.uint32))


@pytest.mark.parametrize("T,K,N,E,k,out", [(300, 512, 256, 64, 8, torch.bfloat16), (5, 128, 384, 4, 2, torch.float32),
                                           (0, 256, 128, 8, 2, torch.bfloat16), (1000, 1024, 512, 16, 4, torch.float32),
                                           (1000, 256, 128, 256, 8, torch.bfloat16)])   # 256 experts
def test_gather_fused_grouped_gemm_matches_gather_then_gemm(T, K, N, E, k, out):
    """Bit-identical to gathering the rows first, padding rows exactly 0, rows past the layout untouched, and
    within the GEMM bound of the oracle on every row."""
    g = np.random.default_rng([23, T, K, N])
    q = g.integers(0, 254, size=(T, K)).astype(np.uint8)
    q[q >= 0x7F] += 1                                     # finite codes only
    s = g.uniform(1e-4, 1e-2, size=(K // 128, T)).astype(np.float32)
    w = wl.bf16_bits((g.standard_normal((E * N, K)) * 0.02).astype(np.float32))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(w).view(E, N, K))
    say(f"gather-fused grouped: T={T} K={K} N={N} E={E} k={k} {out}")
    c1, c2, r = fused_and_separate(q, s, logits_of("normal", T, E, 7), k, qw, sw, out)
    assert same_bits(c1, c2)
    used = r.M
    f = bf16_bits_to_f64(c2) if out == torch.bfloat16 else c2.astype(np.float64)
    assert np.all(np.isnan(f[used:]))
    empty = np.nonzero(r.row_token[:used] < 0)[0]
    assert np.all(f[empty] == 0.0)
    if used:
        oqa, osa = oracle.moe_gather_fp8(q, s, r.row_token[:used])
        C, B = oracle.grouped_gemm_blockscaled(oqa, osa, host(qw), host(sw), r.offsets)
        assert_gemm_within_bound(f[:used], C, B, out == torch.bfloat16, "gather-fused grouped")


def test_gather_fused_tokens_out_of_range_read_as_empty_rows():
    """A row whose token is >= T (as well as -1) gives an exactly zero output row."""
    T, K, N, E = 64, 256, 256, 2
    g = np.random.default_rng(24)
    q = g.integers(0, 0x7E, size=(T, K)).astype(np.uint8)
    s = g.uniform(1e-3, 1e-2, size=(K // 128, T)).astype(np.float32)
    w = wl.bf16_bits((g.standard_normal((E * N, K)) * 0.02).astype(np.float32))
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(w).view(E, N, K))
    rt = np.arange(256, dtype=np.int32) % (T + 40)          # tokens T .. T+39 are out of range
    rt[::7] = -1
    off = torch.tensor([0, 128, 256], dtype=torch.int32, device="cuda")
    c = fq.fp8q_grouped_gemm_blockscaled_gather(u8_dev(q), f32_dev(s), torch.from_numpy(rt).cuda(), qw, sw, off,
                                                out_dtype=torch.float32)
    c = host(c)
    bad = (rt < 0) | (rt >= T)
    assert np.all(c[bad] == 0.0) and np.all(np.abs(c[~bad]).sum(axis=1) > 0)


@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_gather_fused_moe_layer(out):
    """The MoE layer's dispatch (8192 tokens x 7168, top-8 of 64, 64 experts x [2048, 7168]) through the
    gather-fused grouped GEMM: bit-identical to gather + grouped GEMM over the whole routing capacity."""
    d = wl.moe()
    T, E, k, K = d["T"], d["E"], d["topk"], d["K"]
    say(f"gather-fused grouped: moe layer {out}")
    q, s = oracle.quant_act_1x128(d["tokens"])
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    c1, c2, r = fused_and_separate(q, s, d["logits"], k, qw, sw, out)
    assert same_bits(c1, c2)
    say(f"  bit-identical over {r.M} rows")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_moe_layer_timed_path_against_oracle(out):
    """The MoE layer exactly as the benchmark's step runs it: the tokens quantized (1x128) and routed on the
    GPU, the expert weights quantized (128x128) on the GPU, and the grouped GEMM reading the routed token rows
    in place, over the routing capacity.  Against the oracle's quantizers, routing, gather and grouped GEMM:
    four rows of every expert segment (its first and last routed rows and two others) on all 2048 columns,
    and two experts' whole segments (every row, the segment's 128-row half tile included) on two 256-column
    blocks.  fp32 output is held to the literal bound 1e-3 B + 1e-6; bf16 output to that plus its own final
    rounding, with the literal ratio printed.  Empty rows are exactly 0, rows past the layout untouched."""
    d = wl.moe()
    T, E, k, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
    dt = torch.float32 if out == "f32" else torch.bfloat16
    cap = fq.fp8q_moe_route_capacity(T, E, k)
    say(f"moe layer, timed path: T={T} E={E} k={k} N={N} K={K} out={out}, capacity {cap} rows")
    qt, st = fq.fp8q_quant_act_1x128(bf16_dev(d["tokens"]))
    _, off, _, row_token = fq.fp8q_moe_route_topk(f32_dev(d["logits"]), k)
    qw, sw = fq.fp8q_quant_w_128x128(bf16_dev(d["w"]))
    c = torch.full((cap, N), float("nan"), dtype=dt, device="cuda")
    fq.fp8q_grouped_gemm_blockscaled_gather(qt, st, row_token, qw, sw, off, out_dtype=dt, c=c)
    ch = gemm_out_to_f64(c)

    oqt, ost = oracle.quant_act_1x128(d["tokens"])
    r = oracle.moe_route_topk(d["logits"], k, rows=cap)
    assert np.array_equal(host(off), r.offsets) and np.array_equal(host(row_token), r.row_token)
    used = r.M
    oqa, osa = oracle.moe_gather_fp8(oqt, ost, r.row_token[:used])
    oqw, osw = oracle.quant_w_128x128(d["w"])
    g = np.random.default_rng(8)
    rows = []
    for e in range(E):
        lo, cnt = int(r.offsets[e]), int(r.counts[e])
        if cnt:
            rows += [lo, lo + cnt - 1] + [lo + int(i) for i in g.integers(cnt, size=2)]
    rows = np.array(sorted(set(rows)))
    bf = out == "bf16"
    C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, r.offsets, rows=rows)
    r1 = assert_gemm_within_bound(ch[rows], C, B, bf, "moe sampled rows")
    lit = [literal_bound_ratio(ch[rows], C, B)]
    # whole segments: an expert whose padded length is an odd number of 128-row blocks (its last tile is the
    # 128 x 256 layout) and one with an even number, if there is one
    seg = np.diff(r.offsets) // 128
    odd = [e for e in range(E) if seg[e] % 2 == 1]
    even = [e for e in range(E) if seg[e] % 2 == 0 and seg[e] > 0]
    r2 = 0.0
    for e, n0 in [(odd[0] if odd else 0, 1792), (even[0] if even else E - 1, 512)]:
        tr = np.arange(r.offsets[e], r.offsets[e + 1])
        tc = np.arange(n0, n0 + 256)
        C, B = oracle.grouped_gemm_blockscaled(oqa, osa, oqw, osw, r.offsets, rows=tr, cols=tc)
        got = ch[r.offsets[e]:r.offsets[e + 1], n0:n0 + 256]
        r2 = max(r2, assert_gemm_within_bound(got, C, B, bf, f"moe expert {e} segment, columns {n0}.."))
        lit.append(literal_bound_ratio(got, C, B))
    empty = np.nonzero(r.row_token[:used] < 0)[0]
    assert np.all(ch[empty] == 0.0)
    assert np.all(np.isnan(ch[used:]))
    say(f"  {len(rows)} sampled rows max err/bound {r1:.3g}; whole segments {r2:.3g}; "
        f"literal-bound ratio {max(lit):.3g}")
