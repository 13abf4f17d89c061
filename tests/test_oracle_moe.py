"""Pins of the oracle's MoE routing (top-k gating, expert-sorted 128-padded layout) and FP8 row gather.

Independent of the oracle's code: a hand-worked layout (tests/golden/moe_routing_hand.json), the top-k
definition checked pair by pair, library special cases (k = 1 is numpy's argmax, k = E a stable sort),
layout invariants, numpy indexing for the gather, and the gather's commutation with the row-wise 1x128
quantizer.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_routing_hand.json")


def tie_heavy_logits(rng, T, E):
    """Logits from a 5-value set that includes both zeros, so most rows hold ties."""
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
    return vals[rng.integers(0, len(vals), size=(T, E))]


def check_topk_definition(logits, idx, k):
    """Token by token, without sorting: k distinct experts; every chosen expert beats every unchosen one
    (larger logit, or an equal logit and a lower index); consecutive entries are in that order too."""
    T, E = logits.shape
    for t in range(T):
        v = logits[t]
        sel = [int(e) for e in idx[t]]
        assert len(set(sel)) == k and all(0 <= e < E for e in sel)

        def before(a, b):
            return v[a] > v[b] or (v[a] == v[b] and a < b)

        for a in sel:
            for b in range(E):
                if b not in sel:
                    assert before(a, b), (t, a, b)
        for a, b in zip(sel, sel[1:]):
            assert before(a, b), (t, a, b)


def check_layout(r, T, E, k, pad, rows):
    off = r.offsets.astype(np.int64)
    counts = np.bincount(r.topk_idx.ravel(), minlength=E)
    assert off[0] == 0 and np.all(off[1:] - off[:-1] == (counts + pad - 1) // pad * pad)
    assert len(r.row_token) == rows and rows >= off[-1]
    assert np.all(r.row_token[off[-1]:] == -1)
    for e in range(E):
        seg = r.row_token[off[e]:off[e + 1]]
        toks = np.nonzero((r.topk_idx == e).any(axis=1))[0]
        assert np.array_equal(seg[:len(toks)], toks)           # the expert's tokens, ascending
        assert np.all(seg[len(toks):] == -1)                  # then empty rows
    for t in range(T):
        for j in range(k):
            row = r.row_of[t, j]
            assert r.row_token[row] == t
            e = r.topk_idx[t, j]
            assert off[e] <= row < off[e + 1]


def test_hand_worked_routing(olib):
    g = json.load(open(GOLDEN))
    logits = np.array(g["logits"], np.float32)
    assert np.signbit(logits[1, 0]) and not np.signbit(logits[1, 1])
    r = oracle.moe_route_topk(logits, g["k"], pad=g["pad"], lib=olib)
    assert r.topk_idx.tolist() == g["topk_idx"]
    assert r.offsets.tolist() == g["offsets"]
    assert r.row_of.tolist() == g["row_of"]
    want = np.full(g["offsets"][-1], -1, np.int32)
    for row, tok in g["filled_rows"].items():
        want[int(row)] = tok
    assert np.array_equal(r.row_token, want)


@pytest.mark.parametrize("T,E,k,heavy", [(40, 8, 3, False), (40, 8, 3, True), (25, 64, 8, True), (9, 6, 6, True),
                                         (30, 256, 8, False)])
def test_topk_satisfies_the_pairwise_definition(olib, T, E, k, heavy):
    rng = np.random.default_rng([11, T, E, k, int(heavy)])
    logits = tie_heavy_logits(rng, T, E) if heavy else rng.standard_normal((T, E), dtype=np.float32)
    r = oracle.moe_route_topk(logits, k, lib=olib)
    check_topk_definition(logits, r.topk_idx, k)


def test_k1_is_argmax_and_k_equal_E_is_a_stable_sort(olib):
    rng = np.random.default_rng(12)
    for logits in (rng.standard_normal((300, 16), dtype=np.float32), tie_heavy_logits(rng, 300, 16)):
        r1 = oracle.moe_route_topk(logits, 1, lib=olib)
        assert np.array_equal(r1.topk_idx[:, 0], np.argmax(logits, axis=1))   # first maximum
        rE = oracle.moe_route_topk(logits, 16, lib=olib)
        assert np.array_equal(rE.topk_idx, np.argsort(-logits, axis=1, kind="stable"))


@pytest.mark.parametrize("T,E,k,extra", [(8192, 64, 8, 0), (1000, 256, 8, 0), (300, 64, 8, 200), (1, 4, 2, 0),
                                         (0, 8, 2, 0)])
def test_layout_invariants(olib, T, E, k, extra):
    rng = np.random.default_rng([13, T, E])
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if extra:   # skew: experts 0 and 1 win for most tokens
        logits[:extra, :2] += 10.0
    cap = oracle.moe_route_capacity(T, E, k)
    r = oracle.moe_route_topk(logits, k, rows=cap, lib=olib)
    check_layout(r, T, E, k, 128, cap)
    assert cap % 128 == 0 and cap >= T * k + E * 127


def test_route_rejects_bad_input(olib):
    logits = np.zeros((4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.moe_route_topk(logits, 9, lib=olib)                  # k > E
    bad = logits.copy()
    bad[2, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.moe_route_topk(bad, 2, lib=olib)
    with pytest.raises(ValueError):
        oracle.moe_route_topk(logits, 2, rows=100, lib=olib)        # the layout needs 128 rows


def test_gather_hand_case(olib):
    q = np.stack([np.full(256, 0x38, np.uint8), np.full(256, 0xB0, np.uint8)])    # tokens 0 and 1
    s = np.array([[0.5, 2.0], [0.25, 4.0]], np.float32)                             # [K/128 = 2, T = 2]
    qa, sa = oracle.moe_gather_fp8(q, s, np.array([1, -1, 0], np.int32), lib=olib)
    assert np.all(qa[0] == 0xB0) and np.all(qa[1] == 0) and np.all(qa[2] == 0x38)
    assert sa.tolist() == [[2.0, 0.0, 0.5], [4.0, 0.0, 0.25]]


def test_gather_matches_numpy_indexing(olib):
    rng = np.random.default_rng(14)
    T, K = 50, 384
    q = rng.integers(0, 256, size=(T, K), dtype=np.uint8)
    s = rng.uniform(1e-3, 1.0, size=(K // 128, T)).astype(np.float32)
    row_token = rng.integers(-1, T, size=200).astype(np.int32)
    qa, sa = oracle.moe_gather_fp8(q, s, row_token, lib=olib)
    valid = row_token >= 0
    assert np.array_equal(qa[valid], q[row_token[valid]]) and np.all(qa[~valid] == 0)
    assert np.array_equal(sa[:, valid], s[:, row_token[valid]]) and np.all(sa[:, ~valid] == 0)


def test_gather_commutes_with_the_row_quantizer(olib):
    """Quantizing tokens then gathering equals gathering bf16 tokens then quantizing (1x128 groups lie in
    one row), including the empty rows, which quantize to code 0 with scale 0."""
    rng = np.random.default_rng(15)
    T, E, k, K = 40, 8, 3, 512
    x = (rng.standard_normal((T, K), dtype=np.float32) * 3).view(np.uint32) >> 16
    x = x.astype(np.uint16)
    r = oracle.moe_route_topk(rng.standard_normal((T, E), dtype=np.float32), k, lib=olib)
    q, s = oracle.quant_act_1x128(x, lib=olib)
    qa, sa = oracle.moe_gather_fp8(q, s, r.row_token, lib=olib)
    xg = np.zeros((len(r.row_token), K), np.uint16)
    xg[r.row_token >= 0] = x[r.row_token[r.row_token >= 0]]
    q2, s2 = oracle.quant_act_1x128(xg, lib=olib)
    assert np.array_equal(qa, q2) and np.array_equal(sa.view(np.uint32), s2.view(np.uint32))
