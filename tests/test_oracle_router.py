"""Pins of the oracle's router, top-k selection and gates.

Selection is by (fp32 logit descending, expert index ascending) and the gates
are the softmax renormalised over the k selected experts.  The expected
number of distinct experts that 8 independently routed rows touch,
896 (1 - (880/896)^8) ~ 120.3, is printed in "Kimi K3 on GB300: 13 kernels a
layer" (section "What DSpark adds").
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _rand_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_to_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_router_one_hot_x_selects_a_column():
    rng = np.random.default_rng(0)
    H, E = 64, 12
    wr = _rand_bf16(rng, (E, H))
    bias = rng.standard_normal(E).astype(np.float32)
    x = np.zeros((1, H), np.uint16)
    x[0, 17] = 0x3F80  # 1.0
    lg, od = oracle.router_logits(x, wr, None, H, E)
    assert np.array_equal(lg[0].astype(np.float64), _bf16_to_f64(wr[:, 17]))
    lg, od = oracle.router_logits(x, wr, bias, H, E)
    assert np.array_equal(lg[0], (_bf16_to_f64(wr[:, 17]) + bias.astype(np.float64)).astype(np.float32))


def test_router_equals_exact_sum_rounded_once():
    """fp32(exact sum) with the exact sum from math.fsum (Shewchuk)."""
    rng = np.random.default_rng(1)
    H, E, B = 512, 24, 3
    x = _rand_bf16(rng, (B, H))
    wr = _rand_bf16(rng, (E, H), 0.02)
    bias = rng.standard_normal(E).astype(np.float32)
    lg, od = oracle.router_logits(x, wr, bias, H, E)
    assert od == 0
    xd, wd = _bf16_to_f64(x), _bf16_to_f64(wr)
    for b in range(B):
        for e in range(E):
            exact = math.fsum(list(xd[b] * wd[e]) + [float(bias[e])])
            assert lg[b, e] == np.float32(exact)


@pytest.mark.slow
def test_router_k3_shape_sum_is_order_independent():
    """At the K3 shape (H 7168, weights ~N(0, 0.02), x ~N(0, 1)) the double
    sum of the exact products did not depend on the summation order."""
    seed = 3
    x = synth.fill_bf16(seed, synth.tag(0, synth.KIND_X), 1.0, 2 * 7168).reshape(2, 7168)
    wr = synth.fill_bf16(seed, synth.tag(0, synth.KIND_ROUTER), 0.02, 896 * 7168).reshape(896, 7168)
    lg, od = oracle.router_logits(x, wr, None, 7168, 896)
    assert od == 0
    xd, wd = _bf16_to_f64(x), _bf16_to_f64(wr)
    for e in (0, 1, 100, 895):
        assert lg[1, e] == np.float32(math.fsum(xd[1] * wd[e]))


def _dominates(l, a, b):
    return l[a] > l[b] or (l[a] == l[b] and a < b)


@pytest.mark.parametrize("E,k", [(8, 2), (10, 3), (9, 4)])
def test_topk_brute_force_over_all_subsets(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(20):
        # few distinct values so ties are frequent
        lg = rng.integers(-3, 3, (1, E)).astype(np.float32) * np.float32(0.5)
        idx, gate = oracle.topk(lg, k)
        l = lg[0]
        winners = [s for s in itertools.combinations(range(E), k)
                   if all(_dominates(l, a, b) for a in s for b in range(E) if b not in s)]
        assert len(winners) == 1
        assert sorted(idx[0].tolist()) == list(winners[0])
        for j in range(k - 1):
            assert _dominates(l, idx[0, j], idx[0, j + 1])


def test_topk_matches_lexsort():
    rng = np.random.default_rng(11)
    lg = (rng.standard_normal((16, 896)) * 0.02).astype(np.float32)
    lg[3, 10] = lg[3, 500] = lg[3].max() + 1  # a tie at the top
    idx, gate = oracle.topk(lg, 16)
    for b in range(16):
        order = np.lexsort((np.arange(896), -lg[b].astype(np.float64)))
        assert np.array_equal(idx[b], order[:16])
    assert idx[3, 0] == 10 and idx[3, 1] == 500


def test_topk_all_equal_logits():
    for E, k in ((16, 2), (896, 16)):
        idx, gate = oracle.topk(np.zeros((2, E), np.float32), k)
        assert np.array_equal(idx, np.tile(np.arange(k), (2, 1)))
        assert np.all(gate == np.float32(1.0 / k))


def test_topk_signed_zero_is_a_tie():
    lg = np.array([[-1.0, 0.0, -2.0, -0.0, -3.0]], np.float32)
    lg[0, 3] = -0.0
    idx, gate = oracle.topk(lg, 2)
    assert idx[0].tolist() == [1, 3]
    assert gate[0, 0] == gate[0, 1] == np.float32(0.5)


def test_gates_properties_and_closed_form():
    rng = np.random.default_rng(12)
    lg = (rng.standard_normal((32, 64)) * 2).astype(np.float32)
    idx, gate = oracle.topk(lg, 8)
    assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(gate, axis=1) <= 0)
    # k = 2 closed form: g0 = 1 / (1 + exp(l1 - l0)) (logistic function)
    idx2, gate2 = oracle.topk(lg, 2)
    for b in range(32):
        l0, l1 = float(lg[b, idx2[b, 0]]), float(lg[b, idx2[b, 1]])
        assert abs(float(gate2[b, 0]) - 1.0 / (1.0 + math.exp(l1 - l0))) <= 6e-8
    # k = 1 gives exactly one
    idx1, gate1 = oracle.topk(lg, 1)
    assert np.all(gate1 == 1.0)
    # k = E: renormalised top-k is the plain softmax (library routine)
    idxE, gateE = oracle.topk(lg, 64)
    for b in range(4):
        ref = softmax(lg[b].astype(np.float64))[idxE[b]]
        assert np.allclose(gateE[b], ref, rtol=0, atol=1e-7)


def test_exactly_k_distinct_experts_per_row():
    rng = np.random.default_rng(13)
    lg = rng.integers(-2, 2, (64, 896)).astype(np.float32)
    idx, _ = oracle.topk(lg, 16)
    assert all(len(set(r.tolist())) == 16 for r in idx)


@pytest.mark.slow
def test_distinct_experts_at_batch_8_matches_union_model():
    """Mean distinct experts over 8 independent rows ~ 896(1-(880/896)^8)."""
    g = json.load(open(GOLDEN))["expected_union_b8"]
    E, k, H = g["num_experts"], g["top_k"], 7168
    assert round(E * (1 - ((E - k) / E) ** g["batch"]), 1) == g["value"]
    counts = []
    for seed in range(6):
        x = synth.fill_bf16(seed, synth.tag(0, synth.KIND_X), 1.0, 8 * H).reshape(8, H)
        wr = synth.fill_bf16(seed, synth.tag(0, synth.KIND_ROUTER), 0.02, E * H).reshape(E, H)
        lg, _ = oracle.router_logits(x, wr, None, H, E)
        idx, _ = oracle.topk(lg, k)
        counts.append(len(set(idx.ravel().tolist())))
    assert abs(np.mean(counts) / g["value"] - 1) < 0.05, counts
