"""Pins of the oracle's router (scores, top-k selection, router weights).

The router follows "Three axes of Parallelism", Expert Parallel (EP) ->
Producing assignments: every token is scored against all E experts, top-K
selection gives the expert ids and the weight with which each was chosen.
Nothing here compares the oracle with a retyped copy of itself: the scores are
held to a float64 library product within the error bound of fp32 recursive
summation, the exact summation order to hand-derived IEEE cases, the selection
to a brute-force sort and to numpy's stable argsort, the weights to closed
forms and to scipy's softmax.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from expert_dispatch_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24


def _widen(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scores_within_fp32_summation_bound(dtype):
    rng = np.random.default_rng(7)
    T, d, E = 64, 300, 24
    x = rng.standard_normal((T, d), dtype=np.float32)
    w = rng.standard_normal((d, E), dtype=np.float32) * np.float32(0.05)
    b = rng.standard_normal(E, dtype=np.float32)
    if dtype == "bf16":
        x, w = W.f32_to_bf16_bits(x), W.f32_to_bf16_bits(w)
    logits, _, _ = oracle.route(x, w, b, 3)
    xd, wd = _widen(x), _widen(w)
    exact = xd @ wd + b.astype(np.float64)
    absum = np.abs(xd) @ np.abs(wd)
    gamma = d * U32 / (1 - d * U32)
    bound = gamma * absum + U32 * (np.abs(exact) + gamma * absum)
    err = np.abs(logits.astype(np.float64) - exact)
    assert np.all(err <= bound), float((err / bound).max())
    # and the bound is not vacuous: the scores really are close
    assert float(err.max()) < 1e-4


def test_summation_order_golden():
    fx = json.load(open(os.path.join(GOLDEN, "router_order.json")))
    for case in fx["cases"]:
        x = np.array([case["x"]], np.float32)
        w = np.array(case["w"], np.float32).reshape(-1, 1)
        w2 = np.concatenate([w, np.zeros_like(w)], axis=1)  # second expert scores 0
        b = None
        if case["bias"] is not None:
            b = np.array([case["bias"], 0.0], np.float32)
        logits, _, _ = oracle.route(x, w2, b, 1)
        assert float(logits[0, 0]) == case["expected"], case["name"]


def test_topk_matches_bruteforce_sort_and_stable_argsort():
    inp = W.generate(W.get("qwen3_small"))
    logits, idx, _ = oracle.route(inp["x"], inp["w_router"], inp["bias"], inp["k"])
    k = inp["k"]
    for t in range(0, logits.shape[0], 7):
        l = logits[t]
        brute = sorted(range(l.shape[0]), key=lambda e: (-float(l[e]), e))[:k]
        assert list(idx[t]) == brute
    lib = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, lib)


def test_topk_ties_take_lower_index_first():
    # experts 1, 3 and 4 have identical router columns -> identical scores
    rng = np.random.default_rng(3)
    T, d, E = 16, 32, 6
    x = rng.standard_normal((T, d), dtype=np.float32)
    w = rng.standard_normal((d, E), dtype=np.float32)
    w[:, 3] = w[:, 1]
    w[:, 4] = w[:, 1]
    logits, idx, gates = oracle.route(x, w, None, E)
    for t in range(T):
        order = list(idx[t])
        assert order.index(1) < order.index(3) < order.index(4)
        # equal scores get equal weights
        np.testing.assert_allclose(gates[t, order.index(1)], gates[t, order.index(4)], rtol=0, atol=0)


def test_k_equals_E_is_full_argsort():
    inp = W.generate(W.get("tiny_f32"))
    E = inp["w_router"].shape[1]
    logits, idx, _ = oracle.route(inp["x"], inp["w_router"], None, E)
    np.testing.assert_array_equal(idx, np.argsort(-logits, axis=1, kind="stable"))
    for row in idx:
        assert sorted(row) == list(range(E))


def test_bias_forces_selection():
    rng = np.random.default_rng(11)
    T, d, E, k = 40, 64, 16, 3
    x = rng.standard_normal((T, d), dtype=np.float32)
    w = rng.standard_normal((d, E), dtype=np.float32) * np.float32(0.02)
    b = np.zeros(E, np.float32)
    b[[9, 2, 14]] = [300.0, 200.0, 100.0]
    _, idx, _ = oracle.route(x, w, b, k)
    assert (idx == np.array([9, 2, 14])).all()


def test_gates_closed_forms():
    inp = W.generate(W.get("qwen3_small"))
    x, w, b = inp["x"], inp["w_router"], inp["bias"]
    logits, idx, g = oracle.route(x, w, b, 4)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (np.diff(g, axis=1) <= 0).all()  # slots in descending order
    # k = 1: the single weight is exactly 1
    _, _, g1 = oracle.route(x, w, b, 1)
    assert (g1 == 1.0).all()
    # k = 2: g0 = 1 / (1 + exp(l1 - l0)) = sigmoid(l0 - l1)
    l2, i2, g2 = oracle.route(x, w, b, 2)
    l0 = np.take_along_axis(l2, i2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l2, i2[:, 1:], 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(g2[:, 0], scipy.special.expit(l0 - l1), rtol=1e-14, atol=0)
    # all scores equal (zero router, no bias): every weight is 1/k
    _, _, geq = oracle.route(x, np.zeros_like(w), None, 4)
    np.testing.assert_allclose(geq, 0.25, rtol=0, atol=1e-16)


def test_gates_equal_softmax_then_topk_renormalised():
    inp = W.generate(W.get("tiny_f32"))
    logits, idx, g = oracle.route(inp["x"], inp["w_router"], None, 2)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(g, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    # without renormalisation the weights are the full softmax probabilities
    _, idx_n, g_n = oracle.route(inp["x"], inp["w_router"], None, 2, renorm=False)
    np.testing.assert_array_equal(idx_n, idx)
    np.testing.assert_allclose(g_n, sel, rtol=1e-13, atol=0)


def test_nonfinite_score_is_rejected():
    x = np.array([[np.inf, 1.0]], np.float32)
    w = np.ones((2, 3), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.route(x, w, None, 1)


# ---- load statistics (the load-balance statistic the pages report as a
# validation metric; switch-style auxiliary-loss reading)

def test_route_stats_uniform_probabilities_give_one():
    # every logit equal: each probability is 1/E whatever the routing
    T, E, k = 50, 8, 2
    logits = np.full((T, E), 0.25, np.float32)
    rng = np.random.default_rng(0)
    counts = np.bincount(rng.integers(0, E, size=T * k), minlength=E).astype(np.int32)
    pm, aux = oracle.route_stats(logits, counts, k)
    np.testing.assert_allclose(pm, np.full(E, 1.0 / E), rtol=1e-15)
    assert abs(aux - 1.0) < 1e-14


def test_route_stats_collapsed_routing_gives_E():
    # k = 1, every token's probability and assignment on expert 3
    T, E = 40, 6
    logits = np.full((T, E), -200.0, np.float32)
    logits[:, 3] = 0.0
    counts = np.zeros(E, np.int32)
    counts[3] = T
    pm, aux = oracle.route_stats(logits, counts, 1)
    assert abs(pm[3] - 1.0) < 1e-12 and abs(aux - E) < 1e-10


def test_route_stats_probabilities_average_to_one_and_match_scipy():
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    T, E, k = 33, 7, 3
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    counts = rng.integers(0, 20, size=E).astype(np.int32)
    pm, aux = oracle.route_stats(logits, counts, k)
    assert abs(pm.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(pm, softmax(logits.astype(np.float64), axis=1).mean(0), rtol=1e-13)
    # aux is linear in the counts: one count on expert e alone gives E p_mean[e] / (T k)
    c1 = np.zeros(E, np.int32)
    c1[5] = 1
    assert abs(oracle.route_stats(logits, c1, k)[1] - E * pm[5] / (T * k)) < 1e-15
