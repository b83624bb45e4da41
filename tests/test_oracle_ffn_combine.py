"""Pins of the oracle's expert MLPs and weighted combine.

Expert MLPs: "Three axes of Parallelism", Mapping experts to EP ranks (W_gate,
W_val [E,d,f], W_out [E,f,d]) and Dispatch, expert computation and combine
(E_local independent MLPs; weight every expert output by its router weight,
sum the K outputs). Pins: a hand-worked layer (tests/golden/tiny_layer.json);
permutation-matrix experts whose outputs have a closed form per element (a
transposed operand or a swapped W_gate/W_val fails it); E=1, k=1 reducing the
layer to a plain SwiGLU MLP computed with torch's float64 library ops; a
brute-force dense evaluation of every expert on every token masked by the
routing; identity and scaled-identity experts for the combine.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _widen(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("case", ["k1", "k2"])
def test_hand_worked_layer(case):
    fx = json.load(open(os.path.join(GOLDEN, "tiny_layer.json")))
    inp = dict(x=np.array(fx["x"], np.float32), w_router=np.array(fx["w_router"], np.float32),
               bias=None, w_gate=np.array(fx["w_gate"], np.float32),
               w_val=np.array(fx["w_val"], np.float32), w_out=np.array(fx["w_out"], np.float32),
               k=int(case[1:]))
    r = oracle.moe_layer(inp)
    exp = fx["cases"][case]
    np.testing.assert_array_equal(r["idx"], exp["idx"])
    np.testing.assert_allclose(r["gates"], exp["gates"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(r["out"], exp["out"], rtol=1e-15, atol=1e-300)


def _perm_matrix(p, scale=1.0):
    n = len(p)
    m = np.zeros((n, n), np.float32)
    m[np.arange(n), p] = scale
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_permutation_matrix_experts_closed_form(dtype):
    rng = np.random.default_rng(5)
    n, N, E = 24, 40, 2
    # non-involutive permutations so that a transposed matrix gives other values
    pg, pv, po = (np.roll(np.arange(n), s) for s in (1, 5, 11))
    c = 0.5
    wg = np.stack([_perm_matrix(pg, c), _perm_matrix(pv, c)])
    wv = np.stack([_perm_matrix(pv), _perm_matrix(po)])
    wo = np.stack([_perm_matrix(po), _perm_matrix(pg)])
    x = rng.standard_normal((N, n), dtype=np.float32)
    if dtype == "bf16":
        x, wg, wv, wo = (W.f32_to_bf16_bits(a) for a in (x, wg, wv, wo))
    offsets = np.array([0, 17, N], np.int32)
    y = oracle.expert_ffn_rows(x, offsets, wg, wv, wo)
    xd = _widen(x)
    silu = lambda z: z / (1.0 + math.exp(-z))
    mats = [(pg, pv, po), (pv, po, pg)]
    for j in range(N):
        e = 0 if j < 17 else 1
        a, b, o = mats[e]
        # W[i, p[i]] = 1: column p[i] of x.W picks x[i], so (x.W)[p[i]] = x[i]
        g = np.empty(n); v = np.empty(n); h = np.empty(n); out = np.empty(n)
        g[a] = c * xd[j]
        v[b] = xd[j]
        for col in range(n):
            h[col] = silu(g[col]) * v[col]
        out[o] = h
        np.testing.assert_allclose(y[j], out, rtol=1e-15, atol=1e-300)


def test_single_expert_top1_is_plain_swiglu_mlp():
    inp = W.generate(W.get("qwen3_small"))
    x = inp["x"][:50]
    wg, wv, wo = inp["w_gate"][:1], inp["w_val"][:1], inp["w_out"][:1]
    wr = inp["w_router"][:, :1]
    r = oracle.moe_layer(dict(x=x, w_router=wr, bias=None, w_gate=wg, w_val=wv, w_out=wo, k=1))
    X = torch.from_numpy(_widen(x))
    G = torch.from_numpy(_widen(wg[0]))
    V = torch.from_numpy(_widen(wv[0]))
    O = torch.from_numpy(_widen(wo[0]))
    ref = (torch.nn.functional.silu(X @ G) * (X @ V)) @ O
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=1e-11, atol=1e-12)
    assert (r["gates"] == 1.0).all()


@pytest.mark.parametrize("name", ["tiny_f32", "dsv2_small", "odd_f32"])
def test_dense_masked_bruteforce(name):
    """Every expert on every token, masked by the routing and weighted by the
    router weights: no packing, no permutation, no un-permute."""
    inp = W.generate(W.get(name))
    T = min(inp["x"].shape[0], 48)
    inp = dict(inp, x=inp["x"][:T])
    r = oracle.moe_layer(inp)
    E = inp["w_gate"].shape[0]
    X = torch.from_numpy(_widen(inp["x"]))
    dense = torch.zeros(T, X.shape[1], dtype=torch.float64)
    for e in range(E):
        G, V, O = (torch.from_numpy(_widen(inp[n][e])) for n in ("w_gate", "w_val", "w_out"))
        ye = (torch.nn.functional.silu(X @ G) * (X @ V)) @ O
        wgt = np.zeros(T)
        for t in range(T):
            for s in range(inp["k"]):
                if r["idx"][t, s] == e:
                    wgt[t] = r["gates"][t, s]
        dense += torch.from_numpy(wgt)[:, None] * ye
    if inp.get("shared_w_gate") is not None:
        for q in range(inp["shared_w_gate"].shape[0]):
            G, V, O = (torch.from_numpy(_widen(inp["shared_" + n][q]))
                       for n in ("w_gate", "w_val", "w_out"))
            dense += (torch.nn.functional.silu(X @ G) * (X @ V)) @ O
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-10, atol=1e-11)


def test_shared_experts_equal_one_concatenated_swiglu():
    inp = W.generate(W.get("dsv2_small"))
    x = inp["x"][:30]
    two = oracle.swiglu_shared(x, inp["shared_w_gate"], inp["shared_w_val"], inp["shared_w_out"])
    cat_g = np.concatenate(list(inp["shared_w_gate"]), axis=1)[None]
    cat_v = np.concatenate(list(inp["shared_w_val"]), axis=1)[None]
    cat_o = np.concatenate(list(inp["shared_w_out"]), axis=0)[None]
    one = oracle.expert_ffn_rows(x, np.array([0, 30], np.int32), cat_g, cat_v, cat_o)
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-12)


def test_combine_identity_and_scaled_identity_experts():
    inp = W.generate(W.get("qwen3_small"))
    k = inp["k"]
    T = inp["x"].shape[0]
    _, idx, g = oracle.route(inp["x"], inp["w_router"], inp["bias"], k)
    _, _, perm_src, dest = oracle.permute(idx, inp["w_gate"].shape[0])
    xp = _widen(oracle.gather(inp["x"], perm_src, k))
    tok = np.arange(T, dtype=np.int32)
    # identity experts: sum of weights is 1, so the layer returns its input
    out = oracle.combine(tok, k, dest, g, xp)
    np.testing.assert_allclose(out, _widen(inp["x"]), rtol=1e-14, atol=1e-14)
    # expert e scales by (e+1): out[t] = x[t] * sum_s g[t,s] * (idx[t,s]+1)
    flat_e = idx.reshape(-1)[perm_src]
    out2 = oracle.combine(tok, k, dest, g, xp * (flat_e + 1.0)[:, None])
    scale = (g * (idx + 1.0)).sum(axis=1)
    np.testing.assert_allclose(out2, _widen(inp["x"]) * scale[:, None], rtol=1e-13, atol=1e-13)
    # unweighted un-permute with k = 1 restores the packed rows' sources
    out3 = oracle.combine(tok, k, dest, None, xp)
    np.testing.assert_allclose(out3, _widen(inp["x"]) * k, rtol=1e-14, atol=1e-14)


def test_sampled_layer_equals_full_layer():
    inp = W.generate(W.get("dsv2_small"))
    full = oracle.moe_layer(inp)
    toks = np.array([0, 5, 17, 100, 279], np.int32)
    part = oracle.moe_layer(inp, tokens=toks)
    np.testing.assert_array_equal(part["out"], full["out"][toks])


def test_recv_layer_identity_round_trip():
    inp = W.generate(W.get("ep_share_small"))
    r = oracle.moe_recv_layer(inp)
    N = inp["x_recv"].shape[0]
    # y of packed row j unpermuted lands on its source row
    ident = _widen(r["x_perm"])
    out = oracle.combine(np.arange(N, dtype=np.int32), 1, r["dest"], None, ident)
    np.testing.assert_array_equal(out, _widen(inp["x_recv"]))
    assert r["out"].shape == (N, inp["x_recv"].shape[1])


@pytest.mark.parametrize("name,cap", [("tiny_f32", 8), ("dsv2_small", 9)])
def test_capacity_layer_dense_bruteforce(name, cap):
    """Fixed-capacity routing against every expert on every token, masked by
    the assignments each expert keeps (its first `cap` in (token, slot)
    order): dropped assignments add nothing."""
    inp = W.generate(W.get(name))
    T = min(inp["x"].shape[0], 48)
    inp = dict(inp, x=inp["x"][:T])
    r = oracle.moe_layer(inp, capacity=cap)
    E, k = inp["w_gate"].shape[0], inp["k"]
    assert (r["dest"] < 0).any(), "the cap should drop something here"
    X = torch.from_numpy(_widen(inp["x"]))
    dense = torch.zeros(T, X.shape[1], dtype=torch.float64)
    for e in range(E):
        G, V, O = (torch.from_numpy(_widen(inp[n][e])) for n in ("w_gate", "w_val", "w_out"))
        ye = (torch.nn.functional.silu(X @ G) * (X @ V)) @ O
        wgt = np.zeros(T)
        seen = 0
        for t in range(T):
            for s in range(k):
                if r["idx"][t, s] == e:
                    if seen < cap:
                        wgt[t] = r["gates"][t, s]
                    seen += 1
        dense += torch.from_numpy(wgt)[:, None] * ye
    if inp.get("shared_w_gate") is not None:
        for q in range(inp["shared_w_gate"].shape[0]):
            G, V, O = (torch.from_numpy(_widen(inp["shared_" + n][q]))
                       for n in ("w_gate", "w_val", "w_out"))
            dense += (torch.nn.functional.silu(X @ G) * (X @ V)) @ O
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-10, atol=1e-11)


def test_capacity_sampled_layer_equals_full_layer():
    inp = W.generate(W.get("dsv2_small"))
    full = oracle.moe_layer(inp, capacity=30)
    toks = np.array([0, 5, 17, 100, 279], np.int32)
    part = oracle.moe_layer(inp, tokens=toks, capacity=30)
    np.testing.assert_array_equal(part["out"], full["out"][toks])


def test_partial_layers_of_all_ranks_sum_to_the_full_layer():
    """All-gather / reduce-scatter layout: the reduce-scatter sums the ranks'
    partial outputs, which must give the layer over all experts."""
    inp = W.generate(W.get("qwen3_small"))
    full = oracle.moe_layer(inp)
    E = inp["w_gate"].shape[0]
    R = 4
    E_loc = E // R
    total = np.zeros_like(full["out"])
    for r in range(R):
        e0 = r * E_loc
        part = dict(inp, w_gate=inp["w_gate"][e0:e0 + E_loc], w_val=inp["w_val"][e0:e0 + E_loc],
                    w_out=inp["w_out"][e0:e0 + E_loc])
        total += oracle.moe_partial_layer(part, e0)["out"]
    np.testing.assert_allclose(total, full["out"], rtol=1e-12, atol=1e-12)


def test_partial_layer_sampled_equals_full():
    inp = W.generate(W.get("ag_rs_small"))
    full = oracle.moe_partial_layer(inp, inp["e_first"])
    toks = np.array([0, 7, 150, 299], np.int32)
    part = oracle.moe_partial_layer(inp, inp["e_first"], tokens=toks)
    np.testing.assert_array_equal(part["out"], full["out"][toks])


def test_hidden_rounding_with_identity_down_weight_is_bf16_of_h():
    """round_h: with one expert and W_out = I (f = d) the output is h itself,
    so the rounded variant must equal the exact variant's output rounded to
    bf16 by torch (to nearest, ties to even)."""
    rng = np.random.default_rng(501)
    n, d = 48, 64
    bf = W.f32_to_bf16_bits
    x = bf(rng.standard_normal((n, d)).astype(np.float32))
    wg = bf((rng.standard_normal((1, d, d)) / 8).astype(np.float32))
    wv = bf((rng.standard_normal((1, d, d)) / 8).astype(np.float32))
    wo = bf(np.eye(d, dtype=np.float32)[None])
    off = np.array([0, n], np.int32)
    exact = oracle.expert_ffn_rows(x, off, wg, wv, wo)
    rounded = oracle.expert_ffn_rows(x, off, wg, wv, wo, round_h=True)
    want = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(rounded, want)
    assert np.any(rounded != exact)


def test_hidden_rounding_error_within_its_bound():
    """round_h moves every output by at most 2^-8 sum_c |h_c| |W_out[c,o]|
    (one rounding of each h_c to 8 significant bits, relative error at most
    2^-8), and does move it."""
    inp = W.generate(W.get("qwen3_small"))
    o = oracle.moe_layer(inp)
    r = oracle.moe_layer(inp, round_h=True)
    np.testing.assert_array_equal(r["dest"], o["dest"])
    y, yr = o["y"], r["y"]
    # |h| from the exact layer: the identity-weight run gives h for expert e
    # rows directly, so bound with the exact h of each packed row
    E, d, f = inp["w_gate"].shape
    x_perm = o["x_perm"]
    xw = _widen(x_perm)
    bound = np.zeros_like(y)
    off = o["offsets"]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        g = xw[lo:hi] @ _widen(inp["w_gate"][e])
        v = xw[lo:hi] @ _widen(inp["w_val"][e])
        h = g / (1.0 + np.exp(-g)) * v
        bound[lo:hi] = (2.0 ** -8) * (np.abs(h) @ np.abs(_widen(inp["w_out"][e])))
    diff = np.abs(yr - y)
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-300)
    assert diff.max() > 0
