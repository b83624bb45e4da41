"""Pins of the oracle's backward.

The pages' systems train the layer (autograd through the index_select /
index_copy permutation pair: "feat(parallelism): expert parallelism for the
Nemotron-3 Nano MoE layers", Design; expert gradients divided by the EP group
size: "Three axes of Parallelism", EP backward pass) but print no gradient
formula or value. The oracle's hand-derived chain rule is pinned by:
  * torch float64 autograd of a dense formulation written independently here
    (every expert on every token, masked by the routing; capacity and expert
    range as masks from a cumulative count), compared on every gradient;
  * central finite differences of the oracle's own forward (no torch), for
    elements of every weight and of the input;
  * properties that hold exactly: softmax-shift invariance (each token's
    logit gradients sum to 0), k = 1 with renormalised weights (the weight is
    identically 1, so the router gets no gradient), a zero output gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_amd import workloads as W


def _layer(seed, T=14, d=10, f=6, E=5, k=2, dtype="f32", shared=0, router_scale=1.5):
    rng = np.random.default_rng(seed)

    def draw(*shape, std=1.0):
        a = (rng.standard_normal(shape) * std).astype(np.float32)
        if dtype == "bf16":
            return (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy()
                    .view(np.uint16))
        return a

    inp = dict(x=draw(T, d), w_router=draw(d, E, std=router_scale), bias=None,
               w_gate=draw(E, d, f, std=0.5), w_val=draw(E, d, f, std=0.5),
               w_out=draw(E, f, d, std=0.5), k=k)
    if shared:
        inp.update(shared_w_gate=draw(shared, d, f, std=0.5), shared_w_val=draw(shared, d, f, std=0.5),
                   shared_w_out=draw(shared, f, d, std=0.5))
    d_out = draw(T, d)
    return inp, d_out


def _t(a):
    return torch.from_numpy(oracle.widen(a)).requires_grad_(True)


def _torch_grads(inp, d_out, renorm=True, capacity=None, e_first=None, scale=1.0):
    """Autograd of L = sum(out * d_out), the layer written densely."""
    x, wr = _t(inp["x"]), _t(inp["w_router"])
    wg, wv, wo = _t(inp["w_gate"]), _t(inp["w_val"]), _t(inp["w_out"])
    k = inp["k"]
    E_loc = wg.shape[0]
    logits = x @ wr
    if inp.get("bias") is not None:
        logits = logits + torch.from_numpy(inp["bias"].astype(np.float64))
    # the selection is piecewise constant: taken from the values, not differentiated
    idx = torch.topk(logits.detach(), k, dim=1).indices
    sel = logits.gather(1, idx)
    g = torch.softmax(sel, 1) if renorm else torch.softmax(logits, 1).gather(1, idx)
    keep = torch.ones_like(idx, dtype=torch.bool)
    local = idx.clone()
    if e_first is not None:
        keep = (idx >= e_first) & (idx < e_first + E_loc)
        local = idx - e_first
    if capacity is not None:
        flat = idx.reshape(-1)
        onehot = torch.nn.functional.one_hot(flat, E_loc)
        rank = (torch.cumsum(onehot, 0) - onehot).gather(1, flat[:, None]).reshape(idx.shape)
        keep = rank < capacity
    out = torch.zeros_like(x)
    for e in range(E_loc):
        a = x @ wg[e]
        v = x @ wv[e]
        y = (torch.nn.functional.silu(a) * v) @ wo[e]
        w_e = (g * ((local == e) & keep)).sum(1)
        out = out + w_e[:, None] * y
    sh = []
    if inp.get("shared_w_gate") is not None:
        sh = [_t(inp["shared_w_gate"]), _t(inp["shared_w_val"]), _t(inp["shared_w_out"])]
        for q in range(sh[0].shape[0]):
            out = out + (torch.nn.functional.silu(x @ sh[0][q]) * (x @ sh[1][q])) @ sh[2][q]
    L = (out * torch.from_numpy(oracle.widen(d_out))).sum()
    L.backward()
    return dict(idx=idx.numpy(), d_x=x.grad.numpy(), d_w_router=wr.grad.numpy(),
                d_w_gate=wg.grad.numpy() * scale, d_w_val=wv.grad.numpy() * scale,
                d_w_out=wo.grad.numpy() * scale)


def _close(got, ref, rtol, what):
    err = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    assert err <= rtol, f"{what}: max err / max |ref| = {err:.3e} > {rtol}"


def _expert_grads_full(res, E, f):
    """Reassemble the oracle's per-(e,c) pairs into [E,d,f] / [E,f,d]."""
    P = res["pairs"]
    d = res["d_w_gate"].shape[1]
    dg = np.zeros((E, d, f))
    dv = np.zeros((E, d, f))
    do = np.zeros((E, f, d))
    for p, (e, c) in enumerate(P):
        dg[e, :, c] = res["d_w_gate"][p]
        dv[e, :, c] = res["d_w_val"][p]
        do[e, c, :] = res["d_w_out"][p]
    return dg, dv, do


CASES = [
    dict(seed=1),
    dict(seed=2, k=3, E=6),
    dict(seed=3, dtype="bf16"),
    dict(seed=4, shared=2),
    dict(seed=5, k=1),
    dict(seed=6, renorm=False),
    dict(seed=7, capacity=3, T=16, k=2, E=4),
    dict(seed=8, e_first=2, E_global=7, E=3),
    dict(seed=9, scale=0.25),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_backward_matches_float64_autograd(case):
    case = dict(case)
    renorm = case.pop("renorm", True)
    capacity = case.pop("capacity", None)
    e_first = case.pop("e_first", None)
    E_global = case.pop("E_global", None)
    scale = case.pop("scale", 1.0)
    seed = case.pop("seed")
    E = case.pop("E", 5)
    inp, d_out = _layer(seed, E=E, **case)
    if E_global is not None:
        # a rank's slice: the router spans E_global experts, the rank owns E of them
        rng = np.random.default_rng(seed + 100)
        inp["w_router"] = (rng.standard_normal((inp["x"].shape[1], E_global)) * 1.5).astype(
            inp["w_router"].dtype) if inp["w_router"].dtype == np.float32 else inp["w_router"]
    inp["renorm"] = renorm
    res = oracle.moe_backward(inp, d_out, pairs=oracle.all_pairs(E, inp["w_gate"].shape[2]),
                              scale=scale, capacity=capacity, e_first=e_first)
    ref = _torch_grads(inp, d_out, renorm, capacity, e_first, scale)
    np.testing.assert_array_equal(res["idx"], ref["idx"])
    dg, dv, do = _expert_grads_full(res, E, inp["w_gate"].shape[2])
    # the oracle's logits are rounded to fp32 (the router's definition), torch's
    # are float64: the weights and everything downstream differ by ~1e-7
    _close(res["d_x"], ref["d_x"], 1e-6, "d_x")
    if not (renorm and inp["k"] == 1):
        _close(res["d_w_router"], ref["d_w_router"], 1e-6, "d_w_router")
    _close(dg, ref["d_w_gate"], 1e-6, "d_w_gate")
    _close(dv, ref["d_w_val"], 1e-6, "d_w_val")
    _close(do, ref["d_w_out"], 1e-6, "d_w_out")


def _loss(inp, d_out):
    r = oracle.moe_layer(inp)
    return float(np.sum(r["out"] * oracle.widen(d_out)))


@pytest.mark.parametrize("which", ["w_gate", "w_val", "w_out", "x", "w_router"])
def test_backward_matches_finite_differences(which):
    inp, d_out = _layer(21, T=9, d=7, f=5, E=4, k=2)
    E, d, f = 4, 7, 5
    res = oracle.moe_backward(inp, d_out, pairs=oracle.all_pairs(E, f))
    dg, dv, do = _expert_grads_full(res, E, f)
    grads = dict(w_gate=dg, w_val=dv, w_out=do, x=res["d_x"], w_router=res["d_w_router"])
    rng = np.random.default_rng(3)
    # the expert path is double throughout; the router path rounds the logits
    # to fp32, so its differences carry ~1e-7 relative noise / step
    step, tol = (1e-3, 1e-5) if which.startswith("w_") and which != "w_router" else (2e-2, 2e-3)
    g = grads[which]
    for _ in range(6):
        pos = tuple(int(rng.integers(0, n)) for n in inp[which].shape)
        base = inp[which].copy()
        w0 = float(base[pos])
        hi = np.float32(w0 + step)
        lo = np.float32(w0 - step)
        base[pos] = hi
        Lp = _loss(dict(inp, **{which: base}), d_out)
        base[pos] = lo
        Lm = _loss(dict(inp, **{which: base}), d_out)
        fd = (Lp - Lm) / (float(hi) - float(lo))
        assert abs(fd - g[pos]) <= tol * max(1.0, np.max(np.abs(g))), \
            f"{which}{pos}: finite difference {fd:.9g} vs oracle {g[pos]:.9g}"


@pytest.mark.parametrize("renorm", [True, False])
def test_logit_gradients_sum_to_zero_per_token(renorm):
    inp, d_out = _layer(31, T=20, E=6, k=3)
    inp["renorm"] = renorm
    res = oracle.moe_backward(inp, d_out)
    s = res["d_logits"].sum(axis=1)
    assert np.max(np.abs(s)) <= 1e-14 * max(1.0, np.max(np.abs(res["d_logits"])))
    if renorm:
        # only the selected experts' logits move the renormalised weights
        mask = np.zeros_like(res["d_logits"], bool)
        np.put_along_axis(mask, res["idx"], True, axis=1)
        assert np.all(res["d_logits"][~mask] == 0.0)


def test_single_selected_expert_passes_no_router_gradient():
    inp, d_out = _layer(41, k=1)
    res = oracle.moe_backward(inp, d_out)
    assert np.all(res["d_logits"] == 0.0)
    assert np.all(res["d_w_router"] == 0.0)


def test_zero_output_gradient():
    inp, d_out = _layer(51)
    d_out = np.zeros_like(d_out)
    res = oracle.moe_backward(inp, d_out, pairs=oracle.all_pairs(5, 6))
    for key in ("d_x", "d_w_router", "d_gates", "d_w_gate", "d_w_val", "d_w_out"):
        assert np.all(res[key] == 0.0), key


def test_sampled_tokens_equal_full():
    inp, d_out = _layer(61, T=30, E=6, k=2)
    full = oracle.moe_backward(inp, d_out)
    tok = np.array([0, 7, 8, 29], np.int32)
    part = oracle.moe_backward(inp, d_out, tokens=tok)
    np.testing.assert_array_equal(part["d_x"], full["d_x"][tok])
    np.testing.assert_array_equal(part["d_gates"], full["d_gates"][tok])
    np.testing.assert_array_equal(part["d_logits"], full["d_logits"][tok])


def _is_bf16(a):
    a = np.asarray(a, np.float64)
    f = a.astype(np.float32)
    return np.array_equal(f.astype(np.float64), a) and \
        np.all((f.view(np.uint32) & np.uint32(0xFFFF)) == 0)


def test_storage_point_chain_rounds_where_stated_and_stays_close():
    """store_bf16: the values handed between kernels are bf16 numbers (d_y,
    a and v, da and dv, the packed rows' input gradients), every gradient
    stays within a few bf16 roundings of the exact chain (relative L2 below
    1e-2) and differs from it (the roundings happened)."""
    inp = W.generate(W.get("qwen3_small"))
    d_out = W.output_gradient(W.get("qwen3_small"))
    E, f = inp["w_gate"].shape[0], inp["w_gate"].shape[2]
    pairs = oracle.all_pairs(E, f)[:: 7]
    ex = oracle.moe_backward(inp, d_out, pairs=pairs)
    st = oracle.moe_backward(inp, d_out, pairs=pairs, store_bf16=True)
    for key in ("d_y", "act", "d_act", "d_x_perm"):
        assert _is_bf16(st[key]), key
    for key in ("d_y", "d_act", "d_x_perm", "d_x", "d_gates", "d_logits", "d_w_gate", "d_w_val",
                "d_w_out", "d_w_router"):
        a, b = st[key], ex[key]
        l2 = float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b * b)))
        assert 0 < l2 < 1e-2, (key, l2)
    # the router weights' gradients read the expert outputs the forward formed
    # from its bf16-stored h
    x_perm = oracle.gather(inp["x"], st["perm_src"], inp["k"])
    y_h = oracle.expert_ffn_rows(x_perm, st["offsets"], inp["w_gate"], inp["w_val"],
                                 inp["w_out"], round_h=True)
    np.testing.assert_array_equal(st["y"], y_h)
    assert not np.array_equal(st["y"], ex["y"])


def test_storage_point_rounding_of_bf16_exact_values_changes_nothing():
    """With one expert, top-1 routing (weight 1) and a bf16 upstream gradient,
    d_y = d_out is already a bf16 number: rounding it at its storage point
    leaves the input-side chain (ORACLE_STORE_DY alone) unchanged."""
    inp = dict(W.generate(W.get("qwen3_small")))
    inp.update(k=1, w_router=inp["w_router"][:, :1], bias=None, w_gate=inp["w_gate"][:1],
               w_val=inp["w_val"][:1], w_out=inp["w_out"][:1])
    d_out = W.output_gradient(W.get("qwen3_small"))
    T = inp["x"].shape[0]
    off = np.array([0, T], np.int32)
    dy = oracle.widen(d_out)
    base = oracle.expert_ffn_backward_rows(inp["x"], off, inp["w_gate"], inp["w_val"],
                                           inp["w_out"], dy)
    rd = oracle.expert_ffn_backward_rows(inp["x"], off, inp["w_gate"], inp["w_val"],
                                         inp["w_out"], dy, store=oracle.STORE_DY)
    for a, b in zip(base, rd):
        np.testing.assert_array_equal(a, b)
    ra = oracle.expert_ffn_backward_rows(inp["x"], off, inp["w_gate"], inp["w_val"],
                                         inp["w_out"], dy, store=oracle.STORE_ACT)
    assert not np.array_equal(ra[1], base[1])


def test_round_bf16_matches_torch_cast_on_fp32_values():
    """The oracle's bf16 rounding (to nearest, ties to even) equals torch's
    float32 -> bfloat16 conversion on float32 inputs, ties and subnormals
    included."""
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]                 # finite only
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)       # exactly half-way
    vals = np.concatenate([bits, ties]).view(np.float32)
    vals = vals[np.abs(vals) < 3.0e38]                              # no overflow to inf
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(vals), want)


def test_each_storage_point_rounds_only_its_own_stage():
    """ACT rounds only the stored activations, DACT only their gradients,
    DX only the packed rows' input gradients: each result equals the exact
    chain's value rounded once to bf16, and the stages before it are left
    exactly as the exact chain has them."""
    inp = W.generate(W.get("qwen3_small"))
    d_out = W.output_gradient(W.get("qwen3_small"))
    k = inp["k"]
    idx, gates = oracle.route(inp["x"], inp["w_router"], inp["bias"], k)[1:3]
    _, offsets, perm_src, _ = oracle.permute(idx, inp["w_gate"].shape[0])
    x_perm = oracle.gather(inp["x"], perm_src, k)
    dy = oracle.widen(d_out)[perm_src // k] * gates.reshape(-1)[perm_src][:, None]
    args = (x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"], dy)
    act, dact, dx = oracle.expert_ffn_backward_rows(*args)
    a1, d1, x1 = oracle.expert_ffn_backward_rows(*args, store=oracle.STORE_DX)
    np.testing.assert_array_equal(a1, act)
    np.testing.assert_array_equal(d1, dact)
    np.testing.assert_array_equal(x1, oracle.round_bf16(dx))
    a2, d2, _ = oracle.expert_ffn_backward_rows(*args, store=oracle.STORE_DACT)
    np.testing.assert_array_equal(a2, act)
    np.testing.assert_array_equal(d2, oracle.round_bf16(dact))
    a3, _, _ = oracle.expert_ffn_backward_rows(*args, store=oracle.STORE_ACT)
    np.testing.assert_array_equal(a3, oracle.round_bf16(act))
