"""GPU parity of the layer's backward against the oracle (through the C ABI).

The backward is the chain rule on the forward definitions ("Three axes of
Parallelism", EP backward pass: expert gradients divided by the EP group
size; "feat(parallelism): expert parallelism for the Nemotron-3 Nano MoE
layers", Design: autograd through the permutation pair). Every gradient the
GPU path produces is compared with the oracle's double-precision chain rule:
the router-weight, logit and input gradients per token, the expert-output,
pre-activation and packed-input gradients per packed row, and the expert and
router weight gradients. Reduced workloads are compared in full; the full
Qwen3-30B-A3B-shaped workload in full as well (every token, every packed row
and every hidden column of every expert); the d = 4096 stress workload on
sampled tokens and a few hidden columns of every expert. Floating-point bar
(tests/util.py check_grad): fp32 data as in the forward, max relative error
<= 1e-5; bf16 data, against the oracle's chain with every value rounded to
bf16 at the storage points where training hands it between kernels: the
forward's max error <= 2e-2 of the reference's RMS beyond two bf16 ulps of
each element (room for rounding flips at its own storage point and at one
of its inputs), and relative L2 error <= 2e-2; against the exact chain,
relative L2 error <= 2e-2."""
import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_amd import ops
from expert_dispatch_amd import workloads as W
from util import check_grad, to_numpy, to_torch, widen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _shared(inp):
    if inp.get("shared_w_gate") is None:
        return None
    return (to_torch(np.concatenate(list(inp["shared_w_gate"]), axis=1)[None]),
            to_torch(np.concatenate(list(inp["shared_w_val"]), axis=1)[None]),
            to_torch(np.concatenate(list(inp["shared_w_out"]), axis=0)[None]))


def _check_backward(name, full, capacity=None, scale=1.0, renorm=True, pairs_per_expert=None):
    cfg = W.get(name)
    say(f"[backward] {name}: generate")
    inp = W.generate(cfg)
    inp["renorm"] = renorm
    d_out = W.output_gradient(cfg)
    x, wr = to_torch(inp["x"]), to_torch(inp["w_router"])
    bias = to_torch(inp["bias"]) if inp.get("bias") is not None else None
    wg, wv, wo = to_torch(inp["w_gate"]), to_torch(inp["w_val"]), to_torch(inp["w_out"])
    shared = _shared(inp)
    e_first = inp.get("e_first")
    say(f"[backward] {name}: gpu forward + backward (capacity {capacity}, renorm {renorm})")
    sv = ops.moe_layer_train(x, wr, bias, cfg.k, wg, wv, wo, shared=shared, capacity=capacity,
                             e_first=e_first, renorm=renorm)
    g = ops.moe_layer_backward(sv, to_torch(d_out), x, wr, wg, wv, wo, shared=shared,
                               scale=scale)
    torch.cuda.synchronize()
    T, k, E, f = cfg.T, cfg.k, cfg.E, cfg.f
    tokens = None
    if full:
        rng = np.random.default_rng(1)
        tokens = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=256)])).astype(np.int32)
    if pairs_per_expert is None:
        pairs = oracle.all_pairs(E, f)
    else:
        rng = np.random.default_rng(2)
        cols = [np.unique(np.concatenate([[0, f - 1], rng.integers(0, f, size=pairs_per_expert)]))
                for _ in range(E)]
        pairs = np.array([(e, c) for e in range(E) for c in cols[e]], np.int64)
    say(f"[backward] {name}: oracle ({len(pairs)} weight columns)")
    # bf16 data: the oracle's chain with every value rounded at the storage
    # points where the training step hands it between kernels (all sums
    # exact) is the reference for the element-wise gate; the exact chain is
    # held to the norm-wise bar beside it
    o = oracle.moe_backward(inp, d_out, tokens=tokens, pairs=pairs, scale=scale,
                            capacity=capacity, e_first=e_first, store_bf16=cfg.dtype == "bf16")
    ox = None
    if cfg.dtype == "bf16":
        ox = oracle.moe_backward(inp, d_out, tokens=tokens, pairs=pairs, scale=scale,
                                 capacity=capacity, e_first=e_first)
    tok = o["tokens"]
    dt = cfg.dtype
    # packing as in the forward: bit-exact
    np.testing.assert_array_equal(to_numpy(sv["idx"]), o["idx"])
    np.testing.assert_array_equal(to_numpy(sv["dest"]), o["dest"])
    rows_t = torch.from_numpy(o["y_rows"]).to("cuda")
    e = {}
    e["d_gates"] = check_grad(to_numpy(g["d_gates"])[tok], o["d_gates"], dt, f"{name} d_gates")
    e["d_logits"] = check_grad(to_numpy(g["d_logits"])[tok], o["d_logits"], dt, f"{name} d_logits")
    e["d_y"] = check_grad(to_numpy(g["d_y"].index_select(0, rows_t)), o["d_y"], dt, f"{name} d_y")
    e["d_act"] = check_grad(to_numpy(g["d_act"].index_select(0, rows_t)), o["d_act"], dt,
                            f"{name} d_act")
    e["d_x_perm"] = check_grad(to_numpy(g["d_x_perm"].index_select(0, rows_t)), o["d_x_perm"],
                               dt, f"{name} d_x_perm")
    e["d_x"] = check_grad(to_numpy(g["d_x"])[tok], o["d_x"], dt, f"{name} d_x")
    pe, pc = pairs[:, 0], pairs[:, 1]
    dwg = to_numpy(g["d_w_gate"])[pe, :, pc]
    dwv = to_numpy(g["d_w_val"])[pe, :, pc]
    dwo = to_numpy(g["d_w_out"])[pe, pc, :]
    e["d_w_gate"] = check_grad(dwg, o["d_w_gate"], dt, f"{name} d_w_gate")
    e["d_w_val"] = check_grad(dwv, o["d_w_val"], dt, f"{name} d_w_val")
    e["d_w_out"] = check_grad(dwo, o["d_w_out"], dt, f"{name} d_w_out")
    if o["d_w_router"] is not None:
        e["d_w_router"] = check_grad(to_numpy(g["d_w_router"]), o["d_w_router"], dt,
                                      f"{name} d_w_router")
    if ox is not None:
        # against the exact chain: the norm-wise bar on every gradient
        got = {"d_gates": to_numpy(g["d_gates"])[tok], "d_logits": to_numpy(g["d_logits"])[tok],
               "d_x": to_numpy(g["d_x"])[tok], "d_w_gate": dwg, "d_w_val": dwv, "d_w_out": dwo,
               "d_act": widen(to_numpy(g["d_act"].index_select(0, rows_t))),
               "d_x_perm": widen(to_numpy(g["d_x_perm"].index_select(0, rows_t)))}
        if ox["d_w_router"] is not None:
            got["d_w_router"] = to_numpy(g["d_w_router"])
        for key, val in got.items():
            ref = ox[key]
            l2 = float(np.sqrt(np.sum((np.asarray(val, np.float64) - ref) ** 2) /
                               max(np.sum(ref * ref), 1e-300)))
            assert l2 <= 2e-2, f"{name} {key}: relative L2 error {l2:.3e} > 2e-2 (exact chain)"
            e[key + "_exact_l2"] = l2
    say(f"[backward] {name}: ok " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))


@pytest.mark.parametrize("name", ["tiny_f32", "odd_f32", "qwen3_small", "dsv2_small",
                                  "dsv2_small_empty4", "stress_small", "ag_rs_small"])
def test_backward_small(name):
    _check_backward(name, full=False)


def test_backward_small_capacity_scaled_unnormalised():
    cfg = W.get("qwen3_small")
    cap = int(np.ceil(0.8 * cfg.T * cfg.k / cfg.E))
    _check_backward("qwen3_small", full=False, capacity=cap, scale=0.125, renorm=False)


def test_backward_full_qwen3():
    """Every gradient element of the Qwen3-30B-A3B-shaped layer (all 4096
    tokens, all 32768 packed rows, all 128 x 768 expert weight columns)."""
    _check_backward("qwen3_30b_a3b", full=False)


def test_backward_stress_sampled():
    """The d = 4096, f = 1536 stress layer: sampled tokens and four hidden
    columns (plus the first and last) of every expert's weight gradients,
    each summed over all of the expert's packed rows."""
    _check_backward("stress_zipf", full=True, pairs_per_expert=4)
