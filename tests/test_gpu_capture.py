"""The layer's calls only enqueue work: no device -> host copy, no wait for
the device and no allocation anywhere on the path (the property the
Modalities EP page, "feat(parallelism): expert parallelism for the Nemotron-3
Nano MoE layers", Design, makes the point of its device-built permutation:
its Tests check that the permutation performs no device-to-host readback).

Checked two ways on preallocated buffers:
  * eagerly, with PyTorch's sync debug mode set to raise on any synchronising
    torch call made by the binding;
  * by capturing the whole chain in a HIP graph in global capture mode, where
    any synchronising HIP call (a blocking copy, a device or stream wait, an
    allocation on the legacy stream) from any thread invalidates the capture.
    The captured graph is then replayed several times, with eager work and
    synchronisations between the replays, and every replay must reproduce
    the eager results bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from expert_dispatch_amd import ops
from expert_dispatch_amd import workloads as W
from util import to_torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _device(inp):
    dev = {}
    for key in ("x", "w_router", "bias", "w_gate", "w_val", "w_out", "x_recv", "recv_counts"):
        if inp.get(key) is not None:
            dev[key] = to_torch(inp[key])
    if inp.get("shared_w_gate") is not None:
        dev["shared"] = (to_torch(np.concatenate(list(inp["shared_w_gate"]), axis=1)[None]),
                         to_torch(np.concatenate(list(inp["shared_w_val"]), axis=1)[None]),
                         to_torch(np.concatenate(list(inp["shared_w_out"]), axis=0)[None]))
    return dev


def _allocations() -> int:
    return int(torch.cuda.memory_stats().get("allocation.all.allocated", 0))


def _no_sync_then_replay(run, outputs: dict, what: str, replays: int = 3):
    """run() enqueues the chain on the current stream writing `outputs`."""
    torch.cuda.synchronize()
    # 1. eager: any synchronising torch call raises
    torch.cuda.set_sync_debug_mode("error")
    try:
        n0 = _allocations()
        run()
        n1 = _allocations()
    finally:
        torch.cuda.set_sync_debug_mode(0)
    torch.cuda.synchronize()
    assert n1 == n0, f"{what}: the eager chain allocated {n1 - n0} device blocks"
    ref = {k: v.clone() for k, v in outputs.items()}
    # 2. capture in global mode: a synchronising HIP call from any thread fails it
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side, capture_error_mode="global"):
        # (counted inside the capture: beginning one allocates PyTorch's own
        # random-number state)
        n0 = _allocations()
        run()
        n1 = _allocations()
    assert n1 == n0, f"{what}: the captured chain allocated {n1 - n0} device blocks"
    torch.cuda.synchronize()
    # 3. replays, each after the outputs were overwritten by eager work
    for rep in range(replays):
        for v in outputs.values():
            if v.dtype in (torch.float32, torch.bfloat16):
                v.fill_(float("nan"))
            else:
                v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outputs.items():
            a = v.contiguous().view(torch.uint8) if v.dim() else v
            b = ref[k].contiguous().view(torch.uint8) if v.dim() else ref[k]
            assert torch.equal(a, b), f"{what}: replay {rep}: {k} differs from the eager run"
        say(f"[capture] {what}: replay {rep} bitwise equal to the eager run")
    del g


@pytest.mark.parametrize("name", ["qwen3_small", "dsv2_small", "qwen3_30b_a3b", "dsv2_lite"])
def test_routed_layer_no_sync_graph(name):
    """route -> permute -> gate_up -> down (+ shared experts) -> combine."""
    inp = W.generate(W.get(name))
    dev = _device(inp)
    k = inp["k"]
    T, d = dev["x"].shape
    E, _, f = dev["w_gate"].shape
    shared_f = dev["shared"][0].shape[2] if "shared" in dev else 0
    bufs = ops.layer_buffers(T, k, d, f, E, dev["x"].dtype, dev["x"].device, shared_f=shared_f)

    def run():
        ops.moe_layer(dev["x"], dev["w_router"], dev.get("bias"), k, dev["w_gate"],
                      dev["w_val"], dev["w_out"], shared=dev.get("shared"), bufs=bufs)

    outs = {key: bufs[key] for key in ("logits", "idx", "gates", "counts", "offsets",
                                       "perm_src", "dest", "y", "out")}
    outs["x_perm"] = bufs["x_perm"]
    if shared_f:
        outs["y_shared"] = bufs["y_shared"]
    _no_sync_then_replay(run, outs, name)


@pytest.mark.parametrize("name", ["ep_share_small", "ep_rank_share"])
def test_receive_chain_no_sync_graph(name):
    """permute_recv -> gate_up -> down -> un-permute, on one EP rank's share."""
    inp = W.generate(W.get(name))
    dev = _device(inp)
    N, d = dev["x_recv"].shape
    E, _, f = dev["w_gate"].shape
    S = dev["recv_counts"].shape[0]
    i32 = torch.int32
    cuda = dev["x_recv"].device
    p = dict(counts=torch.empty(E, dtype=i32, device=cuda),
             offsets=torch.empty(E + 1, dtype=i32, device=cuda),
             perm_src=torch.empty(N, dtype=i32, device=cuda),
             dest=torch.empty(N, dtype=i32, device=cuda),
             x_perm=ops.empty_rows(N, d, dev["x_recv"].dtype, cuda))
    ws = torch.empty(max(1, ops.grouped_ffn_workspace(N, d, f, E, dev["x_recv"].dtype)),
                     dtype=torch.uint8, device=cuda)
    y = torch.empty((N, d), dtype=torch.float32, device=cuda)
    out = torch.empty((N, d), dtype=torch.float32, device=cuda)
    assert S * E <= 4096

    def run():
        ops.permute_recv(dev["recv_counts"], dev["x_recv"], out=p)
        ops.grouped_ffn(p["x_perm"], p["offsets"], dev["w_gate"], dev["w_val"], dev["w_out"],
                        y=y, workspace=ws)
        ops.combine(y, p["dest"], None, 1, out=out)

    outs = dict(p, y=y, out=out)
    _no_sync_then_replay(run, outs, name)
