#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

One step = one pass of the whole hot path over one batch: router (scores,
top-k, weights) -> expert-major packing -> grouped SwiGLU gate/up -> down ->
weighted combine (plus the shared experts where the workload has them; the
receive-side workload runs the device reorder instead of router + packing and
un-permutes back to sender-major order; the gathered-token workload routes every
gathered token over the whole expert set, packs only the rank's own experts and
combines into the rank's partial output). Inputs are seeded synthetic tensors
already resident in HBM; every buffer is allocated before timing, so the timed
region is kernel launches only. After the timed steps the same K steps run
once more (the A/A repeat, reported as the run-to-run noise floor), then K
steps with HIP events recorded between the stages on the stream the kernels
are launched on (the per-stage times; the events slow a step down, so they
stay out of the timed region), and each stage is timed cold: right after a
1 GiB read that evicts its inputs from the L2s and the Infinity Cache.
Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU; % bf16 MFMA peak (GEMM), % HBM BW (permute)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_MFMA_BF16_TFS = 2500.0    # dense bf16 matrix peak
PEAK_MFMA_F32_TFS = 157.3      # used for the fp32 path (vector fp32 peak)
# fp32 vector peak without packed-fp32 instructions (the library is built
# without them): 256 CUs x 4 SIMDs x 16 lanes x 2 flop (one FMA) x 2.4 GHz =
# 78.6 TFLOP/s; the 157.3 TFLOP/s figure counts packed FMAs (two per lane and
# clock)
PEAK_VALU_F32_TFS = 78.6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="stress_zipf",
                    help="workload (default: the largest one-GPU workload, the T=32768, "
                         "d=4096 Zipf stress layer)")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="fixed-capacity packing: each expert keeps at most "
                         "ceil(factor * T * k / E) assignments (token-routed workloads)")
    ap.add_argument("--y-dtype", choices=("f32", "bf16"), default="f32",
                    help="storage type of the expert outputs y_perm between the down GEMM "
                         "and the combine (bf16 inputs only)")
    ap.add_argument("--partial-dtype", choices=("f32", "bf16"), default="bf16",
                    help="gathered-token workload: type of the partial output that the "
                         "reduce-scatter would sum")
    ap.add_argument("--no-renorm", action="store_true",
                    help="un-normalised router weights: the full-softmax probabilities of the "
                         "selected experts instead of a softmax over the k selected logits")
    ap.add_argument("--route-stats", action="store_true",
                    help="add the load statistics (mean full-softmax probability per expert and "
                         "the load-balance statistic) to the step, after the packing")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step instead: the forward keeping what the "
                         "backward needs, then the backward of sum(out * d_out) with a "
                         "seeded d_out (token-routed workloads)")
    ap.add_argument("--cold-reps", type=int, default=3,
                    help="reps of the per-stage cold timing (each stage right after a 1 GiB "
                         "read that evicts the caches); 0 skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the matrix-core-loop and streaming-copy ceilings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU work of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (3 launches), the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n,
                      "copy_calibration_bytes_written_per_launch": n, "launches": 3}), flush=True)


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def stage_work(cfg, counts, es, ys=4, kept=None, os_=4, touched=None):
    """Algorithmic flops and bytes of one launch of each stage: what the method
    must compute or move (s = element size, TK = T*k rows, n_act = experts with
    rows). Router 2*T*d*E flop; packing (T + TK)*d*s bytes + indices; gate_up
    4*TK*d*f flop over TK*d*s + n_act*2*d*f*s + TK*f*s bytes; down 2*TK*f*d flop
    over TK*f*s + n_act*f*d*s + TK*d*ys bytes; combine TK*d*ys + T*d*os bytes
    (ys, os = element sizes of the stored expert outputs and of the layer
    output). For a rank of the all-gather layout the router spans the whole
    expert set, TK is the rank's kept assignments, and the packing reads only
    the ``touched`` tokens that have at least one of them."""
    T, k, d, f, E = cfg.T, cfg.k, cfg.d, cfg.f, cfg.E
    rows = cfg.rows if kept is None else kept   # packed rows the experts process
    active = int((counts > 0).sum())
    w = {}
    if cfg.kind == "routed":
        w["route"] = dict(flops=2.0 * T * d * E,
                          bytes=T * d * es + d * E * es + E * 4 + T * E * 4 + 2 * T * k * 4,
                          bound="alu")
        w["permute"] = dict(flops=0.0, bytes=(T + rows) * d * es + 4 * cfg.rows * 4, bound="hbm")
    elif cfg.kind == "gathered":
        Eg = cfg.E_global
        w["route"] = dict(flops=2.0 * T * d * Eg,
                          bytes=T * d * es + d * Eg * es + Eg * 4 + T * Eg * 4 + 2 * T * k * 4,
                          bound="alu")
        # idx read + dest written for every assignment, perm_src for the kept
        w["permute"] = dict(flops=0.0, bytes=(touched + rows) * d * es + 2 * T * k * 4 + rows * 4,
                            bound="hbm")
    else:
        w["permute_recv"] = dict(flops=0.0, bytes=2 * rows * d * es + 2 * rows * 4, bound="hbm")
    # the expert MLPs' algorithmic bytes: the weights once, x_perm in (gate_up)
    # and y_perm out (down); the hidden activations h between the two launches
    # are implementation traffic, listed apart (impl_bytes)
    w["gate_up"] = dict(flops=4.0 * rows * d * f,
                        bytes=rows * d * es + active * 2 * d * f * es, impl_bytes=rows * f * es)
    w["down"] = dict(flops=2.0 * rows * f * d,
                     bytes=active * f * d * es + rows * d * ys, impl_bytes=rows * f * es)
    if cfg.shared:
        fs = cfg.shared * f
        w["shared_gate_up"] = dict(flops=4.0 * T * d * fs, bytes=T * d * es + 2 * d * fs * es,
                                   impl_bytes=T * fs * es)
        w["shared_down"] = dict(flops=2.0 * T * fs * d, bytes=fs * d * es + T * d * ys,
                                impl_bytes=T * fs * es)
    # load statistics: the logits read (once for the normalisers, once for the
    # probabilities), the counts and the outputs
    w["route_stats"] = dict(flops=0.0, bytes=2 * T * E * 4 + E * 4 + E * 4 + 4, bound="hbm")
    units = cfg.units
    idx_bytes = T * k * 8 if cfg.kind == "gathered" else rows * 8
    w["combine"] = dict(flops=2.0 * rows * d,
                        bytes=rows * d * ys + units * d * os_ + idx_bytes
                        + (units * d * 4 if cfg.shared else 0), bound="hbm")
    mfma_peak = PEAK_MFMA_BF16_TFS if es == 2 else PEAK_MFMA_F32_TFS
    for name, v in w.items():
        if "bound" not in v:
            # the bound follows from all bytes the kernel must move (h included)
            ai = v["flops"] / max(v["bytes"] + v.get("impl_bytes", 0), 1)
            v["bound"] = "mfma" if ai * PEAK_HBM_GBS * 1e9 > mfma_peak * 1e12 else "hbm"
    return w


def roofline_entry(v, us, es):
    if v["bound"] == "hbm":
        ach = v["bytes"] / (us * 1e-6) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS)
    if v["bound"] == "alu":
        ach = v["flops"] / (us * 1e-6) / 1e12
        return dict(bound="alu", achieved=ach, peak=PEAK_VALU_F32_TFS, unit="TFLOP/s",
                    frac=ach / PEAK_VALU_F32_TFS)
    peak = PEAK_MFMA_BF16_TFS if es == 2 else PEAK_MFMA_F32_TFS
    ach = v["flops"] / (us * 1e-6) / 1e12
    return dict(bound="mfma", achieved=ach, peak=peak, unit="TFLOP/s", frac=ach / peak)


def traffic_for(stage: str, workload: str):
    """HBM bytes (read + write) per launch of a stage, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/traffic.json), if it was
    taken on the current sources of the stage's kernels; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(workload, {}).get(stage)
        if not ent:
            return None
        h = hashlib.sha256()
        for src in ent["sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != ent["sources_sha256"]:
            return None
        return float(ent["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError, TypeError):
        return None


def input_digests(inp: dict) -> dict:
    """xxh64 of the bytes of every generated input array (the seeded values
    both the GPU run and the oracle read), so two runs can show they used the
    same inputs."""
    import xxhash
    out = {}
    for key in sorted(inp):
        v = inp[key]
        parts = [v] if isinstance(v, np.ndarray) else list(v) if isinstance(v, (list, tuple)) else []
        if parts and all(isinstance(a, np.ndarray) for a in parts):
            h = xxhash.xxh64()
            for a in parts:
                h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1))
            out[key] = h.hexdigest()
    return out


def host_info() -> dict:
    """CPU model and thread settings of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_model=model, os_cpu_count=os.cpu_count(),
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"))


def cpu_baseline(cfg, inp, target_s: float, round_h: bool = False):
    """Time the oracle on the first n tokens (rows) of the same workload, n
    calibrated to about target_s seconds of CPU work. Returns the report and
    the oracle's results of the last run (the parity reference for those
    tokens). ``round_h`` (gathered-token workload): the oracle rounds h to
    bf16 at its storage point, the reference the partial output is held to."""
    import oracle
    last = {}
    if cfg.kind == "routed":
        def run(n):
            sub = dict(inp, x=inp["x"][:n])
            t = time.perf_counter()
            last["o"] = oracle.moe_layer(sub)
            return time.perf_counter() - t
        total = cfg.T
    elif cfg.kind == "gathered":
        def run(n):
            sub = dict(inp, x=inp["x"][:n])
            t = time.perf_counter()
            last["o"] = oracle.moe_partial_layer(sub, cfg.e_first, round_h=round_h)
            return time.perf_counter() - t
        total = cfg.T
    else:
        def run(n):
            t = time.perf_counter()
            last["o"] = oracle.moe_recv_layer(inp, rows=np.arange(n, dtype=np.int32))
            return time.perf_counter() - t
        total = cfg.N
    # calibrate in two steps: a 16-token run overstates the cost per token (the
    # per-expert setup of a tiny batch), so size a ~2 s run from it first
    n0 = min(total, 16)
    t0 = run(n0)
    n1 = int(min(total, max(n0, n0 * 2.0 / max(t0, 1e-3))))
    t1 = run(n1) if n1 > n0 else t0
    n = int(min(total, max(n1, n1 * target_s / max(t1, 1e-3))))
    t = run(n)
    reps = 1
    # the whole workload in less than the target time: repeat it
    while n == total and t < 0.6 * target_s and reps < 30:
        t += run(n)
        reps += 1
    unit_name = {"routed": "tokens", "gathered": "gathered tokens"}.get(cfg.kind, "rows")
    what = (f"all {total}" if n == total else f"first {n} of {total}")
    rep = dict(value=reps * n / t, unit=f"{unit_name}/s", cores=oracle.num_threads(),
               kind="oracle",
               sample=f"{what} {unit_name} of the same workload (same weights), whole layer "
                      f"in the oracle, {reps} run(s), {t:.1f} s", **host_info())
    return rep, last["o"], n


def sample_parity(cfg, o, n, g):
    """Parity of the timed GPU run's outputs against the oracle's on the
    cpu_baseline sample (the first n tokens or received rows): integer
    mismatches of the router ids, the fp32 rule on the router weights, and
    the layer output's max error / RMS (the bf16 bar) and normwise error."""
    def num(t):
        t = t.detach().cpu()
        if t.dtype == torch_bf16():
            t = t.float()
        return t.numpy().astype(np.float64) if t.is_floating_point() else t.numpy()

    res = {"sample": n}
    if cfg.kind != "recv":
        idx = g["idx"][:n].cpu().numpy()
        res["idx_mismatches"] = int((idx != o["idx"]).sum())
        gg = num(g["gates"][:n])
        ref = np.asarray(o["gates"], np.float64)
        rms = float(np.sqrt(np.mean(ref * ref)))
        res["gates_max_rel_err"] = float(np.max(np.abs(gg - ref) / np.maximum(np.abs(ref), rms)))
        out = num(g["out"][:n])
    else:
        out = num(g["out"][o["rows"]])
    ref = o["out"]
    rms = float(np.sqrt(np.mean(ref * ref)))
    res["out_max_err_over_rms"] = float(np.max(np.abs(out - ref)) / rms)
    res["out_rel_l2"] = float(np.sqrt(np.sum((out - ref) ** 2) / np.sum(ref * ref)))
    if g["out"].dtype == torch_bf16():
        # an output stored in bf16: its own rounding (at most 2^-8 of each
        # element) taken off each element's error
        u = 2.0 ** -8
        excess = np.maximum(np.abs(out - ref) - u * np.abs(ref), 0.0) / (1 + u)
        res["out_max_err_beyond_storage_over_rms"] = float(np.max(excess) / rms)
    return res


def torch_bf16():
    import torch
    return torch.bfloat16


def ceilings(torch, ops):
    """What the chip reaches on this machine in the plainest kernels: the
    matrix-core loop (bf16 TFLOP/s) and a 2 GiB streaming copy and read
    (GB/s), each the median of 5 event-timed launches."""
    cuda = torch.device("cuda")
    res = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return float(np.median(ts))

    blocks = 256 * 4
    sink = torch.empty(blocks, dtype=torch.float32, device=cuda)
    flops = {}

    def mfma():
        flops["n"] = ops.ceiling_mfma(blocks, 4096, sink)
    t = timed(mfma)
    res["mfma_bf16_tflops"] = round(flops["n"] / t / 1e12, 1)
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=cuda)
    dst = torch.empty_like(src)
    usink = torch.empty(4096, dtype=torch.int32, device=cuda)
    t = timed(lambda: ops.ceiling_copy(src, dst, nbytes, 4096))
    res["copy_gbs"] = round(2 * nbytes / t / 1e9, 1)
    t = timed(lambda: ops.ceiling_read(src, nbytes, usink, 4096))
    res["read_gbs"] = round(nbytes / t / 1e9, 1)
    res["how"] = ("matrix-core loop: 1024 blocks x 4 wavefronts x 4096 x 8 "
                  "v_mfma_f32_32x32x16_bf16 on registers; copy and read: 2 GiB, 16-byte "
                  "non-temporal accesses, 4096 blocks; median of 5 launches")
    del src, dst
    return res


def backward_work(cfg, counts, es):
    """Algorithmic flops and bytes of the backward stages (bf16 data, fp32
    gradients of the weights, fp32 expert outputs y). rows = kept packed rows,
    n_act = experts with rows."""
    T, k, d, f, E = cfg.T, cfg.k, cfg.d, cfg.f, cfg.E
    rows = int(counts.sum())
    active = int((counts > 0).sum())
    w = {}
    # d_out read once per token, y read and d_y written per row, weights and dest
    w["combine_bwd"] = dict(flops=4.0 * rows * d,
                            bytes=T * d * es + rows * d * 4 + rows * d * es + T * k * 12)
    w["down_bwd"] = dict(flops=2.0 * rows * d * f,
                         bytes=rows * d * es + active * f * d * es + 2 * rows * 2 * f * es)
    w["weight_grads"] = dict(flops=6.0 * rows * d * f,
                             bytes=rows * (f + d + d + 2 * f) * es + 3 * E * d * f * 4)
    w["gate_up_bwd"] = dict(flops=4.0 * rows * d * f,
                            bytes=rows * 2 * f * es + active * 2 * d * f * es + rows * d * es)
    # every token's rows of d_x_perm plus k rows of W_r^T (L2-resident), d_x written once
    w["token_grad"] = dict(flops=2.0 * rows * d + 2.0 * T * k * d,
                           bytes=rows * d * es + T * d * 4 + T * k * 16 + d * E * es * 2,
                           bound="hbm")
    w["route_bwd"] = dict(flops=6.0 * T * E, bytes=T * E * 4 + T * k * 16 + T * E * 6,
                          bound="hbm")
    w["router_bwd"] = dict(flops=2.0 * T * d * E, bytes=T * d * es + T * E * es + d * E * 4)
    for v in w.values():
        if "bound" not in v:
            ai = v["flops"] / max(v["bytes"], 1)
            v["bound"] = "mfma" if ai * PEAK_HBM_GBS * 1e9 > PEAK_MFMA_BF16_TFS * 1e12 else "hbm"
    return w


def main_backward(args):
    """One training step of the layer: forward (keeping the pre-activations)
    and backward, every buffer allocated before timing."""
    import torch
    from expert_dispatch_amd import ops
    from expert_dispatch_amd import workloads as W

    cfg = W.get(args.config)
    if cfg.kind != "routed" or cfg.dtype != "bf16" or cfg.shared:
        print("bench.py --backward times the token-routed bf16 workloads without shared "
              "experts", file=sys.stderr)
        sys.exit(2)
    es = 2
    log(f"[bench] generating {cfg.name} (training step)")
    inp = W.generate(cfg)
    torch.cuda.set_device(0)
    dev = {k: to_dev(inp.get(k), torch) for k in ("x", "w_router", "bias", "w_gate", "w_val",
                                                  "w_out")}
    d_out = to_dev(W.output_gradient(cfg), torch)
    T, k, d, f, E = cfg.T, cfg.k, cfg.d, cfg.f, cfg.E
    rows = T * k
    cuda = torch.device("cuda")
    bf = torch.bfloat16
    f32 = torch.float32
    b = dict(
        logits=torch.empty((T, E), dtype=f32, device=cuda),
        idx=torch.empty((T, k), dtype=torch.int32, device=cuda),
        gates=torch.empty((T, k), dtype=f32, device=cuda),
        counts=torch.empty(E, dtype=torch.int32, device=cuda),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=cuda),
        perm_src=torch.empty(rows, dtype=torch.int32, device=cuda),
        dest=torch.empty(rows, dtype=torch.int32, device=cuda),
        x_perm=ops.empty_rows(rows, d, bf, cuda),
        h=torch.empty((rows, f), dtype=bf, device=cuda),
        act=torch.empty((rows, 2 * f), dtype=bf, device=cuda),
        y=torch.empty((rows, d), dtype=f32, device=cuda),
        out=torch.empty((T, d), dtype=f32, device=cuda),
        d_y=torch.empty((rows, d), dtype=bf, device=cuda),
        d_gates=torch.empty((T, k), dtype=f32, device=cuda),
        d_act=torch.empty((rows, 2 * f), dtype=bf, device=cuda),
        d_xp=torch.empty((rows, d), dtype=bf, device=cuda),
        d_x=torch.empty((T, d), dtype=f32, device=cuda),
        dwg=torch.empty((E, d, f), dtype=f32, device=cuda),
        dwv=torch.empty((E, d, f), dtype=f32, device=cuda),
        dwo=torch.empty((E, f, d), dtype=f32, device=cuda),
        d_l=torch.empty((T, E), dtype=f32, device=cuda),
        d_lp=torch.empty((T, E), dtype=bf, device=cuda),
        d_wr=torch.empty((d, E), dtype=f32, device=cuda),
    )
    ws = torch.empty(max(1, ops.permute_workspace(T, k, E)), dtype=torch.uint8, device=cuda)
    rws = torch.empty(max(1, ops.router_backward_workspace(T, d, E)), dtype=torch.uint8,
                      device=cuda)
    tws = torch.empty(d * E * es, dtype=torch.uint8, device=cuda)
    stages = ["route", "permute", "gate_up", "down", "combine", "combine_bwd", "down_bwd",
              "weight_grads", "gate_up_bwd", "token_grad", "route_bwd", "router_bwd"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ops.route(dev["x"], dev["w_router"], dev["bias"], k, out=(b["logits"], b["idx"], b["gates"]))
        mark(1)
        ops.permute(b["idx"], dev["x"], E, out=b, workspace=ws)
        mark(2)
        ops.ffn_gate_up_train(b["x_perm"], b["offsets"], dev["w_gate"], dev["w_val"], h=b["h"],
                              act=b["act"])
        mark(3)
        ops.ffn_down(b["h"], b["offsets"], dev["w_out"], y=b["y"])
        mark(4)
        ops.combine(b["y"], b["dest"], b["gates"], k, out=b["out"])
        mark(5)
        ops.combine_backward(d_out, b["y"], b["dest"], b["gates"], k, d_y=b["d_y"],
                             d_gates=b["d_gates"])
        mark(6)
        ops.ffn_down_backward(b["d_y"], b["offsets"], dev["w_out"], b["act"], d_act=b["d_act"])
        mark(7)
        ops.ffn_weight_grads(b["x_perm"], b["h"], b["d_y"], b["d_act"], b["offsets"], E,
                             out=(b["dwg"], b["dwv"], b["dwo"]))
        mark(8)
        ops.ffn_gate_up_backward(b["d_act"], b["offsets"], dev["w_gate"], dev["w_val"],
                                 d_x=b["d_xp"])   # bf16, as the training step hands it on
        mark(9)
        ops.token_backward(b["d_xp"], b["dest"], b["idx"], b["gates"], b["d_gates"],
                           dev["w_router"], d_x=b["d_x"], workspace=tws)
        mark(10)
        ops.route_backward(b["logits"], b["idx"], b["gates"], b["d_gates"], True,
                           d_logits=b["d_l"], d_logits_lp=b["d_lp"])
        mark(11)
        ops.router_backward(dev["x"], dev["w_router"], b["d_lp"], d_w=b["d_wr"], workspace=rws)
        mark(12)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} training steps")
    torch.cuda.synchronize()
    t0.record()
    for s_ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    # per-stage times from K more steps with events between the stages (kept
    # out of the timed steps, which they would slow down)
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    stage_us = {n: float(np.mean([evs[s_][j].elapsed_time(evs[s_][j + 1])
                                  for s_ in range(args.steps)]) * 1e3)
                for j, n in enumerate(stages)}
    counts = b["counts"].cpu().numpy()
    fw = stage_work(cfg, counts, es, 4, int(counts.sum()))
    bw = backward_work(cfg, counts, es)
    work = dict(fw, **bw)
    rep = {}
    for n in stages:
        r = roofline_entry(work[n], stage_us[n], es)
        rep[n] = dict(us=round(stage_us[n], 2), bound=r["bound"], achieved=round(r["achieved"], 1),
                      unit=r["unit"], frac=round(r["frac"], 4), alg_flops=work[n]["flops"],
                      alg_bytes=work[n]["bytes"])
    bwd = stages[5:]
    dominant = max(bwd, key=lambda n: stage_us[n])
    dom = roofline_entry(work[dominant], stage_us[dominant], es)
    res = {
        "metric": "MoE-layer training step (forward + backward) tokens/sec at 1 GPU",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "forward_ms": round(sum(stage_us[n] for n in stages[:5]) / 1e3, 5),
        "backward_ms": round(sum(stage_us[n] for n in bwd) / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs, weights and output gradient)",
        "config": {"workload": cfg.name, "seed": cfg.seed, "T": T, "k": k, "d": d, "f": f,
                   "E": E, "kept_rows": int(counts.sum())},
        "roofline": {"kernel": dominant, "bound": dom["bound"], "achieved": round(dom["achieved"], 1),
                     "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                     "traffic": traffic_for(dominant, cfg.name + "/backward")},
        "stages": rep,
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.backward:
        if args.gpus != 1:
            print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported",
                  file=sys.stderr)
            sys.exit(2)
        main_backward(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on one GPU's share of an expert-parallel layout)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from expert_dispatch_amd import ops
    from expert_dispatch_amd import workloads as W

    cfg = W.get(args.config)
    es = 2 if cfg.dtype == "bf16" else 4
    log(f"[bench] generating {cfg.name}")
    inp = W.generate(cfg)
    torch.cuda.set_device(0)
    dev = {k: to_dev(inp.get(k), torch) for k in
           ("x", "w_router", "bias", "w_gate", "w_val", "w_out", "x_recv", "recv_counts")}
    E, d, f = cfg.E, cfg.d, cfg.f
    rows = cfg.rows
    xdt = torch.bfloat16 if es == 2 else torch.float32
    cuda = torch.device("cuda")
    # every buffer of the step, allocated once
    bufs = dict(
        counts=torch.empty(E, dtype=torch.int32, device=cuda),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=cuda),
        perm_src=torch.empty(rows, dtype=torch.int32, device=cuda),
        dest=torch.empty(rows, dtype=torch.int32, device=cuda),
        x_perm=ops.empty_rows(rows, d, xdt, cuda),   # the padded packed-row stride
    )
    h = torch.empty((rows, f), dtype=xdt, device=cuda)
    ys = 2 if (args.y_dtype == "bf16" and es == 2) else 4
    y = torch.empty((rows, d), dtype=torch.bfloat16 if ys == 2 else torch.float32, device=cuda)
    units = cfg.units
    gathered = cfg.kind == "gathered"
    os_ = 2 if (gathered and args.partial_dtype == "bf16") else 4
    out = torch.empty((units, d), dtype=torch.bfloat16 if os_ == 2 else torch.float32, device=cuda)
    shared = None
    cap = None
    e_first = cfg.e_first if gathered else None
    if cfg.kind in ("routed", "gathered"):
        Er = cfg.E_global if gathered else E   # experts the router scores
        logits = torch.empty((cfg.T, Er), dtype=torch.float32, device=cuda)
        idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=cuda)
        gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=cuda)
        ws = torch.empty(max(1, ops.permute_workspace(cfg.T, cfg.k, E)), dtype=torch.uint8,
                         device=cuda)
        if args.capacity_factor is not None and not gathered:
            cap = int(np.ceil(args.capacity_factor * cfg.T * cfg.k / E))
            bufs["routed"] = torch.empty(E, dtype=torch.int32, device=cuda)
        if cfg.shared:
            shared = dict(
                wg=to_dev(np.concatenate(list(inp["shared_w_gate"]), axis=1)[None], torch),
                wv=to_dev(np.concatenate(list(inp["shared_w_val"]), axis=1)[None], torch),
                wo=to_dev(np.concatenate(list(inp["shared_w_out"]), axis=0)[None], torch),
                off=None,   # one group of all T tokens
                h=torch.empty((cfg.T, cfg.shared * f), dtype=xdt, device=cuda),
                y=torch.empty((cfg.T, d), dtype=torch.float32, device=cuda))

    renorm = not args.no_renorm
    with_stats = args.route_stats and cfg.kind == "routed"
    if args.route_stats and not with_stats:
        print("--route-stats applies to the token-routed workloads only", file=sys.stderr)
        sys.exit(2)
    if with_stats:
        stats_out = (torch.empty(E, dtype=torch.float32, device=cuda),
                     torch.empty(1, dtype=torch.float32, device=cuda))
        stats_ws = torch.empty(max(1, ops.route_stats_workspace(cfg.T, E)), dtype=torch.uint8,
                               device=cuda)
        stats_counts = bufs["routed"] if "routed" in bufs else bufs["counts"]
    stages = (["route", "permute"] if cfg.kind != "recv" else ["permute_recv"]) + \
        (["route_stats"] if with_stats else []) + \
        ["gate_up", "down"] + (["shared_gate_up", "shared_down"] if shared else []) + ["combine"]

    # the step as its stages' launches, in order
    def _route():
        ops.route(dev["x"], dev["w_router"], dev["bias"], cfg.k, renorm, out=(logits, idx, gates))

    def _permute():
        ops.permute(idx, dev["x"], E, capacity=cap, e_first=e_first, out=bufs, workspace=ws)

    def _shared_up():
        ops.ffn_gate_up(dev["x"], shared["off"], shared["wg"], shared["wv"], h=shared["h"])

    def _combine():
        if cfg.kind != "recv":
            ops.combine(y, bufs["dest"], gates, cfg.k, y_shared=shared["y"] if shared else None,
                        out=out)
        else:
            ops.combine(y, bufs["dest"], None, 1, out=out)

    fns = {
        "route": _route,
        "permute": _permute,
        "route_stats": lambda: ops.route_stats(logits, stats_counts, cfg.k, out=stats_out,
                                               workspace=stats_ws),
        "permute_recv": lambda: ops.permute_recv(dev["recv_counts"], dev["x_recv"], out=bufs),
        "gate_up": lambda: ops.ffn_gate_up(bufs["x_perm"], bufs["offsets"], dev["w_gate"],
                                           dev["w_val"], h=h),
        "down": lambda: ops.ffn_down(h, bufs["offsets"], dev["w_out"], y=y),
        "shared_gate_up": _shared_up,
        "shared_down": lambda: ops.ffn_down(shared["h"], shared["off"], shared["wo"],
                                            y=shared["y"]),
        "combine": _combine,
    }
    stage_fns = [fns[n] for n in stages]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        for j, fn in enumerate(stage_fns):
            fn()
            if ev is not None:
                ev[j + 1].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    n_ev = len(stages) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")

    def timed():
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.steps):
            step()
        t_end.record()
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    ms = timed()
    # A/A: the same K timed steps once more, back to back: the run-to-run noise floor
    ms_repeat = timed()
    # the distribution of single steps: K more steps with an event between
    # consecutive steps (none inside a step)
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    sev[0].record()
    for s in range(args.steps):
        step()
        sev[s + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([sev[s].elapsed_time(sev[s + 1]) for s in range(args.steps)])
    # per-stage times: K more steps with an event between stages (kept out of
    # the timed steps: an event between two launches makes the second wait for
    # the first to drain completely)
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    stage_us = {}
    for j, name in enumerate(stages):
        stage_us[name] = float(np.mean([evs[s][j].elapsed_time(evs[s][j + 1])
                                        for s in range(args.steps)]) * 1e3)
    events_ms = float(np.mean([evs[s][0].elapsed_time(evs[s][-1]) for s in range(args.steps)]))

    # cold stages: before each stage a 1 GiB read evicts its inputs from the
    # L2s and the 256 MB Infinity Cache, so the stage reads them from HBM (a
    # read, not a write: evicting dirty lines would put write-backs to HBM
    # under the timed stage)
    cold_us = {}
    if args.cold_reps > 0:
        log(f"[bench] cold stages, {args.cold_reps} rep(s)")
        flush = torch.ones(1 << 28, dtype=torch.int32, device=cuda)
        flush_sum = torch.empty((), dtype=torch.int64, device=cuda)
        cev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in stages] for _ in range(args.cold_reps)]
        for r in range(args.cold_reps):
            for j, fn in enumerate(stage_fns):
                torch.sum(flush, dim=0, out=flush_sum)
                cev[r][j][0].record()
                fn()
                cev[r][j][1].record()
        torch.cuda.synchronize()
        for j, name in enumerate(stages):
            cold_us[name] = float(np.mean([cev[r][j][0].elapsed_time(cev[r][j][1])
                                           for r in range(args.cold_reps)]) * 1e3)
        del flush, flush_sum

    counts = bufs["counts"].cpu().numpy()
    kept = int(counts.sum())
    touched = None
    if gathered:
        touched = int((bufs["dest"].view(cfg.T, cfg.k) >= 0).any(dim=1).sum().item())
    work = stage_work(cfg, counts, es, ys, kept, os_, touched)
    stage_rep = {}
    for name in stages:
        r = roofline_entry(work[name], stage_us[name], es)
        stage_rep[name] = dict(us=round(stage_us[name], 2), bound=r["bound"],
                               achieved=round(r["achieved"], 1), unit=r["unit"],
                               frac=round(r["frac"], 4), alg_flops=work[name]["flops"],
                               alg_bytes=work[name]["bytes"])
        if "impl_bytes" in work[name]:
            stage_rep[name]["impl_bytes"] = work[name]["impl_bytes"]
        if name in cold_us:
            rc = roofline_entry(work[name], cold_us[name], es)
            stage_rep[name].update(cold_us=round(cold_us[name], 2),
                                   cold_frac=round(rc["frac"], 4))
    gemm = [n for n in stages if n in ("gate_up", "down", "shared_gate_up", "shared_down")]
    dominant = max(stages, key=lambda n: stage_us[n])
    dom = roofline_entry(work[dominant], stage_us[dominant], es)
    traffic = traffic_for(dominant, cfg.name)
    gemm_flops = sum(work[n]["flops"] for n in gemm)
    gemm_us = sum(stage_us[n] for n in gemm)
    value = units / (ms * 1e-3)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": {"routed": "tokens/s", "gathered": "gathered tokens/s"}.get(cfg.kind,
                                                                           "received rows/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if es == 2 else "f32",
        "data": "synthetic (seeded Gaussian inputs and weights of the stated shapes)",
        "config": {"workload": cfg.name, "description": cfg.description, "seed": cfg.seed,
                   "y_perm_dtype": "bf16" if ys == 2 else "f32",
                   "capacity_factor": None if gathered else args.capacity_factor,
                   "router_weights": "softmax over the selected" if renorm else "full softmax",
                   "route_stats": with_stats,
                   "kept_rows": kept, "T": cfg.T,
                   "k": cfg.k, "N": cfg.N, "d": d, "f": f, "E": E, "shared": cfg.shared,
                   "rows": rows, "load_max_over_mean": round(float(counts.max() / max(counts.mean(), 1e-9)), 3),
                   "empty_experts": int((counts == 0).sum()),
                   "input_xxh64": input_digests(inp)},
        **({"partial": {"E_global": cfg.E_global, "e_first": cfg.e_first,
                        "partial_dtype": "bf16" if os_ == 2 else "f32",
                        "tokens_with_local_expert": touched}} if gathered else {}),
        "roofline": {"kernel": dominant, "bound": dom["bound"], "achieved": round(dom["achieved"], 1),
                     "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                     "traffic": traffic},
        "aa": {"ms_per_step": round(ms, 5), "ms_per_step_repeat": round(ms_repeat, 5),
               "rel_delta": round(abs(ms_repeat - ms) / ms, 4)},
        "step_ms": {"median": round(float(np.median(step_ms)), 5),
                    "p10": round(float(np.percentile(step_ms, 10)), 5),
                    "p90": round(float(np.percentile(step_ms, 90)), 5),
                    "how": "K single steps, an event between consecutive steps"},
        "ms_per_step_with_stage_events": round(events_ms, 5),
        "gemm_mfma_frac": round(gemm_flops / (gemm_us * 1e-6) / 1e12 / (PEAK_MFMA_BF16_TFS if es == 2 else PEAK_MFMA_F32_TFS), 4),
        "stages": stage_rep,
    }
    res["ceilings"] = None
    if not args.no_ceilings:
        log("[bench] ceilings")
        res["ceilings"] = ceilings(torch, ops)
    res["parity"] = None
    if not args.no_cpu_baseline:
        log("[bench] oracle CPU baseline")
        # a rank's partial output sums fewer expert rows than the layer output,
        # so its RMS is small beside the bf16 rounding of the h it is formed
        # from: for bf16 data it is compared with the oracle that rounds h at
        # its storage point (as in the parity tests)
        storage_ref = gathered and es == 2
        res["cpu_baseline"], o_sample, n_sample = cpu_baseline(cfg, inp, args.cpu_seconds,
                                                               round_h=storage_ref)
        if cap is None and renorm:
            g = dict(out=out)
            if cfg.kind != "recv":
                g.update(idx=idx, gates=gates)
            res["parity"] = sample_parity(cfg, o_sample, n_sample, g)
            res["parity"]["note"] = ("the timed run's outputs on the oracle sample: router ids "
                                     "(mismatches), router weights (fp32 rule), layer output "
                                     "(max error / RMS against the 2e-2 bf16 bar)")
            res["parity"]["reference"] = ("oracle with h rounded to bf16 at its storage point"
                                          if storage_ref else "exact oracle")
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
