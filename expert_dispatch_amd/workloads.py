"""Seeded synthetic workloads for the routed-expert MoE layer.

This module only draws inputs; it holds none of the layer's arithmetic, so
both the HIP path's tests and the CPU oracle can take their inputs from it.

Recipe:
  * Gaussian values come from ``torch.Generator().manual_seed(seed)`` on the
    CPU (``torch.randn`` in fp32, times the std) in this order: x, router
    weight W_r, router bias, then for each expert e in ascending order
    W_gate[e], W_val[e], W_out[e], then the shared experts in the same way;
  * the structure that is particular to a config (experts forced empty, Zipf
    popularity ranks, Dirichlet count shares) comes from numpy's
    ``default_rng(seed)``;
  * for bf16 configs the fp32 draws are rounded to bf16 (round to nearest,
    ties to even); the rounded values are the inputs of both sides;
  * x ~ N(0, 1); W_r ~ N(0, 0.02); expert weights ~ N(0, 1/sqrt(fan_in)) with
    fan_in = d for W_gate and W_val and f for W_out (the second parameter of
    N is the standard deviation);
  * router bias: N(0, 0.5) for load skew; Zipf(s) popularity as
    b_e = -s * ln(r_e) over a seeded permutation of ranks r_e = 1..E; experts
    forced empty get b_e = -1e4;
  * receive-side share: p ~ Dirichlet(alpha) over the S*E_loc (sender, local
    expert) cells in sender-major order, counts ~ Multinomial(N, p), so the
    total is exact and many cells are small or empty.

bf16 tensors are returned as uint16 arrays holding the bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "routed" (tokens pass the router), "recv" (received buffer) or
                         # "gathered" (one rank of the all-gather / reduce-scatter layout)
    dtype: str           # "f32" or "bf16"
    d: int
    f: int
    E: int               # experts held on this GPU
    seed: int
    T: int = 0           # routed: tokens
    k: int = 0           # routed: top-k
    bias: str = "none"   # "none" | "normal" | "zipf"
    bias_std: float = 0.5
    zipf_s: float = 1.1
    shared: int = 0      # always-on shared experts of the routed shape
    empty: int = 0       # experts forced to receive no token
    N: int = 0           # recv: received rows
    S: int = 0           # recv: senders
    E_global: int = 0    # recv / gathered: experts over the whole EP group
    e_first: int = 0     # gathered: first global expert this rank owns
    alpha: float = 0.3   # recv: Dirichlet concentration
    description: str = ""

    @property
    def rows(self) -> int:
        """Rows the grouped FFN can process: T*k assignments (at most, for a
        rank's expert range) or N received rows."""
        return self.N if self.kind == "recv" else self.T * self.k

    @property
    def units(self) -> int:
        """Tokens (routed / gathered) or received rows (recv) one layer pass handles."""
        return self.N if self.kind == "recv" else self.T


CONFIGS = {
    c.name: c for c in [
        Config("tiny_f32", "routed", "f32", d=64, f=128, E=8, seed=1, T=256, k=2,
               description="tiny fp32 layer: T=256, d=64, E=8, top-2, SwiGLU 64->128->64"),
        Config("qwen3_30b_a3b", "routed", "bf16", d=2048, f=768, E=128, seed=2, T=4096, k=8,
               bias="normal",
               description="Qwen3-30B-A3B-shaped layer: T=4096 (2x2048), d=2048, E=128, "
                           "top-8, SwiGLU 2048->768->2048, router bias N(0,0.5)"),
        Config("dsv2_lite", "routed", "bf16", d=2048, f=1408, E=64, seed=3, T=8192, k=6,
               bias="normal", shared=2,
               description="DeepSeek-V2-Lite-shaped layer: T=8192 (2x4096), d=2048, 64 routed "
                           "experts top-6, SwiGLU 2048->1408->2048, 2 shared experts"),
        Config("dsv2_lite_empty4", "routed", "bf16", d=2048, f=1408, E=64, seed=3, T=8192,
               k=6, bias="normal", shared=2, empty=4,
               description="DeepSeek-V2-Lite-shaped layer with 4 experts receiving no token"),
        Config("ep_rank_share", "recv", "bf16", d=2048, f=1024, E=16, seed=4, N=16384, S=4,
               E_global=64,
               description="one EP rank's received buffer: N=16384 rows sender-major over "
                           "4 senders x 16 local experts (of 64), SwiGLU 2048->1024->2048, "
                           "Dirichlet(0.3) cell counts"),
        Config("ag_rs_rank", "gathered", "bf16", d=2048, f=768, E=16, seed=6, T=32768, k=8,
               E_global=128, e_first=80, bias="normal",
               description="one rank of an 8-rank all-gather / reduce-scatter EP group at the "
                           "Qwen3-30B-A3B shape: 32768 gathered tokens (8x4096), replicated "
                           "router over 128 experts, top-8, local experts 80..95, SwiGLU "
                           "2048->768->2048, partial outputs"),
        Config("stress_zipf", "routed", "bf16", d=4096, f=1536, E=64, seed=5, T=32768, k=8,
               bias="zipf",
               description="large-batch stress: T=32768, d=4096, E=64, top-8, SwiGLU "
                           "4096->1536->4096, Zipf(1.1) expert popularity via the router bias"),
        # Reduced shapes with the same structure: small enough for a full
        # element-by-element oracle comparison, still several tiles and a
        # ragged tail in every dimension the kernels tile.
        Config("qwen3_small", "routed", "bf16", d=256, f=384, E=16, seed=12, T=300, k=4,
               bias="normal", description="reduced Qwen3-shaped layer"),
        Config("dsv2_small", "routed", "bf16", d=256, f=256, E=12, seed=13, T=280, k=3,
               bias="normal", shared=2, description="reduced DeepSeek-V2-Lite-shaped layer"),
        Config("dsv2_small_empty4", "routed", "bf16", d=256, f=256, E=12, seed=13, T=280, k=3,
               bias="normal", shared=2, empty=4,
               description="reduced DeepSeek-V2-Lite-shaped layer, 4 empty experts"),
        Config("ep_share_small", "recv", "bf16", d=256, f=384, E=6, seed=14, N=700, S=4,
               E_global=24, description="reduced EP-rank receive share"),
        Config("stress_small", "routed", "bf16", d=512, f=384, E=16, seed=15, T=520, k=4,
               bias="zipf", description="reduced Zipf stress layer"),
        Config("odd_f32", "routed", "f32", d=48, f=80, E=5, seed=16, T=37, k=3,
               description="fp32 layer with dims that are not tile multiples"),
        Config("ag_rs_small", "gathered", "bf16", d=256, f=384, E=4, seed=17, T=300, k=4,
               E_global=16, e_first=8, bias="normal",
               description="reduced all-gather / reduce-scatter rank: experts 8..11 of 16"),
    ]
}


def get(name: str, **overrides) -> Config:
    c = CONFIGS[name]
    return dataclasses.replace(c, **overrides) if overrides else c


def _draw(gen, shape, std, dtype) -> torch.Tensor:
    a = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        a.mul_(float(np.float32(std)))
    return a.to(torch.bfloat16).view(torch.int16) if dtype == "bf16" else a


def _as_numpy(t: torch.Tensor) -> np.ndarray:
    a = t.numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def _normal(gen, shape, std, dtype):
    return _as_numpy(_draw(gen, shape, std, dtype))


def _experts(gen, n, d, f, dtype):
    # large host buffers are allocated by torch, whose parallel copies also
    # spread the first touch of the pages over the host threads
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    wg = torch.empty((n, d, f), dtype=tdt)
    wv = torch.empty((n, d, f), dtype=tdt)
    wo = torch.empty((n, f, d), dtype=tdt)
    for e in range(n):
        wg[e].copy_(_draw(gen, (d, f), 1.0 / math.sqrt(d), dtype))
        wv[e].copy_(_draw(gen, (d, f), 1.0 / math.sqrt(d), dtype))
        wo[e].copy_(_draw(gen, (f, d), 1.0 / math.sqrt(f), dtype))
    return _as_numpy(wg), _as_numpy(wv), _as_numpy(wo)


def generate(cfg: Config | str) -> dict:
    """Draw every input of one layer pass. Returns a dict of numpy arrays
    plus the integer parameters the calls need."""
    if isinstance(cfg, str):
        cfg = get(cfg)
    gen = torch.Generator().manual_seed(cfg.seed)
    rng = np.random.default_rng(cfg.seed)
    out = dict(config=cfg, dtype=cfg.dtype)
    if cfg.kind == "routed":
        out["x"] = _normal(gen, (cfg.T, cfg.d), 1.0, cfg.dtype)
        out["w_router"] = _normal(gen, (cfg.d, cfg.E), 0.02, cfg.dtype)
        bias = None
        if cfg.bias == "normal":
            bias = _normal(gen, (cfg.E,), cfg.bias_std, "f32")
        out["w_gate"], out["w_val"], out["w_out"] = _experts(gen, cfg.E, cfg.d, cfg.f, cfg.dtype)
        if cfg.shared:
            (out["shared_w_gate"], out["shared_w_val"],
             out["shared_w_out"]) = _experts(gen, cfg.shared, cfg.d, cfg.f, cfg.dtype)
        if cfg.bias == "zipf":
            ranks = rng.permutation(cfg.E) + 1
            bias = (-cfg.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)
        if cfg.empty:
            if bias is None:
                bias = np.zeros(cfg.E, np.float32)
            starved = np.sort(rng.choice(cfg.E, size=cfg.empty, replace=False))
            bias = bias.copy()
            bias[starved] = np.float32(-1.0e4)
            out["starved"] = starved
        out["bias"] = bias
        out["k"] = cfg.k
        out["renorm"] = True
    elif cfg.kind == "gathered":
        out["x"] = _normal(gen, (cfg.T, cfg.d), 1.0, cfg.dtype)
        out["w_router"] = _normal(gen, (cfg.d, cfg.E_global), 0.02, cfg.dtype)
        out["bias"] = (_normal(gen, (cfg.E_global,), cfg.bias_std, "f32")
                       if cfg.bias == "normal" else None)
        out["w_gate"], out["w_val"], out["w_out"] = _experts(gen, cfg.E, cfg.d, cfg.f, cfg.dtype)
        out["k"] = cfg.k
        out["renorm"] = True
        out["e_first"] = cfg.e_first
    elif cfg.kind == "recv":
        out["x_recv"] = _normal(gen, (cfg.N, cfg.d), 1.0, cfg.dtype)
        out["w_gate"], out["w_val"], out["w_out"] = _experts(gen, cfg.E, cfg.d, cfg.f, cfg.dtype)
        p = rng.dirichlet(np.full(cfg.S * cfg.E, cfg.alpha))
        counts = rng.multinomial(cfg.N, p).astype(np.int32)
        out["recv_counts"] = counts.reshape(cfg.S, cfg.E)
    else:
        raise ValueError(cfg.kind)
    return out


def output_gradient(cfg: Config | str) -> np.ndarray:
    """A seeded upstream gradient dL/dout [T,d] for a backward pass, Gaussian
    with unit variance, in the workload's activation type (its own generator,
    so the layer's inputs are the same with or without it)."""
    if isinstance(cfg, str):
        cfg = get(cfg)
    gen = torch.Generator().manual_seed(1_000_003 * (cfg.seed + 1))
    return _normal(gen, (cfg.T, cfg.d), 1.0, cfg.dtype)


def zero_expert_column(inp: dict, j: int) -> dict:
    """Receive-side variant with local expert j emptied: its rows are moved to
    the next expert of the same sender, so the total stays N."""
    rc = inp["recv_counts"].copy()
    E = rc.shape[1]
    for i in range(rc.shape[0]):
        rc[i, (j + 1) % E] += rc[i, j]
        rc[i, j] = 0
    out = dict(inp)
    out["recv_counts"] = rc
    return out
