"""Plain CPU reference (oracle) of the routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only users; the product path
(``expert_dispatch_amd``) never imports this package. It shares no code with
the HIP library: the arithmetic lives in ``oracle.c`` (plain C, fp64 except
for the single-precision router definition), this file only marshals numpy
arrays.

Sources followed (page title, section):
  * "Three axes of Parallelism", Expert Parallel (EP) -> Producing assignments:
    router scores [T,E], top-K ids and router weights, the token-major
    assignment buffer, per-expert counts, offsets and the expert-major pack.
  * same page, Dispatch, expert computation and combine: the receive-side
    count matrix, the source-major -> expert-major reorder, E_local independent
    MLPs, and the weighted sum of the K expert outputs per token.
  * same page, Mapping experts to EP ranks: W_gate, W_val [E,d,f], W_out [E,f,d].
  * "feat(parallelism): expert parallelism for the Nemotron-3 Nano MoE layers",
    Design: the device-built permutation indices for the received buffer, and
    autograd through the index_select / index_copy permutation pair.
  * "Three axes of Parallelism", EP backward pass: expert gradients divided by
    the EP group size. The backward itself is the chain rule on the forward
    definitions (no page writes it out); see oracle.h.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

# The one build line of the oracle (also used by __graft_entry__.build()).
GCC_CMD = [
    "gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
    "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
    os.path.join(_HERE, "oracle.c"), "-o", _SO, "-lm",
]

_lib = None


def build():
    subprocess.run(GCC_CMD, check=True)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32p, i64p, f32p, f64p = (ctypes.c_void_p,) * 5
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_route.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.oracle_permute.argtypes = [vp, ctypes.c_int64, ctypes.c_int, vp, vp, vp, vp]
        L.oracle_permute_capacity.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                              vp, vp, vp, vp, vp]
        L.oracle_permute_range.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           vp, vp, vp, vp]
        L.oracle_permute_recv.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                          vp, vp, vp, vp]
        L.oracle_gather.argtypes = [vp, ctypes.c_int, ctypes.c_int64, vp, ctypes.c_int64,
                                    ctypes.c_int, vp]
        L.oracle_expert_ffn_rows.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                             ctypes.c_int64, ctypes.c_int, vp]
        L.oracle_expert_ffn_rows_h.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                               ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp]
        L.oracle_combine.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, vp, vp,
                                     vp, vp, vp, vp]
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_route_backward.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, vp]
        L.oracle_route_stats.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.oracle_router_grads.argtypes = [vp, vp, i32, i64, i32, i32, vp, vp, i64, vp, vp]
        L.oracle_combine_backward_gates.argtypes = [vp, i64, i32, i64, vp, vp, vp, vp, vp]
        L.oracle_combine_backward_rows.argtypes = [vp, vp, i64, i32, i64, vp, vp, vp]
        L.oracle_expert_ffn_backward_rows.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp,
                                                      vp, vp, i64, i32, vp, vp, vp, vp]
        L.oracle_expert_weight_grads.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp, vp,
                                                 vp, vp, vp, i64, ctypes.c_double, vp, vp, vp]
        L.oracle_expert_ffn_backward_rows_h.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp,
                                                        vp, vp, i64, i32, i32, vp, vp, vp, vp]
        L.oracle_expert_weight_grads_h.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp, vp,
                                                   vp, vp, vp, i64, ctypes.c_double, i32, vp, vp,
                                                   vp]
        L.oracle_round_bf16.argtypes = [vp, i64]
        for name in ("oracle_route", "oracle_permute", "oracle_permute_capacity",
                     "oracle_permute_range",
                     "oracle_permute_recv", "oracle_gather",
                     "oracle_expert_ffn_rows", "oracle_expert_ffn_rows_h", "oracle_combine",
                     "oracle_route_backward", "oracle_router_grads",
                     "oracle_combine_backward_gates", "oracle_combine_backward_rows",
                     "oracle_expert_ffn_backward_rows", "oracle_expert_weight_grads",
                     "oracle_expert_ffn_backward_rows_h", "oracle_expert_weight_grads_h",
                     "oracle_round_bf16",
                     "oracle_route_stats"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _xtype(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:  # bf16 bit patterns
        return 1
    raise TypeError(f"oracle takes fp32 or bf16-as-uint16 arrays, got {a.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _c(a, dtype=None):
    a = np.asarray(a)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


def route(x, w, bias, k: int, renorm: bool = True):
    """Router scores, top-k ids and router weights. Returns (logits fp32 [T,E],
    idx int32 [T,k], gates float64 [T,k])."""
    x, w = _c(x), _c(w)
    xt = _xtype(x)
    if _xtype(w) != xt:
        raise TypeError("x and w_router must have the same element type")
    T, d = x.shape
    d2, E = w.shape
    assert d == d2
    b = None if bias is None else _c(bias, np.float32)
    logits = np.empty((T, E), np.float32)
    idx = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float64)
    _check(lib().oracle_route(_p(x), _p(w), xt, _p(b), T, d, E, k, int(bool(renorm)),
                              _p(logits), _p(idx), _p(gates)), "oracle_route")
    return logits, idx, gates


def permute(idx, E: int):
    """Expert-major packing of the flat assignments. Returns
    (counts [E], offsets [E+1], perm_src [TK], dest [TK]), all int32."""
    flat = _c(np.asarray(idx).reshape(-1), np.int32)
    TK = flat.shape[0]
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_src = np.empty(TK, np.int32)
    dest = np.empty(TK, np.int32)
    _check(lib().oracle_permute(_p(flat), TK, E, _p(counts), _p(offsets), _p(perm_src),
                                _p(dest)), "oracle_permute")
    return counts, offsets, perm_src, dest


def permute_capacity(idx, E: int, capacity: int):
    """Fixed-capacity packing: each expert keeps its first ``capacity``
    assignments in ascending a = t*k+s. Returns (routed [E], counts [E],
    offsets [E+1], perm_src [kept], dest [TK]) int32; dest = -1 when dropped."""
    flat = _c(np.asarray(idx).reshape(-1), np.int32)
    TK = flat.shape[0]
    routed = np.empty(E, np.int32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_src = np.empty(max(TK, 1), np.int32)
    dest = np.empty(TK, np.int32)
    _check(lib().oracle_permute_capacity(_p(flat), TK, E, int(capacity), _p(routed), _p(counts),
                                         _p(offsets), _p(perm_src), _p(dest)),
           "oracle_permute_capacity")
    return routed, counts, offsets, perm_src[:int(offsets[E])].copy(), dest


def permute_range(idx, e_first: int, E_loc: int):
    """Packing of the expert range [e_first, e_first + E_loc) (one rank of the
    all-gather layout). Returns (counts [E_loc], offsets [E_loc+1],
    perm_src [kept], dest [TK]) int32; dest = -1 outside the range."""
    flat = _c(np.asarray(idx).reshape(-1), np.int32)
    TK = flat.shape[0]
    counts = np.empty(E_loc, np.int32)
    offsets = np.empty(E_loc + 1, np.int32)
    perm_src = np.empty(max(TK, 1), np.int32)
    dest = np.empty(TK, np.int32)
    _check(lib().oracle_permute_range(_p(flat), TK, int(e_first), int(E_loc), _p(counts),
                                      _p(offsets), _p(perm_src), _p(dest)),
           "oracle_permute_range")
    return counts, offsets, perm_src[:int(offsets[E_loc])].copy(), dest


def permute_recv(recv_counts, N: int):
    """Sender-major -> expert-major reorder of a received buffer of N rows."""
    recv = _c(recv_counts, np.int32)
    S, E_loc = recv.shape
    counts = np.empty(E_loc, np.int32)
    offsets = np.empty(E_loc + 1, np.int32)
    perm_src = np.empty(N, np.int32)
    dest = np.empty(N, np.int32)
    _check(lib().oracle_permute_recv(_p(recv), S, E_loc, N, _p(counts), _p(offsets),
                                     _p(perm_src), _p(dest)), "oracle_permute_recv")
    return counts, offsets, perm_src, dest


def gather(x, perm_src, k: int):
    """x_perm[j] = x[perm_src[j] // k] (bitwise row copy)."""
    x = _c(x)
    ps = _c(perm_src, np.int32)
    rows = ps.shape[0]
    out = np.empty((rows,) + x.shape[1:], x.dtype)
    d = int(np.prod(x.shape[1:]))
    _check(lib().oracle_gather(_p(x), x.dtype.itemsize, d, _p(ps), rows, k, _p(out)),
           "oracle_gather")
    return out


def expert_ffn_rows(x_perm, offsets, wg, wv, wo, rows=None, N=None, round_h=False):
    """SwiGLU expert MLPs evaluated in double on the listed packed rows
    (all rows if None). Returns float64 [len(rows), d]. With ``N`` given,
    ``x_perm`` holds only the listed rows (row r = packed row rows[r]) of a
    packed buffer of N rows. ``round_h``: the hidden activations are rounded
    once to bf16 before the down product (their storage point for bf16 data
    with fp32 accumulation); otherwise everything is exact."""
    x_perm, wg, wv, wo = _c(x_perm), _c(wg), _c(wv), _c(wo)
    xt = _xtype(x_perm)
    for w in (wg, wv, wo):
        if _xtype(w) != xt:
            raise TypeError("activations and expert weights must share an element type")
    compact = N is not None
    if not compact:
        N = x_perm.shape[0]
    d = x_perm.shape[1]
    E, d2, f = wg.shape
    assert d2 == d and wv.shape == wg.shape and wo.shape == (E, f, d)
    off = _c(offsets, np.int32)
    assert off.shape == (E + 1,)
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    if compact:
        assert x_perm.shape[0] == rows.shape[0]
    y = np.empty((rows.shape[0], d), np.float64)
    _check(lib().oracle_expert_ffn_rows_h(_p(x_perm), xt, N, d, f, E, _p(off), _p(wg), _p(wv),
                                          _p(wo), _p(rows), rows.shape[0], int(compact),
                                          int(bool(round_h)), _p(y)),
           "oracle_expert_ffn_rows_h")
    return y


def combine(tokens, k: int, dest, gates, y, yrow=None, shared=None):
    """out[r] = sum_s gates[t,s] * y[dest[t*k+s]] (+ shared[r]), t = tokens[r],
    in double. gates None = weight 1; yrow maps packed rows to rows of y."""
    tokens = _c(tokens, np.int32)
    dest = _c(np.asarray(dest).reshape(-1), np.int32)
    g = None if gates is None else _c(np.asarray(gates).reshape(-1), np.float64)
    y = _c(y, np.float64)
    yr = None if yrow is None else _c(yrow, np.int64)
    sh = None if shared is None else _c(shared, np.float64)
    d = y.shape[1]
    out = np.empty((tokens.shape[0], d), np.float64)
    _check(lib().oracle_combine(_p(tokens), tokens.shape[0], k, d, _p(dest), _p(g), _p(y),
                                _p(yr), _p(sh), _p(out)), "oracle_combine")
    return out


def swiglu_shared(x, wg, wv, wo, rows=None, round_h=False):
    """Sum of always-on shared experts on token rows: sum_q SwiGLU_q(x[t]),
    in double, q ascending. wg/wv [Q,d,f], wo [Q,f,d]."""
    x = _c(x)
    T = x.shape[0]
    rows = np.arange(T, dtype=np.int64) if rows is None else _c(rows, np.int64)
    total = None
    for q in range(wg.shape[0]):
        part = expert_ffn_rows(x, np.array([0, T], np.int32), wg[q:q + 1], wv[q:q + 1],
                               wo[q:q + 1], rows, round_h=round_h)
        total = part if total is None else total + part
    return total


def moe_layer(inp: dict, tokens=None, capacity=None, round_h=False):
    """The whole layer on a token-routed workload dict (see
    expert_dispatch_amd.workloads). Returns a dict of every intermediate.
    With ``tokens`` given, only the packed rows those tokens need are
    gathered and run through the expert MLPs, and only those tokens are
    combined; ``x_perm`` then holds the rows listed in ``y_rows``. With
    ``capacity`` given, the packing keeps at most that many assignments per
    expert (see permute_capacity); ``routed`` then holds the counts before
    the cap. ``round_h``: the hidden activations rounded to bf16 at their
    storage point (see expert_ffn_rows)."""
    k = inp["k"]
    logits, idx, gates = route(inp["x"], inp["w_router"], inp.get("bias"), k,
                               inp.get("renorm", True))
    E = inp["w_gate"].shape[0]
    if capacity is None:
        counts, offsets, perm_src, dest = permute(idx, E)
        routed = counts
    else:
        routed, counts, offsets, perm_src, dest = permute_capacity(idx, E, capacity)
    T = inp["x"].shape[0]
    kept = int(offsets[E])
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    if tokens is None:
        need = np.arange(kept, dtype=np.int64)
        x_perm = gather(inp["x"], perm_src, k)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"],
                                 round_h=round_h)
    else:
        need = np.unique(dest.reshape(T, k)[tok].reshape(-1)).astype(np.int64)
        need = need[need >= 0]
        x_perm = gather(inp["x"], perm_src[need], k)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"],
                                 need, N=kept, round_h=round_h)
    yrow = np.full(max(kept, 1), -1, np.int64)
    yrow[need] = np.arange(need.shape[0])
    shared = None
    if inp.get("shared_w_gate") is not None:
        shared = swiglu_shared(inp["x"], inp["shared_w_gate"], inp["shared_w_val"],
                               inp["shared_w_out"], tok.astype(np.int64), round_h=round_h)
    out = combine(tok, k, dest, gates, y_rows, yrow, shared)
    return dict(logits=logits, idx=idx, gates=gates, counts=counts, routed=routed,
                offsets=offsets, perm_src=perm_src, dest=dest, x_perm=x_perm, y_rows=need,
                y=y_rows, shared=shared, tokens=tok, out=out)


def moe_partial_layer(inp: dict, e_first: int, tokens=None, round_h=False):
    """One rank of the all-gather / reduce-scatter layout on a gathered-token
    workload: the replicated router over every token, the rank's local experts
    (inp["w_gate"] etc. hold them, global ids e_first..) over the assignments
    routed to them, and the combine into this rank's partial output (the
    reduce-scatter then sums the partials of all ranks). ``round_h`` as in
    moe_layer."""
    k = inp["k"]
    logits, idx, gates = route(inp["x"], inp["w_router"], inp.get("bias"), k,
                               inp.get("renorm", True))
    E_loc = inp["w_gate"].shape[0]
    counts, offsets, perm_src, dest = permute_range(idx, e_first, E_loc)
    T = inp["x"].shape[0]
    kept = int(offsets[E_loc])
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    if tokens is None:
        need = np.arange(kept, dtype=np.int64)
        x_perm = gather(inp["x"], perm_src, k)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"],
                                 round_h=round_h)
    else:
        need = np.unique(dest.reshape(T, k)[tok].reshape(-1)).astype(np.int64)
        need = need[need >= 0]
        x_perm = gather(inp["x"], perm_src[need], k)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"],
                                 need, N=kept, round_h=round_h)
    yrow = np.full(max(kept, 1), -1, np.int64)
    yrow[need] = np.arange(need.shape[0])
    out = combine(tok, k, dest, gates, y_rows, yrow, None)
    return dict(logits=logits, idx=idx, gates=gates, counts=counts, offsets=offsets,
                perm_src=perm_src, dest=dest, x_perm=x_perm, y_rows=need, y=y_rows,
                tokens=tok, out=out)


def moe_recv_layer(inp: dict, rows=None):
    """One EP rank's receive side: reorder, expert MLPs, unweighted un-permute
    back to sender-major order. ``rows`` restricts the evaluated received rows
    (``x_perm`` then holds the packed rows listed in ``y_rows``)."""
    N = inp["x_recv"].shape[0]
    counts, offsets, perm_src, dest = permute_recv(inp["recv_counts"], N)
    r = np.arange(N, dtype=np.int32) if rows is None else _c(rows, np.int32)
    if rows is None:
        need = np.arange(N, dtype=np.int64)
        x_perm = gather(inp["x_recv"], perm_src, 1)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"])
    else:
        need = np.unique(dest[r]).astype(np.int64)
        x_perm = gather(inp["x_recv"], perm_src[need], 1)
        y_rows = expert_ffn_rows(x_perm, offsets, inp["w_gate"], inp["w_val"], inp["w_out"],
                                 need, N=N)
    yrow = np.full(N, -1, np.int64)
    yrow[need] = np.arange(need.shape[0])
    out = combine(r, 1, dest, None, y_rows, yrow, None)
    return dict(counts=counts, offsets=offsets, perm_src=perm_src, dest=dest, x_perm=x_perm,
                y_rows=need, y=y_rows, rows=r, out=out)


# ------------------------------------------------------------------ backward

def widen(a) -> np.ndarray:
    """fp32 or bf16-bit-pattern (uint16) array -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def route_backward(logits, idx, gates, d_gates, renorm: bool = True):
    """d_logits [T,E] float64 from the router-weight gradients d_gates [T,k]."""
    logits = _c(logits, np.float32)
    idx = _c(idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    g = _c(gates, np.float64)
    dg = _c(d_gates, np.float64)
    out = np.empty((T, E), np.float64)
    _check(lib().oracle_route_backward(_p(logits), _p(idx), _p(g), _p(dg), T, E, k,
                                       int(bool(renorm)), _p(out)), "oracle_route_backward")
    return out


def router_grads(x, w, d_logits, want_dx=True, want_dw=True):
    """(d_x [T,d], d_w [d,E]) of the router scores, float64; x holds the
    tokens d_logits belongs to (row for row)."""
    x, w = _c(x), _c(w)
    xt = _xtype(x)
    T, d = x.shape
    E = w.shape[1]
    dl = _c(d_logits, np.float64)
    assert dl.shape == (T, E)
    tok = np.arange(T, dtype=np.int32)
    dx = np.empty((T, d), np.float64) if want_dx else None
    dw = np.empty((d, E), np.float64) if want_dw else None
    _check(lib().oracle_router_grads(_p(x), _p(w), xt, T, d, E, _p(dl), _p(tok), T, _p(dx),
                                     _p(dw)), "oracle_router_grads")
    return dx, dw


def combine_backward_gates(tokens, k: int, dest, y, yrow, d_out_rows):
    tokens = _c(tokens, np.int32)
    dest = _c(np.asarray(dest).reshape(-1), np.int32)
    y = _c(y, np.float64)
    yr = None if yrow is None else _c(yrow, np.int64)
    do = _c(d_out_rows, np.float64)
    d = do.shape[1]
    out = np.empty((tokens.shape[0], k), np.float64)
    _check(lib().oracle_combine_backward_gates(_p(tokens), tokens.shape[0], k, d, _p(dest),
                                               _p(y), _p(yr), _p(do), _p(out)),
           "oracle_combine_backward_gates")
    return out


def combine_backward_rows(perm_src, rows, k: int, gates, d_out):
    ps = _c(perm_src, np.int32)
    rows = _c(rows, np.int64)
    g = None if gates is None else _c(np.asarray(gates).reshape(-1), np.float64)
    do = _c(d_out, np.float64)
    d = do.shape[1]
    out = np.empty((rows.shape[0], d), np.float64)
    _check(lib().oracle_combine_backward_rows(_p(ps), _p(rows), rows.shape[0], k, d, _p(g),
                                              _p(do), _p(out)), "oracle_combine_backward_rows")
    return out


# storage points of bf16 training (oracle.h ORACLE_STORE_*)
STORE_DY, STORE_ACT, STORE_DACT, STORE_DX = 1, 2, 4, 8


def round_bf16(a) -> np.ndarray:
    """float64 copy of ``a`` with every value rounded once to bf16 (to
    nearest, ties to even)."""
    out = np.array(a, dtype=np.float64, copy=True, order="C")
    _check(lib().oracle_round_bf16(_p(out), out.size), "oracle_round_bf16")
    return out


def expert_ffn_backward_rows(x_perm, offsets, wg, wv, wo, d_y, rows=None, N=None, store=0):
    """(act, d_act, d_x) of the listed packed rows, float64: act = [a | v]
    [n,2f], d_act = [da | dv] [n,2f], d_x [n,d]. ``rows`` and ``N`` as in
    expert_ffn_rows; d_y [n,d] the rows' output gradients. ``store``: an OR
    of STORE_* (the values rounded to bf16 at those storage points)."""
    x_perm, wg, wv, wo = _c(x_perm), _c(wg), _c(wv), _c(wo)
    xt = _xtype(x_perm)
    compact = N is not None
    if not compact:
        N = x_perm.shape[0]
    d = x_perm.shape[1]
    E, _, f = wg.shape
    off = _c(offsets, np.int32)
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    dy = _c(d_y, np.float64)
    n = rows.shape[0]
    act = np.empty((n, 2 * f), np.float64)
    dact = np.empty((n, 2 * f), np.float64)
    dx = np.empty((n, d), np.float64)
    _check(lib().oracle_expert_ffn_backward_rows_h(_p(x_perm), xt, N, d, f, E, _p(off), _p(wg),
                                                   _p(wv), _p(wo), _p(rows), n, int(compact),
                                                   int(store), _p(dy), _p(act), _p(dact),
                                                   _p(dx)),
           "oracle_expert_ffn_backward_rows_h")
    return act, dact, dx


def expert_weight_grads(x_perm, offsets, wg, wv, wo, d_y, pairs, scale: float = 1.0, store=0):
    """Weight gradients of the listed (expert, hidden column) pairs:
    (dWg[e][:,c], dWv[e][:,c], dWo[e][c,:]), each float64 [P,d]. x_perm and
    d_y hold every packed row."""
    x_perm, wg, wv, wo = _c(x_perm), _c(wg), _c(wv), _c(wo)
    xt = _xtype(x_perm)
    N, d = x_perm.shape
    E, _, f = wg.shape
    off = _c(offsets, np.int32)
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    pe = _c(pairs[:, 0], np.int32)
    pc = _c(pairs[:, 1], np.int32)
    P = pe.shape[0]
    dy = _c(d_y, np.float64)
    assert dy.shape == (N, d)
    outs = [np.empty((P, d), np.float64) for _ in range(3)]
    _check(lib().oracle_expert_weight_grads_h(_p(x_perm), xt, N, d, f, E, _p(off), _p(wg),
                                              _p(wv), _p(wo), _p(dy), _p(pe), _p(pc), P,
                                              float(scale), int(store), *(_p(o) for o in outs)),
           "oracle_expert_weight_grads_h")
    return tuple(outs)


def all_pairs(E: int, f: int) -> np.ndarray:
    """Every (expert, hidden column) pair, expert-major."""
    e, c = np.meshgrid(np.arange(E), np.arange(f), indexing="ij")
    return np.stack([e.reshape(-1), c.reshape(-1)], axis=1)


def moe_backward(inp: dict, d_out, tokens=None, pairs=None, scale: float = 1.0,
                 capacity=None, e_first=None, store_bf16=False):
    """Gradients of the loss L = sum(out * d_out) through the layer (or, with
    ``e_first``, through one rank's partial output), in double.

    With ``tokens`` None every token is evaluated: d_x [T,d], d_gates [T,k],
    d_logits [T,E] and the router weight gradient d_w_router [d,E]. With
    ``tokens`` given only those tokens' input and router gradients are formed
    (from the packed rows they use, listed in ``y_rows``); d_w_router is then
    None. ``pairs`` lists (expert, hidden column) pairs whose expert weight
    gradients are formed over all packed rows (all_pairs(E, f) for all of
    them), multiplied by ``scale``. Shared experts, where the workload has
    them, add their input gradient to d_x; their weight gradients are the
    same functions on the token rows (expert_weight_grads with offsets [0,T]).

    ``store_bf16``: the chain as bf16 training hands values between its
    kernels, every value rounded once to bf16 at those storage points (the
    forward's h; the backward's d_y, the kept pre-activations a and v, their
    gradients da and dv, the packed rows' input gradients, and the logit
    gradients that the router weight gradient's product reads); all sums
    exact. Otherwise every value is exact."""
    k = inp["k"]
    renorm = inp.get("renorm", True)
    x = inp["x"]
    T = x.shape[0]
    logits, idx, gates = route(x, inp["w_router"], inp.get("bias"), k, renorm)
    E = inp["w_gate"].shape[0]
    if e_first is not None:
        counts, offsets, perm_src, dest = permute_range(idx, e_first, E)
    elif capacity is not None:
        _, counts, offsets, perm_src, dest = permute_capacity(idx, E, capacity)
    else:
        counts, offsets, perm_src, dest = permute(idx, E)
    kept = int(offsets[E])
    dout = widen(d_out)
    full = tokens is None
    tok = np.arange(T, dtype=np.int32) if full else _c(tokens, np.int32)
    if full:
        need = np.arange(kept, dtype=np.int64)
    else:
        need = np.unique(dest.reshape(T, k)[tok].reshape(-1)).astype(np.int64)
        need = need[need >= 0]
    wg, wv, wo = inp["w_gate"], inp["w_val"], inp["w_out"]
    xp = gather(x, perm_src[need], k)
    y = expert_ffn_rows(xp, offsets, wg, wv, wo, need, N=kept, round_h=store_bf16)
    yrow = np.full(max(kept, 1), -1, np.int64)
    yrow[need] = np.arange(need.shape[0])
    # combine: out[t] = sum_s g[t,s] y[dest[t,s]]
    d_gates = combine_backward_gates(tok, k, dest, y, yrow, dout[tok])
    d_y = combine_backward_rows(perm_src, need, k, gates, dout)
    routed_store = (STORE_DY | STORE_ACT | STORE_DACT | STORE_DX) if store_bf16 else 0
    act, d_act, d_xp = expert_ffn_backward_rows(xp, offsets, wg, wv, wo, d_y, need, N=kept,
                                                store=routed_store)
    if store_bf16:
        d_y = round_bf16(d_y)
    # the packing's backward: each token sums the input gradients of its rows
    d_x = combine(tok, k, dest, None, d_xp, yrow)
    # router
    d_logits = route_backward(logits[tok], idx[tok], gates[tok], d_gates, renorm)
    dxr, _ = router_grads(x[tok], inp["w_router"], d_logits, True, False)
    dwr = None
    if full:
        _, dwr = router_grads(x[tok], inp["w_router"],
                              round_bf16(d_logits) if store_bf16 else d_logits, False, True)
    d_x += dxr
    if inp.get("shared_w_gate") is not None:
        sg, sv, so = inp["shared_w_gate"], inp["shared_w_val"], inp["shared_w_out"]
        for q in range(sg.shape[0]):
            _, _, dxs = expert_ffn_backward_rows(x, np.array([0, T], np.int32), sg[q:q + 1],
                                                 sv[q:q + 1], so[q:q + 1], dout[tok],
                                                 tok.astype(np.int64),
                                                 store=(STORE_DY | STORE_ACT | STORE_DACT)
                                                 if store_bf16 else 0)
            d_x += dxs
    res = dict(logits=logits, idx=idx, gates=gates, counts=counts, offsets=offsets,
               perm_src=perm_src, dest=dest, tokens=tok, y_rows=need, y=y, d_y=d_y, act=act,
               d_act=d_act, d_x_perm=d_xp, d_gates=d_gates, d_logits=d_logits, d_x=d_x,
               d_w_router=dwr)
    if pairs is not None:
        xall = gather(x, perm_src, k)
        dyall = combine_backward_rows(perm_src, np.arange(kept, dtype=np.int64), k, gates, dout)
        res["pairs"] = np.asarray(pairs, np.int64).reshape(-1, 2)
        res["d_w_gate"], res["d_w_val"], res["d_w_out"] = expert_weight_grads(
            xall, offsets, wg, wv, wo, dyall, res["pairs"], scale,
            store=(STORE_DY | STORE_ACT | STORE_DACT) if store_bf16 else 0)
    return res


def route_stats(logits, counts, k: int):
    """(p_mean [E] float64, aux float): mean full-softmax probability per expert
    and the load-balance statistic E * sum_e (counts_e / (T*k)) * p_mean_e."""
    logits = _c(logits, np.float32)
    counts = _c(counts, np.int32)
    T, E = logits.shape
    pm = np.empty(E, np.float64)
    aux = np.empty(1, np.float64)
    _check(lib().oracle_route_stats(_p(logits), _p(counts), T, E, k, _p(pm), _p(aux)),
           "oracle_route_stats")
    return pm, float(aux[0])
