"""Thin Python binding of libmoe (include/moe.h) over PyTorch device tensors.

Argument marshalling only: every step runs in the HIP library. PyTorch
provides device memory and the current stream. If ``libmoe.so`` has not been
built the first call raises; there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported before libmoe so that both share torch's HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
_lib = None

MOE_F32, MOE_BF16 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def debug_lib_path() -> str:
    """The MOE_DEBUG build (device precondition checks; tests only)."""
    return os.path.join(os.path.dirname(_LIB_PATH), "libmoe_debug.so")


def lib():
    """Open libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = bind(_LIB_PATH)
    return _lib


def bind(path: str):
    """Open a build of libmoe at `path` and declare its entry points."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m expert_dispatch_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [i]
    L.moe_version.restype = i
    L.moe_x_perm_ld.restype = i
    L.moe_x_perm_ld.argtypes = [i, i]
    sigs = {
        "moe_route": [vp, i, vp, vp, i, i, i, i, i, vp, vp, vp, vp],
        "moe_permute": [vp, i, i, i, vp, i, i, vp, vp, vp, vp, vp, i, vp, sz, vp],
        "moe_permute_noalloc": [vp, i, i, i, vp, i, i, vp, vp, vp, vp, vp, i, vp],
        "moe_permute_capacity": [vp, i, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp, i, vp, sz,
                                 vp],
        "moe_permute_range": [vp, i, i, i, i, vp, i, i, vp, vp, vp, vp, vp, i, vp, sz, vp],
        "moe_permute_recv": [vp, i, i, i, vp, i, i, vp, vp, vp, vp, vp, i, vp, sz, vp],
        "moe_grouped_ffn": [vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, i, vp, sz, vp],
        "moe_ffn_gate_up": [vp, i, i, i, i, i, i, vp, vp, vp, vp, vp],
        "moe_ffn_down": [vp, i, i, i, i, i, vp, vp, vp, i, vp],
        "moe_combine": [vp, i, vp, vp, i, i, i, vp, i, vp, i, vp],
        "moe_ffn_gate_up_train": [vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp],
        "moe_combine_backward": [vp, i, vp, i, vp, vp, i, i, i, vp, i, vp, vp],
        "moe_ffn_down_backward": [vp, i, i, i, i, i, vp, vp, vp, vp, vp],
        "moe_ffn_gate_up_backward": [vp, i, i, i, i, i, vp, vp, vp, vp, i, i, vp],
        "moe_ffn_weight_grads": [vp, i, vp, vp, vp, i, i, i, i, i, vp, ctypes.c_float, vp, vp,
                                 vp, vp],
        "moe_route_backward": [vp, vp, vp, vp, i, i, i, i, vp, vp, vp],
        "moe_router_backward": [vp, vp, i, vp, i, i, i, vp, i, vp, vp, sz, vp],
        "moe_route_stats": [vp, vp, i, i, i, vp, vp, vp, sz, vp],
        "moe_token_backward": [vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = i
    # measurement helpers (include/moe_ceiling.h)
    L.moe_ceiling_mfma.argtypes = [i, i, vp, vp]
    L.moe_ceiling_mfma.restype = ctypes.c_longlong
    L.moe_ceiling_copy.argtypes = [vp, vp, ctypes.c_longlong, i, vp]
    L.moe_ceiling_copy.restype = i
    L.moe_ceiling_read.argtypes = [vp, ctypes.c_longlong, vp, i, vp]
    L.moe_ceiling_read.restype = i
    for name, args in {"moe_permute_workspace": [i, i, i],
                       "moe_permute_recv_workspace": [i, i, i],
                       "moe_grouped_ffn_workspace": [i, i, i, i, i],
                       "moe_router_backward_workspace": [i, i, i],
                       "moe_route_stats_workspace": [i, i],
                       "moe_token_backward_workspace": [i, i, i]}.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = sz
    L.moe_debug_status.argtypes = [vp, i]
    L.moe_debug_status.restype = i
    return L


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dt_of(dtype: torch.dtype) -> int:
    return MOE_BF16 if dtype == torch.bfloat16 else MOE_F32


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D device tensor whose rows are contiguous
    (packed rows may sit in a wider buffer: x_perm = buf[:, :d])."""
    if not t.is_cuda or t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1) \
            or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be a 2-D device tensor with contiguous rows")
    return int(t.stride(0))


def x_perm_ld(d: int, dtype) -> int:
    """The library's recommended row stride for packed rows of width d."""
    return int(lib().moe_x_perm_ld(d, _dt_of(dtype)))


def empty_rows(rows: int, d: int, dtype, device) -> torch.Tensor:
    """[rows, d] view of a [rows, x_perm_ld(d)] buffer: packed rows laid out
    with the recommended padded stride."""
    ld = x_perm_ld(d, dtype)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :d]


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def route(x, w_router, bias, k: int, renorm: bool = True, *, out=None, stream=None):
    """Router scores, top-k ids and router weights."""
    _dev(x, "x"); _dev(w_router, "w_router")
    T, d = x.shape
    E = w_router.shape[1]
    if out is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        gates = torch.empty((T, k), dtype=torch.float32, device=x.device)
    else:
        logits, idx, gates = out
    _check("moe_route", lib().moe_route(_p(x), _dt(x), _p(w_router), _p(bias), T, d, E, k,
                                        int(bool(renorm)), _p(logits), _p(idx), _p(gates),
                                        _stream(stream)))
    return logits, idx, gates


def route_stats_workspace(T: int, E: int) -> int:
    return int(lib().moe_route_stats_workspace(T, E))


def route_stats(logits, counts, k: int, *, out=None, workspace=None, stream=None):
    """(p_mean [E] fp32, aux [1] fp32): the mean full-softmax probability of
    every expert and the load-balance statistic E * sum_e (counts_e/(T*k)) p_mean_e."""
    _dev(logits, "logits"); _dev(counts, "counts")
    T, E = logits.shape
    if out is None:
        out = (torch.empty(E, dtype=torch.float32, device=logits.device),
               torch.empty(1, dtype=torch.float32, device=logits.device))
    p_mean, aux = out
    ws = workspace
    if ws is None:
        ws = torch.empty(max(1, route_stats_workspace(T, E)), dtype=torch.uint8,
                         device=logits.device)
    _check("moe_route_stats", lib().moe_route_stats(
        _p(logits), _p(counts), T, E, k, _p(p_mean), _p(aux), _p(ws), ws.numel(),
        _stream(stream)))
    return p_mean, aux


def permute_workspace(T: int, k: int, E: int) -> int:
    return int(lib().moe_permute_workspace(T, k, E))


def permute(topk_idx, x, E: int, *, capacity=None, e_first=None, out=None, workspace=None,
            stream=None):
    """Expert-major packing. Returns dict(counts, offsets, perm_src, dest, x_perm);
    with ``capacity`` (fixed-capacity packing) also ``routed``, the counts
    before the cap. With ``e_first`` only global experts [e_first, e_first + E)
    are packed (one rank of the all-gather layout)."""
    _dev(topk_idx, "topk_idx"); _dev(x, "x")
    T, k = topk_idx.shape
    d = x.shape[1]
    dev = x.device
    if out is None:
        out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   perm_src=torch.empty(T * k, dtype=torch.int32, device=dev),
                   dest=torch.empty(T * k, dtype=torch.int32, device=dev),
                   x_perm=empty_rows(T * k, d, x.dtype, dev))
        if capacity is not None:
            out["routed"] = torch.empty(E, dtype=torch.int32, device=dev)
    ldx = _rows(out["x_perm"], "x_perm")
    nbytes = permute_workspace(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if e_first is not None:
        _check("moe_permute_range", lib().moe_permute_range(
            _p(topk_idx), T, k, int(e_first), E, _p(x), _dt(x), d, _p(out["counts"]),
            _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]), ldx,
            _p(workspace), workspace.numel(), _stream(stream)))
    elif capacity is None:
        _check("moe_permute", lib().moe_permute(
            _p(topk_idx), T, k, E, _p(x), _dt(x), d, _p(out["counts"]), _p(out["offsets"]),
            _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]), ldx, _p(workspace),
            workspace.numel(), _stream(stream)))
    else:
        _check("moe_permute_capacity", lib().moe_permute_capacity(
            _p(topk_idx), T, k, E, int(capacity), _p(x), _dt(x), d, _p(out.get("routed")),
            _p(out["counts"]), _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]),
            _p(out["x_perm"]), ldx, _p(workspace), workspace.numel(), _stream(stream)))
    return out


def permute_recv(recv_counts, x_recv, *, out=None, stream=None):
    """Receive-side reorder (sender-major -> expert-major) of N = len(x_recv) rows."""
    _dev(recv_counts, "recv_counts"); _dev(x_recv, "x_recv")
    S, E_loc = recv_counts.shape
    N, d = x_recv.shape
    dev = x_recv.device
    if out is None:
        out = dict(counts=torch.empty(E_loc, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E_loc + 1, dtype=torch.int32, device=dev),
                   perm_src=torch.empty(N, dtype=torch.int32, device=dev),
                   dest=torch.empty(N, dtype=torch.int32, device=dev),
                   x_perm=empty_rows(N, d, x_recv.dtype, dev))
    ldx = _rows(out["x_perm"], "x_perm")
    _check("moe_permute_recv", lib().moe_permute_recv(
        _p(recv_counts), S, E_loc, N, _p(x_recv), _dt(x_recv), d, _p(out["counts"]),
        _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]), ldx, None,
        0, _stream(stream)))
    return out


def grouped_ffn_workspace(N: int, d: int, f: int, E: int, dtype) -> int:
    return int(lib().moe_grouped_ffn_workspace(N, d, f, E, _dt_of(dtype)))


def _offsets(offsets, E: int):
    """Device offsets [E+1], or None: one group of all rows (E must be 1)."""
    if offsets is None:
        if E != 1:
            raise ValueError("offsets may be None only for a single expert (E = 1)")
        return
    _dev(offsets, "offsets")


def grouped_ffn(x_perm, offsets, w_gate, w_val, w_out, *, y_dtype=torch.float32, y=None,
                workspace=None, stream=None):
    """y[j] = (silu(x_perm[j] W_gate[e]) * (x_perm[j] W_val[e])) W_out[e] per expert segment
    (offsets None: one expert over all rows)."""
    for t, n in ((w_gate, "w_gate"), (w_val, "w_val"), (w_out, "w_out")):
        _dev(t, n)
    _offsets(offsets, w_gate.shape[0])
    ldx = _rows(x_perm, "x_perm")
    N, d = x_perm.shape
    E, _, f = w_gate.shape
    if y is None:
        y = torch.empty((N, d), dtype=y_dtype, device=x_perm.device)
    nbytes = grouped_ffn_workspace(N, d, f, E, x_perm.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x_perm.device)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _p(x_perm), ldx, _dt(x_perm), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(w_out),
        _p(y), _dt(y), _p(workspace), workspace.numel(), _stream(stream)))
    return y


def ffn_gate_up(x_perm, offsets, w_gate, w_val, *, h=None, stream=None):
    """h = silu(x_perm W_gate[e]) * (x_perm W_val[e]) per expert segment."""
    for t, n in ((w_gate, "w_gate"), (w_val, "w_val")):
        _dev(t, n)
    _offsets(offsets, w_gate.shape[0])
    ldx = _rows(x_perm, "x_perm")
    N, d = x_perm.shape
    E, _, f = w_gate.shape
    if h is None:
        h = torch.empty((N, f), dtype=x_perm.dtype, device=x_perm.device)
    _check("moe_ffn_gate_up", lib().moe_ffn_gate_up(
        _p(x_perm), ldx, _dt(x_perm), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(h),
        _stream(stream)))
    return h


def ffn_down(h, offsets, w_out, *, y_dtype=torch.float32, y=None, stream=None):
    """y = h W_out[e] per expert segment."""
    for t, n in ((h, "h"), (w_out, "w_out")):
        _dev(t, n)
    _offsets(offsets, w_out.shape[0])
    N, f = h.shape
    E, _, d = w_out.shape
    if y is None:
        y = torch.empty((N, d), dtype=y_dtype, device=h.device)
    _check("moe_ffn_down", lib().moe_ffn_down(
        _p(h), _dt(h), N, f, d, E, _p(offsets), _p(w_out), _p(y), _dt(y), _stream(stream)))
    return y


def combine(y_perm, dest, gates, k: int, *, y_shared=None, out_dtype=torch.float32, out=None,
            stream=None):
    """out[t] = sum_s gates[t,s] * y_perm[dest[t*k+s]] (+ y_shared[t])."""
    _dev(y_perm, "y_perm"); _dev(dest, "dest")
    TK = dest.numel()
    T = TK // k
    d = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y_perm.device)
    sh_dt = _dt(y_shared) if y_shared is not None else MOE_F32
    _check("moe_combine", lib().moe_combine(
        _p(y_perm), _dt(y_perm), _p(dest), _p(gates), T, k, d, _p(y_shared), sh_dt, _p(out),
        _dt(out), _stream(stream)))
    return out


def moe_partial_layer(x, w_router, bias, k: int, e_first: int, w_gate, w_val, w_out, *,
                      y_dtype=torch.float32, out_dtype=torch.float32, stream=None):
    """One rank of the all-gather / reduce-scatter layout: the replicated router
    over the gathered tokens, the rank's local experts (global ids e_first..,
    weights w_gate etc.), the combine into this rank's partial output."""
    E_loc = w_gate.shape[0]
    logits, idx, gates = route(x, w_router, bias, k, stream=stream)
    p = permute(idx, x, E_loc, e_first=e_first, stream=stream)
    y = grouped_ffn(p["x_perm"], p["offsets"], w_gate, w_val, w_out, y_dtype=y_dtype,
                    stream=stream)
    out = combine(y, p["dest"], gates, k, out_dtype=out_dtype, stream=stream)
    return dict(logits=logits, idx=idx, gates=gates, y=y, out=out, **p)


def layer_buffers(T: int, k: int, d: int, f: int, E: int, dtype, device, *, shared_f: int = 0,
                  capacity: bool = False, y_dtype=torch.float32, out_dtype=torch.float32) -> dict:
    """Every output and workspace of one moe_layer pass, allocated once, so
    that later passes allocate nothing (a caller that captures the layer in
    a HIP graph passes them as ``bufs``). ``shared_f``: width of the fused
    shared-expert SwiGLU (0: none)."""
    rows = T * k
    i32 = torch.int32
    b = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=device),
        idx=torch.empty((T, k), dtype=i32, device=device),
        gates=torch.empty((T, k), dtype=torch.float32, device=device),
        counts=torch.empty(E, dtype=i32, device=device),
        offsets=torch.empty(E + 1, dtype=i32, device=device),
        perm_src=torch.empty(rows, dtype=i32, device=device),
        dest=torch.empty(rows, dtype=i32, device=device),
        x_perm=empty_rows(rows, d, dtype, device),
        permute_ws=torch.empty(max(1, permute_workspace(T, k, E)), dtype=torch.uint8,
                               device=device),
        ffn_ws=torch.empty(max(1, grouped_ffn_workspace(rows, d, f, E, dtype)),
                           dtype=torch.uint8, device=device),
        y=torch.empty((rows, d), dtype=y_dtype, device=device),
        out=torch.empty((T, d), dtype=out_dtype, device=device),
    )
    if capacity:
        b["routed"] = torch.empty(E, dtype=i32, device=device)
    if shared_f:
        b["shared_ws"] = torch.empty(max(1, grouped_ffn_workspace(T, d, shared_f, 1, dtype)),
                                     dtype=torch.uint8, device=device)
        b["y_shared"] = torch.empty((T, d), dtype=y_dtype, device=device)
    return b


def moe_layer(x, w_router, bias, k: int, w_gate, w_val, w_out, *, shared=None, capacity=None,
              y_dtype=torch.float32, out_dtype=torch.float32, bufs=None, stream=None):
    """The whole token-routed layer: route -> permute -> grouped FFN -> combine.
    ``shared`` = (w_gate, w_val, w_out) of the always-on shared experts
    concatenated along f (one SwiGLU of width q*f equals the sum of q).
    ``y_dtype`` is the storage type of the expert outputs between the down
    GEMM and the combine. ``capacity``: fixed-capacity packing (at most that
    many rows per expert; dropped assignments add nothing to their token).
    ``bufs``: outputs and workspaces from layer_buffers (then nothing is
    allocated and the dtypes are the buffers'); every call only enqueues
    work on the stream, none waits for the device."""
    E = w_gate.shape[0]
    if bufs is None:
        T, d = x.shape
        bufs = layer_buffers(T, k, d, w_gate.shape[2], E, x.dtype, x.device,
                             shared_f=0 if shared is None else shared[0].shape[2],
                             capacity=capacity is not None, y_dtype=y_dtype,
                             out_dtype=out_dtype)
    b = bufs
    logits, idx, gates = route(x, w_router, bias, k, out=(b["logits"], b["idx"], b["gates"]),
                               stream=stream)
    p = permute(idx, x, E, capacity=capacity, out=b, workspace=b["permute_ws"], stream=stream)
    y = grouped_ffn(p["x_perm"], p["offsets"], w_gate, w_val, w_out, y=b["y"],
                    workspace=b["ffn_ws"], stream=stream)
    y_sh = None
    if shared is not None:
        # one group of all T tokens: offsets NULL
        y_sh = grouped_ffn(x, None, *shared, y=b["y_shared"], workspace=b["shared_ws"],
                           stream=stream)
    out = combine(y, p["dest"], gates, k, y_shared=y_sh, out=b["out"], stream=stream)
    res = {key: b[key] for key in ("counts", "offsets", "perm_src", "dest", "x_perm")}
    if "routed" in b:
        res["routed"] = b["routed"]
    return dict(logits=logits, idx=idx, gates=gates, y=y, y_shared=y_sh, out=out, **res)


# ------------------------------------------------------------------ backward

def ffn_gate_up_train(x_perm, offsets, w_gate, w_val, *, h=None, act=None, stream=None):
    """h = silu(x W_gate[e]) * (x W_val[e]) and the pre-activations act = [a | v]
    [N,2f] that the backward needs."""
    for t, n in ((w_gate, "w_gate"), (w_val, "w_val")):
        _dev(t, n)
    _offsets(offsets, w_gate.shape[0])
    ldx = _rows(x_perm, "x_perm")
    N, d = x_perm.shape
    E, _, f = w_gate.shape
    if h is None:
        h = torch.empty((N, f), dtype=x_perm.dtype, device=x_perm.device)
    if act is None:
        act = torch.empty((N, 2 * f), dtype=x_perm.dtype, device=x_perm.device)
    _check("moe_ffn_gate_up_train", lib().moe_ffn_gate_up_train(
        _p(x_perm), ldx, _dt(x_perm), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(h),
        _p(act),
        _stream(stream)))
    return h, act


def combine_backward(d_out, y_perm, dest, gates, k: int, *, d_y=None, d_y_dtype=None,
                     d_gates=None, stream=None):
    """d_y[dest[t,s]] = gates[t,s] d_out[t]; d_gates[t,s] = <d_out[t], y_perm[dest[t,s]]>."""
    _dev(d_out, "d_out"); _dev(y_perm, "y_perm"); _dev(dest, "dest"); _dev(gates, "gates")
    T, d = d_out.shape
    if d_y is None:
        d_y = torch.empty((y_perm.shape[0], d), dtype=d_y_dtype or d_out.dtype,
                          device=d_out.device)
    if d_gates is None:
        d_gates = torch.empty((T, k), dtype=torch.float32, device=d_out.device)
    _check("moe_combine_backward", lib().moe_combine_backward(
        _p(d_out), _dt(d_out), _p(y_perm), _dt(y_perm), _p(dest), _p(gates), T, k, d, _p(d_y),
        _dt(d_y), _p(d_gates), _stream(stream)))
    return d_y, d_gates


def ffn_down_backward(d_y, offsets, w_out, act, *, d_act=None, stream=None):
    """d_act = [da | dv]: the SwiGLU backward of dh = d_y W_out[e]^T."""
    N, d = d_y.shape
    E, f, _ = w_out.shape
    if d_act is None:
        d_act = torch.empty((N, 2 * f), dtype=d_y.dtype, device=d_y.device)
    _check("moe_ffn_down_backward", lib().moe_ffn_down_backward(
        _p(d_y), _dt(d_y), N, d, f, E, _p(offsets), _p(w_out), _p(act), _p(d_act),
        _stream(stream)))
    return d_act


def ffn_gate_up_backward(d_act, offsets, w_gate, w_val, *, d_x=None, dx_dtype=torch.float32,
                         accumulate=False, stream=None):
    """d_x = da W_gate[e]^T + dv W_val[e]^T (added into d_x with accumulate)."""
    N = d_act.shape[0]
    E, d, f = w_gate.shape
    if d_x is None:
        d_x = torch.empty((N, d), dtype=dx_dtype, device=d_act.device)
    _check("moe_ffn_gate_up_backward", lib().moe_ffn_gate_up_backward(
        _p(d_act), _dt(d_act), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(d_x), _dt(d_x),
        int(bool(accumulate)), _stream(stream)))
    return d_x


def ffn_weight_grads(x_perm, h, d_y, d_act, offsets, E: int, *, scale: float = 1.0, out=None,
                     stream=None):
    """(dW_gate [E,d,f], dW_val [E,d,f], dW_out [E,f,d]) in fp32, times ``scale``."""
    ldx = _rows(x_perm, "x_perm")
    N, d = x_perm.shape
    f = h.shape[1]
    dev = x_perm.device
    if out is None:
        out = (torch.empty((E, d, f), dtype=torch.float32, device=dev),
               torch.empty((E, d, f), dtype=torch.float32, device=dev),
               torch.empty((E, f, d), dtype=torch.float32, device=dev))
    dwg, dwv, dwo = out
    _check("moe_ffn_weight_grads", lib().moe_ffn_weight_grads(
        _p(x_perm), ldx, _p(h), _p(d_y), _p(d_act), _dt(x_perm), N, d, f, E, _p(offsets),
        float(scale), _p(dwg), _p(dwv), _p(dwo), _stream(stream)))
    return dwg, dwv, dwo


def route_backward(logits, idx, gates, d_gates, renorm: bool = True, *, lp_dtype=None,
                   d_logits=None, d_logits_lp=None, stream=None):
    """d_logits [T,E] fp32, plus a bf16 copy when ``lp_dtype`` is bfloat16."""
    T, E = logits.shape
    k = idx.shape[1]
    d_l = d_logits
    if d_l is None:
        d_l = torch.empty((T, E), dtype=torch.float32, device=logits.device)
    d_lp = d_logits_lp
    if d_lp is None and lp_dtype == torch.bfloat16:
        d_lp = torch.empty((T, E), dtype=torch.bfloat16, device=logits.device)
    _check("moe_route_backward", lib().moe_route_backward(
        _p(logits), _p(idx), _p(gates), _p(d_gates), T, E, k, int(bool(renorm)), _p(d_l),
        _p(d_lp), _stream(stream)))
    return d_l, d_lp


def token_backward(d_x_perm, dest, idx, gates, d_gates, w_router, *, d_x=None, workspace=None,
                   stream=None):
    """d_x = sum_s d_x_perm[dest] + sum_s d_l[t,e_s] W_r[:,e_s] for renormalised
    router weights (d_l formed from gates and d_gates), fp32 [T,d]."""
    T, k = idx.shape
    d, E = w_router.shape
    if d_x is None:
        d_x = torch.empty((T, d), dtype=torch.float32, device=idx.device)
    nbytes = int(lib().moe_token_backward_workspace(d, E, _dt(w_router)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=idx.device)
    _check("moe_token_backward", lib().moe_token_backward(
        _p(d_x_perm), _dt(d_x_perm), _p(dest), _p(idx), _p(gates), _p(d_gates), _p(w_router),
        _dt(w_router), T, k, d, E, _p(d_x), _p(workspace), workspace.numel(), _stream(stream)))
    return d_x


def router_backward_workspace(T: int, d: int, E: int) -> int:
    return int(lib().moe_router_backward_workspace(T, d, E))


def router_backward(x, w_router, d_logits, *, d_x=None, accumulate=False, want_dw=True,
                    d_w=None, workspace=None, stream=None):
    """d_x (+)= d_logits W_r^T; dW_r = x^T d_logits (fp32). d_logits in x's dtype."""
    T, d = x.shape
    E = w_router.shape[1]
    dw = d_w
    if dw is None and want_dw:
        dw = torch.empty((d, E), dtype=torch.float32, device=x.device)
    nbytes = router_backward_workspace(T, d, E) if dw is not None else 0
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _check("moe_router_backward", lib().moe_router_backward(
        _p(x), _p(w_router), _dt(x), _p(d_logits), T, d, E, _p(d_x), int(bool(accumulate)),
        _p(dw), _p(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return d_x, dw


def moe_layer_train(x, w_router, bias, k: int, w_gate, w_val, w_out, *, shared=None,
                    capacity=None, e_first=None, renorm=True, y_dtype=torch.float32,
                    stream=None):
    """Forward of the layer keeping what the backward needs (the pre-activations
    of every SwiGLU besides the forward's intermediates)."""
    E = w_gate.shape[0]
    logits, idx, gates = route(x, w_router, bias, k, renorm, stream=stream)
    p = permute(idx, x, E, capacity=capacity, e_first=e_first, stream=stream)
    h, act = ffn_gate_up_train(p["x_perm"], p["offsets"], w_gate, w_val, stream=stream)
    y = ffn_down(h, p["offsets"], w_out, y_dtype=y_dtype, stream=stream)
    sv = dict(logits=logits, idx=idx, gates=gates, h=h, act=act, y=y, renorm=renorm, k=k, **p)
    y_sh = None
    if shared is not None:
        # one group of all T tokens: offsets NULL
        h_sh, act_sh = ffn_gate_up_train(x, None, shared[0], shared[1], stream=stream)
        y_sh = ffn_down(h_sh, None, shared[2], y_dtype=y_dtype, stream=stream)
        sv.update(shared_off=None, h_shared=h_sh, act_shared=act_sh, y_shared=y_sh)
    sv["out"] = combine(y, p["dest"], gates, k, y_shared=y_sh, stream=stream)
    return sv


def moe_layer_backward(sv, d_out, x, w_router, w_gate, w_val, w_out, *, shared=None,
                       scale: float = 1.0, dx_perm_dtype=None, stream=None):
    """Gradients of sum(out * d_out) through the layer given the saved forward
    ``sv`` of moe_layer_train. Expert weight gradients are multiplied by
    ``scale`` (1/P for an EP group of P ranks). The packed rows' input
    gradient d_x_perm is kept in the activation type unless ``dx_perm_dtype``
    says otherwise (bf16 training hands every tensor between kernels over in
    bf16; the tokens' d_x sums it in fp32)."""
    if dx_perm_dtype is None:
        dx_perm_dtype = x.dtype
    k = sv["k"]
    E = w_gate.shape[0]
    T = x.shape[0]
    g = {}
    d_y, d_gates = combine_backward(d_out, sv["y"], sv["dest"], sv["gates"], k,
                                    d_y_dtype=x.dtype, stream=stream)
    d_act = ffn_down_backward(d_y, sv["offsets"], w_out, sv["act"], stream=stream)
    g["d_w_gate"], g["d_w_val"], g["d_w_out"] = ffn_weight_grads(
        sv["x_perm"], sv["h"], d_y, d_act, sv["offsets"], E, scale=scale, stream=stream)
    d_xp = ffn_gate_up_backward(d_act, sv["offsets"], w_gate, w_val, dx_dtype=dx_perm_dtype,
                                stream=stream)
    renorm = sv["renorm"]
    if renorm:
        # the packing's backward and the router's input term in one pass
        d_x = token_backward(d_xp, sv["dest"], sv["idx"], sv["gates"], d_gates, w_router,
                             stream=stream)
    else:
        d_x = combine(d_xp, sv["dest"], None, k, out_dtype=torch.float32, stream=stream)
    if shared is not None:
        off = sv["shared_off"]
        d_act_sh = ffn_down_backward(d_out.to(x.dtype), off, shared[2], sv["act_shared"],
                                     stream=stream)
        g["d_shared"] = ffn_weight_grads(x, sv["h_shared"], d_out.to(x.dtype), d_act_sh, off, 1,
                                         stream=stream)
        ffn_gate_up_backward(d_act_sh, off, shared[0], shared[1], d_x=d_x, accumulate=True,
                             stream=stream)
    d_l, d_lp = route_backward(sv["logits"], sv["idx"], sv["gates"], d_gates, renorm,
                               lp_dtype=x.dtype, stream=stream)
    # full-softmax weights: d_l is dense, the input term is a product with W_r^T
    _, g["d_w_router"] = router_backward(x, w_router, d_lp if d_lp is not None else d_l,
                                         d_x=None if renorm else d_x, accumulate=True,
                                         stream=stream)
    g.update(d_x=d_x, d_gates=d_gates, d_logits=d_l, d_y=d_y, d_act=d_act, d_x_perm=d_xp)
    return g


# ------------------------------------------------------- measurement helpers

def ceiling_mfma(blocks: int, iters: int, sink, stream=None) -> int:
    """Enqueue the matrix-core loop (include/moe_ceiling.h); returns its flops."""
    n = int(lib().moe_ceiling_mfma(blocks, iters, _p(sink), _stream(stream)))
    if n < 0:
        raise MoeError("moe_ceiling_mfma", n, "bad argument or launch")
    return n


def ceiling_copy(src, dst, nbytes: int, blocks: int, stream=None):
    if lib().moe_ceiling_copy(_p(src), _p(dst), nbytes, blocks, _stream(stream)) != 0:
        raise MoeError("moe_ceiling_copy", -1, "bad argument or launch")


def ceiling_read(src, nbytes: int, sink, blocks: int, stream=None):
    if lib().moe_ceiling_read(_p(src), nbytes, _p(sink), blocks, _stream(stream)) != 0:
        raise MoeError("moe_ceiling_read", -1, "bad argument or launch")
