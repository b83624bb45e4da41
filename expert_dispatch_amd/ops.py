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


def lib():
    """Open libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m expert_dispatch_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [i]
    L.moe_version.restype = i
    sigs = {
        "moe_route": [vp, i, vp, vp, i, i, i, i, i, vp, vp, vp, vp],
        "moe_permute": [vp, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_capacity": [vp, i, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_range": [vp, i, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_recv": [vp, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_grouped_ffn": [vp, i, i, i, i, i, vp, vp, vp, vp, vp, i, vp, sz, vp],
        "moe_ffn_gate_up": [vp, i, i, i, i, i, vp, vp, vp, vp, vp],
        "moe_ffn_down": [vp, i, i, i, i, i, vp, vp, vp, i, vp],
        "moe_combine": [vp, i, vp, vp, i, i, i, vp, i, vp, i, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = i
    for name, args in {"moe_permute_workspace": [i, i, i],
                       "moe_permute_recv_workspace": [i, i, i],
                       "moe_grouped_ffn_workspace": [i, i, i, i, i]}.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = sz
    _lib = L
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
                   x_perm=torch.empty((T * k, d), dtype=x.dtype, device=dev))
        if capacity is not None:
            out["routed"] = torch.empty(E, dtype=torch.int32, device=dev)
    nbytes = permute_workspace(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if e_first is not None:
        _check("moe_permute_range", lib().moe_permute_range(
            _p(topk_idx), T, k, int(e_first), E, _p(x), _dt(x), d, _p(out["counts"]),
            _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]),
            _p(workspace), workspace.numel(), _stream(stream)))
    elif capacity is None:
        _check("moe_permute", lib().moe_permute(
            _p(topk_idx), T, k, E, _p(x), _dt(x), d, _p(out["counts"]), _p(out["offsets"]),
            _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]), _p(workspace),
            workspace.numel(), _stream(stream)))
    else:
        _check("moe_permute_capacity", lib().moe_permute_capacity(
            _p(topk_idx), T, k, E, int(capacity), _p(x), _dt(x), d, _p(out.get("routed")),
            _p(out["counts"]), _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]),
            _p(out["x_perm"]), _p(workspace), workspace.numel(), _stream(stream)))
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
                   x_perm=torch.empty((N, d), dtype=x_recv.dtype, device=dev))
    _check("moe_permute_recv", lib().moe_permute_recv(
        _p(recv_counts), S, E_loc, N, _p(x_recv), _dt(x_recv), d, _p(out["counts"]),
        _p(out["offsets"]), _p(out["perm_src"]), _p(out["dest"]), _p(out["x_perm"]), None, 0,
        _stream(stream)))
    return out


def grouped_ffn_workspace(N: int, d: int, f: int, E: int, dtype) -> int:
    return int(lib().moe_grouped_ffn_workspace(N, d, f, E, _dt_of(dtype)))


def grouped_ffn(x_perm, offsets, w_gate, w_val, w_out, *, y_dtype=torch.float32, y=None,
                workspace=None, stream=None):
    """y[j] = (silu(x_perm[j] W_gate[e]) * (x_perm[j] W_val[e])) W_out[e] per expert segment."""
    for t, n in ((x_perm, "x_perm"), (offsets, "offsets"), (w_gate, "w_gate"),
                 (w_val, "w_val"), (w_out, "w_out")):
        _dev(t, n)
    N, d = x_perm.shape
    E, _, f = w_gate.shape
    if y is None:
        y = torch.empty((N, d), dtype=y_dtype, device=x_perm.device)
    nbytes = grouped_ffn_workspace(N, d, f, E, x_perm.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x_perm.device)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _p(x_perm), _dt(x_perm), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(w_out),
        _p(y), _dt(y), _p(workspace), workspace.numel(), _stream(stream)))
    return y


def ffn_gate_up(x_perm, offsets, w_gate, w_val, *, h=None, stream=None):
    N, d = x_perm.shape
    E, _, f = w_gate.shape
    if h is None:
        h = torch.empty((N, f), dtype=x_perm.dtype, device=x_perm.device)
    _check("moe_ffn_gate_up", lib().moe_ffn_gate_up(
        _p(x_perm), _dt(x_perm), N, d, f, E, _p(offsets), _p(w_gate), _p(w_val), _p(h),
        _stream(stream)))
    return h


def ffn_down(h, offsets, w_out, *, y_dtype=torch.float32, y=None, stream=None):
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


def moe_layer(x, w_router, bias, k: int, w_gate, w_val, w_out, *, shared=None, capacity=None,
              y_dtype=torch.float32, out_dtype=torch.float32, stream=None):
    """The whole token-routed layer: route -> permute -> grouped FFN -> combine.
    ``shared`` = (w_gate, w_val, w_out) of the always-on shared experts
    concatenated along f (one SwiGLU of width q*f equals the sum of q).
    ``y_dtype`` is the storage type of the expert outputs between the down
    GEMM and the combine. ``capacity``: fixed-capacity packing (at most that
    many rows per expert; dropped assignments add nothing to their token)."""
    E = w_gate.shape[0]
    logits, idx, gates = route(x, w_router, bias, k, stream=stream)
    p = permute(idx, x, E, capacity=capacity, stream=stream)
    y = grouped_ffn(p["x_perm"], p["offsets"], w_gate, w_val, w_out, y_dtype=y_dtype,
                    stream=stream)
    y_sh = None
    if shared is not None:
        T = x.shape[0]
        off = torch.tensor([0, T], dtype=torch.int32, device=x.device)
        y_sh = grouped_ffn(x, off, *shared, y_dtype=y_dtype, stream=stream)
    out = combine(y, p["dest"], gates, k, y_shared=y_sh, out_dtype=out_dtype, stream=stream)
    return dict(logits=logits, idx=idx, gates=gates, y=y, y_shared=y_sh, out=out, **p)
