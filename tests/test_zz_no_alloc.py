"""moe_permute_noalloc (the packing for callers that cannot allocate: its
chunk histograms live in the library's static per-GPU array) against
moe_permute with a caller workspace, through the C ABI: every output bit for
bit, on two calls in a row, the second with a smaller input (the static
array keeps the first call's contents, which the second must not read)."""
import ctypes

import numpy as np
import pytest
import torch

from expert_dispatch_amd import ops
from util import to_numpy

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _outs(T, k, E, d, dtype):
    rows = T * k
    return dict(counts=torch.full((E,), -5, dtype=torch.int32, device="cuda"),
                offsets=torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"),
                perm_src=torch.full((rows,), -5, dtype=torch.int32, device="cuda"),
                dest=torch.full((rows,), -5, dtype=torch.int32, device="cuda"),
                x_perm=ops.empty_rows(rows, d, dtype, "cuda").fill_(0))


def _case(T, k, E, d, seed, skew):
    L = ops.lib()
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, skew))
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    idx_t = torch.from_numpy(idx).cuda()
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda().to(torch.bfloat16)
    ref = _outs(T, k, E, d, x.dtype)
    got = _outs(T, k, E, d, x.dtype)
    ws = torch.empty(max(1, ops.permute_workspace(T, k, E)), dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ld = ref["x_perm"].stride(0)
    assert L.moe_permute(_p(idx_t), T, k, E, _p(x), ops.MOE_BF16, d, _p(ref["counts"]),
                         _p(ref["offsets"]), _p(ref["perm_src"]), _p(ref["dest"]),
                         _p(ref["x_perm"]), ld, _p(ws), ws.numel(), st) == 0
    assert L.moe_permute_noalloc(_p(idx_t), T, k, E, _p(x), ops.MOE_BF16, d, _p(got["counts"]),
                                 _p(got["offsets"]), _p(got["perm_src"]), _p(got["dest"]),
                                 _p(got["x_perm"]), ld, st) == 0
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm_src", "dest"):
        np.testing.assert_array_equal(to_numpy(got[key]), to_numpy(ref[key]), err_msg=key)
    assert torch.equal(got["x_perm"].view(torch.int16), ref["x_perm"].view(torch.int16))
    # and the packing is the stable expert-major one
    counts = np.bincount(idx.reshape(-1), minlength=E)
    np.testing.assert_array_equal(to_numpy(got["counts"]), counts)
    order = np.argsort(idx.reshape(-1), kind="stable")
    np.testing.assert_array_equal(to_numpy(got["perm_src"]), order)
    print(f"[no-alloc] T={T} k={k} E={E}: equal to the workspace packing", flush=True)


def test_noalloc_packing_equals_workspace_packing_twice():
    _case(32768, 8, 64, 4096, seed=71, skew=0.5)    # the stress shape: 64 ranking chunks
    _case(300, 4, 16, 256, seed=72, skew=2.0)       # smaller: 3 chunks, stale ones ignored
