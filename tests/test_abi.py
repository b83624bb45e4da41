"""The C ABI library loads, exports every entry point include/*.h declares,
and rejects bad host-side arguments before touching the device (no compute
call is made here, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
HEADERS = sorted(os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))
                 if h.endswith(".h"))


def _declared(headers=(HEADER,)):
    names = set()
    for h in headers:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from expert_dispatch_amd import ops
    return ops.lib()


def test_header_declares_the_path():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_permute_capacity", "moe_permute_range",
              "moe_permute_recv",
              "moe_grouped_ffn", "moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = _declared(HEADERS)
    assert "moe_ceiling_mfma" in names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(3) == b"workspace too small"
    assert L.moe_version() >= 101
    # recommended packed-row stride: one 128-byte line past the row
    assert L.moe_x_perm_ld(2048, 1) == 2112
    assert L.moe_x_perm_ld(64, 0) == 96
    assert L.moe_x_perm_ld(0, 1) == 0
    assert L.moe_x_perm_ld(64, 7) == 0


def test_workspace_queries(L):
    assert L.moe_permute_workspace(4096, 8, 128) >= 8 * 128 * 4
    assert L.moe_grouped_ffn_workspace(32768, 2048, 768, 128, 1) >= 32768 * 768 * 2
    assert L.moe_grouped_ffn_workspace(512, 64, 128, 8, 0) >= 512 * 128 * 4


def test_host_side_errors_return_before_launch(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    # k > E, k <= 0, E too large, unknown dtype
    assert L.moe_route(fake, 1, fake, None, 16, 64, 4, 5, 1, fake, fake, fake, None) == 1
    assert L.moe_route(fake, 1, fake, None, 16, 64, 4, 0, 1, fake, fake, fake, None) == 1
    assert L.moe_route(fake, 1, fake, None, 16, 64, 2048, 2, 1, fake, fake, fake, None) == 2
    assert L.moe_route(fake, 7, fake, None, 16, 64, 8, 2, 1, fake, fake, fake, None) == 1
    # required outputs NULL
    assert L.moe_route(fake, 1, fake, None, 16, 64, 8, 2, 1, None, fake, fake, None) == 1
    assert L.moe_route(fake, 1, fake, None, 16, 64, 8, 2, 1, fake, None, fake, None) == 1
    # permute: too small a workspace, NULL workspace
    need = L.moe_permute_workspace(100, 2, 8)
    assert L.moe_permute(fake, 100, 2, 8, fake, 1, 64, fake, fake, fake, fake, fake, 0, fake,
                         need - 1, None) == 3
    assert L.moe_permute(fake, 100, 2, 8, fake, 1, 64, fake, fake, fake, fake, fake, 0, None,
                         0, None) == 3
    # packed-row stride below the row width
    assert L.moe_permute(fake, 100, 2, 8, fake, 1, 64, fake, fake, fake, fake, fake, 63, fake,
                         need, None) == 1
    # capacity packing: negative capacity, small workspace
    assert L.moe_permute_capacity(fake, 100, 2, 8, -1, fake, 1, 64, None, fake, fake, fake,
                                  fake, fake, 0, fake, need, None) == 1
    assert L.moe_permute_capacity(fake, 100, 2, 8, 10, fake, 1, 64, None, fake, fake, fake,
                                  fake, fake, 0, fake, need - 1, None) == 3
    # range packing: negative first expert, E_loc too large
    assert L.moe_permute_range(fake, 100, 2, -1, 8, fake, 1, 64, fake, fake, fake, fake, fake,
                               0, fake, need, None) == 1
    assert L.moe_permute_range(fake, 100, 2, 0, 2048, fake, 1, 64, fake, fake, fake, fake, fake,
                               0, fake, need, None) == 2
    # permute_recv: too many cells
    assert L.moe_permute_recv(fake, 64, 128, 10, fake, 1, 64, fake, fake, fake, fake, fake,
                              0, None, 0, None) == 2
    assert L.moe_permute_recv(fake, 4, 16, 10, fake, 1, 64, fake, fake, fake, fake, fake,
                              32, None, 0, None) == 1
    # grouped ffn: NULL offsets, small workspace, bad y dtype
    assert L.moe_grouped_ffn(fake, 0, 1, 10, 64, 64, 2, None, fake, fake, fake, fake, 0, fake,
                             1 << 20, None) == 1
    assert L.moe_grouped_ffn(fake, 0, 1, 10, 64, 64, 2, fake, fake, fake, fake, fake, 0, fake,
                             16, None) == 3
    assert L.moe_grouped_ffn(fake, 0, 1, 10, 64, 64, 2, fake, fake, fake, fake, fake, 9, fake,
                             1 << 20, None) == 1
    # packed-row stride below d, for the readers of x_perm
    assert L.moe_grouped_ffn(fake, 32, 1, 10, 64, 64, 2, fake, fake, fake, fake, fake, 0, fake,
                             1 << 20, None) == 1
    assert L.moe_ffn_gate_up(fake, 60, 1, 10, 64, 64, 2, fake, fake, fake, fake, None) == 1
    assert L.moe_ffn_weight_grads(fake, 8, fake, fake, fake, 1, 10, 64, 64, 2, fake, 1.0,
                                  fake, fake, fake, None) == 1
    # combine: k too large
    assert L.moe_combine(fake, 0, fake, None, 4, 33, 64, None, 0, fake, 0, None) == 2
    # backward: combine without weights, k = 0
    assert L.moe_combine_backward(fake, 1, fake, 0, fake, None, 4, 2, 64, fake, 1, fake, None) == 1
    assert L.moe_combine_backward(fake, 1, fake, 0, fake, fake, 4, 0, 64, fake, 1, fake, None) == 1
    # gate_up backward: accumulating into bf16, fp32 data into a bf16 gradient, NULL d_x
    assert L.moe_ffn_gate_up_backward(fake, 1, 10, 64, 64, 2, fake, fake, fake, fake, 1, 1,
                                      None) == 2
    assert L.moe_ffn_gate_up_backward(fake, 0, 10, 64, 64, 2, fake, fake, fake, fake, 1, 0,
                                      None) == 2
    assert L.moe_ffn_gate_up_backward(fake, 1, 10, 64, 64, 2, fake, fake, fake, None, 0, 0,
                                      None) == 1
    # down backward: NULL saved pre-activations; training forward: NULL act
    assert L.moe_ffn_down_backward(fake, 1, 10, 64, 64, 2, fake, fake, None, fake, None) == 1
    assert L.moe_ffn_gate_up_train(fake, 0, 1, 10, 64, 64, 2, fake, fake, fake, fake, None,
                                   None) == 1
    # router backward: no output asked for, k > E, NULL inputs with rows
    assert L.moe_route_backward(fake, fake, fake, fake, 4, 8, 2, 1, None, None, None) == 1
    assert L.moe_route_backward(fake, fake, fake, fake, 4, 8, 9, 1, fake, None, None) == 1
    assert L.moe_router_backward(None, fake, 1, fake, 4, 64, 8, fake, 0, None, None, 0,
                                 None) == 1
    # token input gradient: too small a workspace
    assert L.moe_token_backward(fake, 0, fake, fake, fake, fake, fake, 1, 64, 2, 128, 8, fake,
                                fake, 16, None) == 3
    # load statistics: too small a workspace, k > E
    assert L.moe_route_stats(fake, fake, 64, 8, 2, fake, fake, fake, 16, None) == 3
    need_s = L.moe_route_stats_workspace(64, 8)
    assert L.moe_route_stats(fake, fake, 64, 8, 2, fake, fake, fake, need_s - 1, None) == 3
    assert L.moe_route_stats_workspace(4096, 128) > L.moe_route_stats_workspace(4096, 8)
    assert L.moe_route_stats(fake, fake, 64, 8, 9, fake, fake, fake, 1 << 20, None) == 1
    # router W_r gradient at large T needs the split workspace
    need_r = L.moe_router_backward_workspace(4096, 64, 8)
    assert need_r > 0 and L.moe_router_backward_workspace(64, 64, 8) == 0
    assert L.moe_router_backward(fake, fake, 1, fake, 4096, 64, 8, None, 0, fake, None, 0,
                                 None) == 3


def test_empty_inputs_are_no_ops(L):
    # T = 0 / N = 0 enqueue nothing and succeed
    assert L.moe_route(None, 1, None, None, 0, 64, 8, 2, 1, None, None, None, None) == 0
    assert L.moe_grouped_ffn(None, 0, 1, 0, 64, 64, 2, ctypes.c_void_p(0x1000), None, None,
                             None, None, 0, None, 0, None) == 0
    assert L.moe_combine(None, 0, None, None, 0, 2, 64, None, 0, None, 0, None) == 0
    assert L.moe_combine_backward(None, 1, None, 0, None, None, 0, 2, 64, None, 1, None,
                                  None) == 0
    assert L.moe_route_backward(None, None, None, None, 0, 8, 2, 1, None, None, None) == 0


def test_debug_status_release_and_debug_builds(L):
    """The release library reports that it checks no device preconditions;
    the debug build (MOE_DEBUG) loads beside it and exports the same calls."""
    from expert_dispatch_amd import ops
    f = ctypes.c_uint(7)
    assert L.moe_debug_status(ctypes.byref(f), 0) == 2   # MOE_ERR_UNSUPPORTED
    assert f.value == 0
    assert L.moe_debug_status(None, 0) == 1              # MOE_ERR_INVALID_ARG
    if not os.path.exists(ops.debug_lib_path()):
        pytest.skip("libmoe_debug.so not built")
    D = ops.bind(ops.debug_lib_path())
    for n in _declared(HEADERS):
        assert hasattr(D, n), n
    assert D.moe_version() == L.moe_version()


def test_noalloc_packing_rejects_sizes_past_its_static_array(L):
    """moe_permute_noalloc keeps its chunk histograms in a 1 MiB static
    array per GPU: a request that needs more returns MOE_ERR_WORKSPACE
    before anything is enqueued (the pointers here are never dereferenced)."""
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_permute_workspace(1 << 20, 2, 1024) > (1 << 20)
    assert L.moe_permute_noalloc(fake, 1 << 20, 2, 1024, fake, 1, 64, fake, fake, fake, fake, fake,
                                 0, None) == 3
    assert L.moe_permute_noalloc(fake, 16, 2, 1025, fake, 1, 64, fake, fake, fake, fake, fake,
                                 0, None) == 2   # E past the packing's limit
    assert L.moe_permute_noalloc(fake, 16, 0, 8, fake, 1, 64, fake, fake, fake, fake, fake,
                                 0, None) == 1   # k <= 0
