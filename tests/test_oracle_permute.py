"""Pins of the oracle's expert-major packing and receive-side reorder.

"Three axes of Parallelism", Expert Parallel (EP) -> Producing assignments:
count the assignments per expert, offsets from the cumulative counts, write
each assignment into its expert's region. The Modalities EP page's tests check
the same three things held here: the result is a permutation, it groups by
expert, and it matches a loop reference; on top of that the packing is held
to numpy's stable argsort and bincount, and the receive-side reorder to a
closed form built block by block from the count matrix.
"""
import numpy as np
import pytest

import oracle
from expert_dispatch_amd import workloads as W


def _check_invariants(key, E, counts, offsets, perm_src, dest):
    n = key.shape[0]
    assert counts.sum() == n and offsets[-1] == n and offsets[0] == 0
    assert (np.diff(offsets) == counts).all()
    # bijection between assignments and packed rows
    assert sorted(perm_src.tolist()) == list(range(n))
    np.testing.assert_array_equal(dest[perm_src], np.arange(n))
    for e in range(E):
        seg = perm_src[offsets[e]:offsets[e + 1]]
        assert (key[seg] == e).all()          # groups by expert
        assert (np.diff(seg) > 0).all()       # stable: ascending flat order


def _loop_reference(flat, E):
    # for every expert, its assignments in row-major (token, slot) order
    parts = [np.argwhere(flat == e)[:, 0] for e in range(E)]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_small", "dsv2_small_empty4", "stress_small"])
def test_pack_matches_libraries_and_loop(name):
    inp = W.generate(W.get(name))
    _, idx, _ = oracle.route(inp["x"], inp["w_router"], inp["bias"], inp["k"])
    E = inp["w_gate"].shape[0]
    counts, offsets, perm_src, dest = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets[1:], np.cumsum(np.bincount(flat, minlength=E)))
    np.testing.assert_array_equal(perm_src, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(perm_src, _loop_reference(flat, E))
    _check_invariants(flat, E, counts, offsets, perm_src, dest)


def test_pack_empty_and_single_expert_cases():
    counts, offsets, perm_src, dest = oracle.permute(np.zeros(0, np.int32), 5)
    assert counts.tolist() == [0] * 5 and offsets.tolist() == [0] * 6
    flat = np.full(37, 3, np.int32)               # every assignment to one expert
    counts, offsets, perm_src, dest = oracle.permute(flat, 5)
    assert counts.tolist() == [0, 0, 0, 37, 0]
    np.testing.assert_array_equal(perm_src, np.arange(37))
    with pytest.raises(oracle.OracleError):
        oracle.permute(np.array([0, 5], np.int32), 5)


def _recv_closed_form(recv):
    """dest(r) = offsets[j] + sum_{i'<i} recv[i',j] + (r - start of block (i,j))."""
    S, E = recv.shape
    offsets = np.concatenate([[0], np.cumsum(recv.sum(axis=0))])
    dest = []
    for i in range(S):
        for j in range(E):
            base = offsets[j] + recv[:i, j].sum()
            dest.extend(range(base, base + recv[i, j]))
    return np.array(dest, np.int64)


@pytest.mark.parametrize("name", ["ep_share_small", "ep_rank_share"])
def test_recv_reorder_closed_form_and_stable_sort(name):
    cfg = W.get(name)
    rng = np.random.default_rng(cfg.seed)
    p = rng.dirichlet(np.full(cfg.S * cfg.E, cfg.alpha))
    recv = rng.multinomial(cfg.N, p).astype(np.int32).reshape(cfg.S, cfg.E)
    counts, offsets, perm_src, dest = oracle.permute_recv(recv, cfg.N)
    np.testing.assert_array_equal(dest, _recv_closed_form(recv))
    keys = np.repeat(np.tile(np.arange(cfg.E), cfg.S), recv.reshape(-1))
    np.testing.assert_array_equal(perm_src, np.argsort(keys, kind="stable"))
    np.testing.assert_array_equal(counts, recv.sum(axis=0))
    _check_invariants(keys, cfg.E, counts, offsets, perm_src, dest)


def test_recv_reorder_round_trip_and_errors():
    inp = W.generate(W.get("ep_share_small"))
    inp = W.zero_expert_column(inp, 2)
    N = inp["x_recv"].shape[0]
    counts, offsets, perm_src, dest = oracle.permute_recv(inp["recv_counts"], N)
    assert counts[2] == 0
    xp = oracle.gather(inp["x_recv"], perm_src, 1)
    np.testing.assert_array_equal(xp[dest], inp["x_recv"])      # un-permute restores it
    bad = inp["recv_counts"].copy()
    bad[0, 0] += 1
    with pytest.raises(oracle.OracleError):
        oracle.permute_recv(bad, N)


def test_gather_reads_each_token_for_each_slot():
    inp = W.generate(W.get("qwen3_small"))
    k = inp["k"]
    _, idx, _ = oracle.route(inp["x"], inp["w_router"], inp["bias"], k)
    _, _, perm_src, dest = oracle.permute(idx, inp["w_gate"].shape[0])
    xp = oracle.gather(inp["x"], perm_src, k)
    T = inp["x"].shape[0]
    for a in range(0, T * k, 5):
        np.testing.assert_array_equal(xp[dest[a]], inp["x"][a // k])


def _capacity_reference(flat, E, cap):
    """Each expert keeps its first `cap` assignments in ascending flat order
    (written out with Python lists, one expert at a time)."""
    kept, dest = [], np.full(flat.shape[0], -1, np.int64)
    routed = np.bincount(flat, minlength=E)
    for e in range(E):
        mine = [a for a in range(flat.shape[0]) if flat[a] == e][:cap]
        for a in mine:
            dest[a] = len(kept)
            kept.append(a)
    counts = np.minimum(routed, cap)
    return routed, counts, np.concatenate([[0], np.cumsum(counts)]), np.array(kept, np.int64), dest


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_capacity_pack_bruteforce(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 40)), int(rng.integers(1, 4)), int(rng.integers(1, 7))
    k = min(k, E)
    # skewed ids so some experts overflow
    flat = np.minimum(rng.geometric(0.4, size=T * k) - 1, E - 1).astype(np.int32)
    for cap in (0, 1, 2, 5, T * k):
        r = oracle.permute_capacity(flat.reshape(T, k), E, cap)
        ref = _capacity_reference(flat, E, cap)
        for got, want, what in zip(r, ref, ("routed", "counts", "offsets", "perm_src", "dest")):
            np.testing.assert_array_equal(got, want, err_msg=f"{what} cap={cap}")
        assert (r[4] < 0).sum() == int(np.maximum(ref[0] - cap, 0).sum())


@pytest.mark.parametrize("name", ["qwen3_small", "stress_small"])
def test_capacity_at_least_every_count_is_the_plain_pack(name):
    inp = W.generate(W.get(name))
    _, idx, _ = oracle.route(inp["x"], inp["w_router"], inp["bias"], inp["k"])
    E = inp["w_gate"].shape[0]
    plain = oracle.permute(idx, E)
    cap = int(plain[0].max())
    routed, counts, offsets, perm_src, dest = oracle.permute_capacity(idx, E, cap)
    np.testing.assert_array_equal(routed, plain[0])
    for got, want in zip((counts, offsets, perm_src, dest), plain):
        np.testing.assert_array_equal(got, want)
    # one below the largest count drops exactly the largest expert's last assignment
    routed, counts, offsets, perm_src, dest = oracle.permute_capacity(idx, E, cap - 1)
    assert (dest < 0).sum() == int((plain[0] == cap).sum())


def test_capacity_rejects_negative():
    with pytest.raises(RuntimeError):
        oracle.permute_capacity(np.zeros((2, 1), np.int32), 1, -1)


@pytest.mark.parametrize("seed", [0, 1])
def test_range_packing_is_the_ranks_slice_of_the_global_packing(seed):
    """All-gather layout: rank r owns experts [r*E_loc, (r+1)*E_loc). Its packing
    is exactly its experts' slice of the global packing, shifted to start at 0,
    and every assignment is kept by exactly one rank."""
    rng = np.random.default_rng(seed)
    R, E_loc, T, k = 4, 3, 57, 3
    E = R * E_loc
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    g_counts, g_off, g_src, g_dest = oracle.permute(idx, E)
    owners = np.zeros(T * k, np.int64)
    for r in range(R):
        e0 = r * E_loc
        counts, offsets, perm_src, dest = oracle.permute_range(idx, e0, E_loc)
        np.testing.assert_array_equal(counts, g_counts[e0:e0 + E_loc])
        lo, hi = g_off[e0], g_off[e0 + E_loc]
        np.testing.assert_array_equal(perm_src, g_src[lo:hi])
        mine = (idx.reshape(-1) >= e0) & (idx.reshape(-1) < e0 + E_loc)
        np.testing.assert_array_equal(dest[mine], g_dest[mine] - lo)
        assert (dest[~mine] == -1).all()
        owners += mine
    assert (owners == 1).all()
