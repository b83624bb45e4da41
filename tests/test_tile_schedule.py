"""The grouped FFN's tile list (expert_dispatch_amd/csrc/mfma_common.hpp:
build_tile_list, tail_cost, decode_tile), restated in Python: the device
builds it per launch from the expert offsets, so its arithmetic is checked
here on the CPU, and on the GPU by the parity tests of the EP-share and
gathered-token workloads, whose lists split their last round.

Checked: the closed-form cost of the busiest block equals a brute-force
deal of the list over the grid; every (packed row, column tile) is computed
exactly once, by a tile inside its expert's segment, whether or not the last
round of 256-row tiles is split into 128-row halves."""
import random

import numpy as np

kGroupM = 4


def tail_cost(nb, ns, G, c8):
    qb, rb, qs, ms = nb // G, nb % G, ns // G, ns % G
    extra = 0
    if rb > 0:
        extra = 8 + (c8 if rb + ms > G else 0)
    if ms > 0:
        extra = max(extra, c8)
    return 8 * qb + c8 * qs + extra


def dealt_cost(nb, ns, G, c8):
    """Brute force: position r of the grid takes list entries r, r + G, ..."""
    cost = np.zeros(G, np.int64)
    for t in range(nb + ns):
        cost[t % G] += 8 if t < nb else c8
    return int(cost.max())


def build(off, n_tiles, G, c8):
    E = len(off) - 1
    big, small, pb, ps, rb, rs = [], [], [], [], 0, 0
    for e in range(E):
        n = max(0, off[e + 1] - off[e])
        rem = n & 255
        big.append(((n >> 8) + (1 if rem > 128 else 0)) * n_tiles)
        small.append(n_tiles if 0 < rem <= 128 else 0)
    for e in range(E):
        pb.append(rb)
        rb += big[e]
        ps.append(rs)
        rs += small[e]
    L = dict(off=off, big=pb, small=ps, E=E, n_tiles=n_tiles, total_big=rb, total_small=rs,
             split=0)
    rem = rb % G
    if c8 > 0 and rem > 0 and tail_cost(rb - rem, rs + 2 * rem, G, c8) < tail_cost(rb, rs, G, c8):
        L["split"] = rem
    return L


def _owner(pre, E, t):
    lo, hi = 0, E - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if pre[mid] <= t:
            lo = mid
        else:
            hi = mid - 1
    return lo


def decode(L, t):
    """(expert, column tile, first row, segment end, rows) of list entry t."""
    half = -1
    B, s = L["total_big"], L["split"]
    if B - s <= t < B + s:
        u = t - (B - s)
        half = u & 1
        t = B - s + (u >> 1)
    elif t >= B + s:
        t -= s
    off = L["off"]
    if t < B:
        e = _owner(L["big"], L["E"], t)
        lo, hi = off[e], max(off[e], off[e + 1])
        n = hi - lo
        mt = (n >> 8) + (1 if (n & 255) > 128 else 0)
        local = t - L["big"][e]
        grp = local // (kGroupM * L["n_tiles"])
        within = local - grp * (kGroupM * L["n_tiles"])
        gsz = min(kGroupM, mt - grp * kGroupM)
        m0 = lo + (grp * kGroupM + within % gsz) * 256
        if half >= 0:
            return e, within // gsz, m0 + 128 * half, hi, 128
        return e, within // gsz, m0, hi, 256
    t -= B
    e = _owner(L["small"], L["E"], t)
    lo, hi = off[e], max(off[e], off[e + 1])
    return e, t - L["small"][e], lo + ((hi - lo) >> 8) * 256, hi, 128


def test_tail_cost_closed_form_equals_brute_force():
    rng = random.Random(7)
    for _ in range(3000):
        G = 8 * rng.randint(1, 32)
        nb, ns, c8 = rng.randint(0, 4 * G), rng.randint(0, 4 * G), rng.randint(1, 8)
        assert tail_cost(nb, ns, G, c8) == dealt_cost(nb, ns, G, c8), (nb, ns, G, c8)


def test_every_row_and_column_tile_once_split_or_not():
    rng = random.Random(3)
    splits = 0
    for it in range(1500):
        E, G, n_tiles = rng.randint(1, 40), 8 * rng.randint(1, 32), rng.randint(1, 12)
        sizes = [rng.choice([0, rng.randint(1, 300), rng.randint(1, 1500), 256 * rng.randint(1, 4)])
                 for _ in range(E)]
        off = [0]
        for z in sizes:
            off.append(off[-1] + z)
        L = build(off, n_tiles, G, rng.choice([0, 6, 7]))
        splits += L["split"] > 0
        seen = np.zeros((off[-1], n_tiles), np.int32)
        for t in range(L["total_big"] + L["split"] + L["total_small"]):
            e, nt, m0, hi, bm = decode(L, t)
            assert 0 <= nt < n_tiles and off[e] <= m0 < hi, (it, t)
            seen[m0:min(m0 + bm, hi), nt] += 1
        assert np.all(seen == 1), it
    assert splits > 300


def test_the_measured_workloads_split_where_it_pays():
    """The realised tile counts of the EP-share gate_up (520 256-row and 64
    128-row tiles on 256 blocks) split the 8 tiles of their last round; the
    Qwen3-shaped gate_up (750 and 432), whose 128-row tiles already fill
    that round, stays whole."""
    assert tail_cost(520 - 8, 64 + 2 * 8, 256, 7) < tail_cost(520, 64, 256, 7)
    assert not tail_cost(750 - 238, 432 + 2 * 238, 256, 7) < tail_cost(750, 432, 256, 7)
