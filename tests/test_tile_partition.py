"""CPU check of how the row-grouped GEMMs deal their tiles to the XCDs
(csrc/gemm.hip tile decode, csrc/common.hpp tile_starts_block,
csrc/kernels.hpp chain_bounds_block and rowgrouped_slots / chain_slots).

The rules, restated here from the kernels:
  - the tile list of a GEMM with nt column tiles runs expert by expert,
    column tile by column tile, m-tile by m-tile; expert e owns m-tiles
    tstart[e] .. tstart[e+1]-1 (256 routed rows each, the last one ragged);
  - tile cost in eighths of a full tile: 8, except an expert's last m-tile
    with at most 192 rows when the expert has other m-tiles: 4 + one per
    64-row piece that holds rows; cpre = exclusive prefix of the experts'
    summed m-tile costs;
  - separate launches: XCD x starts at the tile where the cumulative cost
    reaches x / 8 of the total (or, with equal counts, at x * ceil(M nt / 8));
    a workgroup is the XCD's slot-th and takes tile start + slot if that is
    below the next XCD's start;
  - chained launches: XCD x takes m-tiles xcd_mt[x] .. xcd_mt[x+1]-1, the
    m-tile boundary nearest x / 8 of the cost, clamped to within 3 m-tiles of
    x M / 8, and every column tile of them;
  - the grids hold 8 * rowgrouped_slots (separate; with equal counts exactly
    the equal share) or 8 * chain_slots (chained) workgroups.
Every (m-tile, column tile) must be run exactly once, within the grid, and in
a chained launch on the XCD whose range holds its m-tile.

The weight-gradient GEMMs (gemm.hip dW decode, dw_chunkmap_block): expert e's
rows split into chunks of at most 4096 rows (at least one chunk); the chunk
list runs expert by expert; corder lists the chunks heaviest first (the
4096-row chunks in list order, then each expert's shorter chunk by rows
descending, ties by expert); the (chunk, matrix) groups in that order are
dealt to the XCDs in snake order (row r of 8 groups: XCD x takes group
8r + x for even r, 8r + 7 - x for odd r), and an XCD's slot s runs tile
s mod per_c of its group s div per_c.  The grid holds ceil(nmat * (E +
ceil(R / 4096)) / 8) * per_c slots per XCD.
"""
import bisect

import numpy as np
import pytest

BM, X, SLACK = 256, 8, 3


def tile_map(counts):
    mt = [(c + BM - 1) // BM for c in counts]
    cost = []
    for c, m in zip(counts, mt):
        if m == 0:
            cost.append(0)
            continue
        last = c - BM * (m - 1)
        cost.append(8 * (m - 1) + (4 + (last + 63) // 64 if last <= 192 and m >= 2 else 8))
    return np.concatenate([[0], np.cumsum(mt)]), np.concatenate([[0], np.cumsum(cost)])


def expert_of(starts, f, key):
    """Count of experts i with f(starts[i]) <= key, less one (the kernel's
    ballot; f(starts[]) is nondecreasing, so a bisection counts the same)."""
    vals = [f(v) for v in starts[:-1]]
    return bisect.bisect_right(vals, key) - 1


def first_tile(x, nt, tstart, cpre):
    M = tstart[-1]
    if x == 0:
        return 0
    if x == X:
        return M * nt
    t = x * cpre[-1] // X
    e = expert_of(cpre, lambda v: v, t)
    c0, ce = cpre[e], cpre[e + 1] - cpre[e]
    t0, mc = tstart[e], tstart[e + 1] - tstart[e]
    if ce == 0:
        return t0 * nt
    rem = (t - c0) * nt
    q = rem // ce
    r = min((rem - q * ce + 4) // 8, mc - 1)
    return t0 * nt + q * mc + r


def chain_bounds(tstart, cpre):
    M, out = tstart[-1], []
    for x in range(X + 1):
        if x in (0, X):
            out.append(0 if x == 0 else M)
            continue
        t = x * cpre[-1] // X
        lo, hi = 0, len(tstart) - 1
        while hi - lo > 1:
            mid = (lo + hi) // 2
            lo, hi = (mid, hi) if cpre[mid] <= t else (lo, mid)
        mc = tstart[lo + 1] - tstart[lo]
        v = tstart[lo] + min((t - cpre[lo] + 4) // 8, mc)
        base = x * M // X
        out.append(min(max(min(max(v, base - SLACK), base + SLACK), 0), M))
    return out


def decode(xcd, slot, nt, tstart, cpre, xcd_mt=None, even=False):
    """(expert, m-tile, column tile) of workgroup slot of XCD xcd, or None."""
    if xcd_mt is not None:
        lo, hi = xcd_mt[xcd], xcd_mt[xcd + 1]
        if slot >= (hi - lo) * nt:
            return None
        key = lo * nt + slot
    else:
        lo, hi = 0, tstart[-1]
        if even:
            per = -(-(hi * nt) // X)
            key = xcd * per + slot
            if slot >= per or key >= hi * nt:
                return None
        else:
            k0, k1 = first_tile(xcd, nt, tstart, cpre), first_tile(xcd + 1, nt, tstart, cpre)
            key = k0 + slot
            if key >= k1:
                return None

    def clip(v):
        return min(max(v, lo), hi)
    e = expert_of(tstart, lambda v: clip(v) * nt, key)
    cs, mcnt = clip(tstart[e]), clip(tstart[e + 1]) - clip(tstart[e])
    local = key - cs * nt
    j = local // mcnt
    return e, cs + (local - j * mcnt), j


def routings():
    rng = np.random.default_rng(20)
    out = [[537, 538, 486, 539, 530, 523, 541, 489, 518, 480, 524, 514, 494, 495, 492, 492],
           [1, 63, 64, 65, 192, 193, 256, 257, 448, 449], [40000], [0, 0, 5, 0],
           [4096, 8192, 4097, 1, 0], [4095, 4096, 12288, 0, 0, 3]]
    for _ in range(24):
        E = int(rng.choice([1, 3, 8, 16, 128, 300]))
        R = int(rng.integers(1, 40000))
        out.append(list(rng.multinomial(R, rng.dirichlet(np.ones(E) * rng.choice([0.05, 1, 10])))))
    return out


@pytest.mark.parametrize("counts", routings())
def test_every_tile_runs_once_within_the_grid(counts):
    tstart, cpre = tile_map(counts)
    M, E = tstart[-1], len(counts)
    mt_bound = (sum(counts) + E * (BM - 1)) // BM
    xm = chain_bounds(tstart, cpre)
    assert xm[0] == 0 and xm[-1] == M and all(a <= b for a, b in zip(xm, xm[1:]))
    for nt in (1, 6, 20):
        for mode in ("cost", "even", "chain"):
            share = -(-(mt_bound * nt) // X)
            slots = {"chain": ((mt_bound + X - 1) // X + 2 * SLACK) * nt,
                     "even": share, "cost": 2 * share + 2}[mode]
            seen = set()
            for xcd in range(X):
                for s in range(slots):
                    r = decode(xcd, s, nt, tstart, cpre, xm if mode == "chain" else None,
                               mode == "even")
                    if r is None:
                        continue
                    e, g, j = r
                    assert tstart[e] <= g < tstart[e + 1] and 0 <= j < nt
                    assert (g, j) not in seen
                    seen.add((g, j))
                    if mode == "chain":
                        assert xm[xcd] <= g < xm[xcd + 1]
            assert len(seen) == M * nt


def test_scout_routing_costs_balance():
    """At the Scout routing the cost split gives every XCD within 3% of the
    mean cost (equal counts left one XCD 9% over: it holds no cheap tiles)."""
    counts = routings()[0]
    tstart, cpre = tile_map(counts)
    nt = 64

    def tile_cost(g):
        e = max(i for i in range(len(counts)) if tstart[i] <= g)
        m = tstart[e + 1] - tstart[e]
        last = counts[e] - BM * (m - 1)
        return 4 + (last + 63) // 64 if g == tstart[e + 1] - 1 and last <= 192 and m >= 2 else 8

    costs = []
    for xcd in range(X):
        c = 0
        for s in range(10000):
            r = decode(xcd, s, nt, tstart, cpre)
            if r is None:
                break
            c += tile_cost(r[1])
        costs.append(c)
    assert max(costs) <= 1.03 * np.mean(costs)


CH = 4096


def chunk_map(counts):
    nch = [max(1, -(-c // CH)) for c in counts]
    full = [c // CH for c in counts]
    cstart = np.concatenate([[0], np.cumsum(nch)]).astype(int)
    fpre = np.concatenate([[0], np.cumsum(full)]).astype(int)
    corder = [None] * cstart[-1]
    for e in range(len(counts)):
        for c in range(full[e]):
            corder[fpre[e] + c] = cstart[e] + c
    keys = [counts[e] - full[e] * CH if nch[e] > full[e] else -1 for e in range(len(counts))]
    for e, k in enumerate(keys):
        if k >= 0:
            rank = sum(1 for j, kj in enumerate(keys) if kj > k or (kj == k and j < e))
            corder[fpre[-1] + rank] = cstart[e] + full[e]
    return cstart, corder


def chunk_rows(counts, cstart, gc):
    e = expert_of(cstart, lambda v: v, gc)
    return min(CH, counts[e] - (gc - cstart[e]) * CH) if counts[e] else 0


def dw_decode(xcd, slot, per_c, nmat, cstart, corder):
    row = slot // per_c
    pos = row * X + (X - 1 - xcd if row & 1 else xcd)
    if pos >= nmat * cstart[-1]:
        return None
    return pos % nmat, corder[pos // nmat], slot - row * per_c


@pytest.mark.parametrize("counts", routings())
def test_dw_groups_run_once_heaviest_first(counts):
    cstart, corder = chunk_map(counts)
    assert sorted(corder) == list(range(cstart[-1]))
    rows = [chunk_rows(counts, cstart, g) for g in corder]
    assert all(a >= b for a, b in zip(rows, rows[1:]))
    bound = len(counts) + -(-sum(counts) // CH)
    for nmat, per_c in ((1, 3), (2, 5)):
        slots = -(-(nmat * bound) // X) * per_c
        seen = set()
        for xcd in range(X):
            for s in range(slots):
                r = dw_decode(xcd, s, per_c, nmat, cstart, corder)
                if r is not None:
                    assert r not in seen
                    seen.add(r)
        assert len(seen) == nmat * cstart[-1] * per_c


def test_dw_snake_dealing_balances_skewed_routing():
    """Zipf(1.2)-skewed routing over 128 experts (a tile costs its 64-row
    stages plus about 6 stages of prologue and epilogue): dealing the groups
    heaviest first in snake order never leaves an XCD more loaded than dealing
    them round-robin in list order, and with at least 32768 routed rows keeps
    every XCD within 3% of the mean (round-robin: 4-9% over).  With fewer rows
    one 4096-row chunk can outweigh the rest of its XCD's share."""
    rng = np.random.default_rng(7)
    p = 1.0 / np.arange(1, 129) ** 1.2
    for R in (8192, 32768, 65536, 131072):
        counts = list(rng.multinomial(R, p / p.sum()))
        cstart, corder = chunk_map(counts)
        n = cstart[-1]

        def cost(gc):
            return -(-chunk_rows(counts, cstart, gc) // 64) + 6

        snake, rr = np.zeros(X), np.zeros(X)
        for xcd in range(X):
            for s in range(-(-(2 * (128 + -(-R // CH))) // X)):
                r = dw_decode(xcd, s, 1, 2, cstart, corder)
                if r is not None:
                    snake[xcd] += cost(r[1])
        for pos in range(2 * n):
            rr[pos % X] += cost(pos % n)
        assert snake.max() <= rr.max(), (R, snake, rr)
        if R >= 32768:
            assert snake.max() <= 1.03 * snake.mean(), (R, snake)
