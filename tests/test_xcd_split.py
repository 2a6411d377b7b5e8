"""Host-side model of how the tiled prefill GEMM hands its work items to the
eight XCDs, checked on random routings.

The kernel (gemm_prefill_tiled_kernel) orders items (expert, row stripe,
token tile), gives XCD x a contiguous range whose estimated work (a fixed
cost per item plus its active 16-token sub-tiles) is about an eighth of the
total, and clamps every range to the G workgroups the grid holds per XCD.
An expert's token tiles share its 16-token sub-tiles evenly (the first
ones one more).
This file restates that integer arithmetic and checks what the kernel's
correctness rests on: the ranges partition the items exactly, none exceeds
G, every lookup stays inside the tile table, and on skewed routings the
ranges carry near-equal work.  The GPU parity tests cover the kernel itself.
"""
import numpy as np
import pytest

TOKENS = 128      # tokens per prefill tile
ROWS = 256        # weight rows per workgroup
TILE_COST = 4     # the kernel's fixed cost per item, in 16-token sub-tiles


def cdiv(a, b):
    return -(-a // b)


def token_tile(c, q):
    """(first row, rows) of token tile q of an expert with c tokens."""
    nt, nsub = cdiv(c, TOKENS), cdiv(c, 16)
    base, extra = divmod(nsub, nt)
    first = 16 * (q * base + min(q, extra))
    return first, min(16 * (base + (1 if q < extra else 0)), c - first)


def weighted_bounds(cnt, R, c0):
    """The nine weighted range bounds before clamping, the grid's G per XCD,
    the item count and the tile and cost prefixes."""
    E = len(cnt)
    ns = cdiv(R, ROWS)
    toff = np.concatenate([[0], np.cumsum([cdiv(c, TOKENS) for c in cnt])]).astype(np.int64)
    max_tiles = cdiv(int(sum(cnt)), TOKENS) + E      # the host's grid bound
    G = cdiv(max_tiles * ns, 8)
    nvalid = int(toff[E]) * ns
    cost = [c0 * cdiv(c, TOKENS) + cdiv(c, 16) for c in cnt]
    woff = np.concatenate([[0], np.cumsum(cost)]).astype(np.int64)
    W = int(woff[E]) * ns
    bnd = []
    for lane in range(9):
        target = (W * lane + 7) // 8
        if lane == 0:
            b = 0
        elif lane < 8 and target < W:
            j = upper(woff, target, E, ns)
            gc = int(woff[j + 1] - woff[j])
            nt = int(toff[j + 1] - toff[j])
            assert gc > 0 and nt > 0
            rem = target - int(woff[j]) * ns
            st, r2 = rem // gc, rem % gc
            assert 0 <= st < ns
            b = int(toff[j]) * ns + st * nt + first_tile_at(r2, gc, nt, c0)
        else:
            b = nvalid
        bnd.append(b)
    return bnd, G, nvalid, ns, toff


def first_tile_at(r2, gc, nt, c0):
    """First token tile q of an expert whose cost prefix reaches r2 (nt if
    none): the expert's gc - c0 * nt sub-tiles are split evenly over its nt
    tiles, the first `extra` taking one more."""
    nsub = gc - c0 * nt
    base, extra = divmod(nsub, nt)
    costs = [c0 + base + (1 if q < extra else 0) for q in range(nt)]
    p = 0
    for q in range(nt):
        if p >= r2:
            return q
        p += costs[q]
    return nt


def upper(arr, v, E, ns):
    """Largest j in [0, E) with arr[j] * ns <= v (arr[0] = 0)."""
    lo, hi = 0, E
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if arr[mid] * ns <= v:
            lo = mid
        else:
            hi = mid
    return lo


def split(cnt, R, c0):
    """Per-XCD work of the clamped ranges, checking the partition."""
    E = len(cnt)
    bnd, G, nvalid, ns, toff = weighted_bounds(cnt, R, c0)
    bnd = list(bnd)
    for x in range(8):
        bnd[x + 1] = min(max(bnd[x + 1], bnd[x]), bnd[x] + G)
    bnd[8] = nvalid
    for x in range(7, 0, -1):
        bnd[x] = max(bnd[x], bnd[x + 1] - G)

    seen = np.zeros(nvalid, np.int64)
    work = np.zeros(8)
    for x in range(8):
        first, last = bnd[x], bnd[x + 1]
        assert 0 <= first <= last <= nvalid and last - first <= G
        for item in range(first, last):
            j = upper(toff, item, E, ns)
            nt = int(toff[j + 1] - toff[j])
            assert nt > 0
            local = item - int(toff[j]) * ns
            stripe, tile = local // nt, int(toff[j]) + local % nt
            assert 0 <= stripe < ns and toff[j] <= tile < toff[j + 1]
            ntok = token_tile(cnt[j], tile - int(toff[j]))[1]
            assert ntok > 0
            seen[item] += 1
            work[x] += c0 + cdiv(ntok, 16)
    assert np.all(seen == 1)
    return work


@pytest.mark.parametrize("seed", range(6))
def test_ranges_partition_the_items(seed):
    rng = np.random.default_rng(seed)
    for trial in range(60):
        E = int(rng.integers(2, 257))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 3000))
        mode = trial % 4
        if mode == 0:
            p = rng.dirichlet(np.full(E, 0.3))
        elif mode == 1:
            p = np.full(E, 1.0 / E)
        elif mode == 2:          # a tenth of the experts take everything
            p = np.zeros(E)
            p[: max(1, E // 10)] = 1.0
            p /= p.sum()
        else:
            p = rng.dirichlet(np.full(E, 5.0))
        cnt = rng.multinomial(T * k, p).tolist()
        split(cnt, int(rng.choice([64, 96, 300, 2880, 5760])), int(rng.choice([0, 2, 4])))


def test_token_tiles_split_evenly():
    """An expert's tiles cover its rows in order, hold at most 128 rows,
    and differ by at most one 16-row sub-tile (the last may be ragged)."""
    for c in range(1, 3000):
        nt = cdiv(c, TOKENS)
        tiles = [token_tile(c, q) for q in range(nt)]
        assert tiles[0][0] == 0 and sum(r for _, r in tiles) == c
        assert all(tiles[q][0] + tiles[q][1] == tiles[q + 1][0] for q in range(nt - 1))
        assert all(0 < r <= TOKENS for _, r in tiles)
        subs = [cdiv(r, 16) for _, r in tiles]
        assert sum(subs) == cdiv(c, 16) and max(subs) - min(subs) <= 1


def test_single_token_and_empty_experts():
    split([0, 1, 0, 0], 64, TILE_COST)
    split([0] * 255 + [3], 5760, TILE_COST)
    split([1] * 256, 5760, TILE_COST)


def test_skewed_routing_balances_work():
    """A 120b-sized skewed routing (128 experts, counts from 3 to ~940): the
    busiest XCD carries within 1% of the mean work."""
    rng = np.random.default_rng(7)
    p = rng.dirichlet(np.full(128, 1.0))
    cnt = rng.multinomial(4096 * 4, p).tolist()
    w = split(cnt, 5760, TILE_COST)
    assert w.max() / w.mean() < 1.01
