"""Host-side check of the persistent causal schedule's index arithmetic, as the
forward kernel and both backward kernels compute it: pairs of blocks
(n - 1 - r, r) of every head, contiguous pair ranges per XCD (workgroup id mod
8), each XCD's workgroups taking its pairs in turn, the heavy block of a pair
first and a lone middle block (odd n) once. Every block of every head must be
run exactly once, by a workgroup of the XCD that owns its pair, and the busiest
workgroup may run at most one pair more than the least busy one. The GPU side
(tests/test_persistent_gpu.py) checks the kernels' outputs against
one-block-per-workgroup launches bit for bit.
"""

from __future__ import annotations

import collections

import pytest


def schedule(n_bh: int, nb: int, grid: int):
    """{workgroup: [(bh, block), ...]} in the order the kernel runs them."""
    npair = (nb + 1) // 2
    all_pairs = n_bh * npair
    per_xcd = grid >> 3
    out = {}
    for wg in range(grid):
        xcd = wg & 7
        p_lo, p_hi = all_pairs * xcd // 8, all_pairs * (xcd + 1) // 8
        work = []
        wi = 0
        while True:
            p = p_lo + (wg >> 3) + (wi >> 1) * per_xcd
            if p >= p_hi:
                break
            bh, r = divmod(p, npair)
            blk = r if wi & 1 else nb - 1 - r
            if not ((wi & 1) and blk == nb - 1 - r):
                work.append((bh, blk))
            wi += 1
        out[wg] = work
    return out


@pytest.mark.parametrize("n_bh,nb,grid", [
    (128, 16, 256), (16, 63, 256), (128, 32, 512), (256, 3, 512), (128, 4, 256),
    (4096, 1, 256), (7, 5, 24), (3, 9, 8), (1000, 2, 256), (13, 64, 256),
])
def test_every_block_once(n_bh, nb, grid):
    sched = schedule(n_bh, nb, grid)
    count = collections.Counter(item for work in sched.values() for item in work)
    assert set(count) == {(bh, b) for bh in range(n_bh) for b in range(nb)}
    assert max(count.values()) == 1
    # pairs stay on the XCD that owns them: the heads in flight on an XCD
    # are a contiguous range
    for wg, work in sched.items():
        npair = (nb + 1) // 2
        xcd = wg & 7
        lo, hi = n_bh * npair * xcd // 8, n_bh * npair * (xcd + 1) // 8
        for bh, b in work:
            r = min(b, nb - 1 - b)
            assert lo <= bh * npair + r < hi
    # balance in pairs: at most one pair apart
    pairs = [sum(1 for _, b in work if b >= nb - 1 - b) for work in sched.values()]
    assert max(pairs) - min(pairs) <= 1


def test_paired_costs_are_equal():
    """Block r of a causal self-attention head costs about r + 1 key tiles (or
    n - r query tiles for a key block); paired blocks add up to n + 1."""
    for nb in (1, 2, 3, 16, 63):
        npair = (nb + 1) // 2
        sums = {(nb - 1 - r + 1) + (r + 1 if r != nb - 1 - r else 0) for r in range(npair)}
        assert sums <= {nb + 1, (nb + 1) // 2}
