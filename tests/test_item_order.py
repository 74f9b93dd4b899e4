"""CPU model of the forward kernel's block -> work item map for batch
entries with their own key counts (no GPU).

The kernel deals blocks to the 8 XCDs round-robin (block i runs on XCD
i mod 8, in order of i) and map_block turns block i into a position so that
each XCD receives a contiguous eighth of the positions.  kvlen_item then
turns a position into (entry, head, query tile): group x of the positions
holds, for every entry, the items [x M / 8, (x + 1) M / 8) of that entry
(M = heads x query tiles), entry after entry in order of decreasing key
count (ties by index; index order beyond 64 entries).  The formulas restate
the kernel's (attn_fwd_kernel.hip); the checks are what the map must give:
every item exactly once, every XCD an equal share of each entry, and each
XCD's blocks longest entry first.
"""
import numpy as np
import pytest


def map_block(bid, n):
    xcd, slot = bid & 7, bid >> 3
    per, rem = n >> 3, n & 7
    return xcd * per + min(xcd, rem) + slot


def kvlen_item(pos, B, H, nq, lens, skv):
    M = H * nq
    base = 0
    x = 0
    while x < 7:
        c = ((x + 1) * M >> 3) - (x * M >> 3)
        if pos < base + B * c:
            break
        base += B * c
        x += 1
    c = ((x + 1) * M >> 3) - (x * M >> 3)
    assert c > 0
    t = pos - base
    r, k = t // c, (x * M >> 3) + t % c
    b = r
    if B <= 64:
        ln = [min(max(v, 0), skv) for v in lens]
        rank = [sum(1 for u in range(B) if ln[u] > ln[t_] or (ln[u] == ln[t_] and u < t_)) for t_ in range(B)]
        assert sorted(rank) == list(range(B))
        b = rank.index(r)
    return b, k // nq, k % nq


SHAPES = [(1, 1, 1), (3, 4, 2), (4, 12, 32), (5, 3, 7), (2, 1, 3), (70, 2, 1), (64, 3, 5), (7, 16, 9)]


@pytest.mark.parametrize("B,H,nq", SHAPES)
def test_every_item_once_and_balanced(B, H, nq):
    rng = np.random.default_rng(B * 1000 + H * 10 + nq)
    skv = 5000
    lens = [int(v) for v in rng.integers(-3, skv + 200, size=B)]
    if B > 2:
        lens[1] = lens[2]                                  # a tie
    n = B * H * nq
    seen = set()
    per_xcd = [[] for _ in range(8)]
    for bid in range(n):
        item = kvlen_item(map_block(bid, n), B, H, nq, lens, skv)
        assert 0 <= item[0] < B and 0 <= item[1] < H and 0 <= item[2] < nq
        seen.add(item)
        per_xcd[bid & 7].append(item)
    assert len(seen) == n
    clamp = [min(max(v, 0), skv) for v in lens]
    M = H * nq
    if M % 8 == 0:
        # each XCD: M / 8 items of every entry, in dispatch order longest entry first
        for x in range(8):
            got = per_xcd[x]
            for b in range(B):
                assert sum(1 for it in got if it[0] == b) == M // 8
            if B <= 64:
                keys = [clamp[it[0]] for it in got]
                assert keys == sorted(keys, reverse=True)


def test_longest_first_on_the_paged_workload():
    """The paged-cache workload (4 entries, 12 heads, 32 query tiles): every
    XCD starts with the longest entry and ends with the shortest."""
    B, H, nq = 4, 12, 32
    lens = [12000, 32760, 4100, 20480]
    n = B * H * nq
    for x in range(8):
        bids = [bid for bid in range(n) if bid & 7 == x]
        ents = [kvlen_item(map_block(bid, n), B, H, nq, lens, 32760)[0] for bid in bids]
        assert ents == [1] * 48 + [3] * 48 + [0] * 48 + [2] * 48
