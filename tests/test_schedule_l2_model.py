"""How often the causal forward's dispatch order makes one XCD fetch each K/V tile.

A least-recently-used model of one XCD's L2 (capacity counted in 128-key tiles of K plus V,
64 KiB each at d = 128) replays the causal forward's work order at the headline shape
(H = 32, N = 32768, BM = 256, BN = 128): every query tile of a head runs on one XCD (heads
dealt to XCDs round-robin, so 4 heads per XCD, one after the other), longest query tile
first, one workgroup per CU on the XCD's 32 CUs, a freed CU taking the next workgroup, and
every workgroup reading one key tile per step.  Generation g is the g-th group of 32
workgroups of a head; with the snake order, odd generations walk their keys down from the
diagonal, so that they start on the tiles the previous generation read last.

The I/O floor ("I/O Analysis is All You Need", abstract: I/O-optimal tiling and
scheduling; "IO-Aware Algorithms", How it works: each tile of K and V brought on chip as
few times as the on-chip capacity allows) is one read of every K/V tile.  With 32 resident
256-row query tiles the causal triangle needs 2.5 K/V reads per head if no tile survives in
L2 between generations; the snake order's reuse at each change of generation brings the
model to 2.0-2.13 reads for 64-48 tiles of L2 (the measured kernel: 2.09), and none of
the orders below does better by more than 0.5% at any of those capacities.  Bytes fetched
beyond L2 come to (Q + O + r * (K + V)) / T_min, i.e. 1.5x T_min at r = 2.0: the traffic
target sits exactly at this order's model with the whole 4 MiB L2 holding K and V.
"""

import collections

import pytest

N_QTILES = 128        # 32768 rows / BM 256
KT_PER_QTILE = 2      # key tiles of 128 per query tile (BM / BN)
HEADS_PER_XCD = 4     # 32 heads over 8 XCDs
CUS_PER_XCD = 32
RESIDENT = 32         # one 8-wave workgroup per CU


def kv_reads_per_tile(order, cap_tiles):
    """Replay `order` (a list of (head, key tiles in visiting order)) on CUS_PER_XCD CUs
    that each take the next workgroup when free, through an LRU cache of cap_tiles key
    tiles; return fetched tiles / distinct (head, tile) pairs."""
    lru = collections.OrderedDict()
    misses = 0
    it = iter(order)
    slots = [None] * CUS_PER_XCD

    def take(c):
        nxt = next(it, None)
        slots[c] = None if nxt is None else [nxt[0], nxt[1], 0]

    for c in range(CUS_PER_XCD):
        take(c)
    while any(s is not None for s in slots):
        for c in range(CUS_PER_XCD):
            s = slots[c]
            if s is None:
                continue
            key = (s[0], s[1][s[2]])
            if key in lru:
                lru.move_to_end(key)
            else:
                misses += 1
                lru[key] = True
                if len(lru) > cap_tiles:
                    lru.popitem(last=False)
            s[2] += 1
            if s[2] == len(s[1]):
                take(c)
    return misses / (HEADS_PER_XCD * N_QTILES * KT_PER_QTILE)


def work_order(longest_first=True, direction=lambda gen: "down" if gen % 2 else "up", period=RESIDENT):
    """The XCD's workgroups in dispatch order: for each head, its query tiles (longest
    first, as the kernel does for causal masks, or shortest first), each with its key
    tiles 0 .. 2 qt + 1 walked up or down by its generation (position // period)."""
    order = []
    for h in range(HEADS_PER_XCD):
        for pos in range(N_QTILES):
            qt = N_QTILES - 1 - pos if longest_first else pos
            tiles = list(range((qt + 1) * KT_PER_QTILE))
            if direction(pos // period) == "down":
                tiles.reverse()
            order.append((h, tiles))
    return order


def test_model_floor_and_no_reuse_bounds():
    # with L2 large enough for a whole head's K/V (256 tiles) every tile is fetched once
    assert kv_reads_per_tile(work_order(), 256) == pytest.approx(1.0)
    # all generations walking up with enough L2 for one generation's spread: every
    # generation refetches its whole key range, 1 + 3/4 + 1/2 + 1/4 = 2.5
    assert kv_reads_per_tile(work_order(direction=lambda g: "up"), 64) == pytest.approx(2.5)


@pytest.mark.parametrize("cap", [48, 56, 64])
def test_kernel_order_is_within_half_a_percent_of_the_best(cap):
    kernel = kv_reads_per_tile(work_order(), cap)
    assert 1.99 <= kernel <= 2.14
    alternatives = {
        "all up": work_order(direction=lambda g: "up"),
        "all down": work_order(direction=lambda g: "down"),
        "inverted snake": work_order(direction=lambda g: "up" if g % 2 else "down"),
        "shortest first, snake": work_order(longest_first=False),
        "snake every 16": work_order(period=16),
        "snake every 64": work_order(period=64),
    }
    # none reads fewer tiles by more than 0.5% (at 64 tiles the inverted snake reads 2.000
    # against 2.008; below that it thrashes: 51-54)
    for name, order in alternatives.items():
        assert kv_reads_per_tile(order, cap) >= kernel * 0.995, name


def test_traffic_at_two_reads_is_the_target():
    # Q, O and one copy of K, V are a quarter of T_min each (N_q = N_kv, same d and dtype)
    def traffic_over_tmin(r):
        return (1 + 1 + r * 2) / 4

    assert traffic_over_tmin(2.0) == pytest.approx(1.5)
    assert traffic_over_tmin(2.09) == pytest.approx(1.545)
