"""CPU model of the LDS ring hand-over in the bf16 forward kernel.

The ping-pong form runs two wave groups half a tile apart; K and V tiles each
have two LDS buffers (K(t) in buffer t % 2, V(t) in buffer 2 + t % 2), filled
by direct-to-LDS DMAs.  Workgroup barriers are numbered globally; half step
h is the interval between barriers h - 1 and h.  The schedule (group 1 passes
one extra barrier first, so it runs half a tile behind group 0):

    group 0, half step 2s+1: MFMA(s)  = reads V(s-1) (P x V), then K(s) (S = K Q^T)
    group 0, half step 2s+2: softmax(s); issues the DMA of V(s) at its start and
                             waits for it at its end
    group 1, half step 2s+2: MFMA(s); waits for its DMA of K(s+1) at its end
    group 1, half step 2s+3: softmax(s); issues the DMA of K(s+2) at its start
    group 1, half step 1:    issues the DMA of K(1) (prologue; K(0) lands
                             before barrier 0)

A DMA issued in half step a and waited for in half step b writes its buffer
at any time in [a, b]; a read in half step r happens at any time in r; a
barrier orders everything before it against everything after it, and nothing
orders two things inside one half step.  The invariant: every read of tile t
from a buffer happens in a half step after the one in which tile t's DMA
completed (so a barrier publishes the data), and before the half step in
which the next DMA into that buffer is issued (so no write lands while a wave
still reads).  The tests check that invariant for the kernel's schedule and
for the sequential ring, and show that moving each group's DMA to the end of
its own MFMA half step (a variant tried and dropped because its outputs
changed from run to run) breaks it: group 1's DMA of K(s+2) into K(s)'s buffer
is issued in the half step in which the other waves of group 1 still read
K(s).
"""

import itertools

import pytest


def pingpong_events(ntiles, dma_at_end_of_mfma=False):
    """(buffer, tile, kind, first_half_step, last_half_step) for every LDS
    access of one workgroup; kind is 'w' (DMA) or 'r' (operand read)."""
    ev = []
    kbuf = lambda t: ("K", t % 2)      # noqa: E731
    vbuf = lambda t: ("V", t % 2)      # noqa: E731
    ev.append((kbuf(0), 0, "w", -1, 0))           # before barrier 0: all waves, then wait
    if ntiles > 1:
        ev.append((kbuf(1), 1, "w", 1, 2))        # group 1 prologue; waited after its MFMA(0)
    for s in range(ntiles):
        # reads: group 0 MFMA(s) in half step 2s+1, group 1 MFMA(s) in 2s+2
        for h in (2 * s + 1, 2 * s + 2):
            ev.append((kbuf(s), s, "r", h, h))
            if s >= 1:
                ev.append((vbuf(s - 1), s - 1, "r", h, h))
        # group 0: DMA of V(s)
        if dma_at_end_of_mfma:
            ev.append((vbuf(s), s, "w", 2 * s + 1, 2 * s + 2))
        else:
            ev.append((vbuf(s), s, "w", 2 * s + 2, 2 * s + 2))
        # group 1: DMA of K(s+2), waited after its MFMA(s+1) (half step 2s+4)
        if s + 2 < ntiles:
            if dma_at_end_of_mfma:
                ev.append((kbuf(s + 2), s + 2, "w", 2 * s + 2, 2 * s + 4))
            else:
                ev.append((kbuf(s + 2), s + 2, "w", 2 * s + 3, 2 * s + 4))
    # the last P x V (tile ntiles-1) after the loop: group 0 in 2n+1, group 1 in 2n+2
    n = ntiles
    for h in (2 * n + 1, 2 * n + 2):
        ev.append((vbuf(n - 1), n - 1, "r", h, h))
    return ev


def sequential_events(ntiles, stages):
    """The sequential form: tile t (K and V) in ring slot t % stages; the DMAs
    of tile t + stages - 1 are issued at the start of step t, and tile t + 1
    is waited for at its end; every wave reads tile t in step t; one barrier
    ends each step (half step h = step h here)."""
    ahead = stages - 1
    ev = []
    for t in range(min(ahead, ntiles)):
        ev.append((("KV", t % stages), t, "w", -1, 0))
    for t in range(ntiles):
        if t + ahead < ntiles:
            # issued in step t, completed by the end of step t + ahead - 1
            ev.append((("KV", (t + ahead) % stages), t + ahead, "w", t + 1, t + ahead))
        ev.append((("KV", t % stages), t, "r", t + 1, t + 1))
    return ev


def check(events):
    """Violations of the hand-over invariant, as readable strings."""
    bad = []
    by_buf = {}
    for e in events:
        by_buf.setdefault(e[0], []).append(e)
    for buf, evs in by_buf.items():
        writes = {e[1]: e for e in evs if e[2] == "w"}
        for (_, tile, kind, r0, r1) in evs:
            if kind != "r":
                continue
            w = writes[tile]
            if not r0 > w[4]:
                bad.append(f"{buf}: tile {tile} read in half step {r0} before its DMA completed ({w[4]})")
            nxt = [x for t, x in writes.items() if t > tile]
            if nxt:
                n = min(nxt, key=lambda x: x[1])
                if not r1 < n[3]:
                    bad.append(f"{buf}: tile {tile} read in half step {r1} while tile {n[1]}'s DMA "
                               f"(issued in {n[3]}) writes the buffer")
    return bad


@pytest.mark.parametrize("ntiles", [1, 2, 3, 4, 7, 12])
def test_pingpong_schedule_keeps_the_invariant(ntiles):
    assert check(pingpong_events(ntiles)) == []


@pytest.mark.parametrize("ntiles,stages", list(itertools.product([1, 2, 5, 9], [2, 3, 4])))
def test_sequential_ring_keeps_the_invariant(ntiles, stages):
    assert check(sequential_events(ntiles, stages)) == []


def test_dma_at_end_of_mfma_half_step_races():
    """The dropped variant: group 1 issues K(s+2) into K(s)'s buffer at the end
    of its own MFMA(s) half step, in which the other waves of group 1 may
    still read K(s); nothing but a barrier orders waves of one group."""
    bad = check(pingpong_events(6, dma_at_end_of_mfma=True))
    assert any(b.startswith("('K', 0): tile 0 read in half step 2 while tile 2") for b in bad), bad
    # the V side of that variant stays ordered: V(s) reuses V(s-2)'s buffer,
    # whose last reader finished in half step 2s
    assert not any(b.startswith("('V'") for b in bad), bad


def test_model_detects_a_missing_wait():
    """A planted fault in the model (the K(s+2) DMA waited one half step too
    late) must be caught: the reads of K(s+2) by group 0 would see it land."""
    ev = [(b, t, k, a, (z + 1 if (k == "w" and b[0] == "K" and t >= 2) else z))
          for (b, t, k, a, z) in pingpong_events(5)]
    assert check(ev)


# ---------------------------------------------------------------------------
# The two-group dK/dV backward kernel: 32-row blocks of Q, dO and their row
# statistics in a five-buffer ring (block X in buffer X % 5); group 0 takes
# the even blocks, group 1 the odd ones.  Block X is read in half step X+1
# (S, dP by rows, its group's MFMA phase), X+2 (its statistics, the group's
# VALU phase) and X+3 (dV, dK by transpose reads, the group's next MFMA
# phase).  In half step h the group on the VALU issues the DMA of block h+1
# and waits for it at the end of half step h+1; the prologue loads blocks 0
# and 1 before barrier 0, and group 1 issues block 2 in half step 1.

def dkdv_events(nqb, nbuf=5, issue_lead=1):
    buf = lambda x: ("QdO", x % nbuf)  # noqa: E731
    ev = []
    for x in range(min(2, nqb)):
        ev.append((buf(x), x, "w", -1, 0))
    for x in range(2, nqb):
        h = x - issue_lead  # issued at the start of half step x - 1
        ev.append((buf(x), x, "w", h, x))
    for x in range(nqb):
        for h in (x + 1, x + 2, x + 3):
            ev.append((buf(x), x, "r", h, h))
    return ev


def dkdv_barriers(nqb, grp):
    """Workgroup barriers one wave of group grp passes in the kernel (the
    prologue, two per step, the count-evening barriers, the final one)."""
    ng = nqb // 2 if grp else (nqb + 1) // 2
    n = 1 + (1 if grp else 0) + 2 * ng
    n += 1 if (nqb % 2 == 0) == (grp == 0) else 0
    return n + 1


@pytest.mark.parametrize("nqb", [1, 2, 3, 4, 5, 6, 7, 11, 64])
def test_dkdv_ring_keeps_the_invariant(nqb):
    assert check(dkdv_events(nqb)) == []


def test_dkdv_ring_of_four_races():
    """With four buffers block X+4 would land in block X's buffer while its
    transpose reads (half step X+3) may still run."""
    bad = check(dkdv_events(9, nbuf=4))
    assert bad and all("while tile" in b for b in bad), bad


@pytest.mark.parametrize("nqb", range(1, 40))
def test_dkdv_groups_pass_the_same_barriers(nqb):
    assert dkdv_barriers(nqb, 0) == dkdv_barriers(nqb, 1)


def test_dkdv_half_step_of_each_phase():
    """Group g's MFMA phase of its block X falls in half step X+1 and its VALU
    phase in X+2: group 0 starts right after barrier 0, group 1 after its
    extra barrier 1, and every step is two half steps."""
    for grp in (0, 1):
        start = 1 + grp  # barriers passed before the first MFMA phase
        for j in range(6):
            x = 2 * j + grp
            assert start + 2 * j == x + 1       # MFMA phase
            assert start + 2 * j + 1 == x + 2   # VALU phase
