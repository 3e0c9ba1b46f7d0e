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
