"""CPU model of the prefill kernel's K/V ring schedule (csrc/prefill_bf16.hip).

Tile t of a pass lives in ring slot t % R (R = 2 for four-wave workgroups,
4 for eight-wave ones); with P = R / 2, step t issues the copies of K(t+P+1)
and V(t+P), reads K(t+1) (the next tile's scores) and V(t) (this tile's
products), and the workgroup barrier -- after each wave has waited for its own
copies (vmcnt) and its LDS reads (lgkmcnt) -- closes every P-th step and the
pass's last one.  The prologue issues K(0..P) and V(0..P-1), waits, takes a
barrier, reads K(0), and takes a second barrier.

Between two barriers the waves of a workgroup may be anywhere, so a copy
counts as landed only after the barrier that follows the step that issued it,
and a slot may be refilled only in a barrier interval after every read of its
previous tile.  The model checks both for every tile count up to 64.
"""

import pytest


def ring_events(R, ntiles):
    """(writes, reads): writes[(kind, tile)] = (slot, epoch); reads = [(kind, tile, slot, epoch)]."""
    P = R // 2
    writes, reads = {}, []
    epoch = 0
    for t in range(min(P + 1, ntiles)):
        writes[("K", t)] = (t % R, epoch)
    for t in range(min(P, ntiles)):
        writes[("V", t)] = (t % R, epoch)
    epoch += 1  # wait + barrier
    reads.append(("K", 0, 0, epoch))
    epoch += 1  # second prologue barrier
    for t in range(ntiles):
        if t + P + 1 < ntiles:
            writes[("K", t + P + 1)] = ((t + P + 1) % R, epoch)
        if t + P < ntiles:
            writes[("V", t + P)] = ((t + P) % R, epoch)
        if t + 1 < ntiles:
            reads.append(("K", t + 1, (t + 1) % R, epoch))
        reads.append(("V", t, t % R, epoch))
        if t % P == P - 1 or t == ntiles - 1:
            epoch += 1
    return writes, reads


def check_schedule(R, ntiles):
    writes, reads = ring_events(R, ntiles)
    for kind, tile, slot, epoch in reads:
        wslot, wepoch = writes[(kind, tile)]
        assert wslot == slot
        assert epoch > wepoch, f"R={R} n={ntiles}: {kind}({tile}) read before its copy landed"
        for (k2, t2), (s2, e2) in writes.items():
            if k2 == kind and s2 == slot and t2 > tile:
                assert epoch < e2, f"R={R} n={ntiles}: {kind}({tile}) read in the interval that refills its slot"


@pytest.mark.parametrize("R", [2, 4])
def test_ring_schedule_is_race_free(R):
    for n in range(1, 65):
        check_schedule(R, n)


def test_model_catches_a_too_early_refill():
    """Planted mistake: with four slots, issuing K three tiles ahead of the
    read (one more than the schedule allows) overwrites a slot still being read."""
    R, n = 4, 12
    writes, reads = ring_events(R, n)
    P = R // 2
    bad = dict(writes)
    epoch = 2
    for t in range(n):  # K(t+P+2) issued at step t instead of K(t+P+1)
        if t + P + 2 < n:
            bad[("K", t + P + 2)] = ((t + P + 2) % R, epoch)
        if t % P == P - 1 or t == n - 1:
            epoch += 1
    failed = False
    for kind, tile, slot, ep in reads:
        for (k2, t2), (s2, e2) in bad.items():
            if k2 == kind and s2 == slot and t2 > tile and ep >= e2:
                failed = True
    assert failed
