"""CPU model of the prefill kernel's work order (csrc/prefill_bf16.hip), dense inputs.

Workgroup ids are dealt round-robin to the 8 XCDs; when the item count is a
multiple of 8 each XCD runs a contiguous range of work items, ordered (block
of KV groups, slot, group in the block, query head of the group), a block
holding at least block_heads query heads.  Under the causal mask slot s runs
query tile n-1-s and then its mirror s (once when they coincide).  The model
re-derives, for every workgroup id of the grid, the (batch-head, query tile)
passes the kernel runs and checks that every query tile of every head is run
exactly once.
"""

import pytest


def block_heads_for(n_slots):
    return 4 if n_slots < 16 else 1


def kernel_passes(B, Hq, Hkv, N, waves, causal, mirror=None):
    rows = 32 * waves
    n_qtiles = (N + rows - 1) // rows
    n_slots = (n_qtiles + 1) // 2 if causal else n_qtiles
    n_items = n_slots * B * Hq
    block_heads = block_heads_for(n_slots)
    G = Hq // Hkv
    n_groups = n_items // (n_slots * G)
    BG = 1 if G >= block_heads else (block_heads + G - 1) // G
    per_block = BG * G * n_slots
    mirror = mirror or (lambda n, s: n - 1 - s)
    runs = []
    for blk_id in range(n_items):
        item = blk_id
        if n_items % 8 == 0:
            item = (blk_id & 7) * (n_items >> 3) + (blk_id >> 3)
        blk = item // per_block
        rem = item - blk * per_block
        gib = min(BG, n_groups - blk * BG)
        tslot = rem // (gib * G)
        r2 = rem - tslot * gib * G
        gi = r2 // G
        grp = blk * BG + gi
        b, g = divmod(grp, Hkv)
        h = g * G + (r2 - gi * G)
        for p in range(2 if causal else 1):
            qtile = tslot if not causal else (mirror(n_qtiles, tslot) if p == 0 else tslot)
            if causal and (tslot > n_qtiles - 1 - tslot or (p == 1 and tslot == n_qtiles - 1 - tslot)):
                continue
            runs.append((blk_id, b * Hq + h, qtile))
    return runs, n_qtiles


def coverage(runs):
    seen = {}
    for blk_id, bh, qtile in runs:
        seen[(bh, qtile)] = seen.get((bh, qtile), 0) + 1
    return seen


@pytest.mark.parametrize("B,Hq,Hkv,N,waves,causal", [
    (4, 32, 32, 4096, 4, True),      # causal MHA 4K
    (2, 32, 8, 16384, 8, True),      # causal GQA 16K
    (1, 64, 8, 131072, 8, True),     # causal GQA 128K
    (2, 32, 8, 8192, 8, True), (1, 3, 1, 1000, 4, True), (1, 8, 2, 4500, 8, True), (3, 5, 5, 777, 4, True),
    (1, 1, 1, 1, 4, True), (2, 6, 3, 300, 4, True), (1, 16, 16, 2049, 4, True), (2, 12, 4, 700, 4, True),
    (4, 32, 32, 4096, 8, False), (1, 3, 1, 1000, 4, False), (2, 6, 3, 300, 4, False)])
def test_every_query_tile_runs_once(B, Hq, Hkv, N, waves, causal):
    runs, n_qtiles = kernel_passes(B, Hq, Hkv, N, waves, causal)
    seen = coverage(runs)
    assert all(0 <= q < n_qtiles and 0 <= bh < B * Hq for bh, q in seen)
    assert len(seen) == B * Hq * n_qtiles and set(seen.values()) == {1}


def test_causal_workgroups_carry_equal_work():
    """Paired causal tiles: every workgroup of the 4K workload streams
    n + 1 key-tile rows in all (tile i of 128 rows sees i + 1 such rows)."""
    runs, n_qtiles = kernel_passes(4, 32, 32, 4096, 4, True)
    per_wg = {}
    for blk_id, bh, q in runs:
        per_wg[blk_id] = per_wg.get(blk_id, 0) + q + 1
    assert set(per_wg.values()) == {n_qtiles + 1}


def test_model_catches_a_wrong_mirror():
    """Planted mistake: the heavy tile of slot s taken as n - s instead of
    n - 1 - s leaves one tile of every head unrun."""
    runs, n_qtiles = kernel_passes(2, 32, 8, 16384, 8, True, mirror=lambda n, s: n - s if s else n - 1)
    seen = coverage(runs)
    assert len(seen) < 2 * 32 * n_qtiles or max(seen.values()) > 1
