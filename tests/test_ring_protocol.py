"""Host model of the attention kernel's LDS ring protocols (no GPU).

Each loop is replayed as per-wave event lists cut by the workgroup barriers:
a wave's LDS reads of a tile (QK reads K, the V fragment reads) and its
issue of a tile's loads into a slot. The checks are the two conditions the
kernel relies on:

* a slot is refilled only after every wave has passed a barrier that follows
  its last read of the tile the slot held;
* a tile is read only after a barrier that follows every wave's wait for its
  own share of that tile's loads.

Modelled here: the dense two-tile loop with lagged pairs (ring of 4
[K | V] slots, the lagging half's PV of the step's second tile deferred past
the next barrier from registers, its loads issued after that PV) and the
vertical-slash loop with separate rings (K in 3 slots two tiles ahead, V in 2
slots one tile ahead).
"""
from __future__ import annotations

import itertools

import pytest


def _check(events, n_waves):
    """events[w]: list of (phase, kind, ring, tile, slot) in program order, phase =
    number of barriers the wave has passed. kind: 'issue' (loads of `tile`
    into `slot`, landed by the wave's wait before its next barrier) or 'read'."""
    holder = {}                      # slot -> (tile, phase of its issue)
    issued = {}                      # (tile, ring) -> phase the loads were issued in
    last_read = {}                   # (tile, ring) -> max phase of a read, over all waves
    for w in range(n_waves):
        for phase, kind, ring, tile, slot in events[w]:
            if kind == "read":
                last_read[(tile, ring)] = max(last_read.get((tile, ring), -1), phase)
    issues = sorted((phase, ring, tile, slot) for w in range(n_waves)
                    for phase, kind, ring, tile, slot in events[w] if kind == "issue")
    for phase, ring, tile, slot in issues:           # all waves, in barrier order
        prev = holder.get((ring, slot))
        if prev is not None and prev[0] != tile:
            # every read of the previous tile happened in an earlier phase
            assert last_read.get((prev[0], ring), -1) < phase, (ring, slot, prev[0], tile, phase)
        holder[(ring, slot)] = (tile, phase)
        issued[(tile, ring)] = min(issued.get((tile, ring), 1 << 30), phase)
    for w in range(n_waves):
        for phase, kind, ring, tile, slot in events[w]:
            if kind == "read":
                # loads issued in phase p land before barrier p+1 (each wave waits for its own first)
                assert issued[(tile, ring)] < phase, (ring, tile, phase)
                assert holder_at(events, ring, slot, tile, phase, n_waves), (ring, tile, slot, phase)


def holder_at(events, ring, slot, tile, phase, n_waves):
    """No other tile is issued into `slot` in a phase <= `phase` after `tile` was."""
    issues = sorted({(p, t) for w in range(n_waves) for p, k, r, t, s in events[w]
                     if k == "issue" and r == ring and s == slot})
    current = None
    for p, t in issues:
        if p <= phase:
            current = t
    return current == tile


def dense_lagged(n_tiles, active, n_waves=8, ns=4):
    """active[w][j]: whether wave w computes tile j (its rows reach it)."""
    ev = [[] for _ in range(n_waves)]
    for w in range(n_waves):
        lag = w >= n_waves // 2
        phase = 0
        for j in (0, 1):             # prologue loads, before the first barrier
            if j < n_tiles:
                ev[w].append((phase, "issue", "kv", j, j % ns))
        pend = False
        n = 0
        while 2 * n < n_tiles:
            phase = n + 1            # barrier n passed
            nxt = [t for t in (2 * n + 2, 2 * n + 3) if t < n_tiles]
            if not lag:
                for t in nxt:
                    ev[w].append((phase, "issue", "kv", t, t % ns))
            if pend:
                pend = False         # deferred PV: registers only, no LDS read
            if lag:
                for t in nxt:
                    ev[w].append((phase, "issue", "kv", t, t % ns))
            for i in (0, 1):
                t = 2 * n + i
                if t < n_tiles and active[w][t]:
                    ev[w].append((phase, "read", "kv", t, t % ns))     # QK reads K, then V fragments
                    if lag and i == 1:
                        pend = True
            n += 1
    return ev


def sparse_split(n_tiles, active, n_waves=4):
    ev = [[] for _ in range(n_waves)]
    for w in range(n_waves):
        phase = 0
        if n_tiles > 0:
            ev[w].append((phase, "issue", "k", 0, 0))
            ev[w].append((phase, "issue", "v", 0, 0))
        if n_tiles > 1:
            ev[w].append((phase, "issue", "k", 1, 1))
        for n in range(n_tiles):
            phase = n + 1
            if n + 1 < n_tiles:
                ev[w].append((phase, "issue", "v", n + 1, (n + 1) % 2))
            if n + 2 < n_tiles:
                ev[w].append((phase, "issue", "k", n + 2, (n + 2) % 3))
            if active[w][n]:
                ev[w].append((phase, "read", "k", n, n % 3))
                ev[w].append((phase, "read", "v", n, n % 2))
    return ev


@pytest.mark.parametrize("n_tiles", range(1, 12))
def test_dense_lagged_ring(n_tiles):
    # causal activity: wave w's rows reach tile j when j <= w // 2 + base (waves 0..7 of a 256-row block)
    for base in (0, 1, n_tiles):
        active = [[j <= base + w // 2 for j in range(n_tiles)] for w in range(8)]
        _check(dense_lagged(n_tiles, active), 8)
    _check(dense_lagged(n_tiles, [[True] * n_tiles for _ in range(8)]), 8)


@pytest.mark.parametrize("n_tiles", range(1, 9))
def test_sparse_split_rings(n_tiles):
    # every pattern of which query tile (waves 0-1 or 2-3) each visited tile is active for
    for bits in itertools.product((1, 2, 3), repeat=min(n_tiles, 6)):
        bits = list(bits) + [3] * (n_tiles - len(bits))
        active = [[(bits[j] >> (w // 2)) & 1 == 1 for j in range(n_tiles)] for w in range(4)]
        _check(sparse_split(n_tiles, active), 4)


def test_model_catches_a_broken_ring():
    """The checks fire on a ring one slot too small (three [K | V] slots with
    two tiles in flight) and on loads issued before the slot's readers pass
    the barrier."""
    active = [[True] * 6 for _ in range(8)]
    with pytest.raises(AssertionError):
        _check(dense_lagged(6, active, ns=3), 8)
    ev = sparse_split(5, [[True] * 5 for _ in range(4)])
    # move wave 0's issue of K(3), which refills K(0)'s slot, one phase early
    for idx, e in enumerate(ev[0]):
        if e[1] == "issue" and e[2] == "k" and e[3] == 3:
            ev[0][idx] = (e[0] - 1,) + e[1:]
            break
    with pytest.raises(AssertionError):
        _check(ev, 4)
