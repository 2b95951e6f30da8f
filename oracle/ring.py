"""Plain CPU oracle of the raw-input ring (RawInputRing) and of the snapshot
route it is compared with.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check of the package entry file and the CPU-baseline leg of the
benchmark may import it; the GPU library shares no code with it.

[Serve demo] Tab 4 ("ReplaySSM", §7.1-7.3): during verification each draft
step's raw inputs (q, k, v, g, beta) are written, as they arrive, into a ring
window of fixed capacity per slot; once the window is full a push overwrites
the oldest entry; window() hands the entries back, oldest first, in the
draft-projection layout (draft, B, H, D), row i holding the i-th entry; at
commit the accepted prefix is replayed from the committed state by the same
verify-and-replay engine as the batch path (fold-every-commit: no state
snapshot is kept).  §1.1 route A instead keeps one full state snapshot per
step and rolls back by taking the snapshot of the accepted prefix.

Readings: a slot's window is emptied at commit (the fold-every-commit cycle
starts over); window() of a slot with n < capacity entries fills rows
n..capacity-1 with zeros and reports n.
"""

import numpy as np

__all__ = ["RING_FIELDS", "ring_new", "ring_push", "ring_window", "ring_reset",
           "snapshot_push", "snapshot_restore"]

RING_FIELDS = ("q", "k", "v", "a", "beta")


def ring_new(n_slots, capacity, H, dk, dv):
    """Empty rings: per field an array (n_slots, capacity, H, D) and a count
    of pushes per slot."""
    shp = {"q": (H, dk), "k": (H, dk), "v": (H, dv), "a": (H, dk), "beta": (H,)}
    ring = {f: np.zeros((n_slots, capacity) + shp[f]) for f in RING_FIELDS}
    ring["count"] = np.zeros(n_slots, dtype=np.int64)
    return ring


def ring_push(ring, slots, step):
    """One draft step for a batch: step[f] has shape (B, H, D); entry b goes
    into the ring of slot slots[b] at position count % capacity."""
    cap = ring["q"].shape[1]
    for b, s in enumerate(slots):
        pos = ring["count"][s] % cap
        for f in RING_FIELDS:
            ring[f][s, pos] = step[f][b]
        ring["count"][s] += 1


def ring_window(ring, slots):
    """The windows of a batch of slots: per field (capacity, B, H, D), row i
    the i-th oldest entry still held, zero past the held ones; and n_valid
    (B,) = min(count, capacity)."""
    cap = ring["q"].shape[1]
    B = len(slots)
    out = {f: np.zeros((cap, B) + ring[f].shape[2:]) for f in RING_FIELDS}
    n_valid = np.zeros(B, dtype=np.int64)
    for b, s in enumerate(slots):
        c = int(ring["count"][s])
        n = min(c, cap)
        n_valid[b] = n
        for i in range(n):
            pos = (c - n + i) % cap
            for f in RING_FIELDS:
                out[f][i, b] = ring[f][s, pos]
    return out, n_valid


def ring_reset(ring, slots):
    for s in slots:
        ring["count"][s] = 0


def snapshot_push(snaps, counts, slots, state):
    """Route A: keep the full state of every slot after this step."""
    cap = snaps.shape[1]
    for b, s in enumerate(slots):
        snaps[s, counts[s] % cap] = state[b]
        counts[s] += 1


def snapshot_restore(snaps, slots, n_accepted, committed):
    """Route A rollback: the state after n accepted steps is snapshot n-1
    (the committed state when n = 0)."""
    out = np.array(committed, dtype=np.float64, copy=True)
    for b, s in enumerate(slots):
        if n_accepted[b] > 0:
            out[b] = snaps[s, n_accepted[b] - 1]
    return out
