"""Pins of the raw-input ring oracle (oracle/ring.py) against the values
[Serve demo] Tab 4 prints (tests/golden/ring_tab4.json) and against the
recurrence itself.  CPU only."""
import json
import os

import numpy as np

from oracle import (kda_recurrent, ring_new, ring_push, ring_reset, ring_window, snapshot_push,
                    snapshot_restore, kda_step, verify_and_replay)
from tests.conftest import GOLDEN

G = json.load(open(os.path.join(GOLDEN, "ring_tab4.json")))


def _full(H, dk, dv, B, value):
    return {"q": np.full((B, H, dk), value), "k": np.full((B, H, dk), value),
            "v": np.full((B, H, dv), value), "a": np.full((B, H, dk), value),
            "beta": np.full((B, H), value)}


def test_tab4_panel_a_window_sizes():
    pa = G["panel_a"]
    ring = ring_new(1, pa["capacity"], 1, 2, 2)
    sizes = []
    for i in range(pa["pushes"]):
        ring_push(ring, [0], _full(1, 2, 2, 1, float(i)))
        sizes.append(int(ring_window(ring, [0])[1][0]))
    assert sizes == pa["window_sizes"]


def test_tab4_panel_b_layout():
    pb = G["panel_b"]
    H, D = pb["H"], pb["D"]
    ring = ring_new(1, pb["pushes"], H, D, D)
    for i in range(pb["pushes"]):
        ring_push(ring, [0], _full(H, D, D, 1, float(i)))
    win, n = ring_window(ring, [0])
    assert list(win["q"].shape) == pb["shape"] and n[0] == pb["pushes"]
    for i, val in enumerate(pb["row_values"]):
        assert np.all(win["q"][i] == val) and np.all(win["v"][i] == val)


def test_overwrite_keeps_the_newest_oldest_first_and_pads_with_zeros():
    ring = ring_new(3, 4, 1, 2, 2)
    for i in range(6):
        ring_push(ring, [0, 2], _full(1, 2, 2, 2, float(i)))
    ring_push(ring, [1], _full(1, 2, 2, 1, 9.0))
    win, n = ring_window(ring, [2, 1])
    assert list(n) == [4, 1]
    assert [float(win["k"][i, 0, 0, 0]) for i in range(4)] == [2.0, 3.0, 4.0, 5.0]
    assert float(win["beta"][0, 1, 0]) == 9.0 and not win["beta"][1:, 1].any()
    ring_reset(ring, [2])
    assert ring_window(ring, [2])[1][0] == 0 and ring_window(ring, [0])[1][0] == 4


def test_tab4_panel_c_replay_through_the_ring_equals_the_recurrence():
    """Streaming pushes, window(), then verify-and-replay reproduce the
    token-by-token recurrence exactly (panel (c): error 0)."""
    rng = np.random.default_rng(7)
    B, H, dk, dv, Td = 3, 2, 4, 3, 5
    q = rng.standard_normal((Td, B, H, dk))
    k = rng.standard_normal((Td, B, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((Td, B, H, dv))
    a = -np.abs(rng.standard_normal((Td, B, H, dk)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((Td, B, H))))
    S0 = rng.standard_normal((B, H, dk, dv))
    ring = ring_new(B, Td, H, dk, dv)
    for t in range(Td):
        ring_push(ring, list(range(B)), {"q": q[t], "k": k[t], "v": v[t], "a": a[t], "beta": beta[t]})
    win, n = ring_window(ring, list(range(B)))
    n_acc = np.array([0, 2, 5])
    s_new, o = verify_and_replay(S0, win["q"], win["k"], win["v"], win["a"], win["beta"], n_acc)
    for b in range(B):
        o_r, S_r, _ = kda_recurrent(q[:n_acc[b], b], k[:n_acc[b], b], v[:n_acc[b], b],
                                    a[:n_acc[b], b], beta[:n_acc[b], b], S0[b])
        assert np.max(np.abs(s_new[b] - S_r), initial=0.0) == G["panel_c"]["max_err"]
        assert np.max(np.abs(o[b, :, :n_acc[b]] - np.moveaxis(o_r, 0, 1)), initial=0.0) == 0.0


def test_route_a_snapshots_roll_back_to_the_accepted_prefix():
    rng = np.random.default_rng(8)
    B, H, dk, dv, Td = 2, 2, 3, 3, 4
    S0 = rng.standard_normal((B, H, dk, dv))
    snaps = np.zeros((B, Td, H, dk, dv))
    counts = np.zeros(B, dtype=np.int64)
    S = S0.copy()
    states = []
    for t in range(Td):
        q, k, v = (rng.standard_normal((B, H, d)) for d in (dk, dk, dv))
        a = -np.abs(rng.standard_normal((B, H, dk)))
        beta = rng.random((B, H))
        _, S = kda_step(q, k, v, a, beta, S)
        snapshot_push(snaps, counts, [0, 1], S)
        states.append(S.copy())
    out = snapshot_restore(snaps, [0, 1], np.array([0, 3]), S0)
    assert np.array_equal(out[0], S0[0]) and np.array_equal(out[1], states[2][1])
