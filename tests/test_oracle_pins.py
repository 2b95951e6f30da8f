"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: closed
forms, brute force through explicit transition matrices, invariants, values
printed on the pages (tests/golden, each fixture citing its passage).
CPU only.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (compose_segments, kda_chunked_ref, kda_prefill, kda_recurrent, kda_step,
                    pack_heads, projection_bytes_per_step, segment_summary,
                    snapshot_bytes_per_step, snapshot_cost_ratio, unpack_heads,
                    verify_and_replay)
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_inputs(rng, T, H, dk, dv, g_min=-1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    a = g_min / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, a, beta


# ---------------------------------------------------------------- kda_step
def test_step_worked_example_by_hand():
    g = _golden("step_worked_example.json")
    S = np.array(g["S"])
    a = np.log(np.array(g["exp_a"]))
    k, v, q = map(np.array, (g["k"], g["v"], g["q"]))
    o, Sn = kda_step(q, k, v, a, g["beta"], S)
    np.testing.assert_allclose(Sn, g["decay_then_error"]["S_new"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o, g["decay_then_error"]["o"], rtol=0, atol=1e-15)
    o2, Sn2 = kda_step(q, k, v, a, g["beta"], S, error_before_decay=True)
    np.testing.assert_allclose(Sn2, g["error_before_decay"]["S_new"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o2, g["error_before_decay"]["o"], rtol=0, atol=1e-15)


def test_step_beta_zero_only_decays():
    rng = np.random.default_rng(1)
    q, k, v, a, _ = _rand_inputs(rng, 1, 3, 8, 5)
    S = rng.standard_normal((3, 8, 5))
    o, Sn = kda_step(q[0], k[0], v[0], a[0], np.zeros(3), S)
    np.testing.assert_allclose(Sn, np.exp(a[0])[:, :, None] * S, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.einsum("hij,hi->hj", Sn, q[0]), rtol=0, atol=1e-14)


def test_step_delta_rule_write_then_read():
    # No decay, beta=1, unit-norm k: after the write the state maps k to v exactly.
    rng = np.random.default_rng(2)
    q, k, v, _, _ = _rand_inputs(rng, 1, 4, 16, 12)
    S = rng.standard_normal((4, 16, 12))
    _, Sn = kda_step(q[0], k[0], v[0], np.zeros((4, 16)), np.ones(4), S)
    np.testing.assert_allclose(np.einsum("hij,hi->hj", Sn, k[0]), v[0], rtol=0, atol=1e-12)


def test_step_from_zero_state_is_rank_one():
    rng = np.random.default_rng(3)
    q, k, v, a, beta = _rand_inputs(rng, 1, 2, 6, 7)
    o, Sn = kda_step(q[0], k[0], v[0], a[0], beta[0], np.zeros((2, 6, 7)))
    want_S = beta[0][:, None, None] * k[0][:, :, None] * v[0][:, None, :]
    np.testing.assert_allclose(Sn, want_S, rtol=0, atol=1e-15)
    want_o = (beta[0] * np.sum(k[0] * q[0], -1))[:, None] * v[0]
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-15)


def test_step_no_write_no_decay_reads_state():
    rng = np.random.default_rng(4)
    q, k, v, _, _ = _rand_inputs(rng, 1, 2, 5, 3)
    S = rng.standard_normal((2, 5, 3))
    o, Sn = kda_step(q[0], k[0], v[0], np.zeros((2, 5)), np.zeros(2), S)
    np.testing.assert_array_equal(Sn, S)
    np.testing.assert_allclose(o, np.einsum("hij,hi->hj", S, q[0]), rtol=0, atol=1e-15)


def test_orthonormal_keys_store_pairs_exactly():
    # a=0, beta=1, orthonormal keys, S0=0: the state is sum_i k_i v_i^T and
    # every stored value is retrieved exactly (classic delta-rule memory).
    rng = np.random.default_rng(5)
    dk, dv, m = 8, 4, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :m].T
    vals = rng.standard_normal((m, dv))
    S = np.zeros((1, dk, dv))
    for i in range(m):
        _, S = kda_step(keys[i][None], keys[i][None], vals[i][None], np.zeros((1, dk)),
                        np.ones(1), S)
    np.testing.assert_allclose(S[0], keys.T @ vals, rtol=0, atol=1e-13)
    np.testing.assert_allclose(keys @ S[0], vals, rtol=0, atol=1e-13)


def test_pre_and_post_decay_readings_differ():
    rng = np.random.default_rng(6)
    q, k, v, a, beta = _rand_inputs(rng, 1, 1, 4, 4)
    S = rng.standard_normal((1, 4, 4))
    o1, _ = kda_step(q[0], k[0], v[0], a[0], beta[0], S)
    o2, _ = kda_step(q[0], k[0], v[0], a[0], beta[0], S, error_before_decay=True)
    assert np.max(np.abs(o1 - o2)) > 1e-3


# ------------------------------------------------------------ kda_recurrent
def _brute_force(q, k, v, a, beta, S0):
    """S_t = M_t S_{t-1} + beta_t k_t v_t^T, M_t = (I - beta_t k_t k_t^T) diag(exp(a_t)),
    one dense dk x dk matrix per step and head."""
    T, H, dk = k.shape
    S = S0.copy()
    o = np.zeros((T, H, v.shape[-1]))
    for t in range(T):
        for h in range(H):
            M = (np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(a[t, h]))
            S[h] = M @ S[h] + beta[t, h] * np.outer(k[t, h], v[t, h])
            o[t, h] = S[h].T @ q[t, h]
    return o, S


@pytest.mark.parametrize("T,H,dk,dv", [(1, 1, 3, 2), (5, 2, 4, 6), (8, 3, 7, 5)])
def test_recurrent_matches_transition_matrix_brute_force(T, H, dk, dv):
    rng = np.random.default_rng(10 + T)
    q, k, v, a, beta = _rand_inputs(rng, T, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((H, dk, dv))
    o, S, _ = kda_recurrent(q, k, v, a, beta, S0)
    o_bf, S_bf = _brute_force(q, k, v, a, beta, S0)
    np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_bf, rtol=0, atol=1e-12)


def test_recurrent_beta_zero_closed_form():
    rng = np.random.default_rng(11)
    q, k, v, a, _ = _rand_inputs(rng, 20, 2, 6, 3)
    S0 = rng.standard_normal((2, 6, 3))
    _, S, _ = kda_recurrent(q, k, v, a, np.zeros((20, 2)), S0)
    np.testing.assert_allclose(S, np.exp(a.sum(0))[:, :, None] * S0, rtol=1e-13, atol=0)


def test_recurrent_value_columns_are_independent():
    # Column j of the state depends only on column j of v: permuting v's
    # columns permutes S's and o's columns.
    rng = np.random.default_rng(12)
    q, k, v, a, beta = _rand_inputs(rng, 12, 2, 5, 6)
    S0 = rng.standard_normal((2, 5, 6))
    perm = rng.permutation(6)
    o1, S1, _ = kda_recurrent(q, k, v, a, beta, S0)
    o2, S2, _ = kda_recurrent(q, k, v[..., perm], a, beta, S0[..., perm])
    np.testing.assert_allclose(o2, o1[..., perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S2, S1[..., perm], rtol=0, atol=1e-14)


def test_recurrent_is_linear_in_values_and_initial_state():
    rng = np.random.default_rng(13)
    q, k, v1, a, beta = _rand_inputs(rng, 10, 1, 4, 3)
    v2 = rng.standard_normal(v1.shape)
    A1, A2 = rng.standard_normal((2, 1, 4, 3))
    o1, S1, _ = kda_recurrent(q, k, v1, a, beta, A1)
    o2, S2, _ = kda_recurrent(q, k, v2, a, beta, A2)
    o3, S3, _ = kda_recurrent(q, k, 2.0 * v1 - v2, a, beta, 2.0 * A1 - A2)
    np.testing.assert_allclose(o3, 2 * o1 - o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S3, 2 * S1 - S2, rtol=0, atol=1e-12)


def test_recurrent_rejects_bad_checkpoint():
    rng = np.random.default_rng(14)
    q, k, v, a, beta = _rand_inputs(rng, 4, 1, 2, 2)
    with pytest.raises(ValueError):
        kda_recurrent(q, k, v, a, beta, None, [5])
    with pytest.raises(ValueError):
        kda_recurrent(q, k, v, a, beta, None, [0])


# ------------------------------------------------------------- chunk form
@pytest.mark.parametrize("chunk,T,dk,dv", [(1, 9, 4, 3), (16, 40, 16, 12), (16, 128, 16, 16),
                                           (64, 150, 8, 24), (64, 64, 32, 32)])
def test_chunked_form_equals_recurrence(chunk, T, dk, dv):
    rng = np.random.default_rng(20 + chunk + T)
    q, k, v, a, beta = _rand_inputs(rng, T, 1, dk, dv)
    S0 = 0.1 * rng.standard_normal((dk, dv))
    o_c, S_c = kda_chunked_ref(q[:, 0], k[:, 0], v[:, 0], a[:, 0], beta[:, 0], S0, chunk)
    o_r, S_r, _ = kda_recurrent(q, k, v, a, beta, S0[None])
    np.testing.assert_allclose(o_c, o_r[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_c, S_r[0], rtol=0, atol=1e-12)


# ----------------------------------------------------- varlen + checkpoints
def test_prefill_sequences_are_independent_and_zero_length_keeps_s0():
    rng = np.random.default_rng(30)
    lens = [7, 0, 12, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, a, beta = _rand_inputs(rng, int(cu[-1]), 2, 4, 3)
    S0 = rng.standard_normal((4, 2, 4, 3))
    o, Sf, _ = kda_prefill(q, k, v, a, beta, cu, S0)
    for n, L in enumerate(lens):
        lo, hi = cu[n], cu[n + 1]
        if L == 0:
            np.testing.assert_array_equal(Sf[n], S0[n])
            continue
        o_n, S_n, _ = kda_recurrent(q[lo:hi], k[lo:hi], v[lo:hi], a[lo:hi], beta[lo:hi], S0[n])
        np.testing.assert_array_equal(o[lo:hi], o_n)
        np.testing.assert_array_equal(Sf[n], S_n)


def test_checkpoint_then_resume_equals_one_pass():
    # One-way reuse: the state after p tokens, advanced over the rest, gives the
    # one-pass result; the committed S0 is never written.
    rng = np.random.default_rng(31)
    T, p = 37, 16
    q, k, v, a, beta = _rand_inputs(rng, T, 2, 5, 4)
    S0 = rng.standard_normal((1, 2, 5, 4))
    S0_copy = S0.copy()
    o_all, S_all, ck = kda_prefill(q, k, v, a, beta, [0, T], S0, [[p, 30, T]])
    np.testing.assert_array_equal(S0, S0_copy)
    o_a, S_a, _ = kda_recurrent(q[:p], k[:p], v[:p], a[:p], beta[:p], S0[0])
    np.testing.assert_array_equal(ck[0][p], S_a)
    o_b, S_b, _ = kda_recurrent(q[p:], k[p:], v[p:], a[p:], beta[p:], ck[0][p])
    np.testing.assert_allclose(o_all[p:], o_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_all[0], S_b, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ck[0][T], S_all[0])


def test_prefill_rejects_bad_offsets():
    rng = np.random.default_rng(32)
    q, k, v, a, beta = _rand_inputs(rng, 4, 1, 2, 2)
    with pytest.raises(ValueError):
        kda_prefill(q, k, v, a, beta, [0, 3, 2, 4])
    with pytest.raises(ValueError):
        kda_prefill(q, k, v, a, beta, [0, 3])


# ----------------------------------------------------------------- replay
def _replay_inputs(seed, Td, B, H, dk, dv):
    rng = np.random.default_rng(seed)
    q, k, v, a, beta = _rand_inputs(rng, Td * B, H, dk, dv)
    shp = lambda x: x.reshape((Td, B) + x.shape[1:])
    committed = 0.1 * rng.standard_normal((B, H, dk, dv))
    return committed, shp(q), shp(k), shp(v), shp(a), shp(beta)


@pytest.mark.parametrize("scenario", _golden("replay_scenarios.json")["scenarios"],
                         ids=lambda s: s["name"])
def test_replay_scenarios_match_full_recurrence(scenario):
    g = _golden("replay_scenarios.json")
    Td, n = g["t_draft"], scenario["n_accepted"]
    committed, q, k, v, a, beta = _replay_inputs(40 + n, Td, 2, 3, 4, 5)
    before = committed.copy()
    S_new, O = verify_and_replay(committed, q, k, v, a, beta, [n, n])
    np.testing.assert_array_equal(committed, before)
    for b in range(2):
        if n == 0:
            np.testing.assert_array_equal(S_new[b], committed[b])
            assert not O[b].any()
            continue
        o_r, S_r, _ = kda_recurrent(q[:n, b], k[:n, b], v[:n, b], a[:n, b], beta[:n, b],
                                    committed[b])
        assert np.max(np.abs(S_new[b] - S_r)) < g["tolerance_fp64"]
        assert np.max(np.abs(O[b, :, :n] - o_r.transpose(1, 0, 2))) < g["tolerance_fp64"]
        assert not O[b, :, n:].any()


def test_replay_ragged_batch_and_draft_order():
    Td = 6
    committed, q, k, v, a, beta = _replay_inputs(50, Td, 4, 2, 3, 3)
    n_acc = [0, 3, 6, 1]
    S_new, O = verify_and_replay(committed, q, k, v, a, beta, n_acc)
    for b, n in enumerate(n_acc):
        S = committed[b].copy()
        for i in range(n):
            O_i, S = kda_step(q[i, b], k[i, b], v[i, b], a[i, b], beta[i, b], S)
            np.testing.assert_array_equal(O[b, :, i], O_i)
        np.testing.assert_array_equal(S_new[b], S)
    # draft order matters: reversing the draft axis changes the state
    S_rev, _ = verify_and_replay(committed, q[::-1], k[::-1], v[::-1], a[::-1], beta[::-1],
                                 [Td] * 4)
    S_fwd, _ = verify_and_replay(committed, q, k, v, a, beta, [Td] * 4)
    assert np.max(np.abs(S_rev - S_fwd)) > 1e-6


# ------------------------------------------------------------ pack/unpack
def test_pack_matches_hand_written_layout():
    g = _golden("pack_layout.json")
    state = np.array(g["state_kv"], dtype=np.float64)[None]
    pool = np.full((3, g["page_elems"]), -7.0)
    pack_heads(state, [1], pool)
    np.testing.assert_array_equal(pool[1], g["page"])
    np.testing.assert_array_equal(pool[0], -7.0)
    np.testing.assert_array_equal(pool[2], -7.0)
    # the same page from the transposed [.., dv, dk] source
    pool2 = np.zeros((3, g["page_elems"]))
    pack_heads(state.transpose(0, 1, 3, 2).copy(), [1], pool2, layout="vk")
    np.testing.assert_array_equal(pool2[1], g["page"])


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_pack_unpack_roundtrip_is_bit_exact(dtype):
    rng = np.random.default_rng(60)
    B, H, dk, dv = 3, 2, 4, 5
    state = rng.standard_normal((B, H, dk, dv)).astype(dtype)
    pool = np.full((5, H * dk * dv + 7), np.nan, dtype=dtype)
    slots = [4, 0, 2]
    pack_heads(state, slots, pool)
    for s in slots:
        assert not pool[s, H * dk * dv:].any()
    back = unpack_heads(pool, slots, H, dk, dv)
    assert back.dtype == dtype
    np.testing.assert_array_equal(back.view(np.uint8), state.view(np.uint8))
    back_vk = unpack_heads(pool, slots, H, dk, dv, layout="vk")
    np.testing.assert_array_equal(back_vk, state.transpose(0, 1, 3, 2))
    assert np.isnan(pool[1]).all() and np.isnan(pool[3]).all()


def test_pack_rejects_small_page_and_bad_slot():
    state = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        pack_heads(state, [0], np.zeros((1, 3)))
    with pytest.raises(ValueError):
        pack_heads(state, [1], np.zeros((1, 4)))


# ------------------------------------------------------------ byte ratio
def test_snapshot_ratio_printed_values():
    g = _golden("snapshot_ratio.json")
    for p in g["printed"]:
        r = snapshot_cost_ratio(p["H"], p["dk"], p["dv"])
        assert round(float(r), p["decimals"]) == p["value"], p
    bp = g["bytes_plot"]
    snap = bp["draft_max"] * snapshot_bytes_per_step(bp["H"], bp["dk"], bp["dv"], bp["itemsize"])
    proj = bp["draft_max"] * projection_bytes_per_step(bp["H"], bp["dk"], bp["dv"], bp["itemsize"])
    assert snap == bp["snapshot_bytes_at_draft_max"] and snap >= bp["y_axis_reaches"]
    assert proj < snap
    inc = g["inconsistent"]
    r = snapshot_cost_ratio(inc["H"], inc["dk"], inc["dv"])
    assert r == Fraction(*inc["formula_exact"])
    assert r >= Fraction(4) and r != Fraction(4)


def test_snapshot_ratio_exceeds_one_grows_with_state_and_ignores_draft():
    prev = Fraction(0)
    for d in (4, 8, 16, 32, 64, 128):
        r = snapshot_cost_ratio(16, d, d)
        assert r > prev
        prev = r
    assert snapshot_cost_ratio(1, 8, 8) > 1
    assert snapshot_cost_ratio(3, 16, 32) == snapshot_cost_ratio(32, 16, 32)
    for draft in (1, 2, 4, 8, 16, 32):
        s = draft * snapshot_bytes_per_step(2, 8, 8, 8)
        p = draft * projection_bytes_per_step(2, 8, 8, 8)
        assert Fraction(s, p) == snapshot_cost_ratio(2, 8, 8)


# ------------------------------------------------- context-parallel segments
@pytest.mark.parametrize("T,H,dk,dv", [(1, 1, 3, 2), (9, 2, 5, 4), (40, 2, 8, 8)])
def test_segment_summary_is_the_affine_map_of_the_recurrence(T, H, dk, dv):
    """A S0 + B equals the token-by-token recurrence from any S0 (and B alone
    is the recurrence from S0 = 0)."""
    rng = np.random.default_rng(60 + T)
    q, k, v, a, beta = _rand_inputs(rng, T, H, dk, dv)
    A, B = segment_summary(k, v, a, beta)
    _, S_zero, _ = kda_recurrent(q, k, v, a, beta, np.zeros((H, dk, dv)))
    np.testing.assert_allclose(B, S_zero, rtol=0, atol=1e-12)
    for trial in range(2):
        S0 = rng.standard_normal((H, dk, dv))
        _, S_end, _ = kda_recurrent(q, k, v, a, beta, S0)
        np.testing.assert_allclose(A @ S0 + B, S_end, rtol=0, atol=1e-12)


def test_segment_summary_closed_forms():
    rng = np.random.default_rng(61)
    q, k, v, a, beta = _rand_inputs(rng, 6, 2, 4, 3)
    # beta = 0: the state only decays, A = diag(exp(sum a)), B = 0.
    A, B = segment_summary(k, v, a, np.zeros_like(beta))
    for h in range(2):
        np.testing.assert_allclose(A[h], np.diag(np.exp(a[:, h].sum(0))), rtol=1e-14, atol=0)
    assert not B.any()
    # One token, no decay, beta = 1, unit key: A = I - k k^T (a projector), B = k v^T.
    k1 = np.array([[[0.6, 0.0, 0.8, 0.0]]])
    v1 = np.array([[[1.0, -2.0, 0.5]]])
    A, B = segment_summary(k1, v1, np.zeros((1, 1, 4)), np.ones((1, 1)))
    np.testing.assert_allclose(A[0], np.eye(4) - np.outer(k1[0, 0], k1[0, 0]), atol=1e-15)
    np.testing.assert_allclose(A[0] @ A[0], A[0], atol=1e-15)
    np.testing.assert_allclose(A[0] @ k1[0, 0], 0.0, atol=1e-15)
    np.testing.assert_allclose(B[0], np.outer(k1[0, 0], v1[0, 0]), atol=1e-15)


def test_segment_maps_compose_and_scan_to_the_sequential_states():
    """(A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2), and the exclusive scan of the
    segment maps gives every segment's start state of the one-pass run."""
    rng = np.random.default_rng(62)
    T, H, dk, dv = 30, 2, 6, 5
    q, k, v, a, beta = _rand_inputs(rng, T, H, dk, dv)
    S_in = rng.standard_normal((H, dk, dv))
    cuts = [0, 7, 8, 19, 30]
    maps = [segment_summary(k[lo:hi], v[lo:hi], a[lo:hi], beta[lo:hi])
            for lo, hi in zip(cuts[:-1], cuts[1:])]
    A_all, B_all = segment_summary(k, v, a, beta)
    A12 = maps[1][0] @ maps[0][0]
    B12 = maps[1][0] @ maps[0][1] + maps[1][1]
    A_ref, B_ref = segment_summary(k[:8], v[:8], a[:8], beta[:8])
    np.testing.assert_allclose(A12, A_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(B12, B_ref, rtol=0, atol=1e-12)
    starts, S_end = compose_segments(np.stack([m[0] for m in maps]), np.stack([m[1] for m in maps]),
                                     S_in)
    for i, lo in enumerate(cuts[:-1]):
        if lo == 0:
            np.testing.assert_array_equal(starts[i], S_in)
        else:
            _, S_lo, _ = kda_recurrent(q[:lo], k[:lo], v[:lo], a[:lo], beta[:lo], S_in)
            np.testing.assert_allclose(starts[i], S_lo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_end, A_all @ S_in + B_all, rtol=0, atol=1e-12)
    starts0, _ = compose_segments(np.stack([m[0] for m in maps]), np.stack([m[1] for m in maps]))
    assert not starts0[0].any()

