"""Pins of the bfloat16-state oracle (reading R14): the rounding function
against a library cast and hand-made ties, and the bf16-state decode and
replay against their definitions.  CPU only."""
import numpy as np
import torch

from oracle import (decode_bf16_state, kda_step, round_bf16, verify_and_replay,
                    verify_and_replay_bf16_state)


def test_round_bf16_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-20,
                        rng.standard_normal(2000) * 1e20]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), want)


def test_round_bf16_ties_and_fixed_points():
    u = 2.0 ** -7  # one bf16 ulp at 1
    # Halfway cases go to the even neighbour.
    assert round_bf16(1 + u / 2) == 1.0
    assert round_bf16(1 + 3 * u / 2) == 1 + 2 * u
    assert round_bf16(-(1 + u / 2)) == -1.0
    # Just past halfway goes up; representable values are fixed points.
    assert round_bf16(1 + u / 2 + 2.0 ** -20) == 1 + u
    for v in (1.0, 1 + u, -3.5, 2.0 ** -100, 0.0):
        assert round_bf16(v) == v
    x = np.random.default_rng(2).standard_normal(1000)
    np.testing.assert_array_equal(round_bf16(round_bf16(x)), round_bf16(x))
    # The rounding error is at most half an ulp of 8 significant bits.
    r = round_bf16(x)
    assert np.all(np.abs(r - x) <= 2.0 ** (np.floor(np.log2(np.abs(x))) - 8))


def test_bf16_state_calls_round_only_what_they_store():
    rng = np.random.default_rng(3)
    B, H, dk, dv, Td = 2, 2, 4, 3, 3
    S = round_bf16(rng.standard_normal((B, H, dk, dv)))
    q, k = rng.standard_normal((B, H, dk)), rng.standard_normal((B, H, dk))
    v, a = rng.standard_normal((B, H, dv)), -np.abs(rng.standard_normal((B, H, dk)))
    beta = rng.random((B, H))
    o, S1 = decode_bf16_state(q, k, v, a, beta, S)
    o_ref, S_ref = kda_step(q, k, v, a, beta, S)
    np.testing.assert_array_equal(o, o_ref)            # the output is not rounded
    np.testing.assert_array_equal(S1, round_bf16(S_ref))
    assert not np.array_equal(S1, S_ref)
    qs = rng.standard_normal((Td, B, H, dk))
    ks = rng.standard_normal((Td, B, H, dk))
    vs = rng.standard_normal((Td, B, H, dv))
    as_ = -np.abs(rng.standard_normal((Td, B, H, dk)))
    bs = rng.random((Td, B, H))
    n = np.array([0, 3])
    s_new, o2 = verify_and_replay_bf16_state(S, qs, ks, vs, as_, bs, n)
    s_ref, o2_ref = verify_and_replay(S, qs, ks, vs, as_, bs, n)
    np.testing.assert_array_equal(s_new[0], S[0])      # n = 0: the committed state
    np.testing.assert_array_equal(s_new[1], round_bf16(s_ref[1]))   # rounded once, at the end
    np.testing.assert_array_equal(o2, o2_ref)
