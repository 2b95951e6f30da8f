"""GPU parity: the fused front end (convolution, SiLU, L2Norm, gates) and its
convolution windows against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu

G_MIN = -1.0
LENS = [1, 2, 3, 64, 0, 65, 130, 200]


def _dev(w, dtype):
    return {n: (None if w[n] is None else dev_tensor(w[n], dtype))
            for n in ("x", "z_a", "z_b", "conv_w", "windows")}


def _exact(got, want, what):
    g, t = to_np(got), np.asarray(want, dtype=np.float64)
    assert np.array_equal(g, t), f"{what}: not bit-exact (max diff {np.max(np.abs(g - t)):.3e})"


@pytest.mark.parametrize("dk,dv,dtype,K", [(16, 16, "fp32", 4), (32, 64, "bf16", 4),
                                           (64, 32, "fp32", 3), (128, 128, "bf16", 4),
                                           (128, 16, "bf16", 2), (64, 128, "fp32", 1),
                                           (64, 32, "bf16", 3), (16, 64, "bf16", 1)])
@pytest.mark.parametrize("carried", [True, False])
def test_front_end_matches_oracle(dk, dv, dtype, K, carried):
    H = 2
    w = inputs.front_end_inputs(100 + dk + dv + K, LENS, H, dk, dv, K, dtype, windows=carried)
    d = _dev(w, dtype)
    C = H * (2 * dk + dv)
    ck = [sorted({p for p in (1, 2, 5, 64, L) if 1 <= p <= L}) for L in LENS]
    n_ck = sum(len(c) for c in ck)
    order = np.random.default_rng(3).permutation(n_ck + 2)[:n_ck]
    slots, i = [], 0
    for c in ck:
        slots.append([int(s) for s in order[i:i + len(c)]])
        i += len(c)
    pool = torch.full((n_ck + 2, (K - 1) * C + 8), float("nan"), device="cuda",
                      dtype=d["x"].dtype)
    r = kda.front_end(d["x"], d["z_a"], d["z_b"], d["conv_w"], H, dk, dv, G_MIN, w["cu_seqlens"],
                      win_in=d["windows"], checkpoints=ck, ckpt_slots=slots, conv_pool=pool)
    torch.cuda.synchronize()
    want = oracle.front_end(w["x"], w["z_a"], w["z_b"], w["conv_w"], G_MIN, H, dk, dv,
                            w["cu_seqlens"], windows=w["windows"], checkpoints=ck)
    for f in ("q", "k", "v", "a", "beta"):
        assert_parity(r[f], want[f], dtype, f)
    # Windows are copies of raw rows: bit-exact, and the slot padding is zero.
    _exact(r["window"], want["window_end"], "end windows")
    for n, c in enumerate(ck):
        for j, p in enumerate(c):
            page = to_np(pool[slots[n][j]])
            _exact(page[:(K - 1) * C].reshape(K - 1, C), want["window_ckpt"][n][p],
                   f"window of seq {n} at {p}")
            assert not page[(K - 1) * C:].any(), "slot padding must be zero"


@pytest.mark.parametrize("dk,dv,dtype,K", [(128, 128, "bf16", 4), (32, 16, "fp32", 3),
                                           (64, 64, "bf16", 1), (64, 32, "bf16", 3),
                                           (32, 128, "bf16", 2)])
def test_front_end_step_matches_oracle(dk, dv, dtype, K):
    B, H = 5, 3
    w = inputs.front_end_inputs(120 + dk + K, [1] * B, H, dk, dv, K, dtype)
    d = _dev(w, dtype)
    win = d["windows"] if K > 1 else None
    r = kda.front_end_step(d["x"], d["z_a"], d["z_b"], d["conv_w"], H, dk, dv, G_MIN, win)
    torch.cuda.synchronize()
    q, k, v, a, beta, nw = oracle.front_end_step(w["x"], w["z_a"], w["z_b"], w["conv_w"], G_MIN,
                                                 H, dk, dv, w["windows"])
    for f, want in (("q", q), ("k", k), ("v", v), ("a", a), ("beta", beta)):
        assert_parity(r[f], want, dtype, f)
    if K > 1:
        _exact(win, nw, "shifted window")


def test_decode_steps_continue_the_prefill_front_end():
    """front_end over T tokens, then decode steps from its window, equals the
    front end over T + 3 tokens."""
    H, dk, dv, K, T = 2, 64, 64, 4, 37
    w = inputs.front_end_inputs(130, [T + 3], H, dk, dv, K, "fp32", windows=False)
    d = _dev(w, "fp32")
    head = kda.front_end(d["x"][:T], d["z_a"][:T], d["z_b"][:T], d["conv_w"], H, dk, dv, G_MIN,
                         [0, T])
    win = head["window"]
    full = kda.front_end(d["x"], d["z_a"], d["z_b"], d["conv_w"], H, dk, dv, G_MIN, [0, T + 3])
    for s in range(3):
        t = T + s
        r = kda.front_end_step(d["x"][t:t + 1], d["z_a"][t:t + 1], d["z_b"][t:t + 1],
                               d["conv_w"], H, dk, dv, G_MIN, win)
        for f in ("q", "k", "v", "a", "beta"):
            assert_parity(r[f][0], full[f][t], "fp32", f"{f} of step {s}")
    torch.cuda.synchronize()
    assert torch.equal(win[0], full["window"][0])


def test_front_end_single_sequence_workload_sampled():
    """The front end at the single-sequence prefill's shape (T=8192, H=32,
    d=128, K=4, bf16), checked on tokens at tile edges and the ends."""
    H, dk, dv, K, T = 32, 128, 128, 4, 8192
    w = inputs.front_end_inputs(131, [T], H, dk, dv, K, "bf16")
    d = _dev(w, "bf16")
    r = kda.front_end(d["x"], d["z_a"], d["z_b"], d["conv_w"], H, dk, dv, G_MIN, [0, T],
                      win_in=d["windows"])
    torch.cuda.synchronize()
    for t in (0, 1, 2, 3, 63, 64, 65, 127, 128, 4095, 4096, 8190, 8191):
        lo = max(0, t - (K - 1))
        win = w["windows"][0] if lo == 0 else None
        # The oracle on rows lo..t: with lo > 0 its "window" is the raw rows before lo.
        pre = None
        if lo > 0:
            pre = w["x"][lo - (K - 1):lo][None]
        elif win is not None:
            pre = win[None]
        want = oracle.front_end(w["x"][lo:t + 1], w["z_a"][lo:t + 1], w["z_b"][lo:t + 1],
                                w["conv_w"], G_MIN, H, dk, dv, [0, t + 1 - lo], windows=pre)
        for f in ("q", "k", "v", "a", "beta"):
            assert_parity(r[f][t], want[f][-1], "bf16", f"{f} at token {t}")
    _exact(r["window"][0], w["x"][T - (K - 1):], "end window")
