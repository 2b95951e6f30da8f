"""Pins of the float64 front-end oracle (oracle/front_end.py) against what the
pages and the mathematics fix: a library correlation, closed forms of special
kernels, the channel layout, continuation across a carried window, and the
gate ranges of [Serve demo] §1.3.  CPU only."""
import math

import numpy as np
import pytest

from oracle import conv_window, front_end, front_end_step, short_conv, sigmoid, silu


def _rand(rng, T, H, dk, dv, K):
    C = H * (2 * dk + dv)
    return (rng.standard_normal((T, C)), rng.standard_normal((T, H, dk)),
            rng.standard_normal((T, H)), rng.standard_normal((C, K)) * 0.5)


# ------------------------------------------------------------- activations
def test_sigmoid_and_silu_values_and_identities():
    assert sigmoid(0.0) == 0.5
    assert math.isclose(float(silu(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    x = np.linspace(-8, 8, 33)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    np.testing.assert_allclose(silu(x) - silu(-x), x, atol=1e-13)
    assert silu(0.0) == 0.0 and abs(float(silu(-40.0))) < 1e-15
    assert math.isclose(float(silu(40.0)), 40.0, rel_tol=1e-15)


# ------------------------------------------------------------ convolution
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_short_conv_is_a_library_correlation(K):
    rng = np.random.default_rng(1)
    T, C = 11, 5
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    win = rng.standard_normal((K - 1, C))
    y = short_conv(x, w, win)
    xp = np.concatenate([win, x])
    for c in range(C):
        np.testing.assert_allclose(y[:, c], np.correlate(xp[:, c], w[c], "valid"), atol=1e-12)


def test_short_conv_special_kernels():
    rng = np.random.default_rng(2)
    T, C, K = 9, 4, 4
    x = rng.standard_normal((T, C))
    win = rng.standard_normal((K - 1, C))
    # Only the current-token tap: the identity, scaled per channel.
    w = np.zeros((C, K))
    w[:, K - 1] = [1.0, 2.0, -1.0, 0.5]
    np.testing.assert_array_equal(short_conv(x, w, win), x * w[:, K - 1])
    # Only the oldest tap: a delay of K-1 rows, the window's rows first.
    w = np.zeros((C, K))
    w[:, 0] = 1.0
    np.testing.assert_array_equal(short_conv(x, w, win), np.concatenate([win, x])[:T])
    # A fresh sequence (no window) sees zeros before its start.
    np.testing.assert_array_equal(short_conv(x, w), np.concatenate([np.zeros((K - 1, C)), x])[:T])


def test_conv_window_rows():
    x = np.arange(12.0).reshape(6, 2)
    win = -np.arange(1.0, 7.0).reshape(3, 2)
    np.testing.assert_array_equal(conv_window(x, 4, win), x[3:])         # last K-1 rows
    np.testing.assert_array_equal(conv_window(x[:1], 4, win), np.concatenate([win[1:], x[:1]]))
    np.testing.assert_array_equal(conv_window(x[:0], 4, win), win)        # empty: unchanged
    np.testing.assert_array_equal(conv_window(x[:2], 4), np.concatenate([np.zeros((1, 2)), x[:2]]))


# ------------------------------------------------------------ the layout
def test_channel_layout_q_then_k_then_v():
    H, dk, dv, K = 2, 4, 3, 4
    C = H * (2 * dk + dv)
    x = np.concatenate([np.full(H * dk, 1.0), np.full(H * dk, 2.0), np.full(H * dv, 3.0)])[None]
    x[0, 1] = 5.0                     # q of head 0, channel 1
    x[0, H * dk + dk + 2] = -4.0      # k of head 1, channel 2
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    r = front_end(x, np.zeros((1, H, dk)), np.zeros((1, H)), w, -1.0, H, dk, dv, [0, 1])
    np.testing.assert_allclose(r["v"][0], np.full((H, dv), float(silu(3.0))), rtol=1e-15)
    q0 = silu(np.array([1.0, 5.0, 1.0, 1.0]))
    np.testing.assert_allclose(r["q"][0, 0], q0 / np.sqrt(q0 @ q0 + 1e-6), rtol=1e-14)
    np.testing.assert_allclose(r["q"][0, 1], np.full(dk, 0.5), rtol=1e-6)   # equal entries -> 1/sqrt(dk)
    k1 = silu(np.array([2.0, 2.0, -4.0, 2.0]))
    np.testing.assert_allclose(r["k"][0, 1], k1 / np.sqrt(k1 @ k1 + 1e-6), rtol=1e-14)


def test_l2norm_closed_form_and_gates():
    rng = np.random.default_rng(3)
    T, H, dk, dv, K = 7, 2, 8, 4, 3
    x, z_a, z_b, w = _rand(rng, T, H, dk, dv, K)
    r = front_end(x, z_a, z_b, w, -2.0, H, dk, dv, [0, T])
    y = silu(short_conv(x, w))
    raw_q = y[:, :H * dk].reshape(T, H, dk)
    n = np.linalg.norm(raw_q, axis=-1)
    # ||q|| = ||u|| / sqrt(||u||^2 + eps) and q is parallel to u.
    np.testing.assert_allclose(np.linalg.norm(r["q"], axis=-1), n / np.sqrt(n * n + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(np.sum(r["q"] * raw_q, -1), n * np.linalg.norm(r["q"], axis=-1), rtol=1e-12)
    assert np.all(r["a"] <= 0) and np.all(r["a"] >= -2.0)
    assert np.all((r["beta"] > 0) & (r["beta"] < 1))
    r0 = front_end(x, np.zeros_like(z_a), np.zeros_like(z_b), w, -2.0, H, dk, dv, [0, T])
    assert np.all(r0["a"] == -1.0) and np.all(r0["beta"] == 0.5)
    # A large logit gives the full decay g_min and a full write; a very
    # negative one no decay and no write ([Serve demo] §1.3 ranges, ends).
    big = front_end(x, np.full_like(z_a, 40.0), np.full_like(z_b, 40.0), w, -2.0, H, dk, dv, [0, T])
    assert np.all(big["a"] == -2.0) and np.all(big["beta"] == 1.0)
    small = front_end(x, np.full_like(z_a, -40.0), np.full_like(z_b, -40.0), w, -2.0, H, dk, dv, [0, T])
    assert np.all(np.abs(small["a"]) < 1e-16) and np.all(small["beta"] < 1e-16)


# ------------------------------------------------------------ continuation
def test_continuation_through_the_window_equals_one_pass():
    """front_end(0..T) == front_end(0..p), then front_end(p..T) with the
    window after p tokens; and a checkpoint's window is that window."""
    rng = np.random.default_rng(4)
    T, H, dk, dv, K, p = 13, 2, 4, 4, 4, 5
    x, z_a, z_b, w = _rand(rng, T, H, dk, dv, K)
    win0 = rng.standard_normal((1, K - 1, x.shape[1]))
    full = front_end(x, z_a, z_b, w, -1.0, H, dk, dv, [0, T], windows=win0, checkpoints=[[1, p, T]])
    first = front_end(x[:p], z_a[:p], z_b[:p], w, -1.0, H, dk, dv, [0, p], windows=win0)
    rest = front_end(x[p:], z_a[p:], z_b[p:], w, -1.0, H, dk, dv, [0, T - p],
                     windows=first["window_end"])
    for f in ("q", "k", "v", "a", "beta"):
        np.testing.assert_array_equal(full[f], np.concatenate([first[f], rest[f]]))
    np.testing.assert_array_equal(full["window_ckpt"][0][p], first["window_end"][0])
    np.testing.assert_array_equal(full["window_ckpt"][0][T], full["window_end"][0])
    np.testing.assert_array_equal(rest["window_end"], full["window_end"])
    # Varlen: sequences do not see each other.
    both = front_end(np.concatenate([x, x[:4]]), np.concatenate([z_a, z_a[:4]]),
                     np.concatenate([z_b, z_b[:4]]), w, -1.0, H, dk, dv, [0, T, T + 4])
    alone = front_end(x[:4], z_a[:4], z_b[:4], w, -1.0, H, dk, dv, [0, 4])
    np.testing.assert_array_equal(both["q"][T:], alone["q"])


def test_decode_step_shifts_the_window():
    rng = np.random.default_rng(5)
    B, H, dk, dv, K = 3, 2, 4, 2, 4
    C = H * (2 * dk + dv)
    x = rng.standard_normal((B, C))
    win = rng.standard_normal((B, K - 1, C))
    w = rng.standard_normal((C, K))
    z_a, z_b = rng.standard_normal((B, H, dk)), rng.standard_normal((B, H))
    q, k, v, a, beta, nw = front_end_step(x, z_a, z_b, w, -1.0, H, dk, dv, win)
    np.testing.assert_array_equal(nw, np.concatenate([win[:, 1:], x[:, None]], axis=1))
    for b in range(B):
        r = front_end(x[b:b + 1], z_a[b:b + 1], z_b[b:b + 1], w, -1.0, H, dk, dv, [0, 1],
                      windows=win[b:b + 1])
        np.testing.assert_array_equal(q[b], r["q"][0])
        np.testing.assert_array_equal(v[b], r["v"][0])
        # The convolution of the step reads the window then the token.
        y = np.einsum("cj,jc->c", w, np.concatenate([win[b], x[b:b + 1]]))
        np.testing.assert_allclose(v[b].reshape(-1), silu(y[2 * H * dk:]), rtol=1e-13)
