"""Plain float64 CPU oracle of the KDA front end: what turns a layer's
projections into the recurrence inputs q, k, v, a, beta, and the ShortConv
window that a checkpoint has to keep next to the recurrent state.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check of the package entry file and the CPU-baseline leg of the
benchmark may import it; the GPU library shares no code with it.

Pages cited (titles as published; sections named as on the page):
  [Serve demo]  "【轻量化复刻大模型 / KIMI K3】Serve 模块交互式演示"
  [KDA cache]   "Kimi Linear 的 KDA 缓存：SGLang、vLLM 与 Mooncake Store 全链路"

[KDA cache] ("KDA 的递推与充分状态") says the layer input is projected, passed
through a causal short convolution and an activation, and that Q and K are
then L2-normalised; so the recurrent matrix alone cannot continue the next
token, the ShortConv window is part of the state.  Its checkpoint section
("检查点同时包含两部分") takes the convolution checkpoint as the last
kernel_size - 1 rows of mixed_qkv before the boundary.  [Serve demo] §1.3
gives the gates: alpha = g_min * sigmoid(.) in [g_min, 0] and
beta = sigmoid(.) in [0, 1].  The formulas of that passage were lost in
extraction; the readings taken for what they leave open:

  F1  mixed_qkv holds, per token, the q channels of all heads, then the k
      channels, then the v channels: C = H*dk + H*dk + H*dv, head-major
      inside each part.
  F2  The short convolution is depthwise and causal with kernel size K, one
      weight row w[c, 0..K-1] per channel and no bias:
        y[t, c] = sum_j w[c, j] * x[t - (K-1) + j, c],
      where rows before the sequence start come from the carried window
      (or are zero for a fresh sequence).  w[c, K-1] weights the current token.
  F3  The activation is SiLU, x * sigmoid(x), on all three parts.
  F4  L2Norm over each head's dk channels of q and of k:
        u / sqrt(sum(u^2) + eps), eps = 1e-6.
  F5  a = g_min * sigmoid(z_a) per key channel (the log-decay of the
      recurrence, reading R2) and beta = sigmoid(z_beta) per head.
  F6  The window after p tokens of a sequence is the last K-1 raw (pre-
      convolution) rows before the boundary, taken from the carried window
      where the sequence is shorter than K-1.
"""

import numpy as np

__all__ = ["silu", "sigmoid", "short_conv", "conv_window", "front_end", "front_end_step"]

L2_EPS = 1e-6


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """F3: x * sigmoid(x)."""
    x = _f64(x)
    return x * sigmoid(x)


def short_conv(x, w, window=None):
    """F2: causal depthwise convolution of one sequence.

    x : (T, C) raw rows   w : (C, K)   window : (K-1, C) rows before the start, or None (zero).
    Returns y : (T, C).
    """
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    K = w.shape[1]
    pre = np.zeros((K - 1, C)) if window is None else _f64(window).reshape(K - 1, C)
    xp = np.concatenate([pre, x], axis=0)  # row t + K - 1 of xp is x[t]
    y = np.zeros((T, C))
    for t in range(T):
        for j in range(K):
            y[t] += w[:, j] * xp[t + j]
    return y


def conv_window(x, K, window=None):
    """F6: the last K-1 raw rows before the boundary after all rows of x.

    x : (T, C)   window : (K-1, C) carried in, or None (zero).  Returns (K-1, C).
    """
    x = _f64(x)
    C = x.shape[1]
    pre = np.zeros((K - 1, C)) if window is None else _f64(window).reshape(K - 1, C)
    xp = np.concatenate([pre, x], axis=0)
    return xp[xp.shape[0] - (K - 1):].copy() if K > 1 else np.zeros((0, C))


def _l2norm(u):
    """F4 over the last axis."""
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + L2_EPS)


def _split(y, H, dk, dv):
    """F1: (T, C) -> q (T, H, dk), k (T, H, dk), v (T, H, dv)."""
    T = y.shape[0]
    q = y[:, :H * dk].reshape(T, H, dk)
    k = y[:, H * dk:2 * H * dk].reshape(T, H, dk)
    v = y[:, 2 * H * dk:].reshape(T, H, dv)
    return q, k, v


def front_end(x, z_a, z_b, w, g_min, H, dk, dv, cu_seqlens, windows=None, checkpoints=None):
    """Token-packed front end of independent sequences.

    x : (T_tot, C) mixed_qkv rows (F1)   z_a : (T_tot, H, dk)   z_b : (T_tot, H)
    w : (C, K)   windows : (N, K-1, C) carried windows or None (zero)
    checkpoints : per sequence a list of token counts p (1 <= p <= len), or None.
    Returns a dict with q, k, v (after convolution, SiLU and, for q and k,
    L2Norm), a, beta, the end window of every sequence "window_end"
    (N, K-1, C) and "window_ckpt": per sequence {p: window after p tokens}.
    """
    x, z_a, z_b, w = _f64(x), _f64(z_a), _f64(z_b), _f64(w)
    K = w.shape[1]
    C = x.shape[1]
    assert C == H * (2 * dk + dv)
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    T = cu[-1]
    out = {"q": np.zeros((T, H, dk)), "k": np.zeros((T, H, dk)), "v": np.zeros((T, H, dv)),
           "window_end": np.zeros((N, K - 1, C)), "window_ckpt": []}
    out["a"] = g_min * sigmoid(z_a)    # F5
    out["beta"] = sigmoid(z_b)
    for n in range(N):
        lo, hi = cu[n], cu[n + 1]
        win = None if windows is None else _f64(windows[n])
        y = silu(short_conv(x[lo:hi], w, win))
        q, k, v = _split(y, H, dk, dv)
        out["q"][lo:hi] = _l2norm(q)
        out["k"][lo:hi] = _l2norm(k)
        out["v"][lo:hi] = v
        out["window_end"][n] = conv_window(x[lo:hi], K, win)
        saved = {}
        for p in ([] if checkpoints is None else checkpoints[n]):
            if not 1 <= p <= hi - lo:
                raise ValueError(f"checkpoint {p} outside 1..{hi - lo}")
            saved[int(p)] = conv_window(x[lo:lo + p], K, win)
        out["window_ckpt"].append(saved)
    return out


def front_end_step(x, z_a, z_b, w, g_min, H, dk, dv, window):
    """One decode token per session: the carried window supplies the K-1 rows
    before it and comes back shifted by one row.

    x : (B, C)   z_a : (B, H, dk)   z_b : (B, H)   window : (B, K-1, C)
    Returns (q, k, v, a, beta, new_window), shapes (B, H, *) and (B, K-1, C).
    """
    x, window = _f64(x), _f64(window)
    B, C = x.shape
    K = _f64(w).shape[1]
    q = np.zeros((B, H, dk))
    k = np.zeros((B, H, dk))
    v = np.zeros((B, H, dv))
    new_window = np.zeros((B, K - 1, C))
    for b in range(B):
        r = front_end(x[b:b + 1], _f64(z_a)[b:b + 1], _f64(z_b)[b:b + 1], w, g_min, H, dk, dv,
                      [0, 1], windows=window[b:b + 1])
        q[b], k[b], v[b] = r["q"][0], r["k"][0], r["v"][0]
        new_window[b] = r["window_end"][0]
    return q, k, v, g_min * sigmoid(z_a), sigmoid(z_b), new_window
