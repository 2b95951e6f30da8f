"""Plain float64 CPU oracle for the Kimi Delta Attention (KDA) state recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import this module.
The GPU library never imports it, and this module imports nothing from the GPU
library: the two share no code.  It is slow on purpose: every step is written
out in the order and notation of the pages so that it can be checked by eye.

Pages cited (titles as published; sections named as on the page):
  [Serve demo]  "【轻量化复刻大模型 / KIMI K3】Serve 模块交互式演示"
                (cveoy.top/t/topic/qHUG)
  [KDA cache]   "Kimi Linear 的 KDA 缓存：SGLang、vLLM 与 Mooncake Store 全链路"
                (imreese.github.io/blogs/kimi-kda-cache-sglang-vllm-mooncake-store)

Readings taken where the pages are silent, garbled or disagree (each one is
listed again, with the reason, in the design notes of the repository):
  R1  Decay, then error: the error term is formed against the state after the
      per-key-channel decay ([KDA cache], "KDA 的递推与充分状态", which says the
      old state is decayed per key channel first and the prediction error is
      formed next).  [Serve demo] §1.3 writes the error against the undecayed
      state; that variant is kept behind ``error_before_decay=True`` only to
      show that the two differ.
  R2  The per-channel gate ``a`` is a log-decay in [g_min, 0] ([Serve demo]
      §1.3 bounds it this way), so the decay factor applied to row i of S is
      exp(a_i), not a_i itself.
  R3  No query scaling, output gate or normalisation of o: o_t = S_t^T q_t,
      read from the state after the write ([Serve demo] §1.3 "读出").
  R4  Canonical state layout [.., dk, dv], row-major ([Serve demo] §1.5, the
      (B,H,dk,dv) shape of pack_heads); the transposed layout [.., dv, dk]
      that [KDA cache] ("先统一记号") says some kernels and pools use is
      accepted as a pack source / unpack destination.
  R5  A checkpoint at position p of a sequence is the state after exactly p
      tokens of that sequence, 1 <= p <= len; no rounding to a chunk size
      ([KDA cache], "Kimi K3 预览版与 vLLM 的细粒度检查点", exact tail C(P6976)).
  R6  A page slot holds one flattened state (B=1 view: H*dk*dv values, head
      after head); the rest of the page is zero ([Serve demo] §1.5 and Tab 7
      "KDA 存储", "后续为 pad 零").
  R7  Replay with n_accepted = 0 leaves the state equal to the committed one
      and yields no output rows; for a batch with ragged n_accepted the output
      is padded to the draft length with zeros ([Serve demo] Tab 3 §6.4).
  R14 A bf16 state (a variant; the pages keep the recurrent state in FP32,
      [KDA cache] "检查点状态池的内存成本": in the fixed vLLM snapshot the conv
      state uses the cache dtype and the recurrent state FP32): the state is
      stored in bfloat16 between calls, computed in wider precision within a
      call, and rounded to the nearest bfloat16 (ties to even) when stored.
      A decode call is one step; a replay call rounds once, at its end.
  R13 Context parallelism (KCP): [Serve demo] §1.7 says its exchange does not
      grow with the sequence length and §7.2 calls it a prefix scan, without
      a formula.  Every step is affine in the state,
      S_t = (I - beta_t k_t k_t^T) diag(exp(a_t)) S_{t-1} + beta_t k_t v_t^T,
      so a segment of a sequence maps its start state to its end state by
      S_end = A S_start + B (A is dk x dk, B is dk x dv, independent of the
      length); segments compose by (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2),
      and the exchange is an exclusive scan of these pairs.
"""

from fractions import Fraction

import numpy as np

__all__ = [
    "kda_step",
    "kda_recurrent",
    "kda_prefill",
    "verify_and_replay",
    "pack_heads",
    "unpack_heads",
    "snapshot_cost_ratio",
    "snapshot_bytes_per_step",
    "projection_bytes_per_step",
    "kda_chunked_ref",
    "segment_summary",
    "compose_segments",
    "round_bf16",
    "decode_bf16_state",
    "verify_and_replay_bf16_state",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# One step of the recurrence.
# [Serve demo] §1.3 "KDA 递推核心 (kda_step / kda_recurrent)";
# [KDA cache] "KDA 的递推与充分状态" (decay first, then the error, then the
# write of the increment only).
# ---------------------------------------------------------------------------
def kda_step(q, k, v, a, beta, S, error_before_decay=False):
    """One KDA step for any leading batch shape.

    q, k, a : (..., dk)     v : (..., dv)     beta : (...)     S : (..., dk, dv)
    Returns (o, S_new) with o : (..., dv) and S_new : (..., dk, dv).

    Decay:   S_dec[i, j] = exp(a_i) * S[i, j]                       (R2)
    Error:   delta_j     = v_j - sum_i S_dec[i, j] * k_i            (R1)
    Write:   S_new[i, j] = S_dec[i, j] + beta * k_i * delta_j
    Readout: o_j         = sum_i S_new[i, j] * q_i                  (R3)
    """
    q, k, v, a, beta, S = map(_f64, (q, k, v, a, beta, S))
    S_dec = np.exp(a)[..., :, None] * S
    if error_before_decay:
        # [Serve demo] §1.3 as printed: error against the undecayed state.
        pred = np.einsum("...ij,...i->...j", S, k)
    else:
        pred = np.einsum("...ij,...i->...j", S_dec, k)
    delta = v - pred
    S_new = S_dec + beta[..., None, None] * k[..., :, None] * delta[..., None, :]
    o = np.einsum("...ij,...i->...j", S_new, q)
    return o, S_new


def kda_recurrent(q, k, v, a, beta, S0=None, checkpoints=(), error_before_decay=False):
    """Run the recurrence over one sequence, token after token.

    q, k, a : (T, H, dk)   v : (T, H, dv)   beta : (T, H)   S0 : (H, dk, dv) or None
    checkpoints : token counts p (1 <= p <= T) at which to record the state (R5).
    Returns (o (T, H, dv), S_final (H, dk, dv), {p: state after p tokens}).

    This is the "standard answer" that replay is compared with in
    [Serve demo] Tab 3 §6.4.
    """
    q, k, v, a, beta = map(_f64, (q, k, v, a, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0).copy()
    want = set(int(p) for p in checkpoints)
    for p in want:
        if not 1 <= p <= T:
            raise ValueError(f"checkpoint position {p} outside 1..{T}")
    o = np.zeros((T, H, dv))
    saved = {}
    for t in range(T):
        o[t], S = kda_step(q[t], k[t], v[t], a[t], beta[t], S, error_before_decay)
        if (t + 1) in want:
            saved[t + 1] = S.copy()
    return o, S, saved


def kda_prefill(q, k, v, a, beta, cu_seqlens, S0=None, checkpoints=None):
    """Token-packed, variable-length prefill: independent sequences, one state each.

    q, k, a : (T_tot, H, dk)  v : (T_tot, H, dv)  beta : (T_tot, H)
    cu_seqlens : (N+1,) offsets, cu[0] = 0, non-decreasing, cu[N] = T_tot.
    S0 : (N, H, dk, dv) committed states (read, never written) or None for zero.
    checkpoints : list of N lists of token counts (R5), or None.
    Returns (o (T_tot, H, dv), S_final (N, H, dk, dv), ckpt) where ckpt[n] maps
    p -> state of sequence n after p tokens.

    A sequence of length 0 leaves its state equal to S0 and emits nothing.
    A state restored from a checkpoint can only be advanced, never rewound
    ([KDA cache], "KDA 的递推与充分状态", one-way reuse).
    """
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    T_tot, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    if cu[0] != 0 or cu[-1] != T_tot or any(cu[i + 1] < cu[i] for i in range(N)):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_tot")
    o = np.zeros((T_tot, H, dv))
    S_final = np.zeros((N, H, dk, dv))
    ckpt = []
    for n in range(N):
        lo, hi = cu[n], cu[n + 1]
        s_init = None if S0 is None else _f64(S0)[n].copy()
        pos = () if checkpoints is None else checkpoints[n]
        if hi == lo:
            if len(pos):
                raise ValueError("a zero-length sequence has no checkpoint positions")
            S_final[n] = 0.0 if s_init is None else s_init
            ckpt.append({})
            continue
        o_n, s_n, saved = kda_recurrent(q[lo:hi], k[lo:hi], v[lo:hi], a[lo:hi],
                                        beta[lo:hi], s_init, pos)
        o[lo:hi] = o_n
        S_final[n] = s_n
        ckpt.append(saved)
    return o, S_final, ckpt


# ---------------------------------------------------------------------------
# Speculative verify-and-replay.
# [Serve demo] §1.2 "verify_and_replay 重演一致性" (clone the committed state,
# step n_accepted times, stack the outputs as (B, H, n, Dv)); §1.1 route B for
# the projection layout (draft, B, H, D).
# ---------------------------------------------------------------------------
def verify_and_replay(committed, q, k, v, a, beta, n_accepted):
    """committed : (B, H, dk, dv) — never modified.
    q, k, a : (Td, B, H, dk)   v : (Td, B, H, dv)   beta : (Td, B, H)
    n_accepted : (B,) ints in 0..Td
    Returns (S_new (B, H, dk, dv), O (B, H, Td, dv)) with O[b, :, n_b:] = 0 (R7).
    """
    committed = _f64(committed)
    q, k, v, a, beta = map(_f64, (q, k, v, a, beta))
    Td, B, H, dk = k.shape
    dv = v.shape[-1]
    S_new = np.zeros((B, H, dk, dv))
    O = np.zeros((B, H, Td, dv))
    for b in range(B):
        n = int(n_accepted[b])
        if not 0 <= n <= Td:
            raise ValueError("n_accepted must lie in 0..Td")
        S = committed[b].copy()  # the clone: the committed state is shared
        for i in range(n):
            O[b, :, i], S = kda_step(q[i, b], k[i, b], v[i, b], a[i, b], beta[i, b], S)
        S_new[b] = S
    return S_new, O


# ---------------------------------------------------------------------------
# Head packing into flat page slots.
# [Serve demo] §1.5 "统一页池 (PagedCache)": pack_heads (B,H,dk,dv) -> flat,
# each head laid out contiguously, unpack_heads flat -> (B,H,dk,dv) losslessly;
# Tab 7 "KDA 存储": the state is written flat into the page and the rest of
# the page is zero padding.
# ---------------------------------------------------------------------------
def pack_heads(state, slots, page_pool, layout="kv"):
    """Write state[b] into page_pool[slots[b]], flattened head after head.

    state : (B, H, dk, dv) for layout "kv" or (B, H, dv, dk) for layout "vk"
    page_pool : (n_slots, page_elems), modified in place and returned.
    Element (h, i, j) of a slot (i over dk, j over dv) sits at h*dk*dv + i*dv + j;
    elements at H*dk*dv and beyond are set to zero.
    """
    state = np.asarray(state)
    B, H = state.shape[:2]
    if layout == "kv":
        dk, dv = state.shape[2], state.shape[3]
    elif layout == "vk":
        dv, dk = state.shape[2], state.shape[3]
    else:
        raise ValueError("layout must be 'kv' or 'vk'")
    n_slots, page_elems = page_pool.shape
    if page_elems < H * dk * dv:
        raise ValueError("page too small for one state")
    for b in range(B):
        s = int(slots[b])
        if not 0 <= s < n_slots:
            raise ValueError("slot out of range")
        page = page_pool[s]
        page[:] = 0
        for h in range(H):
            for i in range(dk):
                for j in range(dv):
                    x = state[b, h, i, j] if layout == "kv" else state[b, h, j, i]
                    page[h * dk * dv + i * dv + j] = x
    return page_pool


def unpack_heads(page_pool, slots, H, dk, dv, layout="kv"):
    """Inverse of pack_heads: read page_pool[slots[b]] back into a state tensor."""
    page_pool = np.asarray(page_pool)
    B = len(slots)
    shape = (B, H, dk, dv) if layout == "kv" else (B, H, dv, dk)
    out = np.zeros(shape, dtype=page_pool.dtype)
    for b in range(B):
        page = page_pool[int(slots[b])]
        for h in range(H):
            for i in range(dk):
                for j in range(dv):
                    x = page[h * dk * dv + i * dv + j]
                    if layout == "kv":
                        out[b, h, i, j] = x
                    else:
                        out[b, h, j, i] = x
    return out


# ---------------------------------------------------------------------------
# Byte accounting of the two rollback routes.
# [Serve demo] §1.1 "KDA 投机回放：投影缓存 vs 完整快照": per step a snapshot
# holds H*dk*dv values and a projection holds H*(3*dk + dv + 1) values
# (q, k, g of length dk, v of length dv, and the scalar beta).
# ---------------------------------------------------------------------------
def snapshot_bytes_per_step(H, dk, dv, itemsize):
    return H * dk * dv * itemsize


def projection_bytes_per_step(H, dk, dv, itemsize):
    return H * (3 * dk + dv + 1) * itemsize


def snapshot_cost_ratio(H, dk, dv):
    """Exact ratio snapshot bytes / projection bytes (independent of draft length)."""
    return Fraction(H * dk * dv, H * (3 * dk + dv + 1))


# ---------------------------------------------------------------------------
# Chunked form, float64.  Not the oracle of record: it exists to pin, against
# the plain recurrence, the algebra that a chunked GPU kernel relies on.
# [KDA cache] "预填充为什么能分块并行": within a chunk the transitions are each
# "diagonal minus rank one" and are compressed with a WY representation and a
# UT transform into matrix products plus a small lower-triangular solve.
# The equations below are derived from the recurrence in kda_step:
#   S_r = (I - beta_r k_r k_r^T) diag(exp(a_r)) S_{r-1} + beta_r k_r v_r^T.
# With G_r = sum_{i<=r} a_i (cumulative over the chunk), g_r = exp(G_r) and
# u_r = beta_r * delta_r, unrolling gives
#   S_r = diag(g_r) S + sum_{i<=r} diag(g_r / g_i) k_i u_i^T,
# hence the lower-triangular system
#   (I + diag(beta) tril_{-1}(Kp Km^T)) U = diag(beta) (V - Kp S)
# with Kp_r = k_r*g_r and Km_r = k_r/g_r, whose solution gives
#   O = Qp S + tril_0(Qp Km^T) U,   S_next = diag(g_n) S + Kh^T U,
# where Qp_r = q_r*g_r and Kh_r = k_r*g_n/g_r.
# ---------------------------------------------------------------------------
def kda_chunked_ref(q, k, v, a, beta, S0=None, chunk=64):
    """One sequence, one head: q, k, a (T, dk), v (T, dv), beta (T,), S0 (dk, dv)."""
    q, k, v, a, beta = map(_f64, (q, k, v, a, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, dv))
    for lo in range(0, T, chunk):
        hi = min(lo + chunk, T)
        n = hi - lo
        G = np.cumsum(a[lo:hi], axis=0)          # (n, dk)
        g = np.exp(G)
        Kp = k[lo:hi] * g
        Km = k[lo:hi] / g
        Qp = q[lo:hi] * g
        Kh = k[lo:hi] * (g[n - 1] / g)
        b = beta[lo:hi]
        M = np.eye(n) + b[:, None] * np.tril(Kp @ Km.T, -1)
        rhs = b[:, None] * (v[lo:hi] - Kp @ S)
        U = np.linalg.solve(M, rhs)
        o[lo:hi] = Qp @ S + np.tril(Qp @ Km.T) @ U
        S = g[n - 1][:, None] * S + Kh.T @ U
    return o, S


# ---------------------------------------------------------------------------
# Context-parallel segments (reading R13)

def segment_summary(k, v, a, beta):
    """Affine map of one segment of a sequence, per head.

    k, a : (T, H, dk)   v : (T, H, dv)   beta : (T, H)
    Returns (A, B), A (H, dk, dk) and B (H, dk, dv), with S_end = A @ S_start + B
    for every start state.  Written as the plain product of the per-token maps
    S <- (I - beta k k^T) diag(exp(a)) S + beta k v^T (decay, then error: R1).
    """
    k, v, a, beta = (_f64(x) for x in (k, v, a, beta))
    T, H, dk = k.shape
    dv = v.shape[2]
    A = np.tile(np.eye(dk), (H, 1, 1))
    B = np.zeros((H, dk, dv))
    for t in range(T):
        for h in range(H):
            kk = k[t, h]
            M = (np.eye(dk) - beta[t, h] * np.outer(kk, kk)) * np.exp(a[t, h])[None, :]
            A[h] = M @ A[h]
            B[h] = M @ B[h] + beta[t, h] * np.outer(kk, v[t, h])
    return A, B


def compose_segments(A, B, S_in=None):
    """Exclusive scan of segment maps: the start state of every segment.

    A : (n, H, dk, dk)   B : (n, H, dk, dv)   S_in : (H, dk, dv) or None (zero)
    Returns (starts (n, H, dk, dv), S_end (H, dk, dv)) with starts[0] = S_in and
    starts[i+1] = A[i] @ starts[i] + B[i].
    """
    A, B = _f64(A), _f64(B)
    n, H, dk, dv = B.shape
    S = np.zeros((H, dk, dv)) if S_in is None else _f64(S_in).copy()
    starts = np.zeros((n, H, dk, dv))
    for i in range(n):
        starts[i] = S
        S = A[i] @ S + B[i]
    return starts, S


# ---------------------------------------------------------------------------
# A bfloat16 state (reading R14).
# ---------------------------------------------------------------------------
def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even, returned as float64.

    bfloat16 keeps 8 significant bits (7 stored) and float32's exponent range.
    With x = m * 2**e, 0.5 <= |m| < 1, the nearest value with 8 significant
    bits is rint(m * 2**8) * 2**(e - 8), rint rounding halves to even.  For
    values in the normal range (|x| >= 2**-126) and below the overflow
    threshold, which is where states live.
    """
    x = _f64(x)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def decode_bf16_state(q, k, v, a, beta, S_bf16):
    """One decode step on a bfloat16 state: the step in float64 from the
    stored values, the new state rounded to bfloat16 (R14).  Returns (o, S)."""
    o, S = kda_step(q, k, v, a, beta, _f64(S_bf16))
    return o, round_bf16(S)


def verify_and_replay_bf16_state(committed_bf16, q, k, v, a, beta, n_accepted):
    """verify_and_replay from a bfloat16 committed state; the replayed state
    is rounded to bfloat16 once, at the end of the call (R14)."""
    s_new, o = verify_and_replay(_f64(committed_bf16), q, k, v, a, beta, n_accepted)
    return round_bf16(s_new), o
