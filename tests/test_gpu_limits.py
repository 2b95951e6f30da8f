"""GPU parity at the method's limits.

- The decay bound: log-decays a in [g_min, 0] ("【轻量化复刻大模型 / KIMI K3】
  Serve 模块交互式演示" §1.3) down to the prefill's documented edge,
  a = -160/chunk (-2.5 at chunk 64, -5 at chunk 32), and the flag raised for a
  value just past it (or a NaN, or a growth a > 0), with nothing written.
- Closed forms the pages fix, run through the kernels (prefill, decode,
  replay), not only through the oracle:
  beta = 0: the state only decays, S_t = diag(exp(sum a)) S0 and
  o_t = S_t^T q_t;
  a = 0, beta = 1, unit k: after the write S^T k = v ("Kimi Linear 的 KDA 缓存"
  page, "KDA 的递推与充分状态": the delta rule writes only the increment), so
  with q = k every output equals its own v;
  one token from S0 = 0: S = beta k v^T and o = beta (k . q) v.
Each closed form is computed here in float64 from the inputs alone; the
oracle is compared as well where it is cheap.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu

FIELDS = ("q", "k", "v", "a", "beta")
LENS = [1, 15, 64, 0, 65, 100, 130, 200]


def _prefill(w, dtype, chunk, err_flag=None, ck=None, o=None, s_final=None, pool=None):
    d = {n: dev_tensor(w[n], dtype) for n in FIELDS}
    s0 = None if w.get("s0") is None else torch.from_numpy(w["s0"]).cuda()
    slots = None
    if ck is not None:
        slots, i = [], 0
        for c in ck:
            slots.append(list(range(i, i + len(c))))
            i += len(c)
    res = kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], s0=s0,
                            chunk=chunk, checkpoints=ck, ckpt_slots=slots, page_pool=pool, o=o,
                            s_final=s_final, err_flag=err_flag)
    torch.cuda.synchronize()
    return res, slots


def _workload(wid, dtype, H=2, d=128, a_fill=None, s0_std=0.1, g_min=-1.0):
    w = inputs.prefill_workload(wid, LENS, H, d, d, dtype, s0_std=s0_std, g_min=g_min)
    if a_fill is not None:
        w["a"][...] = a_fill(w["a"].shape)
        if dtype == "bf16":
            w["a"] = inputs.round_to_bf16(w["a"])
    return w


def _oracle_check(w, dtype, o, sf, pool, slots, ck):
    o_r, s_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"],
                                        w["s0"], ck)
    cu = w["cu_seqlens"]
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        if hi > lo:
            assert_parity(o[lo:hi], o_r[lo:hi], dtype, f"o seq {n}")
        assert_parity(sf[n], s_r[n], dtype, f"s_final seq {n}")
        for j, p in enumerate(ck[n]):
            assert_parity(pool[slots[n][j]].reshape(s_r[n].shape), ck_r[n][p], dtype, f"ckpt {p} seq {n}")


# ---------------------------------------------------------------- decay edge
EDGE = [("bf16", 64, "const"), ("bf16", 64, "uniform"), ("fp32", 32, "const"), ("fp32", 32, "uniform"),
        ("bf16", 32, "const"), ("bf16", 32, "uniform")]


@pytest.mark.parametrize("dtype,chunk,kind", EDGE)
def test_prefill_at_the_decay_bound(dtype, chunk, kind):
    """a = -160/chunk on every channel of every token (the decay bound the
    header promises), or uniform in [-160/chunk, 0]: ragged sequences with
    nonzero S0 and checkpoints, against the oracle at the usual bars; the
    error flag stays clear."""
    lo = -160.0 / chunk
    rng = np.random.default_rng(chunk)
    fill = (lambda shp: np.full(shp, lo, np.float32)) if kind == "const" else \
        (lambda shp: rng.uniform(lo, 0.0, shp).astype(np.float32))
    w = _workload(300 + chunk, dtype, a_fill=fill)
    assert w["a"].min() >= lo
    ck = [sorted({p for p in (1, 16, 33, L) if 1 <= p <= L}) for L in LENS]
    H, d = 2, 128
    pool = torch.full((sum(len(c) for c in ck), H * d * d), float("nan"), device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    (o, sf), slots = _prefill(w, dtype, chunk, err_flag=flag, ck=ck, pool=pool)
    assert int(flag.item()) == 0
    assert torch.isfinite(o.float()).all() and torch.isfinite(sf).all()
    _oracle_check(w, dtype, o, sf, pool, slots, ck)


BAD = [("below", -2.515625), ("nan", float("nan")), ("growth", 0.5)]


@pytest.mark.parametrize("kind,value", BAD)
@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("fp32", 32)])
def test_prefill_flags_a_decay_out_of_range(kind, value, dtype, chunk):
    """One log-decay out of [-160/chunk, 0] (just below the bound, a NaN, or a
    growth a > 0) in one token of one sequence: the flag is raised and the
    call writes nothing (o, s_final and the page slots keep their bytes)."""
    w = _workload(320, dtype)
    if kind == "below" and chunk == 32:
        value = -5.03125  # the next bf16 value below -5
    w["a"][140, 1, 77] = value
    ck = [[L] if L else [] for L in LENS]
    H, d = 2, 128
    T = int(w["cu_seqlens"][-1])
    sentinel = 0.375
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((T, H, d), sentinel, dtype=dt, device="cuda")
    sf = torch.full((len(LENS), H, d, d), sentinel, device="cuda")
    pool = torch.full((sum(len(c) for c in ck), H * d * d), sentinel, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    _prefill(w, dtype, chunk, err_flag=flag, ck=ck, o=o, s_final=sf, pool=pool)
    assert int(flag.item()) == 1
    assert bool((o.float() == sentinel).all()), "o was written"
    assert bool((sf == sentinel).all()), "s_final was written"
    assert bool((pool == sentinel).all()), "a page slot was written"
    # The same call with the value back in range runs and leaves the flag alone.
    w["a"][140, 1, 77] = -0.5
    flag.zero_()
    (o2, sf2), _ = _prefill(w, dtype, chunk, err_flag=flag, ck=ck, pool=pool)
    assert int(flag.item()) == 0 and torch.isfinite(o2.float()).all()


def test_gated_prefill_flags_a_nan_logit():
    """A NaN gate logit makes a NaN decay: flagged, nothing written."""
    w = _workload(321, "bf16")
    z_a = inputs.round_to_bf16(np.random.default_rng(3).standard_normal(w["a"].shape).astype(np.float32))
    z_b = inputs.round_to_bf16(np.random.default_rng(4).standard_normal(w["beta"].shape).astype(np.float32))
    z_a[10, 0, 3] = np.nan
    d = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v")}
    T, H, dd = int(w["cu_seqlens"][-1]), 2, 128
    o = torch.full((T, H, dd), 0.375, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.chunk_prefill(d["q"], d["k"], d["v"], dev_tensor(z_a, "bf16"), dev_tensor(z_b, "bf16"),
                      w["cu_seqlens"], chunk=64, o=o, gate_g_min=-1.0, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1 and bool((o.float() == 0.375).all())


# ---------------------------------------------------------------- closed forms
def _decay_only(w):
    """beta = 0: S_t = diag(exp(G_t)) S0 with G_t the running sum of a, and
    o_t = S_t^T q_t (float64, from the inputs alone)."""
    cu = w["cu_seqlens"]
    o = np.zeros(w["v"].shape)
    sf = np.zeros(w["s0"].shape)
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        S0 = w["s0"][n].astype(np.float64)
        G = np.cumsum(w["a"][lo:hi].astype(np.float64), axis=0)          # (L, H, dk)
        St = np.exp(G)[..., None] * S0[None]                              # (L, H, dk, dv)
        o[lo:hi] = np.einsum("thij,thi->thj", St, w["q"][lo:hi].astype(np.float64))
        sf[n] = St[-1] if hi > lo else S0
    return o, sf


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("fp32", 32), ("bf16", 32)])
def test_prefill_beta_zero_only_decays(dtype, chunk):
    w = _workload(330, dtype, g_min=-0.05)
    w["beta"][...] = 0.0
    (o, sf), _ = _prefill(w, dtype, chunk)
    o_c, sf_c = _decay_only(w)
    assert_parity(o, o_c, dtype, "o (beta = 0)")
    assert_parity(sf, sf_c, dtype, "s_final (beta = 0)")


def _unit_write(w, seed=0):
    """a = 0, beta = 1 and q = k with keys of norm exactly 1 in any dtype:
    sixteen entries of +-1/4 at random places, the rest 0."""
    w["a"][...] = 0.0
    w["beta"][...] = 1.0
    rng = np.random.default_rng(seed)
    k = np.zeros(w["k"].shape, np.float32)
    flat = k.reshape(-1, k.shape[-1])
    for r in range(flat.shape[0]):
        idx = rng.choice(flat.shape[1], 16, replace=False)
        flat[r, idx] = rng.choice([-0.25, 0.25], 16)
    w["k"] = k
    w["q"] = k.copy()
    return w


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("fp32", 32), ("bf16", 32)])
def test_prefill_delta_write_reads_back_v(dtype, chunk):
    """a = 0, beta = 1, unit k and q = k: every output is its token's own v,
    and the state at a checkpoint p reproduces v_p through S_p^T k_p."""
    w = _unit_write(_workload(331, dtype))
    ck = [[L] if L else [] for L in LENS]
    H, d = 2, 128
    pool = torch.zeros((sum(len(c) for c in ck), H * d * d), device="cuda")
    (o, sf), slots = _prefill(w, dtype, chunk, ck=ck, pool=pool)
    assert_parity(o, w["v"].astype(np.float64), dtype, "o = v")
    cu = w["cu_seqlens"]
    for n, L in enumerate(LENS):
        if L == 0:
            continue
        last = int(cu[n + 1]) - 1
        S = to_np(pool[slots[n][0]]).reshape(H, d, d)
        back = np.einsum("hij,hi->hj", S, w["k"][last].astype(np.float64))
        assert_parity(back, w["v"][last].astype(np.float64), dtype, f"S_p^T k_p = v_p, seq {n}")
        assert_parity(np.einsum("hij,hi->hj", to_np(sf[n]), w["k"][last].astype(np.float64)),
                      w["v"][last].astype(np.float64), dtype, f"s_final^T k = v, seq {n}")


@pytest.mark.parametrize("dtype,chunk,dk", [("bf16", 64, 64), ("fp32", 32, 64), ("bf16", 32, 128)])
def test_prefill_single_tokens_from_zero(dtype, chunk, dk):
    """Sequences of one token from S0 = 0: S = beta k v^T, o = beta (k . q) v.
    (bf16 at chunk 32 with dk = 128 runs the fused kernel.)"""
    w = inputs.prefill_workload(332, [1] * 7, 2, dk, 128, dtype)
    (o, sf), _ = _prefill(w, dtype, chunk)
    k, q, v, b = (w[n].astype(np.float64) for n in ("k", "q", "v", "beta"))
    S = b[..., None, None] * k[..., :, None] * v[..., None, :]
    assert_parity(sf, S, dtype, "S = beta k v^T")
    assert_parity(o, (b * np.einsum("thi,thi->th", k, q))[..., None] * v, dtype, "o = beta (k.q) v")


def _decode_steps(state, steps, dtype):
    st = torch.from_numpy(state.astype(np.float32)).cuda()
    outs = []
    for t in steps:
        d = {n: dev_tensor(x, dtype) for n, x in t.items()}
        outs.append(kda.decode_step(d["q"], d["k"], d["v"], d["a"], d["beta"], st))
    torch.cuda.synchronize()
    return torch.stack(outs), st


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_closed_forms(dtype):
    B, H, dk, dv = 4, 2, 128, 64
    S0 = inputs.state_normal(340, 0, (B, H, dk, dv), 0.1)
    # beta = 0 over five steps: diag(exp(sum a)) S0, o_t = S_t^T q_t
    steps = [inputs.token_inputs(340, s, (B,), H, dk, dv, dtype, g_min=-0.05) for s in range(5)]
    for t in steps:
        t["beta"][...] = 0.0
    o, st = _decode_steps(S0, steps, dtype)
    G = np.zeros((B, H, dk))
    for i, t in enumerate(steps):
        G += t["a"]
        St = np.exp(G)[..., None] * S0
        assert_parity(o[i], np.einsum("bhij,bhi->bhj", St, t["q"].astype(np.float64)), dtype, f"o step {i}")
    assert_parity(st, np.exp(G)[..., None] * S0, dtype, "state (beta = 0)")
    # a = 0, beta = 1, q = k: o = v at every step
    steps = [_unit_write(inputs.token_inputs(341, s, (B,), H, dk, dv, dtype), s) for s in range(5)]
    o, st = _decode_steps(S0, steps, dtype)
    for i, t in enumerate(steps):
        assert_parity(o[i], t["v"].astype(np.float64), dtype, f"o = v step {i}")
    # one step from the zero state: S = beta k v^T, o = beta (k.q) v
    t = inputs.token_inputs(342, 0, (B,), H, dk, dv, dtype)
    o, st = _decode_steps(np.zeros((B, H, dk, dv)), [t], dtype)
    k, q, v, b = (t[n].astype(np.float64) for n in ("k", "q", "v", "beta"))
    assert_parity(st, b[..., None, None] * k[..., :, None] * v[..., None, :], dtype, "S = beta k v^T")
    assert_parity(o[0], (b * np.einsum("bhi,bhi->bh", k, q))[..., None] * v, dtype, "o = beta (k.q) v")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_replay_closed_forms(dtype):
    """Replay of t_draft = 6 steps with n_accepted = 0..6 per session."""
    B, H, dk, dv, Td = 7, 2, 64, 64, 6
    S0 = inputs.state_normal(350, 0, (B, H, dk, dv), 0.1)
    n_acc = np.arange(B, dtype=np.int32) % (Td + 1)
    committed = torch.from_numpy(S0).cuda()
    nacc = torch.from_numpy(n_acc).cuda()

    def replay(t):
        d = {n: dev_tensor(x, dtype) for n, x in t.items()}
        s_new, o = kda.verify_and_replay(committed, d["q"], d["k"], d["v"], d["a"], d["beta"], nacc)
        torch.cuda.synchronize()
        return s_new, to_np(o)

    # beta = 0
    t = inputs.token_inputs(350, 1, (Td, B), H, dk, dv, dtype, g_min=-0.05)
    t["beta"][...] = 0.0
    s_new, o = replay(t)
    G = np.cumsum(t["a"].astype(np.float64), axis=0)  # (Td, B, H, dk)
    for b in range(B):
        n = int(n_acc[b])
        for i in range(n):
            St = np.exp(G[i, b])[..., None] * S0[b]
            assert_parity(o[b, :, i], np.einsum("hij,hi->hj", St, t["q"][i, b].astype(np.float64)), dtype,
                          f"o b={b} i={i}")
        want = S0[b] if n == 0 else np.exp(G[n - 1, b])[..., None] * S0[b]
        assert_parity(s_new[b], want, dtype, f"s_new b={b} (beta = 0)")
        assert not o[b, :, n:].any()
    # a = 0, beta = 1, q = k: every accepted row is its own v
    t = _unit_write(inputs.token_inputs(351, 1, (Td, B), H, dk, dv, dtype))
    s_new, o = replay(t)
    for b in range(B):
        n = int(n_acc[b])
        if n:
            assert_parity(o[b, :, :n], np.moveaxis(t["v"][:n, b], 0, 1).astype(np.float64), dtype, f"o = v b={b}")
    assert torch.equal(committed, torch.from_numpy(S0).cuda()), "committed was written"
