"""GPU parity: segment summaries (A, B) and their composition, against the
float64 oracle, and the context-parallel identity: summaries -> composed start
states -> prefill of each segment from its start reproduces one pass over the
whole sequence."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu

FIELDS = ("q", "k", "v", "a", "beta")


def _dev(w, dtype):
    return {n: dev_tensor(w[n], dtype) for n in FIELDS}


SEG_LENS = [1, 17, 64, 0, 100, 130]


def _summary(w, dtype, chunk):
    d = _dev(w, dtype)
    A, B = kda.segment_summary(d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], chunk=chunk)
    torch.cuda.synchronize()
    return to_np(A), to_np(B)


def _oracle_summary(w, s):
    cu = w["cu_seqlens"]
    lo, hi = int(cu[s]), int(cu[s + 1])
    return oracle.segment_summary(w["k"][lo:hi], w["v"][lo:hi], w["a"][lo:hi], w["beta"][lo:hi])


def _check_map(An, Bn, A_r, B_r, X, dtype, what):
    """B, and the end state A X + B from the unit-scale start state X (the
    map as composition uses it), per head."""
    for h in range(A_r.shape[0]):
        assert_parity(Bn[h], B_r[h], dtype, f"B {what} head {h}")
        assert_parity(An[h] @ X[h] + Bn[h], A_r[h] @ X[h] + B_r[h], dtype,
                      f"A X + B {what} head {h}")


@pytest.mark.parametrize("dk,dv,dtype,chunk", [(16, 16, "fp32", 16), (32, 64, "bf16", 64),
                                               (64, 32, "fp32", 32), (128, 128, "bf16", 64),
                                               (128, 16, "bf16", 16), (128, 128, "fp32", 32)])
def test_segment_summary_matches_oracle(dk, dv, dtype, chunk):
    """Ragged segments of the standard workload (g_min = -1).  Its decay takes
    the linear part A below fp32's range within a few hundred tokens (the
    oracle's A for 256 tokens is ~1e-52), so A is checked through the end
    state it produces; test_segment_linear_part_weak_decay checks A itself."""
    H = 2
    w = inputs.prefill_workload(60 + dk + dv, SEG_LENS, H, dk, dv, dtype)
    An, Bn = _summary(w, dtype, chunk)
    X = inputs.state_normal(61, 0, (H, dk, dv), 1.0).astype(np.float64)
    for s in range(len(SEG_LENS)):
        A_r, B_r = _oracle_summary(w, s)
        if SEG_LENS[s] == 0:  # the empty segment: exactly the identity map
            assert np.array_equal(An[s], A_r) and not Bn[s].any()
            continue
        _check_map(An[s], Bn[s], A_r, B_r, X, dtype, f"seg {s}")


@pytest.mark.parametrize("dk,dv,dtype,chunk", [(32, 64, "bf16", 64), (128, 128, "bf16", 64),
                                               (64, 64, "fp32", 32), (128, 32, "fp32", 16)])
def test_segment_linear_part_weak_decay(dk, dv, dtype, chunk):
    """Weak decay (g_min = -0.05) keeps A in range over hundreds of tokens.
    fp32: A itself at every length.  bf16: A itself up to two chunks, since
    each token's map adds operand rounding to the product and A's relative
    error grows like sqrt(length) (about 0.5% at 100 tokens and dk = 32, 1%
    at 2048 tokens and dk = 128); its effect on the end state is checked at
    every length."""
    H, lens = 2, [16, 100, 300, 513]
    w = inputs.prefill_workload(62 + dk + dv, lens, H, dk, dv, dtype, g_min=-0.05)
    An, Bn = _summary(w, dtype, chunk)
    X = inputs.state_normal(63, 0, (H, dk, dv), 1.0).astype(np.float64)
    for s, L in enumerate(lens):
        A_r, B_r = _oracle_summary(w, s)
        _check_map(An[s], Bn[s], A_r, B_r, X, dtype, f"seg {s}")
        if dtype == "fp32" or L <= 2 * chunk:
            for h in range(H):
                assert_parity(An[s, h], A_r[h], dtype, f"A seg {s} (length {L}) head {h}")


@pytest.mark.parametrize("dk,dv,with_s_in", [(16, 16, True), (64, 32, False), (128, 128, True)])
def test_compose_matches_oracle(dk, dv, with_s_in):
    n, H = 5, 3
    A = inputs.state_normal(70, 0, (n, H, dk, dk), 1.0 / np.sqrt(dk))
    B = inputs.state_normal(70, 1, (n, H, dk, dv), 0.3)
    s_in = inputs.state_normal(70, 2, (H, dk, dv), 0.5) if with_s_in else None
    dev = lambda x: None if x is None else torch.from_numpy(x).cuda()
    starts, s_end = kda.compose_segments(dev(A), dev(B), dev(s_in))
    torch.cuda.synchronize()
    st_r, end_r = oracle.compose_segments(A, B, s_in)
    for i in range(n):
        assert_parity(starts[i], st_r[i], "fp32", f"start {i}")
    assert_parity(s_end, end_r, "fp32", "end")
    if s_in is not None:
        assert torch.equal(starts[0], dev(s_in)), "starts[0] must be s_in exactly"


def test_compose_zero_segments_returns_s_in():
    H, dk, dv = 2, 32, 16
    s_in = torch.from_numpy(inputs.state_normal(71, 0, (H, dk, dv), 1.0)).cuda()
    A = torch.empty((0, H, dk, dk), device="cuda")
    B = torch.empty((0, H, dk, dv), device="cuda")
    _, s_end = kda.compose_segments(A, B, s_in)
    torch.cuda.synchronize()
    assert torch.equal(s_end, s_in)


def test_empty_segments_only():
    H, dk, dv = 2, 64, 64
    z = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    A, B = kda.segment_summary(z(0, H, dk), z(0, H, dv), z(0, H, dk), z(0, H), [0, 0, 0])
    torch.cuda.synchronize()
    eye = torch.eye(dk, device="cuda").expand(2, H, dk, dk)
    assert torch.equal(A, eye) and not B.any()


@pytest.mark.parametrize("dtype,chunk,d,g_min", [("bf16", 64, 128, -1.0), ("fp32", 32, 64, -1.0),
                                                 ("bf16", 16, 32, -1.0), ("bf16", 64, 128, -0.05),
                                                 ("fp32", 32, 32, -0.05)])
def test_sequential_equals_composed(dtype, chunk, d, g_min):
    """One pass over the whole sequence == summaries, composition, then a
    prefill of every segment from its composed start state.  With weak decay
    (g_min = -0.05) the start states carry into the segments' ends, so the
    linear parts A matter to the result."""
    T, H = 1000, 2
    cut = [0, 250, 251, 600, 1000]  # ragged, one single-token segment
    w = inputs.prefill_workload(80 + d, [T], H, d, d, dtype, s0_std=0.1, g_min=g_min)
    dd = _dev(w, dtype)
    s0 = torch.from_numpy(w["s0"]).cuda()
    o_all, sf_all = kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dd["a"], dd["beta"], [0, T],
                                      s0=s0, chunk=chunk)
    A, B = kda.segment_summary(dd["k"], dd["v"], dd["a"], dd["beta"], cut, chunk=chunk)
    starts, s_end = kda.compose_segments(A, B, s0[0])
    o_seg, sf_seg = kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dd["a"], dd["beta"], cut,
                                      s0=starts, chunk=chunk)
    torch.cuda.synchronize()
    # Against the oracle: the true states at the cuts and the outputs.
    for h in range(H):
        o_r, S_r, saved = oracle.kda_recurrent(*(w[f][:, h:h + 1] for f in ("q", "k", "v", "a")),
                                               w["beta"][:, h:h + 1], w["s0"][0, h][None], cut[1:-1])
        for i, p in enumerate(cut[1:-1], start=1):
            assert_parity(starts[i, h], saved[p][0], dtype, f"composed start {i} head {h}")
        assert_parity(s_end[h], S_r[0], dtype, f"composed end head {h}")
        assert_parity(o_seg[:, h], o_r[:, 0], dtype, f"segmented o head {h}")
        assert_parity(sf_seg[-1, h], S_r[0], dtype, f"segmented final state head {h}")
    # Against the one pass on the GPU.
    assert_parity(o_seg, o_all, dtype, "segmented o vs one pass")
    assert_parity(s_end, sf_all[0], dtype, "composed end vs one pass")
    for i in range(len(cut) - 2):
        assert_parity(sf_seg[i], starts[i + 1], dtype, f"segment {i} end vs composed start")
