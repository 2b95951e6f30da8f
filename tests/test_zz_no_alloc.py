"""kda_chunk_prefill_static (its workspace is the library's static device
array, so the call allocates nothing) against kda_chunk_prefill with a caller
workspace, both through the C ABI: two calls in a row, the second on a
smaller input, on the fused path (chunk 32) and on the two-kernel path
(chunk 64); and the refusal of a call whose workspace does not fit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor

pytestmark = pytest.mark.gpu

I32 = ctypes.c_int32


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _arr(xs):
    return (I32 * max(1, len(xs)))(*xs)


def _call(w, chunk, static, ck=None):
    """One prefill of workload w (bf16, S0; checkpoints ck per sequence, by
    default one at min(length, 40)) through kda_chunk_prefill_static or
    kda_chunk_prefill with a fresh workspace."""
    L = kda.lib()
    cu = [int(x) for x in w["cu_seqlens"]]
    N, T = len(cu) - 1, cu[-1]
    H, dk = w["k"].shape[1:]
    dv = w["v"].shape[2]
    t = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v", "a", "beta")}
    s0 = torch.from_numpy(w["s0"]).cuda()
    if ck is None:
        ck = [[min(int(L_), 40)] for L_ in np.diff(cu)]  # one checkpoint per sequence (no empty ones here)
    ck_pos = [p for c in ck for p in c]
    assert min(ck_pos) > 0
    ck_cu = [0] + np.cumsum([len(c) for c in ck]).tolist()
    n_ck = len(ck_pos)
    slots = list(range(n_ck))[::-1]
    pool = torch.full((n_ck, H * dk * dv), float("nan"), device="cuda")
    o = torch.full((T, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    sf = torch.full((N, H, dk, dv), float("nan"), device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["a"]), _p(t["beta"]), kda.KDA_BF16, H, dk, dv, chunk,
              _arr(cu), N, _p(s0), _p(o), _p(sf), _arr(ck_cu), _arr(ck_pos), _arr(slots), n_ck, _p(pool),
              H * dk * dv, n_ck)
    if static:
        st = L.kda_chunk_prefill_static(*common, _p(flag), stream)
    else:
        need = ctypes.c_size_t(0)
        assert L.kda_chunk_prefill_workspace_size(N, T, H, dk, dv, chunk, n_ck, kda.KDA_BF16,
                                                  ctypes.byref(need)) == 0
        ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
        st = L.kda_chunk_prefill(*common, _p(ws), need.value, _p(flag), stream)
    assert st == kda.KDA_OK, L.kda_last_error()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    return o, sf, pool, slots, ck


@pytest.mark.parametrize("chunk", [32, 64])
def test_static_matches_workspace_entry_twice(chunk):
    """Two calls in a row (the second smaller): each output of the static entry
    equals the workspace entry's bit for bit (same kernels, same work list),
    and both meet the oracle's bar."""
    assert kda.lib().kda_static_scratch_bytes() == 64 << 20
    big = inputs.prefill_workload(500 + chunk, [300, 77, 1, 150], 4, 128, 128, "bf16", s0_std=0.1)
    small = inputs.prefill_workload(501 + chunk, [40, 9], 4, 128, 128, "bf16", s0_std=0.1)
    for w in (big, small):
        o_s, sf_s, pool_s, slots, ck = _call(w, chunk, static=True)
        o_w, sf_w, pool_w, _, _ = _call(w, chunk, static=False)
        assert torch.equal(o_s, o_w) and torch.equal(sf_s, sf_w) and torch.equal(pool_s, pool_w)
        o_r, sf_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"],
                                             w["s0"], ck)
        assert_parity(o_s, o_r, "bf16", "o")
        assert_parity(sf_s, sf_r, "bf16", "s_final")
        for n, (p,) in enumerate(ck):
            assert_parity(pool_s[slots[n]].reshape(sf_r[n].shape), ck_r[n][p], "bf16", f"ckpt seq {n}")


def test_static_matches_workspace_entry_with_segments():
    """A sequence long enough to be cut into segments (three, whose buffers fit
    the static array at H=4), checkpoints in its first and later segments: two
    calls in a row, the second smaller, bit for bit against the workspace
    entry, and at the oracle's bar."""
    big = inputs.prefill_workload(600, [3000, 40], 4, 128, 128, "bf16", s0_std=0.1)
    small = inputs.prefill_workload(601, [2100, 9], 4, 128, 128, "bf16", s0_std=0.1)
    for w, ck in ((big, [[500, 1500, 2900, 3000], [40]]), (small, [[700, 1900], [9]])):
        _, names = kda.prefill_plan(w["cu_seqlens"], 4, 128, 128, 32, ck)
        assert "segments" in names
        o_s, sf_s, pool_s, slots, _ = _call(w, 32, static=True, ck=ck)
        o_w, sf_w, pool_w, _, _ = _call(w, 32, static=False, ck=ck)
        assert torch.equal(o_s, o_w) and torch.equal(sf_s, sf_w) and torch.equal(pool_s, pool_w)
        o_r, sf_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"],
                                             w["s0"], ck)
        assert_parity(o_s, o_r, "bf16", "o")
        assert_parity(sf_s, sf_r, "bf16", "s_final")
        n = 0
        for s, ps in enumerate(ck):
            for p in ps:
                assert_parity(pool_s[slots[n]].reshape(sf_r[s].shape), ck_r[s][p], "bf16", f"ckpt seq {s} at {p}")
                n += 1


def test_static_refuses_a_call_beyond_its_scratch():
    """A two-kernel-path prefill of 4096 tokens at H = 32 needs more than the
    64 MiB scratch for its chunk records: refused with KDA_EWORKSPACE by the
    host checks, before any pointer is used (so placeholders stand in)."""
    L = kda.lib()
    H, d, T = 32, 128, 4096
    assert kda.prefill_workspace_size(1, T, H, d, d, 64, 0) > L.kda_static_scratch_bytes()
    fake = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(7)]
    st = L.kda_chunk_prefill_static(*fake[:5], kda.KDA_BF16, H, d, d, 64, _arr([0, T]), 1, None, fake[5], None,
                                    None, None, None, 0, None, 0, 0, None,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kda.KDA_EWORKSPACE
    assert b"static scratch" in L.kda_last_error()
