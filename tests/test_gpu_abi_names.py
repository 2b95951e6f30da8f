"""The entry points the boundary names (kda_chunk_prefill, kda_decode_step,
kda_verify_and_replay, kda_pack_heads, kda_unpack_heads), called directly
through ctypes with raw device pointers on small shapes and compared with the
float64 oracle; and run-twice bit identity of decode and replay."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu

I32 = ctypes.c_int32


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _arr(xs):
    return (I32 * max(1, len(xs)))(*xs)


def test_kda_chunk_prefill_direct():
    """Two sequences (70 and 33 tokens), H=2, dk=dv=64, bf16, chunk 64,
    nonzero S0, checkpoints at 64 and 70 / 33 in slots 2, 0, 1."""
    L = kda.lib()
    H, d = 2, 64
    w = inputs.prefill_workload(360, [70, 33], H, d, d, "bf16", s0_std=0.1)
    ck = [[64, 70], [33]]
    t = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v", "a", "beta")}
    s0 = torch.from_numpy(w["s0"]).cuda()
    T = 103
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((2, H, d, d), device="cuda")
    page = H * d * d + 64
    pool = torch.full((3, page), float("nan"), device="cuda")
    need = ctypes.c_size_t(0)
    assert L.kda_chunk_prefill_workspace_size(2, T, H, d, d, 64, 3, kda.KDA_BF16, ctypes.byref(need)) == 0
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = L.kda_chunk_prefill(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["a"]), _p(t["beta"]), kda.KDA_BF16,
                             H, d, d, 64, _arr([0, 70, 103]), 2, _p(s0), _p(o), _p(sf), _arr([0, 2, 3]),
                             _arr([64, 70, 33]), _arr([2, 0, 1]), 3, _p(pool), page, 3, _p(ws),
                             need.value, _p(flag), _stream())
    assert st == kda.KDA_OK, L.kda_last_error()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    o_r, sf_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"], w["s0"],
                                         ck)
    assert_parity(o, o_r, "bf16", "o")
    assert_parity(sf, sf_r, "bf16", "s_final")
    for slot, (n, p) in zip([2, 0, 1], [(0, 64), (0, 70), (1, 33)]):
        assert_parity(pool[slot, :H * d * d].reshape(H, d, d), ck_r[n][p], "bf16", f"ckpt {p} seq {n}")
        assert not pool[slot, H * d * d:].any()


def test_kda_decode_step_direct():
    """Three in-place steps, B=3, H=2, dk=32, dv=64, fp32 inputs."""
    L = kda.lib()
    B, H, dk, dv = 3, 2, 32, 64
    S0 = inputs.state_normal(361, 0, (B, H, dk, dv), 0.1)
    st = torch.from_numpy(S0).cuda()
    steps = [inputs.token_inputs(361, s, (B,), H, dk, dv, "fp32") for s in range(3)]
    outs = []
    for t in steps:
        d = {n: dev_tensor(x, "fp32") for n, x in t.items()}
        o = torch.empty((B, H, dv), device="cuda")
        assert L.kda_decode_step(_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["a"]), _p(d["beta"]), kda.KDA_F32,
                                 B, H, dk, dv, _p(st), _p(o), _stream()) == kda.KDA_OK
        outs.append(o)
    torch.cuda.synchronize()
    for b in range(B):
        seq = {n: np.stack([t[n][b] for t in steps]) for n in steps[0]}
        o_r, S_r, _ = oracle.kda_recurrent(seq["q"], seq["k"], seq["v"], seq["a"], seq["beta"], S0[b])
        assert_parity(torch.stack([x[b] for x in outs]), o_r, "fp32", f"o b={b}")
        assert_parity(st[b], S_r, "fp32", f"S b={b}")


def test_kda_verify_and_replay_direct():
    """B=5 sessions, 4 drafts, n_accepted = 0, 1, 2, 4 and 9 (clamped to 4,
    flagged); the committed state is left untouched."""
    L = kda.lib()
    B, H, dk, dv, Td = 5, 2, 64, 32, 4
    t = inputs.token_inputs(362, 0, (Td, B), H, dk, dv, "bf16")
    S0 = inputs.state_normal(362, 0, (B, H, dk, dv), 0.1)
    com = torch.from_numpy(S0).cuda()
    d = {n: dev_tensor(x, "bf16") for n, x in t.items()}
    nacc = torch.tensor([0, 1, 2, 4, 9], dtype=torch.int32, device="cuda")
    s_new = torch.empty_like(com)
    o = torch.full((B, H, Td, dv), 5.0, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert L.kda_verify_and_replay(_p(com), _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["a"]), _p(d["beta"]),
                                   kda.KDA_BF16, _p(nacc), B, H, dk, dv, Td, _p(s_new), _p(o), _p(flag),
                                   _stream()) == kda.KDA_OK
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    assert torch.equal(com, torch.from_numpy(S0).cuda())
    S_r, O_r = oracle.verify_and_replay(S0, t["q"], t["k"], t["v"], t["a"], t["beta"], [0, 1, 2, 4, 4])
    assert torch.equal(s_new[0], com[0])  # n = 0: a bit-exact copy
    assert_parity(s_new, S_r, "bf16", "s_new")
    assert_parity(o, O_r, "bf16", "o")
    assert not o[0].float().any() and not o[1, :, 1:].float().any()


def test_kda_pack_unpack_direct():
    """pack (KV source) into slots 3, 0, 2 of a 5-slot pool with padding, then
    unpack into the VK layout: bit-exact against the oracle's layout."""
    L = kda.lib()
    B, H, dk, dv = 3, 2, 32, 16
    S = inputs.state_normal(363, 0, (B, H, dk, dv), 1.0)
    st = torch.from_numpy(S).cuda()
    slots = [3, 0, 2]
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    page = H * dk * dv + 40
    pool = torch.full((5, page), 9.0, device="cuda")
    assert L.kda_pack_heads(_p(st), kda.KDA_LAYOUT_KV, B, H, dk, dv, _p(sl), _p(pool), page, 5, None,
                            _stream()) == kda.KDA_OK
    back = torch.empty((B, H, dv, dk), device="cuda")
    assert L.kda_unpack_heads(_p(pool), page, 5, _p(sl), B, H, dk, dv, kda.KDA_LAYOUT_VK, _p(back), None,
                              _stream()) == kda.KDA_OK
    torch.cuda.synchronize()
    want = np.full((5, page), 9.0)
    oracle.pack_heads(S, slots, want)
    assert np.array_equal(to_np(pool), want)
    assert np.array_equal(to_np(back), np.swapaxes(S, 2, 3))


def test_decode_and_replay_run_twice_bit_identical():
    """Decode (B=64, H=32, d=128, bf16, four steps from the same state) and
    replay (B=64, H=16, d=32) twice each: the same bits."""
    B, H, d = 64, 32, 128
    S0 = torch.from_numpy(inputs.state_normal(364, 0, (B, H, d, d), 0.05)).cuda()
    steps = [{n: dev_tensor(x, "bf16") for n, x in inputs.token_inputs(364, s, (B,), H, d, d, "bf16").items()}
             for s in range(4)]
    res = []
    for _ in range(2):
        st = S0.clone()
        outs = [kda.decode_step(t["q"], t["k"], t["v"], t["a"], t["beta"], st) for t in steps]
        torch.cuda.synchronize()
        res.append((torch.stack(outs), st))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    w = inputs.replay_workload()
    d2 = {n: dev_tensor(w[n], "fp32") for n in ("q", "k", "v", "a", "beta")}
    com = torch.from_numpy(w["committed"]).cuda()
    nacc = torch.from_numpy(w["n_accepted"]).cuda()
    r = [kda.verify_and_replay(com, d2["q"], d2["k"], d2["v"], d2["a"], d2["beta"], nacc) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(r[0][0], r[1][0]) and torch.equal(r[0][1], r[1][1])
