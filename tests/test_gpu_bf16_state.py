"""GPU parity of the bfloat16-state variant (reading R14) against the oracle.

Tolerance.  One decode step or one replay call computes in fp32 from the
same bf16 values the oracle reads, and both sides round the stored state to
the nearest bf16.  With s the exact value, s' = s + e the fp32 one and |e|
within a few fp32 roundings of the terms summed (bounded here by
2^-20 * max|s|), the two rounded results differ by at most
|rnd(s') - s'| + |e| + |s - rnd(s)| <= ulp_bf16(s) + |e|: so every element is
within one bf16 ulp of its own value plus 2^-20 * max|s|, and they are equal
except near a rounding boundary or where the terms cancel, at most 1 % of
the elements (expected about 0.1 %).  Over many steps those differences feed
later steps, and the bf16 bar (relative Frobenius 1e-2) applies.  Pages of a
bf16 state are copied bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu
FIELDS = ("q", "k", "v", "a", "beta")


def _bf16_state(x):
    return torch.from_numpy(inputs.round_to_bf16(x)).to(torch.bfloat16).cuda()


def _check_one_rounding(got, want, what):
    """got: device bf16 tensor; want: float64 values already rounded to bf16."""
    g = got.float().cpu().numpy().astype(np.float64)
    w = np.asarray(want, dtype=np.float64)
    mag = np.abs(w)
    ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    err = np.abs(g - w)
    bound = ulp + 2.0 ** -20 * mag.max()
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{what}: an element beyond one bf16 ulp + fp32 error ({worst:.2f} of the bound)"
    share = float(np.mean(err > 0))
    assert share <= 0.01, f"{what}: {share:.3%} of the elements differ"
    return share


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (32, 64, "fp32"), (16, 16, "bf16")])
def test_decode_one_step(dk, dv, dtype):
    B, H = 64, 4
    S0 = inputs.round_to_bf16(inputs.state_normal(150, 0, (B, H, dk, dv), 0.05))
    t = inputs.token_inputs(151, 0, (B,), H, dk, dv, dtype)
    state = _bf16_state(S0)
    o = kda.decode_step(*(dev_tensor(t[f], dtype) for f in FIELDS), state)
    torch.cuda.synchronize()
    o_r, S_r = oracle.decode_bf16_state(t["q"], t["k"], t["v"], t["a"], t["beta"], S0)
    _check_one_rounding(state, S_r, "state")
    assert_parity(o, o_r, dtype, "o")


def test_decode_many_steps():
    B, H, dk, dv, steps = 16, 4, 128, 128, 32
    S = inputs.round_to_bf16(inputs.state_normal(152, 0, (B, H, dk, dv), 0.05)).astype(np.float64)
    state = _bf16_state(S)
    for s in range(steps):
        t = inputs.token_inputs(153, s, (B,), H, dk, dv, "bf16")
        o = kda.decode_step(*(dev_tensor(t[f], "bf16") for f in FIELDS), state)
        o_r, S = oracle.decode_bf16_state(t["q"], t["k"], t["v"], t["a"], t["beta"], S)
    torch.cuda.synchronize()
    assert_parity(state.float(), S, "bf16", "state after 32 steps")
    assert_parity(o, o_r, "bf16", "o of the last step")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_replay(dtype):
    w = inputs.replay_workload(wid=154, B=32, H=8, dk=64, dv=64, t_draft=8, dtype=dtype)
    committed = inputs.round_to_bf16(w["committed"])
    c_dev = _bf16_state(committed)
    c_before = c_dev.clone()
    n = torch.from_numpy(w["n_accepted"]).cuda()
    s_new, o = kda.verify_and_replay(c_dev, *(dev_tensor(w[f], dtype) for f in FIELDS), n)
    torch.cuda.synchronize()
    assert torch.equal(c_dev, c_before), "committed state was written"
    assert s_new.dtype == torch.bfloat16
    s_r, o_r = oracle.verify_and_replay_bf16_state(committed, *(w[f] for f in FIELDS), w["n_accepted"])
    _check_one_rounding(s_new, s_r, "s_new")
    for b in np.flatnonzero(w["n_accepted"] == 0):
        assert torch.equal(s_new[b], c_dev[b]), "n = 0 must copy the committed state bit for bit"
    assert_parity(o, o_r, dtype, "o")


@pytest.mark.parametrize("layout", [kda.KDA_LAYOUT_KV, kda.KDA_LAYOUT_VK])
def test_bf16_pages_round_trip(layout):
    B, H, dk, dv = 5, 3, 64, 32
    g = torch.Generator(device="cuda").manual_seed(9)
    shp = (B, H, dk, dv) if layout == kda.KDA_LAYOUT_KV else (B, H, dv, dk)
    state = torch.randn(shp, generator=g, device="cuda").to(torch.bfloat16)
    page = H * dk * dv + 24
    pool = torch.full((B + 2, page), float("nan"), device="cuda").to(torch.bfloat16)
    slots = torch.tensor([6, 0, 3, 2, 5], dtype=torch.int32, device="cuda")
    kda.pack_heads(state, slots, pool, layout=layout)
    back = kda.unpack_heads(pool, slots, H, dk, dv, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(back, state)
    canon = state if layout == kda.KDA_LAYOUT_KV else state.transpose(2, 3)
    for b, s in enumerate(slots.tolist()):
        assert torch.equal(pool[s, :H * dk * dv], canon[b].reshape(-1))
        assert not pool[s, H * dk * dv:].float().any(), "page padding must be zero"
