"""GPU parity: the raw-input ring against its oracle (bit-exact: it only moves
data), the Tab 4 timeline and layout of [Serve demo], and replay through the
ring window against replay of the batch-built draft projections."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.conftest import GOLDEN
from tests.parity import assert_parity, dev_tensor, to_np

pytestmark = pytest.mark.gpu
FIELDS = ("q", "k", "v", "a", "beta")


def _step(rng, B, H, dk, dv, dtype):
    s = {"q": rng.standard_normal((B, H, dk)), "k": rng.standard_normal((B, H, dk)),
         "v": rng.standard_normal((B, H, dv)), "a": -np.abs(rng.standard_normal((B, H, dk))),
         "beta": rng.random((B, H))}
    return {f: inputs.round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32) for f, x in s.items()}


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 16, 32), ("fp32", 32, 16), ("bf16", 128, 128)])
def test_ring_matches_oracle(dtype, dk, dv):
    n_slots, cap, H = 6, 4, 2
    rng = np.random.default_rng(11)
    ring = kda.RawInputRing(n_slots, cap, H, dk, dv, torch.bfloat16 if dtype == "bf16" else torch.float32)
    ref = oracle.ring_new(n_slots, cap, H, dk, dv)
    plan = [[0, 2, 5], [2, 5], [5, 0, 1], [5], [5, 2], [3], [5, 0], [1]]  # slot 5 wraps around
    for i, slots in enumerate(plan):
        st = _step(rng, len(slots), H, dk, dv, dtype)
        ring.push(torch.tensor(slots, dtype=torch.int32, device="cuda"),
                  *(dev_tensor(st[f], dtype) for f in FIELDS))
        oracle.ring_push(ref, slots, st)
        if i == 4:
            ring.reset(torch.tensor([2], dtype=torch.int32, device="cuda"))
            oracle.ring_reset(ref, [2])
    query = [5, 4, 0, 2, 1, 3]
    got = ring.window(torch.tensor(query, dtype=torch.int32, device="cuda"))
    want, n_valid = oracle.ring_window(ref, query)
    torch.cuda.synchronize()
    assert to_np(got["n_valid"]).tolist() == n_valid.tolist()
    for f in FIELDS:
        assert np.array_equal(to_np(got[f]), want[f]), f
    assert to_np(ring.count).tolist() == ref["count"].tolist()


def test_tab4_timeline_and_layout_on_the_device():
    g = json.load(open(os.path.join(GOLDEN, "ring_tab4.json")))
    pa, pb = g["panel_a"], g["panel_b"]
    ring = kda.RawInputRing(1, pa["capacity"], 2, 16, 16, torch.float32)
    slot = torch.zeros(1, dtype=torch.int32, device="cuda")
    sizes = []
    for i in range(pa["pushes"]):
        ring.push(slot, *(torch.full((1,) + ring.shapes[f], float(i), device="cuda") for f in FIELDS))
        sizes.append(int(ring.window(slot)["n_valid"][0]))
    assert sizes == pa["window_sizes"]
    ring = kda.RawInputRing(1, pb["pushes"], pb["H"], 16, 16, torch.float32)
    for i in range(pb["pushes"]):
        ring.push(slot, *(torch.full((1,) + ring.shapes[f], float(i), device="cuda") for f in FIELDS))
    w = ring.window(slot)
    assert list(w["q"].shape[:3]) == pb["shape"][:3]
    for i, val in enumerate(pb["row_values"]):
        assert bool((w["q"][i] == val).all()) and bool((w["beta"][i] == val).all())


@pytest.mark.parametrize("shape", ["pages", "big"])
def test_replay_through_the_ring_equals_batch_replay(shape):
    """Streaming pushes + window() give verify_and_replay the same tensors as
    the batch-built draft projections: identical results, and the oracle's."""
    if shape == "pages":
        w = inputs.replay_workload()
        dt, tdt = "fp32", torch.float32
    else:
        w = inputs.replay_workload(wid=12, B=16, H=32, dk=128, dv=128, t_draft=8, dtype="bf16")
        dt, tdt = "bf16", torch.bfloat16
    Td, B, H, dk = w["q"].shape
    dv = w["v"].shape[-1]
    d = {f: dev_tensor(w[f], dt) for f in FIELDS}
    committed = torch.from_numpy(w["committed"]).cuda()
    n = torch.from_numpy(w["n_accepted"]).cuda()
    slots = torch.randperm(2 * B, generator=torch.Generator().manual_seed(3))[:B].to(torch.int32).cuda()
    ring = kda.RawInputRing(2 * B, Td, H, dk, dv, tdt)
    for t in range(Td):
        ring.push(slots, *(d[f][t].contiguous() for f in FIELDS))
    win = ring.window(slots)
    s_ring, o_ring = kda.verify_and_replay(committed, win["q"], win["k"], win["v"], win["a"],
                                           win["beta"], n)
    s_batch, o_batch = kda.verify_and_replay(committed, d["q"], d["k"], d["v"], d["a"], d["beta"], n)
    torch.cuda.synchronize()
    assert bool((win["n_valid"] == Td).all())
    assert torch.equal(s_ring, s_batch) and torch.equal(o_ring, o_batch)
    s_ref, o_ref = oracle.verify_and_replay(w["committed"], *(w[f] for f in FIELDS), w["n_accepted"])
    assert_parity(s_ring, s_ref, dt, "replayed state")
    assert_parity(o_ring, o_ref, dt, "replayed outputs")


def test_ring_bad_slots_are_skipped_and_flagged():
    ring = kda.RawInputRing(3, 2, 1, 16, 16, torch.float32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = torch.tensor([1, 7, -1], dtype=torch.int32, device="cuda")
    ring.push(slots, *(torch.ones((3,) + ring.shapes[f], device="cuda") for f in FIELDS), err_flag=flag)
    w = ring.window(slots, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag[0]) == 1
    assert ring.count.tolist() == [0, 1, 0]
    assert w["n_valid"].tolist() == [1, 0, 0] and not w["q"][:, 1:].any()
