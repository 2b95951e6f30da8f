"""GPU parity of the fused prefill with sequences split into segments inside
one call (chains of later segments from the zero state and from the
identity, then the composition of the segment maps and the correction of
the later segments' outputs and checkpoints) against the float64 oracle.

Weak decays (a in [-0.002, 0]) keep the start state of every segment far
above rounding at its end, so a wrong composition or correction shows in
every row after the cut, not only in the first few."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, assert_parity_blocks, dev_tensor
from tests.test_gpu_prefill import _check, _run

pytestmark = pytest.mark.gpu

WEAK = -0.002


def _ckpts(lens):
    """Checkpoints on both sides of the cuts (multiples of 32 near L i / n),
    on odd positions, and at the end."""
    out = []
    for L in lens:
        pos = {1, 31, 32, 33, 511, 512, 513, 700, 1023, 1024, 1025, 1056, 1500, 1535, 1536, 2047, L - 1, L}
        out.append(sorted(p for p in pos if 1 <= p <= L))
    return out


@pytest.mark.parametrize("n_seg", [2, 3, 4])
def test_forced_segments_match_oracle(n_seg):
    """Sequences of at least n_seg * 512 tokens in n_seg segments (dv_split =
    -n_seg), the rest whole, nonzero S0, H = 2: outputs (also per 32-token
    chunk), final states and every checkpoint."""
    lens = [2100, 1100, 45, 0, 1300, 2049]
    w = inputs.prefill_workload(700 + n_seg, lens, 2, 128, 128, "bf16", s0_std=0.1, g_min=WEAK)
    w["checkpoints"] = _ckpts(lens)
    _, names = kda.prefill_plan(w["cu_seqlens"], 2, 128, 128, 32, w["checkpoints"], dv_split=-n_seg)
    k = sum(L >= 512 * n_seg for L in lens)  # (the sequences of at least n_seg * 512 tokens)
    assert f"{k} sequences in {k * n_seg} segments" in names, names
    o, sf, pool, slots = _run(w, "bf16", 32, page_extra=8, dv_split=-n_seg)
    _check(w, "bf16", o, sf, pool, slots, block=32)


def test_automatic_segments_match_oracle():
    """One long sequence among short ones at H = 2: the cost model splits it
    by itself (its chain alone would bound the call); no checkpoints, zero
    S0 on a second call."""
    lens = [6000, 300, 64, 17]
    w = inputs.prefill_workload(710, lens, 2, 128, 128, "bf16", s0_std=0.1, g_min=WEAK, ckpt_every=1000)
    _, names = kda.prefill_plan(w["cu_seqlens"], 2, 128, 128, 32, w["checkpoints"])
    assert "segments" in names, names
    o, sf, pool, slots = _run(w, "bf16", 32)
    _check(w, "bf16", o, sf, pool, slots, block=32)
    w["checkpoints"] = None
    o, sf, pool, slots = _run(w, "bf16", 32, with_s0=False)
    w["s0"] = None
    _check(w, "bf16", o, sf, pool, slots, block=32)


def test_segments_run_twice_bit_equal():
    lens = [3000, 700]
    w = inputs.prefill_workload(711, lens, 4, 128, 128, "bf16", s0_std=0.1, g_min=WEAK, ckpt_every=512)
    o, sf, pool, _ = _run(w, "bf16", 32, dv_split=-3)
    o2, sf2, pool2, _ = _run(w, "bf16", 32, dv_split=-3)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert torch.equal(pool.nan_to_num(7.0), pool2.nan_to_num(7.0))


def test_segments_without_final_state():
    """want_final=False: the composition still runs (the later segments need
    their start states) and no final state is written."""
    lens = [1500, 40]
    w = inputs.prefill_workload(712, lens, 2, 128, 128, "bf16", s0_std=0.1, g_min=WEAK)
    d = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v", "a", "beta")}
    s0 = torch.from_numpy(w["s0"]).cuda()
    o, sf = kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], s0=s0, chunk=32,
                              want_final=False, dv_split=-2)
    torch.cuda.synchronize()
    assert sf is None
    o_r, _, _ = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"], w["s0"])
    for n, (lo, hi) in enumerate([(0, 1500), (1500, 1540)]):
        for h in range(2):
            assert_parity_blocks(o[lo:hi, h], o_r[lo:hi, h], "bf16", 32, f"o seq {n} head {h}")


@pytest.mark.parametrize("n_seg", [2, 3])
def test_segments_bad_decay_stops_that_head(n_seg):
    """A decay below the bound in the first segment of a split sequence, head
    0: the flag is raised; as without segments, that (sequence, head) keeps
    what came before the bad chunk and writes no later checkpoint (those of
    the later segments included) and no final state; head 1 of the same
    sequence and the other sequence are complete."""
    lens = [1700, 90]
    H, d = 2, 128
    w = inputs.prefill_workload(713, lens, H, d, d, "bf16", s0_std=0.1, g_min=WEAK)
    w["a"][100, 0, 3] = -6.0
    ck = [[64, 300, 900, 1200, 1700], [50, 90]]
    slots = [[0, 1, 2, 3, 4], [5, 6]]
    T = int(w["cu_seqlens"][-1])
    sentinel = 0.375
    dd = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v", "a", "beta")}
    o = torch.full((T, H, d), sentinel, dtype=torch.bfloat16, device="cuda")
    sf = torch.full((2, H, d, d), sentinel, device="cuda")
    pool = torch.full((7, H * d * d), sentinel, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, names = kda.prefill_plan(w["cu_seqlens"], H, d, d, 32, ck, dv_split=-n_seg)
    assert "1 sequence in" in names, names
    kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dd["a"], dd["beta"], w["cu_seqlens"],
                      s0=torch.from_numpy(w["s0"]).cuda(), chunk=32, checkpoints=ck, ckpt_slots=slots,
                      page_pool=pool, o=o, s_final=sf, err_flag=flag, dv_split=-n_seg)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    o_r, sf_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"], w["s0"], ck)
    page = pool.reshape(7, H, d, d)
    # head 0 of sequence 0: the chunk [96, 128) holds the bad value
    assert_parity_blocks(o[:96, 0], o_r[:96, 0], "bf16", 32, "o seq 0 head 0 before the bad chunk")
    assert_parity(page[0, 0], ck_r[0][64][0], "bf16", "ckpt 64 head 0")
    for j in (1, 2, 3, 4):
        assert bool((page[j, 0] == sentinel).all()), f"checkpoint slot {j} head 0 written"
    assert bool((sf[0, 0] == sentinel).all())
    # head 1 of sequence 0, and sequence 1
    assert_parity_blocks(o[:1700, 1], o_r[:1700, 1], "bf16", 32, "o seq 0 head 1")
    assert_parity(sf[0, 1], sf_r[0, 1], "bf16", "s_final seq 0 head 1")
    for j, p in enumerate(ck[0]):
        assert_parity(page[j, 1], ck_r[0][p][1], "bf16", f"ckpt {p} head 1")
    for h in range(H):
        assert_parity_blocks(o[1700:, h], o_r[1700:, h], "bf16", 32, f"o seq 1 head {h}")
        assert_parity(sf[1, h], sf_r[1, h], "bf16", f"s_final seq 1 head {h}")
        for j, p in enumerate(ck[1]):
            assert_parity(page[slots[1][j], h], ck_r[1][p][h], "bf16", f"ckpt {p} seq 1 head {h}")


def test_segments_with_the_fused_gate():
    """a and beta as logits (the gated entry, g_min = -0.01 so the start
    states carry over) with a sequence in three segments: the identity and
    zero-start chains apply the gate as the others do."""
    lens = [1700, 200]
    H, d, g_min = 2, 128, -0.01
    w = inputs.prefill_workload(714, lens, H, d, d, "bf16", s0_std=0.1)
    rng = np.random.default_rng(715)
    z_a = inputs.round_to_bf16(rng.standard_normal(w["a"].shape).astype(np.float32))
    z_b = inputs.round_to_bf16(rng.standard_normal(w["beta"].shape).astype(np.float32))
    ck = [[300, 600, 1000, 1700], [200]]
    slots = [[0, 1, 2, 3], [4]]
    pool = torch.zeros((5, H * d * d), device="cuda")
    dd = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v")}
    o, sf = kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dev_tensor(z_a, "bf16"), dev_tensor(z_b, "bf16"),
                              w["cu_seqlens"], s0=torch.from_numpy(w["s0"]).cuda(), chunk=32, checkpoints=ck,
                              ckpt_slots=slots, page_pool=pool, gate_g_min=g_min, dv_split=-3)
    torch.cuda.synchronize()
    a = g_min * oracle.sigmoid(z_a)
    beta = oracle.sigmoid(z_b)
    o_r, sf_r, ck_r = oracle.kda_prefill(w["q"], w["k"], w["v"], a, beta, w["cu_seqlens"], w["s0"], ck)
    page = pool.reshape(5, H, d, d)
    for n, (lo, hi) in enumerate([(0, 1700), (1700, 1900)]):
        for h in range(H):
            assert_parity_blocks(o[lo:hi, h], o_r[lo:hi, h], "bf16", 32, f"o seq {n} head {h}")
            assert_parity(sf[n, h], sf_r[n, h], "bf16", f"s_final seq {n} head {h}")
            for j, p in enumerate(ck[n]):
                assert_parity(page[slots[n][j], h], ck_r[n][p][h], "bf16", f"ckpt {p} seq {n} head {h}")


def test_small_workspace_runs_without_segments():
    """A workspace that holds the work list but not the segments' buffers:
    the call runs without segments (same results), through the C entry."""
    import ctypes
    lens = [2100, 300]
    H, d = 2, 128
    w = inputs.prefill_workload(716, lens, H, d, d, "bf16", s0_std=0.1, g_min=WEAK, ckpt_every=700)
    dd = {n: dev_tensor(w[n], "bf16") for n in ("q", "k", "v", "a", "beta")}
    T = int(w["cu_seqlens"][-1])
    ck = w["checkpoints"]
    n_ck = sum(len(c) for c in ck)
    s0 = torch.from_numpy(w["s0"]).cuda()
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((2, H, d, d), device="cuda")
    pool = torch.zeros((n_ck, H * d * d), device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")  # the work list fits, the buffers do not
    assert kda.prefill_workspace_size(2, T, H, d, d, 32, n_ck) > ws.numel()
    cu = (ctypes.c_int32 * 3)(*[int(x) for x in w["cu_seqlens"]])
    ck_cu = (ctypes.c_int32 * 3)(0, len(ck[0]), n_ck)
    ck_pos = (ctypes.c_int32 * n_ck)(*[p for c in ck for p in c])
    ck_slot = (ctypes.c_int32 * n_ck)(*range(n_ck))
    L = kda.lib()
    st = L.kda_chunk_prefill_split(dd["q"].data_ptr(), dd["k"].data_ptr(), dd["v"].data_ptr(), dd["a"].data_ptr(),
                                   dd["beta"].data_ptr(), kda.KDA_BF16, H, d, d, 32, cu, 2, s0.data_ptr(),
                                   o.data_ptr(), sf.data_ptr(), ck_cu, ck_pos, ck_slot, n_ck, pool.data_ptr(),
                                   H * d * d, n_ck, ws.data_ptr(), ws.numel(), -2, None,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.kda_last_error().decode()
    torch.cuda.synchronize()
    slots, i = [], 0
    for c in ck:
        slots.append(list(range(i, i + len(c))))
        i += len(c)
    _check(w, "bf16", o, sf, pool, slots, block=32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_segments_random_shapes(seed):
    """Random lengths (zero and short ones among them), random checkpoint
    positions (a cut and its neighbours among them), S0 or none, and a
    segment count of 0 (the library's choice) or -2 .. -5: every output row
    block, final state and checkpoint against the oracle."""
    rng = np.random.default_rng(720 + seed)
    lens = [int(x) for x in rng.integers(0, 2600, 5)] + [0, 31]
    split = int(rng.choice([0, -2, -3, -4, -5]))
    ck = []
    for L in lens:
        cand = {L, L // 2, (L // 2 + 16) // 32 * 32, (L // 3 + 16) // 32 * 32 + 1, 1}
        cand |= set(int(x) for x in rng.integers(1, max(L, 1) + 1, 3))
        ck.append(sorted(p for p in cand if 1 <= p <= L))
    s0 = None if seed == 1 else 0.1
    w = inputs.prefill_workload(730 + seed, lens, 2, 128, 128, "bf16", s0_std=s0, g_min=WEAK)
    w["checkpoints"] = ck
    o, sf, pool, slots = _run(w, "bf16", 32, page_extra=4, dv_split=split)
    _check(w, "bf16", o, sf, pool, slots, block=32)


@pytest.mark.parametrize("kind", ["const", "uniform"])
def test_segments_at_the_decay_bound(kind):
    """a = -5 (the bound at 32-token chunks) on every channel of every token,
    or uniform in [-5, 0]: a sequence in three segments beside a whole one,
    nonzero S0, checkpoints on both sides of the cuts; the identity chains
    and the corrections at the widest exponents the chunk form admits, against
    the oracle."""
    lens = [2100, 700]
    w = inputs.prefill_workload(720, lens, 2, 128, 128, "bf16", s0_std=0.1)
    rng = np.random.default_rng(720)
    a = np.full(w["a"].shape, -5.0, np.float32) if kind == "const" else \
        rng.uniform(-5.0, 0.0, w["a"].shape).astype(np.float32)
    w["a"] = torch.from_numpy(a).to(torch.bfloat16).float().numpy()  # (the values the device reads)
    assert w["a"].min() >= -5.0
    w["checkpoints"] = _ckpts(lens)
    _, names = kda.prefill_plan(w["cu_seqlens"], 2, 128, 128, 32, w["checkpoints"], dv_split=-3)
    assert "1 sequence in 3 segments" in names, names
    o, sf, pool, slots = _run(w, "bf16", 32, page_extra=8, dv_split=-3)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sf).all()
    _check(w, "bf16", o, sf, pool, slots, block=32)
