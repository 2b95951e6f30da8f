"""GPU parity: chunked prefill (outputs, final states, checkpoints in page
slots) against the float64 recurrent oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import inputs, kda
from tests.parity import assert_parity, assert_parity_blocks, dev_tensor, to_np

pytestmark = pytest.mark.gpu

FIELDS = ("q", "k", "v", "a", "beta")


def _run(w, dtype, chunk, slots_per_seq=None, page_extra=0, dv_split=0, with_s0=True):
    d = {n: dev_tensor(w[n], dtype) for n in FIELDS}
    H, dk = w["k"].shape[1:]
    dv = w["v"].shape[2]
    s0 = None
    if with_s0 and w.get("s0") is not None:
        s0 = torch.from_numpy(w["s0"]).cuda()
    ck = w.get("checkpoints")
    pool = slots = None
    if ck is not None:
        n_ck = sum(len(c) for c in ck)
        order = np.random.default_rng(7).permutation(n_ck + 3)[:n_ck]
        slots, i = [], 0
        for c in ck:
            slots.append([int(x) for x in order[i:i + len(c)]])
            i += len(c)
        pool = torch.full((n_ck + 3, H * dk * dv + page_extra), float("nan"), device="cuda")
    s0_before = None if s0 is None else s0.clone()
    o, sf = kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], s0=s0,
                              chunk=chunk, checkpoints=ck, ckpt_slots=slots, page_pool=pool,
                              dv_split=dv_split)
    torch.cuda.synchronize()
    if s0 is not None:
        assert torch.equal(s0, s0_before), "committed S0 was written"
    return o, sf, pool, slots


def _check(w, dtype, o, sf, pool, slots, heads=None, seqs=None, block=None):
    """Compare against the oracle, optionally on sampled heads / sequences.
    With block set, bf16 outputs also meet the bar on every run of `block`
    tokens of each (sequence, head) on its own."""
    cu = w["cu_seqlens"]
    H, dk = w["k"].shape[1:]
    dv = w["v"].shape[2]
    N = len(cu) - 1
    heads = list(range(H) if heads is None else heads)
    seqs = range(N) if seqs is None else seqs
    ck = w.get("checkpoints")
    on, sfn = to_np(o), to_np(sf)
    for n in seqs:
        lo, hi = int(cu[n]), int(cu[n + 1])
        s0 = None if w.get("s0") is None else w["s0"][n][heads]
        pos = [] if ck is None else ck[n]
        if hi > lo:
            # the requested heads in one oracle pass (heads are independent)
            o_r, S_r, saved = oracle.kda_recurrent(
                *(w[f][lo:hi][:, heads] for f in ("q", "k", "v", "a")), w["beta"][lo:hi][:, heads], s0, pos)
        else:
            S_r = np.zeros((len(heads), dk, dv)) if s0 is None else s0
            saved = {}
        for i, h in enumerate(heads):
            if hi > lo:
                assert_parity(on[lo:hi, h], o_r[:, i], dtype, f"o seq {n} head {h}")
                if block is not None and dtype == "bf16":
                    assert_parity_blocks(on[lo:hi, h], o_r[:, i], dtype, block, f"o seq {n} head {h}")
            assert_parity(sfn[n, h], S_r[i], dtype, f"s_final seq {n} head {h}")
            for j, p in enumerate(pos):
                page = to_np(pool[slots[n][j]])
                got = page[h * dk * dv:(h + 1) * dk * dv].reshape(dk, dv)
                assert_parity(got, saved[p][i], dtype, f"checkpoint seq {n} pos {p} head {h}")
    if pool is not None:
        for n in seqs:
            for s in slots[n]:
                assert not pool[s, H * dk * dv:].any(), "page padding must be zero"


def test_tiny_workload_fp32_chunk16():
    """1 sequence, H=2, dk=dv=16, T=128, fp32, S0 = 0, chunk 16."""
    w = inputs.workload0()
    o, sf, pool, slots = _run(w, "fp32", 16)
    _check(w, "fp32", o, sf, pool, slots)


LENS = [1, 15, 16, 17, 64, 0, 65, 100, 130]


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("fp32", 32), ("bf16", 16)])
def test_varlen_ragged_with_checkpoints(dk, dv, dtype, chunk):
    w = inputs.prefill_workload(30 + dk + dv, LENS, 2, dk, dv, dtype, s0_std=0.1)
    w["checkpoints"] = [sorted({p for p in (1, 7, 16, 33, 64, L) if 1 <= p <= L}) for L in LENS]
    o, sf, pool, slots = _run(w, dtype, chunk, page_extra=8)
    _check(w, dtype, o, sf, pool, slots)


@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_explicit_dv_splits_agree(split):
    """Every dv split of the column-slab kernel at dk = dv = 128, bf16, chunk
    64: one 128-column tile (two column tiles per compute wave) down to eight
    16-column tiles."""
    w = inputs.prefill_workload(40, [200, 77], 2, 128, 128, "bf16", s0_std=0.1, ckpt_every=64)
    o, sf, pool, slots = _run(w, "bf16", 64, dv_split=split)
    _check(w, "bf16", o, sf, pool, slots)


def test_mixed_tile_widths():
    """dv_split = -1: a tile width per sequence in one launch.  With chunk
    counts 20, 14, 6 and 2 (H = 2, so the total work is small) the cost model
    gives the longest sequence 32-column tiles, the second 64 and the others
    one 128-column tile (asserted through the plan query), so every width of
    the mixed launch runs; checkpoints every 256 tokens keep the chunks whole.
    A second identical call gives the same bits (the 32-column tiles run two
    spare waves beside their loaders)."""
    w = inputs.prefill_workload(42, [64 * 20, 64 * 14, 64 * 6, 100], 2, 128, 128, "bf16",
                                s0_std=0.1, ckpt_every=256)
    cols, names = kda.prefill_plan(w["cu_seqlens"], 2, 128, 128, 64, w["checkpoints"], dv_split=-1)
    assert cols == [32, 64, 128, 128] and "slab_mixed_kernel" in names
    o, sf, pool, slots = _run(w, "bf16", 64, dv_split=-1)
    _check(w, "bf16", o, sf, pool, slots, block=64)
    o2, sf2, pool2, _ = _run(w, "bf16", 64, dv_split=-1)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert torch.equal(pool.nan_to_num(7.0), pool2.nan_to_num(7.0))
    o1, sf1, _, _ = _run(w, "bf16", 64, dv_split=1)
    assert_parity(o, o1.float(), "bf16", "o (mixed widths vs one tile per head)")
    assert_parity(sf, sf1, "bf16", "s_final (mixed widths vs one tile per head)")


def test_zero_state_and_no_final():
    w = inputs.prefill_workload(41, [90], 2, 64, 64, "bf16")
    d = {n: dev_tensor(w[n], "bf16") for n in FIELDS}
    o, sf = kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"],
                              want_final=False)
    torch.cuda.synchronize()
    assert sf is None
    o_r, _, _ = oracle.kda_prefill(w["q"], w["k"], w["v"], w["a"], w["beta"], w["cu_seqlens"])
    assert_parity(o, o_r, "bf16", "o")


def test_checkpoint_resume_matches_one_pass():
    """prefill(0..T) == prefill(0..p) -> checkpoint page -> unpack -> prefill(p..T)."""
    T, p, H, d = 300, 128, 2, 128
    w = inputs.prefill_workload(42, [T], H, d, d, "bf16", s0_std=0.1)
    w["checkpoints"] = [[p]]
    o_all, sf_all, pool, slots = _run(w, "bf16", 64)
    s_p = kda.unpack_heads(pool, torch.tensor(slots[0], dtype=torch.int32, device="cuda"), H, d, d)
    tail = {n: dev_tensor(w[n][p:], "bf16") for n in FIELDS}
    o_b, sf_b = kda.chunk_prefill(tail["q"], tail["k"], tail["v"], tail["a"], tail["beta"],
                                  [0, T - p], s0=s_p, chunk=64)
    torch.cuda.synchronize()
    assert_parity(o_b, o_all[p:], "bf16", "resumed outputs")
    assert_parity(sf_b, sf_all, "bf16", "resumed final state")


def test_single_sequence_workload_sampled_heads():
    """T=8192, H=32, dk=dv=128, bf16, S0=0, chunk 64, checkpoints every 512:
    six heads against the oracle (every 64-token chunk on its own as well),
    and a second call bit for bit equal to the first."""
    w = inputs.workload3()
    o, sf, pool, slots = _run(w, "bf16", 64)
    _check(w, "bf16", o, sf, pool, slots, heads=[0, 7, 13, 20, 26, 31], block=64)
    o2, sf2, pool2, _ = _run(w, "bf16", 64)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert torch.equal(pool.nan_to_num(7.0), pool2.nan_to_num(7.0))


def test_varlen_workload_every_sequence():
    """16 sequences, lengths log-uniform in [1024, 32768] (108,886 tokens),
    nonzero S0, checkpoints every 4096 plus the exact tail (35): every
    sequence, every checkpoint and the final states on three heads against
    the oracle, outputs also per 64-token chunk; then a second call in the
    same launch configuration (a tile width per sequence) must give the same
    bits everywhere."""
    w = inputs.workload4()
    cols, _ = kda.prefill_plan(w["cu_seqlens"], 32, 128, 128, 64, w["checkpoints"])
    assert sorted(set(cols)) == [32, 128]  # both widths of the mixed launch run
    o, sf, pool, slots = _run(w, "bf16", 64)
    assert sum(len(c) for c in w["checkpoints"]) == 35
    _check(w, "bf16", o, sf, pool, slots, heads=[0, 17, 31], block=64)
    o2, sf2, pool2, _ = _run(w, "bf16", 64)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert torch.equal(pool.nan_to_num(7.0), pool2.nan_to_num(7.0))


def test_prefill_rejects_bad_checkpoints_and_alias():
    w = inputs.prefill_workload(43, [40], 2, 16, 16, "bf16", s0_std=0.1)
    d = {n: dev_tensor(w[n], "bf16") for n in FIELDS}
    s0 = torch.from_numpy(w["s0"]).cuda()
    pool = torch.zeros((4, 2 * 16 * 16), device="cuda")
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], s0=s0,
                          checkpoints=[[41]], ckpt_slots=[[0]], page_pool=pool)
    assert e.value.status == kda.KDA_EINVAL
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"], s0=s0,
                          s_final=s0)
    assert e.value.status == kda.KDA_EALIAS


@pytest.mark.parametrize("dtype,chunk,bad", [("bf16", 64, (3,)), ("bf16", 32, (3, 5)),
                                             ("fp32", 32, (1, 3))])
def test_prefill_rejects_wide_dv_tile(dtype, chunk, bad):
    """dv tiles are at most 64 columns wide, except on the column-slab path
    (bf16 at chunk 64) and the fused path (bf16 at chunk 32, dk = 128), which
    also take 128; splits that do not divide dv into a supported width are
    refused."""
    w = inputs.prefill_workload(44, [40], 2, 128, 128, dtype)
    d = {n: dev_tensor(w[n], dtype) for n in FIELDS}
    for split in bad:
        with pytest.raises(kda.KDAError) as e:
            kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], w["cu_seqlens"],
                              chunk=chunk, dv_split=split)
        assert e.value.status == kda.KDA_EUNSUPPORTED


@pytest.mark.parametrize("dtype,chunk,g_min,dk", [("bf16", 64, -1.0, 64), ("fp32", 32, -2.0, 64),
                                                 ("bf16", 16, -0.5, 64), ("bf16", 32, -1.0, 128),
                                                 ("bf16", 32, -5.0, 128)])
def test_prefill_with_fused_gate(dtype, chunk, g_min, dk):
    """a and beta given as logits: the prefill applies a = g_min*sigmoid(z_a),
    beta = sigmoid(z_b) itself; the oracle takes the gates in float64 from the
    same logits.  (bf16 at chunk 32, dk = 128: the fused kernel, g_min up to its
    decay bound -160/32.)"""
    import oracle as orc
    lens = [1, 17, 64, 0, 130, 200]
    H, dv = 2, 128
    w = inputs.prefill_workload(170, lens, H, dk, dv, dtype, s0_std=0.1)
    rng = np.random.default_rng(171)
    z_a = rng.standard_normal(w["a"].shape).astype(np.float32)
    z_b = rng.standard_normal(w["beta"].shape).astype(np.float32)
    if dtype == "bf16":
        z_a, z_b = inputs.round_to_bf16(z_a), inputs.round_to_bf16(z_b)
    d = {n: dev_tensor(w[n], dtype) for n in ("q", "k", "v")}
    s0 = torch.from_numpy(w["s0"]).cuda()
    ck = [sorted({p for p in (5, 64, L) if 1 <= p <= L}) for L in lens]
    n_ck = sum(len(c) for c in ck)
    slots, i = [], 0
    for c in ck:
        slots.append(list(range(i, i + len(c))))
        i += len(c)
    pool = torch.zeros((n_ck, H * dk * dv), device="cuda")
    o, sf = kda.chunk_prefill(d["q"], d["k"], d["v"], dev_tensor(z_a, dtype), dev_tensor(z_b, dtype),
                              w["cu_seqlens"], s0=s0, chunk=chunk, checkpoints=ck, ckpt_slots=slots,
                              page_pool=pool, gate_g_min=g_min)
    torch.cuda.synchronize()
    a = g_min * orc.sigmoid(z_a)
    beta = orc.sigmoid(z_b)
    cu = w["cu_seqlens"]
    for n in range(len(lens)):
        lo, hi = int(cu[n]), int(cu[n + 1])
        if hi == lo:
            continue
        o_r, S_r, saved = orc.kda_recurrent(w["q"][lo:hi], w["k"][lo:hi], w["v"][lo:hi], a[lo:hi],
                                            beta[lo:hi], w["s0"][n], ck[n])
        assert_parity(o[lo:hi], o_r, dtype, f"o seq {n}")
        assert_parity(sf[n], S_r, dtype, f"s_final seq {n}")
        for j, p in enumerate(ck[n]):
            assert_parity(pool[slots[n][j]].reshape(H, dk, dv), saved[p], dtype, f"ckpt {p} seq {n}")
