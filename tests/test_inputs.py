"""The seeded input generators: determinism, shapes, ranges, bf16 rounding."""
import numpy as np
import torch

from linear_attention_recurrence_kda_amd import inputs


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 1e-30, 3e38],
                                 dtype=np.float32)])
    got = inputs.round_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert not np.array_equal(got, x)  # input untouched, output rounded


def test_token_inputs_ranges_and_determinism():
    t1 = inputs.token_inputs(0, 3, (50,), 2, 16, 8, "fp32")
    t2 = inputs.token_inputs(0, 3, (50,), 2, 16, 8, "fp32")
    for n in t1:
        np.testing.assert_array_equal(t1[n], t2[n])
    assert t1["q"].shape == (50, 2, 16) and t1["v"].shape == (50, 2, 8)
    assert t1["beta"].shape == (50, 2)
    np.testing.assert_allclose(np.linalg.norm(t1["k"], axis=-1), 1.0, rtol=1e-5)
    assert (t1["a"] <= 0).all() and (t1["a"] >= -1).all()
    assert (t1["beta"] >= 0).all() and (t1["beta"] <= 1).all()
    t3 = inputs.token_inputs(0, 4, (50,), 2, 16, 8, "fp32")
    assert not np.array_equal(t1["q"], t3["q"])


def test_bf16_workload_values_are_bf16():
    t = inputs.token_inputs(3, 0, (10,), 2, 8, 8, "bf16")
    for x in t.values():
        assert (x.view(np.uint32) & 0xFFFF == 0).all()


def test_sequence_slice_regenerates_workload_sequence():
    lens = [5, 9, 3]
    w = inputs.prefill_workload(9, lens, 2, 4, 4, "bf16", s0_std=0.1, ckpt_every=4)
    s = inputs.sequence_slice(9, 1, 9, 2, 4, 4, "bf16", s0_std=0.1)
    np.testing.assert_array_equal(w["q"][5:14], s["q"])
    np.testing.assert_array_equal(w["s0"][1], s["s0"])
    assert w["checkpoints"] == [[4, 5], [4, 8, 9], [3]]
    assert list(w["cu_seqlens"]) == [0, 5, 14, 17]


def test_workload_shapes():
    lens = inputs.prefill_lengths(4)
    assert len(lens) == 16 and all(1024 <= L <= 32768 for L in lens)
    ck = inputs.prefill_checkpoints([8192], 512, tail=False)
    assert ck == [list(range(512, 8193, 512))] and len(ck[0]) == 16
    ck4 = inputs.prefill_checkpoints([6976, 8192], 4096, tail=True)
    assert ck4 == [[4096, 6976], [4096, 8192]]
    r = inputs.replay_workload()
    assert r["q"].shape == (8, 64, 16, 32) and r["committed"].shape == (64, 16, 32, 32)
    assert r["n_accepted"].min() >= 0 and r["n_accepted"].max() <= 8
