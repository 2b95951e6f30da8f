"""GPU parity: head packing into page slots, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_kda_amd import kda

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


@pytest.mark.parametrize("layout", ["kv", "vk"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 16), (64, 128)])
def test_pack_matches_oracle_bit_exact(layout, dk, dv):
    rng = np.random.default_rng(dk * 1000 + dv)
    B, H, n_slots = 3, 2, 6
    page = H * dk * dv + 12
    shp = (B, H, dk, dv) if layout == "kv" else (B, H, dv, dk)
    state = rng.standard_normal(shp).astype(np.float32)
    slots = np.array([4, 0, 2], dtype=np.int32)
    pool0 = rng.standard_normal((n_slots, page)).astype(np.float32)
    want = oracle.pack_heads(state, slots, pool0.copy(), layout=layout)
    pool = torch.from_numpy(pool0).cuda()
    lay = kda.KDA_LAYOUT_KV if layout == "kv" else kda.KDA_LAYOUT_VK
    kda.pack_heads(torch.from_numpy(state).cuda(), torch.from_numpy(slots).cuda(), pool, lay)
    np.testing.assert_array_equal(_bits(pool), want.view(np.int32))
    back = kda.unpack_heads(pool, torch.from_numpy(slots).cuda(), H, dk, dv, lay)
    np.testing.assert_array_equal(_bits(back), state.view(np.int32))


def test_pack_unpack_checkpoint_pages_full_size():
    """16 states of H=32, dk=dv=128 fp32 into 2 MiB page slots and back."""
    B, H, d = 16, 32, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    state = torch.randn((B, H, d, d), device="cuda", generator=g)
    page = H * d * d
    pool = torch.full((40, page + 256), float("nan"), device="cuda")
    slots = torch.arange(39, 39 - 2 * B, -2, dtype=torch.int32, device="cuda")
    kda.pack_heads(state, slots, pool)
    back = kda.unpack_heads(pool, slots, H, d, d)
    torch.cuda.synchronize()
    assert torch.equal(_bits_t(back), _bits_t(state))
    sl = slots.cpu().numpy()
    assert not pool[slots.long(), page:].any()
    # sampled elements against the page index formula h*dk*dv + i*dv + j
    rng = np.random.default_rng(0)
    for _ in range(64):
        b, h, i, j = (int(rng.integers(0, x)) for x in (B, H, d, d))
        assert pool[sl[b], h * d * d + i * d + j].item() == state[b, h, i, j].item()
    untouched = [s for s in range(40) if s not in set(sl.tolist())]
    assert torch.isnan(pool[untouched]).all()
    # transposed source gives the same pages
    pool2 = torch.zeros_like(pool)
    kda.pack_heads(state.transpose(2, 3).contiguous(), slots, pool2, kda.KDA_LAYOUT_VK)
    torch.cuda.synchronize()
    assert torch.equal(_bits_t(pool2[slots.long()]), _bits_t(pool[slots.long()]))


def _bits_t(t):
    return t.contiguous().view(torch.int32)


def test_pack_bad_slot_is_skipped_and_flagged():
    B, H, d = 2, 2, 16
    state = torch.randn((B, H, d, d), device="cuda")
    pool = torch.zeros((3, H * d * d), device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.pack_heads(state, torch.tensor([1, 7], dtype=torch.int32, device="cuda"), pool,
                   err_flag=flag)
    torch.cuda.synchronize()
    assert flag.item() == 1
    assert torch.equal(pool[1], state[0].reshape(-1))
    assert not pool[0].any() and not pool[2].any()


def test_pack_rejects_small_page():
    state = torch.zeros((1, 2, 16, 16), device="cuda")
    pool = torch.zeros((2, 2 * 16 * 16 - 4), device="cuda")
    with pytest.raises(kda.KDAError) as e:
        kda.pack_heads(state, torch.zeros(1, dtype=torch.int32, device="cuda"), pool)
    assert e.value.status == kda.KDA_EINVAL
