"""CPU-only checks of the C ABI: the library loads, exports every entry point
that include/kda.h declares, and rejects bad arguments with a status before it
touches the GPU (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_kda_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(kda_\w+)\s*\(", text, flags=re.M))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so is not built (python -m linear_attention_recurrence_kda_amd.build)")
    return kda.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"kda_chunk_prefill", "kda_decode_step", "kda_verify_and_replay", "kda_pack_heads",
            "kda_unpack_heads", "kda_chunk_prefill_workspace_size"} <= names
    cdll = ctypes.CDLL(kda.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(cdll, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert set(kda.SIGNATURES) == names, "binding signatures out of sync with the header"


def test_status_strings_and_ratio(L):
    assert L.kda_status_string(0) == b"ok"
    assert L.kda_status_string(-3).startswith(b"output aliases")
    assert abs(L.kda_snapshot_cost_ratio(16, 32, 32) - 1024 / 129) < 1e-15
    assert abs(L.kda_snapshot_cost_ratio(2, 8, 8) - 64 / 33) < 1e-15
    assert L.kda_snapshot_cost_ratio(0, 8, 8) < 0


P = ctypes.c_void_p


def _fake(i):
    return P(0x10000000 * (i + 1))  # distinct, never dereferenced


def test_decode_validation(L):
    q, k, v, a, b, s, o = (_fake(i) for i in range(7))
    assert L.kda_decode_step(q, k, v, a, b, 0, 2, 2, 24, 16, s, o, None) == kda.KDA_EUNSUPPORTED
    assert L.kda_decode_step(q, k, v, a, b, 0, -1, 2, 16, 16, s, o, None) == kda.KDA_EINVAL
    assert L.kda_decode_step(q, k, v, a, b, 7, 2, 2, 16, 16, s, o, None) == kda.KDA_EINVAL
    assert L.kda_decode_step(None, k, v, a, b, 0, 2, 2, 16, 16, s, o, None) == kda.KDA_EINVAL
    # o overlapping the state
    assert L.kda_decode_step(q, k, v, a, b, 0, 2, 2, 16, 16, s, s, None) == kda.KDA_EALIAS
    assert b"overlap" in L.kda_last_error()
    # misaligned state
    assert L.kda_decode_step(q, k, v, a, b, 0, 2, 2, 16, 16, P(0x10000004), o, None) == kda.KDA_EINVAL
    # empty batch: nothing to do, status ok
    assert L.kda_decode_step(q, k, v, a, b, 0, 0, 2, 16, 16, s, o, None) == kda.KDA_OK


def test_replay_validation(L):
    c, q, k, v, a, b, n, s, o = (_fake(i) for i in range(9))
    args = lambda **kw: [kw.get("c", c), q, k, v, a, b, 0, n, 2, 2, 16, 16, kw.get("td", 4),
                         kw.get("s", s), kw.get("o", o), None, None]
    assert L.kda_verify_and_replay(*args(td=0)) == kda.KDA_EINVAL
    assert L.kda_verify_and_replay(*args(s=c)) == kda.KDA_EALIAS
    assert L.kda_verify_and_replay(*args(o=c)) == kda.KDA_EALIAS
    assert L.kda_verify_and_replay(*args(o=s)) == kda.KDA_EALIAS


def test_pack_validation(L):
    st, sl, pool = _fake(0), _fake(1), _fake(2)
    H, d = 2, 16
    assert L.kda_pack_heads(st, 0, 1, H, d, d, sl, pool, H * d * d - 4, 4, None, None) == kda.KDA_EINVAL
    assert L.kda_pack_heads(st, 0, 1, H, d, d, sl, pool, H * d * d + 2, 4, None, None) == kda.KDA_EUNSUPPORTED
    assert L.kda_pack_heads(st, 5, 1, H, d, d, sl, pool, H * d * d, 4, None, None) == kda.KDA_EINVAL
    assert L.kda_pack_heads(st, 0, 1, H, d, d, sl, st, H * d * d, 4, None, None) == kda.KDA_EALIAS
    assert L.kda_unpack_heads(pool, H * d * d, 4, sl, 1, H, d, d, 0, pool, None, None) == kda.KDA_EALIAS


def test_prefill_validation(L):
    """Argument checks of the chunked prefill that run on host data only."""
    q, k, v, a, b, o, ws = (_fake(i) for i in range(7))
    I32 = ctypes.c_int32

    def call(dtype=1, H=2, dk=128, dv=128, chunk=64, cu=(0, 40, 100), split=0, ck=None,
             n_slots=0, o_ptr=o):
        cu_a = (I32 * len(cu))(*cu)
        n = len(cu) - 1
        ck_cu = ck_pos = ck_slot = None
        n_ck = 0
        if ck is not None:
            pos, slot, cuv = [], [], [0]
            for p_s in ck:
                pos += [p for p, _ in p_s]
                slot += [s for _, s in p_s]
                cuv.append(len(pos))
            n_ck = len(pos)
            ck_cu, ck_pos, ck_slot = ((I32 * max(len(x), 1))(*x) for x in (cuv, pos, slot))
        pool = _fake(9) if ck is not None else None
        return L.kda_chunk_prefill_split(q, k, v, a, b, dtype, H, dk, dv, chunk, cu_a, n, None, o_ptr,
                                         None, ck_cu, ck_pos, ck_slot, n_ck, pool, H * dk * dv,
                                         n_slots, ws, 1 << 20, split, None, None)

    assert call(dk=24) == kda.KDA_EUNSUPPORTED
    assert call(chunk=48 + 8) == kda.KDA_EUNSUPPORTED
    assert call(chunk=80) == kda.KDA_EUNSUPPORTED
    assert call(dtype=0, chunk=64) == kda.KDA_EUNSUPPORTED  # fp32 inputs: chunk <= 32
    # 128-column tiles: only on the column-slab path (bf16, chunk 64, dk % 32 == 0),
    # where the call then gets as far as the workspace (too small for 4000 tokens).
    assert call(split=1, cu=(0, 4000)) == kda.KDA_EWORKSPACE
    # A width per sequence (-1) only where the column-slab kernel runs at dv = 128.
    assert call(split=-1, dv=64) == kda.KDA_EUNSUPPORTED
    assert call(split=-1, chunk=32, dk=64) == kda.KDA_EUNSUPPORTED
    assert call(split=-1, dtype=0, chunk=32) == kda.KDA_EUNSUPPORTED
    assert call(split=-2) == kda.KDA_EUNSUPPORTED
    assert call(chunk=32, split=1, dk=64) == kda.KDA_EUNSUPPORTED
    # the fused kernel (bf16, chunk 32, dk 128) takes 16- to 128-column tiles
    assert call(chunk=32, split=3) == kda.KDA_EUNSUPPORTED
    # (-n, 2 <= n <= 8: sequences in n segments; beyond that refused)
    assert call(chunk=32, split=-9) == kda.KDA_EUNSUPPORTED
    assert call(dk=16, dv=128, split=1) == kda.KDA_EUNSUPPORTED
    assert call(dtype=0, chunk=32, split=1) == kda.KDA_EUNSUPPORTED
    assert call(split=3) == kda.KDA_EUNSUPPORTED
    assert call(cu=(1, 40)) == kda.KDA_EINVAL
    assert call(cu=(0, 40, 30)) == kda.KDA_EINVAL
    assert call(ck=[[(41, 0)], []], n_slots=2) == kda.KDA_EINVAL          # past the sequence
    assert call(ck=[[(20, 0), (10, 1)], []], n_slots=2) == kda.KDA_EINVAL  # not increasing
    assert call(ck=[[(20, 0)], [(5, 0)]], n_slots=2) == kda.KDA_EINVAL     # slot repeated
    assert call(ck=[[(20, 2)], []], n_slots=2) == kda.KDA_EINVAL           # slot out of range
    assert b"slot" in L.kda_last_error()
    assert call(o_ptr=P(o.value + 8)) == kda.KDA_EINVAL                   # o rows need 16 bytes
    assert b"o must be 16-byte aligned" in L.kda_last_error()
    assert call(H=(1 << 17) + 1, dk=16) == kda.KDA_EUNSUPPORTED           # 32-bit chunk offsets
    assert b"2^24" in L.kda_last_error()


def test_prefill_checkpoint_offsets_checked_before_positions(L):
    """ckpt_cu = [0, 5, 2] with two checkpoints: refused from the offsets alone
    (the five positions the second entry would name are never read)."""
    I32 = ctypes.c_int32
    cu = (I32 * 3)(0, 40, 100)
    ck_cu, ck_pos, ck_slot = (I32 * 3)(0, 5, 2), (I32 * 2)(10, 20), (I32 * 2)(0, 1)
    st = L.kda_chunk_prefill(*(_fake(i) for i in range(5)), 1, 2, 16, 16, 64, cu, 2, None, _fake(5), None,
                             ck_cu, ck_pos, ck_slot, 2, _fake(9), 2 * 16 * 16, 4, _fake(6), 1 << 20,
                             None, None)
    assert st == kda.KDA_EINVAL
    assert b"ckpt_cu" in L.kda_last_error()


def test_gated_prefill_refuses_g_min_below_the_decay_bound(L):
    """The gated a lies in [g_min, 0] ("Serve 模块交互式演示" §1.3); the chunk
    form needs a >= -160/chunk, so g_min below that is refused on the host."""
    I32 = ctypes.c_int32
    cu = (I32 * 2)(0, 40)

    def gated(g_min, chunk=64):
        return L.kda_chunk_prefill_gated(*(_fake(i) for i in range(5)), ctypes.c_float(g_min), 1, 2, 16,
                                         16, chunk, cu, 1, None, _fake(5), None, None, None, None, 0,
                                         None, 0, 0, _fake(6), 1 << 10, 0, None, None)

    assert gated(-2.6) == kda.KDA_EUNSUPPORTED
    assert b"decay bound" in L.kda_last_error()
    assert gated(-5.1, chunk=32) == kda.KDA_EUNSUPPORTED
    assert gated(0.5) == kda.KDA_EINVAL
    # at the bound the call gets as far as the (too small) workspace
    assert gated(-2.5) == kda.KDA_EWORKSPACE
    assert gated(-5.0, chunk=32) == kda.KDA_EWORKSPACE


def test_prefill_plan_widths():
    """The plan query reports each sequence's tile width.  Chunk counts 20,
    14, 6 and 2 at H = 2 with a width per sequence: 32, 64, 128 and 128
    columns (the cost model's balance of the longest chain against the total
    work); one width everywhere for an explicit split."""
    lens = [64 * 20, 64 * 14, 64 * 6, 100]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    ck = [list(range(256, n + 1, 256)) for n in lens]
    cols, names = kda.prefill_plan(cu, 2, 128, 128, 64, ck, dv_split=-1)
    assert cols == [32, 64, 128, 128]
    assert "slab_mixed_kernel" in names
    cols, names = kda.prefill_plan(cu, 2, 128, 128, 64, ck, dv_split=4)
    assert cols == [32] * 4 and "slab_kernel<128> (32-column tiles)" in names
    cols, names = kda.prefill_plan([0, 100, 150], 2, 64, 64, 32, dtype=__import__("torch").float32)
    assert "prop_kernel" in names
    # bf16 at chunk 32 with dk = 128: the fused kernel, a width per sequence
    cols, names = kda.prefill_plan([0, 3000, 3100, 3150], 2, 128, 128, 32)
    assert "fused_kernel" in names and all(c in (16, 32, 64, 128) for c in cols)
    cols, _ = kda.prefill_plan([0, 3000, 3100, 3150], 2, 128, 64, 32, dv_split=2)
    assert cols == [32, 32, 32]


def test_prefill_plan_segments():
    """Fused path (bf16, chunk 32, dk = dv = 128): a sequence whose chain
    would bound the call is cut into segments by the cost model; -n cuts
    every sequence of at least n * 512 tokens into n; dv != dk, an explicit
    tile width or -1 cut nothing."""
    cu = [0, 30000, 31000, 31500]
    _, names = kda.prefill_plan(cu, 32, 128, 128, 32)
    assert "1 sequence in" in names, names
    _, names = kda.prefill_plan([0, 2100, 3200, 3245, 3245, 4545], 2, 128, 128, 32, dv_split=-2)
    assert "3 sequences in 6 segments" in names, names  # (2100, 1100 and 1300 tokens)
    _, names = kda.prefill_plan([0, 2100, 3200, 3245, 3245, 4545], 2, 128, 128, 32, dv_split=-4)
    assert "1 sequence in 4 segments" in names, names
    for kw in ({"dv_split": -1}, {"dv_split": 1}):
        _, names = kda.prefill_plan(cu, 32, 128, 128, 32, **kw)
        assert "segments" not in names, names
    _, names = kda.prefill_plan(cu, 32, 128, 64, 32)
    assert "segments" not in names, names


def test_prefill_plan_is_fast_for_many_sequences():
    """The width choice is O(n log n): 4096 sequences plan in well under a
    tenth of a second."""
    import time
    import numpy as np
    lens = np.random.default_rng(5).integers(1, 4000, 4096)
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    t0 = time.perf_counter()
    cols, _ = kda.prefill_plan(cu, 32, 128, 128, 64)
    assert time.perf_counter() - t0 < 0.1
    assert set(cols) <= {16, 32, 64, 128}
    # the fused path's plan (widths, segments and their list scheduling), with
    # one long sequence among them
    cu[-1] += 60000
    t0 = time.perf_counter()
    cols, _ = kda.prefill_plan(cu, 32, 128, 128, 32)
    assert time.perf_counter() - t0 < 0.5
    assert set(cols) <= {16, 32, 64, 128}


def test_segment_validation(L):
    """Argument checks of the segment summary and the composition."""
    k, v, a, b, A, B, ws = (_fake(i) for i in range(7))
    I32 = ctypes.c_int32

    def summ(dtype=1, H=2, dk=128, dv=128, chunk=64, cu=(0, 40, 100), A_ptr=A, B_ptr=B, ws_ptr=ws):
        cu_a = (I32 * len(cu))(*cu)
        return L.kda_segment_summary(k, v, a, b, dtype, H, dk, dv, chunk, cu_a, len(cu) - 1, A_ptr,
                                     B_ptr, ws_ptr, 1 << 20, None)

    assert summ(dk=24) == kda.KDA_EUNSUPPORTED
    assert summ(dtype=0, chunk=64) == kda.KDA_EUNSUPPORTED
    assert summ(cu=(0, 40, 30)) == kda.KDA_EINVAL
    assert summ(A_ptr=None) == kda.KDA_EINVAL
    assert summ(B_ptr=None) == kda.KDA_EINVAL
    assert summ(A_ptr=P(B.value + 64)) == kda.KDA_EALIAS                 # A overlaps B
    assert summ(ws_ptr=P(ws.value + 16)) == kda.KDA_EINVAL              # 256-byte alignment
    assert summ(cu=(0, 4000, 10000)) == kda.KDA_EWORKSPACE              # 1 MiB is too small
    sz = ctypes.c_size_t(0)
    assert L.kda_segment_summary_workspace_size(3, 300, 2, 128, 128, 64, 1, ctypes.byref(sz)) == 0
    want = ctypes.c_size_t(0)
    assert L.kda_chunk_prefill_workspace_size(3, 300, 2, 128, 128, 64, 0, 1, ctypes.byref(want)) == 0
    assert sz.value == want.value

    s_in, st, end = _fake(7), _fake(8), _fake(9)

    def comp(n=3, H=2, dk=64, dv=32, A_ptr=A, B_ptr=B, st_ptr=st, end_ptr=end):
        return L.kda_compose_segments(A_ptr, B_ptr, n, H, dk, dv, s_in, st_ptr, end_ptr, None)

    assert comp(dk=24) == kda.KDA_EUNSUPPORTED
    assert comp(n=-1) == kda.KDA_EINVAL
    assert comp(H=0) == kda.KDA_EINVAL
    assert comp(A_ptr=None) == kda.KDA_EINVAL
    assert comp(st_ptr=None) == kda.KDA_EINVAL
    assert comp(A_ptr=P(A.value + 4)) == kda.KDA_EINVAL                  # float4 rows of A
    assert comp(st_ptr=P(B.value + 128)) == kda.KDA_EALIAS               # starts overlap B
    assert comp(end_ptr=P(st.value + 4)) == kda.KDA_EALIAS               # end overlaps starts
    assert comp(n=0, end_ptr=None) == kda.KDA_OK                         # nothing to do


def test_front_end_validation(L):
    """Argument checks of the front end and its decode step."""
    x, za, zb, w, q, k, v, a, b, ws = (_fake(i) for i in range(10))
    I32 = ctypes.c_int32
    F = ctypes.c_float

    def fe(dtype=1, H=2, dk=64, dv=64, K=4, g=-1.0, cu=(0, 40, 100), win_in=None, win_out=None,
           x_ptr=x, q_ptr=q, ws_ptr=ws, ck=None, conv_elems=0, n_slots=0):
        cu_a = (I32 * len(cu))(*cu)
        n = len(cu) - 1
        ck_cu = ck_pos = ck_slot = None
        n_ck = 0
        if ck is not None:
            pos, slot, cuv = [], [], [0]
            for p_s in ck:
                pos += [p for p, _ in p_s]
                slot += [s for _, s in p_s]
                cuv.append(len(pos))
            n_ck = len(pos)
            ck_cu, ck_pos, ck_slot = ((I32 * max(len(z), 1))(*z) for z in (cuv, pos, slot))
        pool = _fake(11) if ck is not None else None
        return L.kda_front_end(x_ptr, za, zb, w, dtype, H, dk, dv, K, F(g), cu_a, n, win_in, win_out,
                               ck_cu, ck_pos, ck_slot, n_ck, pool, conv_elems, n_slots, q_ptr, k, v,
                               a, b, ws_ptr, 1 << 20, None)

    assert fe(dk=24) == kda.KDA_EUNSUPPORTED
    assert fe(K=5) == kda.KDA_EUNSUPPORTED and fe(K=0) == kda.KDA_EUNSUPPORTED
    assert fe(g=0.5) == kda.KDA_EINVAL and fe(g=float("nan")) == kda.KDA_EINVAL
    assert fe(cu=(0, 40, 30)) == kda.KDA_EINVAL
    assert fe(x_ptr=P(x.value + 8)) == kda.KDA_EINVAL                     # 16-byte alignment
    assert fe(ws_ptr=P(ws.value + 8)) == kda.KDA_EINVAL                   # 16-byte workspace
    assert fe(q_ptr=P(x.value + 64)) == kda.KDA_EALIAS                    # q overlaps x
    assert fe(ck=[[(41, 0)], []], conv_elems=3 * 2 * 192, n_slots=2) == kda.KDA_EINVAL
    assert fe(ck=[[(20, 0)], [(5, 0)]], conv_elems=3 * 2 * 192, n_slots=2) == kda.KDA_EINVAL
    assert fe(ck=[[(20, 0)], []], conv_elems=10, n_slots=2) == kda.KDA_EINVAL   # slot too small
    sz = ctypes.c_size_t(0)
    assert L.kda_front_end_workspace_size(2, 100, 3, ctypes.byref(sz)) == 0 and sz.value > 0

    def step(K=4, window=_fake(12), B=3, g=-1.0):
        return L.kda_front_end_step(x, za, zb, w, 1, B, 2, 64, 64, K, F(g), window, q, k, v, a, b, None)

    assert step(window=None) == kda.KDA_EINVAL          # K > 1 needs a window
    assert step(B=-1) == kda.KDA_EINVAL
    assert step(B=0) == kda.KDA_OK
    assert step(window=P(x.value + 8)) == kda.KDA_EINVAL            # 16-byte alignment
    assert step(window=P(x.value + 64)) == kda.KDA_EALIAS


def test_ring_validation(L):
    """Argument checks of the raw-input ring."""
    base = [_fake(i) for i in range(6)]

    def ring(**kw):
        args = dict(q=base[0].value, k=base[1].value, v=base[2].value, a=base[3].value,
                    beta=base[4].value, count=base[5].value, n_slots=4, capacity=8, H=2, dk=16, dv=16,
                    dtype=1)
        args.update(kw)
        return kda.KdaRing(**args)

    def push(r, B=2, q=_fake(8)):
        return L.kda_ring_push(ctypes.byref(r), _fake(7), B, q, _fake(9), _fake(10), _fake(11),
                               _fake(12), None, None)

    assert push(ring(capacity=0)) == kda.KDA_EUNSUPPORTED
    assert push(ring(capacity=2000)) == kda.KDA_EUNSUPPORTED
    assert push(ring(dk=24)) == kda.KDA_EUNSUPPORTED
    assert push(ring(q=None)) == kda.KDA_EINVAL
    assert push(ring(q=base[0].value + 8)) == kda.KDA_EINVAL           # 16-byte alignment
    assert push(ring(k=base[0].value + 256)) == kda.KDA_EALIAS          # ring arrays overlap
    assert push(ring(), B=-1) == kda.KDA_EINVAL
    assert push(ring(), B=0) == kda.KDA_OK
    assert push(ring(), q=P(base[0].value + 64)) == kda.KDA_EALIAS     # step input inside the ring
    assert push(ring(), q=P(_fake(8).value + 4)) == kda.KDA_EINVAL
    assert L.kda_ring_window(ctypes.byref(ring()), _fake(7), 2, None, _fake(9), _fake(10), _fake(11),
                             _fake(12), None, None, None) == kda.KDA_EINVAL
    assert L.kda_ring_reset(None, _fake(7), 2, None, None) == kda.KDA_EINVAL
