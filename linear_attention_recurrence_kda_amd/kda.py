"""Thin Python binding of the KDA C ABI (include/kda.h) over ctypes.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their pointers and the current HIP stream are passed to the
library, and a non-zero status raises KDAError with the library's message.
Every step of the computation runs in the HIP kernels of libkda.so; there is
no fallback.  If the library has not been built, loading it raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# (KDA_LIB names another build of the same library, e.g. the sanitized one.)
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_EINVAL, KDA_EUNSUPPORTED, KDA_EALIAS, KDA_EWORKSPACE, KDA_EHIP = 0, -1, -2, -3, -4, -5
KDA_F32, KDA_BF16 = 0, 1
KDA_LAYOUT_KV, KDA_LAYOUT_VK = 0, 1

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/kda.h
class KdaRing(ctypes.Structure):
    """The kda_ring description of include/kda.h."""
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("a", _vp), ("beta", _vp), ("count", _vp),
                ("n_slots", _i64), ("capacity", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
                ("dtype", ctypes.c_int)]


_ringp = ctypes.POINTER(KdaRing)

SIGNATURES = {
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_snapshot_cost_ratio": (ctypes.c_double, [_i32, _i32, _i32]),
    "kda_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32,
                                       _i32, _vp, _vp, _vp]),
    "kda_verify_and_replay": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32,
                                             _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kda_pack_heads": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                                      _i64, _vp, _vp]),
    "kda_unpack_heads": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, ctypes.c_int,
                                        _vp, _vp, _vp]),
    "kda_chunk_prefill_workspace_size": (ctypes.c_int, [_i32, _i64, _i32, _i32, _i32, _i32, _i64,
                                                        ctypes.c_int, ctypes.POINTER(_sz)]),
    "kda_chunk_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32,
                                         _i32, _i32p, _i32, _vp, _vp, _vp, _i32p, _i32p, _i32p,
                                         _i64, _vp, _i64, _i64, _vp, _sz, _vp, _vp]),
    "kda_chunk_prefill_split": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32,
                                               _i32, _i32, _i32p, _i32, _vp, _vp, _vp, _i32p, _i32p,
                                               _i32p, _i64, _vp, _i64, _i64, _vp, _sz, _i32, _vp,
                                               _vp]),
    "kda_chunk_prefill_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32,
                                                _i32, _i32p, _i32, _vp, _vp, _vp, _i32p, _i32p, _i32p,
                                                _i64, _vp, _i64, _i64, _vp, _vp]),
    "kda_static_scratch_bytes": (_sz, []),
    "kda_chunk_prefill_plan": (ctypes.c_int, [ctypes.c_int, _i32, _i32, _i32, _i32, _i32p, _i32,
                                              _i32p, _i32p, _i64, _i32, _i32p, ctypes.c_char_p,
                                              _sz]),
    "kda_chunk_prefill_gated": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_int,
                                               _i32, _i32, _i32, _i32, _i32p, _i32, _vp, _vp, _vp,
                                               _i32p, _i32p, _i32p, _i64, _vp, _i64, _i64, _vp, _sz,
                                               _i32, _vp, _vp]),
    "kda_segment_summary_workspace_size": (ctypes.c_int, [_i32, _i64, _i32, _i32, _i32, _i32,
                                                          ctypes.c_int, ctypes.POINTER(_sz)]),
    "kda_segment_summary": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _i32,
                                           _i32p, _i32, _vp, _vp, _vp, _sz, _vp]),
    "kda_compose_segments": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kda_front_end_workspace_size": (ctypes.c_int, [_i32, _i64, _i64, ctypes.POINTER(_sz)]),
    "kda_front_end": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _i32,
                                     ctypes.c_float, _i32p, _i32, _vp, _vp, _i32p, _i32p, _i32p, _i64,
                                     _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_front_end_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _i32,
                                          _i32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_decode_step_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32,
                                          _i32, ctypes.c_int, _vp, _vp, _vp]),
    "kda_verify_and_replay_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                                                _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp, _vp,
                                                _vp, _vp]),
    "kda_pack_heads_ex": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int, _i32, _i32, _i32, _i32, _vp,
                                         _vp, _i64, _i64, _vp, _vp]),
    "kda_unpack_heads_ex": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _vp, _i32, _i32, _i32,
                                           _i32, ctypes.c_int, _vp, _vp, _vp]),
    "kda_ring_push": (ctypes.c_int, [_ringp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_ring_window": (ctypes.c_int, [_ringp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_ring_reset": (ctypes.c_int, [_ringp, _vp, _i32, _vp, _vp]),
}

_lib = None
_bound = {}


class KDAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"KDA status {status}: {message}")
        self.status = status


class _Lib:
    """libkda.so with each entry point typed from SIGNATURES on first use."""

    def __init__(self, cdll):
        self._cdll = cdll

    def __getattr__(self, name):
        fn = _bound.get(name)
        if fn is None:
            res, args = SIGNATURES[name]
            fn = getattr(self._cdll, name)
            fn.restype, fn.argtypes = res, args
            _bound[name] = fn
        return fn


def lib():
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_recurrence_kda_amd.build`")
        _lib = _Lib(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status):
    if status != KDA_OK:
        msg = lib().kda_last_error().decode()
        raise KDAError(status, msg or lib().kda_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"inputs must be float32 or bfloat16, got {t.dtype}")


def _expect(t, shape, dtype, name, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _i32_array(seq):
    arr = (ctypes.c_int32 * max(1, len(seq)))(*[int(x) for x in seq])
    return arr


def snapshot_cost_ratio(H, dk, dv):
    return lib().kda_snapshot_cost_ratio(H, dk, dv)


def _state_code(t, name):
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    return _dtype_code(t)


def decode_step(q, k, v, a, beta, state, o=None):
    """One token per session; state [B,H,dk,dv] (float32, or bfloat16 for the
    bf16-state variant) is updated in place.  q, k, a [B,H,dk], v [B,H,dv],
    beta [B,H]; returns o [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    for t, shp, n in ((q, (B, H, dk), "q"), (k, (B, H, dk), "k"), (a, (B, H, dk), "a"),
                      (v, (B, H, dv), "v"), (beta, (B, H), "beta")):
        _expect(t, shp, dt, n, dev)
    sd = _state_code(state, "state")
    _expect(state, (B, H, dk, dv), state.dtype, "state", dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _expect(o, (B, H, dv), dt, "o", dev)
    _check(lib().kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _dtype_code(q),
                                    B, H, dk, dv, sd, _ptr(state), _ptr(o), _stream(dev)))
    return o


def verify_and_replay(committed, q, k, v, a, beta, n_accepted, s_new=None, o=None, err_flag=None):
    """Clone committed [B,H,dk,dv] (float32, or bfloat16) and replay
    n_accepted[b] draft steps.  Projections in (t_draft, B, H, D) layout;
    n_accepted int32 [B] on the device.  Returns (s_new [B,H,dk,dv] in the
    committed state's dtype, o [B,H,t_draft,dv])."""
    Td, B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    for t, shp, n in ((q, (Td, B, H, dk), "q"), (k, (Td, B, H, dk), "k"),
                      (a, (Td, B, H, dk), "a"), (v, (Td, B, H, dv), "v"),
                      (beta, (Td, B, H), "beta")):
        _expect(t, shp, dt, n, dev)
    sd = _state_code(committed, "committed")
    _expect(committed, (B, H, dk, dv), committed.dtype, "committed", dev)
    _expect(n_accepted, (B,), torch.int32, "n_accepted", dev)
    if s_new is None:
        s_new = torch.empty_like(committed)
    if o is None:
        o = torch.empty((B, H, Td, dv), dtype=dt, device=dev)
    _expect(s_new, (B, H, dk, dv), committed.dtype, "s_new", dev)
    _expect(o, (B, H, Td, dv), dt, "o", dev)
    if err_flag is not None:
        _expect(err_flag, (1,), torch.int32, "err_flag", dev)
    _check(lib().kda_verify_and_replay_ex(_ptr(committed), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                          _ptr(beta), _dtype_code(q), _ptr(n_accepted), B, H, dk,
                                          dv, Td, sd, _ptr(s_new), _ptr(o), _ptr(err_flag),
                                          _stream(dev)))
    return s_new, o


def pack_heads(state, slot, page_pool, layout=KDA_LAYOUT_KV, err_flag=None, dk=None, dv=None):
    """state [B,H,dk,dv] (KV) or [B,H,dv,dk] (VK) -> page_pool[slot[b]] (zero
    padded); state and pages float32, or both bfloat16."""
    B, H = state.shape[:2]
    if layout == KDA_LAYOUT_KV:
        dk, dv = state.shape[2], state.shape[3]
    else:
        dv, dk = state.shape[2], state.shape[3]
    dev = state.device
    sd = _state_code(state, "state")
    _expect(state, tuple(state.shape), state.dtype, "state", dev)
    _expect(slot, (B,), torch.int32, "slot", dev)
    n_slots, page_elems = page_pool.shape
    _expect(page_pool, (n_slots, page_elems), state.dtype, "page_pool", dev)
    if err_flag is not None:
        _expect(err_flag, (1,), torch.int32, "err_flag", dev)
    _check(lib().kda_pack_heads_ex(_ptr(state), sd, layout, B, H, dk, dv, _ptr(slot),
                                   _ptr(page_pool), page_elems, n_slots, _ptr(err_flag),
                                   _stream(dev)))
    return page_pool


def unpack_heads(page_pool, slot, H, dk, dv, layout=KDA_LAYOUT_KV, state=None, err_flag=None):
    """page_pool[slot[b]] -> state [B,H,dk,dv] (KV) or [B,H,dv,dk] (VK), in
    the pool's dtype (float32 or bfloat16)."""
    dev = page_pool.device
    B = slot.shape[0]
    n_slots, page_elems = page_pool.shape
    sd = _state_code(page_pool, "page_pool")
    _expect(slot, (B,), torch.int32, "slot", dev)
    shp = (B, H, dk, dv) if layout == KDA_LAYOUT_KV else (B, H, dv, dk)
    if state is None:
        state = torch.empty(shp, dtype=page_pool.dtype, device=dev)
    _expect(state, shp, page_pool.dtype, "state", dev)
    if err_flag is not None:
        _expect(err_flag, (1,), torch.int32, "err_flag", dev)
    _check(lib().kda_unpack_heads_ex(_ptr(page_pool), sd, page_elems, n_slots, _ptr(slot), B, H, dk,
                                     dv, layout, _ptr(state), _ptr(err_flag), _stream(dev)))
    return state


def prefill_workspace_size(n_seqs, total_tokens, H, dk, dv, chunk, n_ckpt, dtype=torch.bfloat16):
    out = ctypes.c_size_t(0)
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    _check(lib().kda_chunk_prefill_workspace_size(n_seqs, total_tokens, H, dk, dv, chunk, n_ckpt,
                                                  code, ctypes.byref(out)))
    return out.value


def _ckpt_arrays(checkpoints, ckpt_slots, N):
    """Flatten per-sequence checkpoint lists into (ckpt_cu, ckpt_pos, ckpt_slot)."""
    ck_cu, ck_pos, ck_slot = [0], [], []
    if checkpoints is None:
        return [0] * (N + 1), ck_pos, ck_slot
    if ckpt_slots is None:
        ckpt_slots = [[0] * len(p) for p in checkpoints]
    if len(checkpoints) != N or len(ckpt_slots) != N:
        raise ValueError("checkpoints and ckpt_slots need one list per sequence")
    for pos, sl in zip(checkpoints, ckpt_slots):
        if len(pos) != len(sl):
            raise ValueError("each sequence needs one slot per checkpoint")
        ck_pos += list(pos)
        ck_slot += list(sl)
        ck_cu.append(len(ck_pos))
    return ck_cu, ck_pos, ck_slot


def prefill_plan(cu_seqlens, H, dk, dv, chunk=64, checkpoints=None, dtype=torch.bfloat16,
                 dv_split=0):
    """What chunk_prefill would launch: (dv columns per workgroup of each
    sequence, the kernels' names).  Nothing runs on the device."""
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    ck_cu, ck_pos, _ = _ckpt_arrays(checkpoints, None, N)
    cols = (ctypes.c_int32 * max(1, N))()
    names = ctypes.create_string_buffer(256)
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    _check(lib().kda_chunk_prefill_plan(code, H, dk, dv, chunk, _i32_array(cu), N, _i32_array(ck_cu),
                                        _i32_array(ck_pos), len(ck_pos), dv_split, cols, names,
                                        ctypes.sizeof(names)))
    return [cols[i] for i in range(N)], names.value.decode()


def chunk_prefill(q, k, v, a, beta, cu_seqlens, s0=None, chunk=64, checkpoints=None,
                  ckpt_slots=None, page_pool=None, o=None, s_final=None, want_final=True,
                  workspace=None, dv_split=0, gate_g_min=None, err_flag=None):
    """Token-packed varlen prefill.

    q, k, a [T,H,dk], v [T,H,dv], beta [T,H] (float32 or bfloat16, same dtype)
    cu_seqlens: host sequence of N+1 offsets; s0 [N,H,dk,dv] fp32 or None
    checkpoints: per sequence a list of token counts (or None);
    ckpt_slots: per sequence a list of page slots, same shape as checkpoints;
    page_pool [n_slots, page_elems] fp32 receives the checkpoint states.
    gate_g_min: when given, a and beta are gate logits and the prefill uses
    a = gate_g_min * sigmoid(a), beta = sigmoid(beta) (the fused gate).
    err_flag: int32 [1] on the device, or None; set to 1 when a log-decay
    lies outside [-160/chunk, 0] (what is then written: see kda_chunk_prefill
    in include/kda.h).
    dv_split: 0 (the library's choice), 1/2/4/8 tiles per head, -1 a width
    per sequence, -n (2..8) every sequence of at least n * 512 tokens in n
    segments (fused path).
    Returns (o [T,H,dv], s_final [N,H,dk,dv] or None).
    """
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    for t, shp, n in ((q, (T, H, dk), "q"), (k, (T, H, dk), "k"), (a, (T, H, dk), "a"),
                      (v, (T, H, dv), "v"), (beta, (T, H), "beta")):
        _expect(t, shp, dt, n, dev)
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    if s0 is not None:
        _expect(s0, (N, H, dk, dv), torch.float32, "s0", dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=dt, device=dev)
    _expect(o, (T, H, dv), dt, "o", dev)
    if s_final is None and want_final:
        s_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if s_final is not None:
        _expect(s_final, (N, H, dk, dv), torch.float32, "s_final", dev)
    if checkpoints is not None and (ckpt_slots is None or page_pool is None):
        raise ValueError("checkpoints need ckpt_slots and page_pool")
    ck_cu, ck_pos, ck_slot = _ckpt_arrays(checkpoints, ckpt_slots, N)
    n_ckpt = len(ck_pos)
    if err_flag is not None:
        _expect(err_flag, (1,), torch.int32, "err_flag", dev)
    n_slots, page_elems = (0, 0) if page_pool is None else page_pool.shape
    if page_pool is not None:
        _expect(page_pool, (n_slots, page_elems), torch.float32, "page_pool", dev)
    need = prefill_workspace_size(N, T, H, dk, dv, chunk, n_ckpt, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    common = (H, dk, dv, chunk, _i32_array(cu), N, _ptr(s0), _ptr(o), _ptr(s_final), _i32_array(ck_cu),
              _i32_array(ck_pos), _i32_array(ck_slot), n_ckpt, _ptr(page_pool), page_elems,
              n_slots, _ptr(workspace), workspace.numel(), dv_split, _ptr(err_flag), _stream(dev))
    if gate_g_min is None:
        _check(lib().kda_chunk_prefill_split(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta),
                                             _dtype_code(q), *common))
    else:
        _check(lib().kda_chunk_prefill_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta),
                                             float(gate_g_min), _dtype_code(q), *common))
    return o, s_final


def segment_summary_workspace_size(n_seg, total_tokens, H, dk, dv, chunk, dtype=torch.bfloat16):
    out = ctypes.c_size_t(0)
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    _check(lib().kda_segment_summary_workspace_size(n_seg, total_tokens, H, dk, dv, chunk, code,
                                                    ctypes.byref(out)))
    return out.value


def segment_summary(k, v, a, beta, cu_segments, chunk=64, A=None, B=None, workspace=None):
    """Affine maps S_end = A S_start + B of the segments of a token-packed input.

    k, a [T,H,dk], v [T,H,dv], beta [T,H] (float32 or bfloat16, same dtype);
    cu_segments: host sequence of n+1 segment offsets.
    Returns (A [n,H,dk,dk], B [n,H,dk,dv]), fp32.
    """
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    for t, shp, nm in ((k, (T, H, dk), "k"), (a, (T, H, dk), "a"), (v, (T, H, dv), "v"),
                       (beta, (T, H), "beta")):
        _expect(t, shp, dt, nm, dev)
    cu = [int(x) for x in cu_segments]
    n = len(cu) - 1
    if A is None:
        A = torch.empty((n, H, dk, dk), dtype=torch.float32, device=dev)
    if B is None:
        B = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    _expect(A, (n, H, dk, dk), torch.float32, "A", dev)
    _expect(B, (n, H, dk, dv), torch.float32, "B", dev)
    need = segment_summary_workspace_size(n, T, H, dk, dv, chunk, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().kda_segment_summary(_ptr(k), _ptr(v), _ptr(a), _ptr(beta), _dtype_code(k), H, dk,
                                     dv, chunk, _i32_array(cu), n, _ptr(A), _ptr(B),
                                     _ptr(workspace), workspace.numel(), _stream(dev)))
    return A, B


def compose_segments(A, B, s_in=None, starts=None, s_end=None):
    """Exclusive scan of segment maps: starts[0] = s_in (zero if None),
    starts[i+1] = A[i] starts[i] + B[i].  A [n,H,dk,dk], B [n,H,dk,dv] fp32;
    s_in [H,dk,dv] fp32 or None.  Returns (starts [n,H,dk,dv], s_end [H,dk,dv])."""
    n, H, dk, dv = B.shape
    dev = B.device
    _expect(A, (n, H, dk, dk), torch.float32, "A", dev)
    _expect(B, (n, H, dk, dv), torch.float32, "B", dev)
    if s_in is not None:
        _expect(s_in, (H, dk, dv), torch.float32, "s_in", dev)
    if starts is None:
        starts = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    if s_end is None:
        s_end = torch.empty((H, dk, dv), dtype=torch.float32, device=dev)
    _expect(starts, (n, H, dk, dv), torch.float32, "starts", dev)
    _expect(s_end, (H, dk, dv), torch.float32, "s_end", dev)
    _check(lib().kda_compose_segments(_ptr(A), _ptr(B), n, H, dk, dv, _ptr(s_in), _ptr(starts),
                                      _ptr(s_end), _stream(dev)))
    return starts, s_end


def front_end_workspace_size(n_seqs, total_tokens, n_ckpt=0):
    out = ctypes.c_size_t(0)
    _check(lib().kda_front_end_workspace_size(n_seqs, total_tokens, n_ckpt, ctypes.byref(out)))
    return out.value


def front_end(x, z_a, z_b, conv_w, H, dk, dv, g_min, cu_seqlens, win_in=None, want_window=True,
              checkpoints=None, ckpt_slots=None, conv_pool=None, out=None, workspace=None):
    """Front end of token-packed sequences: causal ShortConv, SiLU, L2Norm of
    q and k, gates.  x [T, H*(2dk+dv)], z_a [T,H,dk], z_b [T,H], conv_w [C,K]
    (one dtype, float32 or bfloat16); win_in [N,K-1,C] or None.
    Returns a dict with q, k, v, a, beta and "window" [N,K-1,C] (or None)."""
    T, C = x.shape
    K = conv_w.shape[1]
    dev, dt = x.device, x.dtype
    for t, shp, nm in ((x, (T, C), "x"), (z_a, (T, H, dk), "z_a"), (z_b, (T, H), "z_b"),
                       (conv_w, (C, K), "conv_w")):
        _expect(t, shp, dt, nm, dev)
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    if win_in is not None:
        _expect(win_in, (N, K - 1, C), dt, "win_in", dev)
    o = dict(out or {})
    for nm, shp in (("q", (T, H, dk)), ("k", (T, H, dk)), ("v", (T, H, dv)), ("a", (T, H, dk)),
                    ("beta", (T, H))):
        if o.get(nm) is None:
            o[nm] = torch.empty(shp, dtype=dt, device=dev)
        _expect(o[nm], shp, dt, nm, dev)
    if want_window and o.get("window") is None:
        o["window"] = torch.empty((N, K - 1, C), dtype=dt, device=dev)
    win_out = o.get("window") if want_window else None
    ck_cu, ck_pos, ck_slot = [0] * (N + 1), [], []
    if checkpoints is not None:
        if ckpt_slots is None or conv_pool is None:
            raise ValueError("checkpoints need ckpt_slots and conv_pool")
        ck_cu = [0]
        for pos, sl in zip(checkpoints, ckpt_slots):
            if len(pos) != len(sl):
                raise ValueError("each sequence needs one slot per checkpoint")
            ck_pos += list(pos)
            ck_slot += list(sl)
            ck_cu.append(len(ck_pos))
    n_ck = len(ck_pos)
    n_slots, conv_elems = (0, 0) if conv_pool is None else conv_pool.shape
    need = front_end_workspace_size(N, T, n_ck)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib().kda_front_end(_ptr(x), _ptr(z_a), _ptr(z_b), _ptr(conv_w), _dtype_code(x), H, dk,
                               dv, K, float(g_min), _i32_array(cu), N, _ptr(win_in), _ptr(win_out),
                               _i32_array(ck_cu), _i32_array(ck_pos), _i32_array(ck_slot), n_ck,
                               _ptr(conv_pool), conv_elems, n_slots, _ptr(o["q"]), _ptr(o["k"]),
                               _ptr(o["v"]), _ptr(o["a"]), _ptr(o["beta"]), _ptr(workspace),
                               workspace.numel(), _stream(dev)))
    o["window"] = win_out
    return o


def front_end_step(x, z_a, z_b, conv_w, H, dk, dv, g_min, window, out=None):
    """One decode token per session; window [B,K-1,C] is shifted in place.
    Returns a dict with q, k, v, a, beta of shape (B, H, *)."""
    B, C = x.shape
    K = conv_w.shape[1]
    dev, dt = x.device, x.dtype
    for t, shp, nm in ((x, (B, C), "x"), (z_a, (B, H, dk), "z_a"), (z_b, (B, H), "z_b"),
                       (conv_w, (C, K), "conv_w")):
        _expect(t, shp, dt, nm, dev)
    if window is not None:
        _expect(window, (B, K - 1, C), dt, "window", dev)
    o = dict(out or {})
    for nm, shp in (("q", (B, H, dk)), ("k", (B, H, dk)), ("v", (B, H, dv)), ("a", (B, H, dk)),
                    ("beta", (B, H))):
        if o.get(nm) is None:
            o[nm] = torch.empty(shp, dtype=dt, device=dev)
        _expect(o[nm], shp, dt, nm, dev)
    _check(lib().kda_front_end_step(_ptr(x), _ptr(z_a), _ptr(z_b), _ptr(conv_w), _dtype_code(x), B,
                                    H, dk, dv, K, float(g_min), _ptr(window), _ptr(o["q"]),
                                    _ptr(o["k"]), _ptr(o["v"]), _ptr(o["a"]), _ptr(o["beta"]),
                                    _stream(dev)))
    return o


class RawInputRing:
    """Per-slot rings of raw draft inputs on the device (kda_ring_*): push one
    step for a batch of slots, window() oldest first in the (draft, B, H, D)
    layout verify_and_replay reads, reset at commit."""

    FIELDS = ("q", "k", "v", "a", "beta")

    def __init__(self, n_slots, capacity, H, dk, dv, dtype=torch.bfloat16, device="cuda"):
        self.n_slots, self.capacity, self.H, self.dk, self.dv = n_slots, capacity, H, dk, dv
        self.dtype, self.device = dtype, torch.device(device)
        shp = {"q": (H, dk), "k": (H, dk), "v": (H, dv), "a": (H, dk), "beta": (H,)}
        self.shapes = shp
        self.t = {f: torch.zeros((n_slots, capacity) + shp[f], dtype=dtype, device=self.device)
                  for f in self.FIELDS}
        self.count = torch.zeros(n_slots, dtype=torch.int32, device=self.device)
        self.device = self.count.device  # the concrete device ("cuda" -> "cuda:0")
        self.desc = KdaRing(*(t.data_ptr() for t in (self.t[f] for f in self.FIELDS)),
                            self.count.data_ptr(), n_slots, capacity, H, dk, dv,
                            _dtype_code(self.t["q"]))

    def push(self, slots, q, k, v, a, beta, err_flag=None):
        B = slots.numel()
        for t, f in zip((q, k, v, a, beta), self.FIELDS):
            _expect(t, (B,) + self.shapes[f], self.dtype, f, self.device)
        _expect(slots, (B,), torch.int32, "slots", self.device)
        _check(lib().kda_ring_push(ctypes.byref(self.desc), _ptr(slots), B, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(a), _ptr(beta), _ptr(err_flag), _stream(self.device)))

    def window(self, slots, out=None, err_flag=None):
        B = slots.numel()
        _expect(slots, (B,), torch.int32, "slots", self.device)
        o = dict(out or {})
        for f in self.FIELDS:
            shp = (self.capacity, B) + self.shapes[f]
            if o.get(f) is None:
                o[f] = torch.empty(shp, dtype=self.dtype, device=self.device)
            _expect(o[f], shp, self.dtype, f, self.device)
        if o.get("n_valid") is None:
            o["n_valid"] = torch.empty(B, dtype=torch.int32, device=self.device)
        _check(lib().kda_ring_window(ctypes.byref(self.desc), _ptr(slots), B, _ptr(o["q"]), _ptr(o["k"]),
                                     _ptr(o["v"]), _ptr(o["a"]), _ptr(o["beta"]), _ptr(o["n_valid"]),
                                     _ptr(err_flag), _stream(self.device)))
        return o

    def reset(self, slots, err_flag=None):
        _expect(slots, (slots.numel(),), torch.int32, "slots", self.device)
        _check(lib().kda_ring_reset(ctypes.byref(self.desc), _ptr(slots), slots.numel(), _ptr(err_flag),
                                    _stream(self.device)))
