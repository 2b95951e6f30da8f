"""Seeded synthetic inputs for the KDA hot path (shared by the tests, the
benchmark and the smoke check; holds none of the recurrence's arithmetic).

Every array is drawn with NumPy's PCG64 from a SeedSequence keyed by
(1000 + workload id, field, block), so one sequence or one decode step can be
regenerated on its own without drawing the whole workload.  Values are
returned as float32 arrays; for bfloat16 workloads each value is first rounded
to the nearest bfloat16 (ties to even), so a float32 -> bfloat16 cast on the
device is exact and the float64 oracle reads the very same numbers.

Input recipe (the pages fix the ranges; the distributions are the workload
descriptions'):
  q, k ~ N(0, 1) per element, then L2-normalised over the key dimension per
  (token, head); v ~ N(0, 1); a = g_min * sigmoid(z), z ~ N(0, 1), one value
  per key channel (the bounded log-decay in [g_min, 0] of the
  "【轻量化复刻大模型 / KIMI K3】Serve 模块交互式演示" page, §1.3);
  beta = sigmoid(z'), z' ~ N(0, 1), in [0, 1] (same section).

Front-end inputs (the layer's side of the recurrence): mixed q|k|v
projection rows x ~ N(0, 1), gate logits z_a, z_b ~ N(0, 1), depthwise
convolution weights ~ N(0, 0.5^2), carried convolution windows ~ N(0, 1).
"""

import concurrent.futures as cf
import math
import os

import numpy as np

# Field ids of the seed key.
_Q, _K, _V, _ZA, _ZB, _S0, _NACC, _LEN, _MIX, _GA, _GB, _CW, _WIN = range(13)

WORKLOADS = {
    0: "tiny recurrence: 1 seq, H=2, dk=dv=16, T=128, fp32, S0=0, chunk 16",
    1: "speculative replay: B=64, H=16, dk=dv=32, Tdraft=8, fp32, S0~N(0,0.1^2)",
    2: "batched decode: B=256, H=32, dk=dv=128, bf16 in, fp32 state~N(0,0.05^2), 64 steps",
    3: "single-sequence prefill: T=8192, H=32, dk=dv=128, bf16, S0=0, chunk 64, ckpt every 512",
    4: "varlen prefill: 16 seqs, len~logU[1024,32768], H=32, dk=dv=128, bf16, S0~N(0,0.1^2), ckpt every 4096 + tail",
}


def _rng(wid, field, block=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + wid, field, block])))


def round_to_bf16(x, inplace=False):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    With inplace=True a contiguous float32 input is overwritten (saves memory
    on the large workloads); otherwise the input is left untouched."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not inplace:
        x = x.copy()
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return x


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _fill(wid, block, field, out, dtype, g_min):
    """Draw one field of one block into the float32 array `out` (in place)."""
    _rng(wid, field, block).standard_normal(out=out, dtype=np.float32)
    if field in (_Q, _K):  # L2-normalise over the key dimension
        out /= np.sqrt(np.einsum("...i,...i->...", out, out))[..., None]
    elif field == _ZA:     # a = g_min * sigmoid(z)
        out[...] = np.float32(g_min) * _sigmoid(out)
    elif field == _ZB:     # beta = sigmoid(z)
        out[...] = _sigmoid(out)
    if dtype == "bf16":
        round_to_bf16(out, inplace=True)
    elif dtype != "fp32":
        raise ValueError("dtype must be 'bf16' or 'fp32'")


_FIELDS = (("q", _Q), ("k", _K), ("v", _V), ("a", _ZA), ("beta", _ZB))


def _shapes(lead, H, dk, dv):
    return {"q": lead + (H, dk), "k": lead + (H, dk), "v": lead + (H, dv), "a": lead + (H, dk),
            "beta": lead + (H,)}


def token_inputs(wid, block, shape_lead, H, dk, dv, dtype, g_min=-1.0):
    """q, k, a of shape shape_lead + (H, dk), v of shape shape_lead + (H, dv),
    beta of shape shape_lead + (H,), drawn from the streams of (wid, block)."""
    shp = _shapes(tuple(shape_lead), H, dk, dv)
    out = {n: np.empty(shp[n], dtype=np.float32) for n, _ in _FIELDS}
    jobs = [_pool().submit(_fill, wid, block, f, out[n], dtype, g_min) for n, f in _FIELDS]
    for j in jobs:
        j.result()
    return out


def state_normal(wid, block, shape, std):
    """Committed / resident fp32 state with N(0, std^2) entries."""
    x = _rng(wid, _S0, block).standard_normal(size=tuple(shape), dtype=np.float32)
    x *= np.float32(std)
    return x


# ---------------------------------------------------------------------------
# Prefill workloads (token-packed, cu_seqlens).
# ---------------------------------------------------------------------------
def prefill_lengths(wid, n_seqs=16, lo=1024, hi=32768):
    """Sequence lengths log-uniform in [lo, hi] (workload 4)."""
    u = _rng(wid, _LEN).random(n_seqs)
    return [int(round(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]


def prefill_checkpoints(lengths, every, tail=True):
    """Per sequence: positions every*m < len, plus len itself when tail=True
    (every*m <= len when tail=False)."""
    out = []
    for L in lengths:
        pos = list(range(every, L, every)) if tail else list(range(every, L + 1, every))
        if tail and L > 0:
            pos.append(L)
        out.append(sorted(set(pos)))
    return out


def prefill_workload(wid, lengths, H, dk, dv, dtype, s0_std=None, ckpt_every=None,
                     ckpt_tail=True, g_min=-1.0):
    """A full token-packed prefill batch.  Sequence n draws from block n; the
    fields of all sequences are drawn in parallel, straight into place."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    shp = _shapes((T,), H, dk, dv)
    out = {n: np.empty(shp[n], dtype=np.float32) for n, _ in _FIELDS}
    jobs = []
    for n, L in enumerate(lengths):
        if L == 0:
            continue
        lo, hi = int(cu[n]), int(cu[n + 1])
        jobs += [_pool().submit(_fill, wid, n, f, out[name][lo:hi], dtype, g_min)
                 for name, f in _FIELDS]
    for j in jobs:
        j.result()
    out["cu_seqlens"] = cu
    out["s0"] = None if s0_std is None else np.stack(
        [state_normal(wid, n, (H, dk, dv), s0_std) for n in range(len(lengths))])
    out["checkpoints"] = (None if ckpt_every is None
                          else prefill_checkpoints(lengths, ckpt_every, ckpt_tail))
    out["lengths"] = list(lengths)
    return out


def sequence_slice(wid, n, L, H, dk, dv, dtype, s0_std=None, g_min=-1.0):
    """Regenerate sequence n of a prefill workload alone (for sampled checks)."""
    t = token_inputs(wid, n, (L,), H, dk, dv, dtype, g_min)
    t["s0"] = None if s0_std is None else state_normal(wid, n, (H, dk, dv), s0_std)
    return t


def workload0():
    return prefill_workload(0, [128], H=2, dk=16, dv=16, dtype="fp32")


def workload3():
    return prefill_workload(3, [8192], H=32, dk=128, dv=128, dtype="bf16",
                            ckpt_every=512, ckpt_tail=False)


def workload4():
    return prefill_workload(4, prefill_lengths(4), H=32, dk=128, dv=128, dtype="bf16",
                            s0_std=0.1, ckpt_every=4096, ckpt_tail=True)


# ---------------------------------------------------------------------------
# Replay workload: projections in (draft, B, H, D) layout.
# ---------------------------------------------------------------------------
def replay_workload(wid=1, B=64, H=16, dk=32, dv=32, t_draft=8, dtype="fp32", s0_std=0.1):
    t = token_inputs(wid, 0, (t_draft, B), H, dk, dv, dtype)
    t["committed"] = state_normal(wid, 0, (B, H, dk, dv), s0_std)
    t["n_accepted"] = _rng(wid, _NACC).integers(0, t_draft + 1, size=B).astype(np.int32)
    return t


# ---------------------------------------------------------------------------
# Decode workload: one token per session per step; step s draws from block s.
# ---------------------------------------------------------------------------
def decode_state(wid=2, B=256, H=32, dk=128, dv=128, std=0.05):
    return state_normal(wid, 0, (B, H, dk, dv), std)


def decode_step_inputs(step, wid=2, B=256, H=32, dk=128, dv=128, dtype="bf16"):
    return token_inputs(wid, step, (B,), H, dk, dv, dtype)


def front_end_inputs(wid, lengths, H, dk, dv, K, dtype, windows=True):
    """Front-end inputs of a token-packed batch: x [T, H*(2dk+dv)] mixed
    projection rows, z_a [T, H, dk], z_b [T, H], conv_w [C, K] and, with
    windows=True, carried windows [N, K-1, C] (None otherwise)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    C = H * (2 * dk + dv)

    def draw(field, shape, scale=1.0, block=0):
        x = _rng(wid, field, block).standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        return round_to_bf16(x, inplace=True) if dtype == "bf16" else x

    return {"x": draw(_MIX, (T, C)), "z_a": draw(_GA, (T, H, dk)), "z_b": draw(_GB, (T, H)),
            "conv_w": draw(_CW, (C, K), 0.5),
            "windows": draw(_WIN, (len(lengths), K - 1, C)) if windows else None,
            "cu_seqlens": cu}
