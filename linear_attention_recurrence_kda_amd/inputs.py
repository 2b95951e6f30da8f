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
"""

import math

import numpy as np

# Field ids of the seed key.
_Q, _K, _V, _ZA, _ZB, _S0, _NACC, _LEN = range(8)

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


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2_normalise(x):
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))
    x /= n[..., None]
    return x


def _sigmoid(z):
    return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)


def token_inputs(wid, block, shape_lead, H, dk, dv, dtype, g_min=-1.0):
    """q, k, a of shape shape_lead + (H, dk), v of shape shape_lead + (H, dv),
    beta of shape shape_lead + (H,), drawn from the streams of (wid, block)."""
    lead = tuple(shape_lead)
    q = _l2_normalise(_normal(_rng(wid, _Q, block), lead + (H, dk)))
    k = _l2_normalise(_normal(_rng(wid, _K, block), lead + (H, dk)))
    v = _normal(_rng(wid, _V, block), lead + (H, dv))
    a = (g_min * _sigmoid(_normal(_rng(wid, _ZA, block), lead + (H, dk)))).astype(np.float32)
    beta = _sigmoid(_normal(_rng(wid, _ZB, block), lead + (H,)))
    out = {"q": q, "k": k, "v": v, "a": a, "beta": beta}
    if dtype == "bf16":
        out = {n: round_to_bf16(x, inplace=True) for n, x in out.items()}
    elif dtype != "fp32":
        raise ValueError("dtype must be 'bf16' or 'fp32'")
    return out


def state_normal(wid, block, shape, std):
    """Committed / resident fp32 state with N(0, std^2) entries."""
    return (std * _normal(_rng(wid, _S0, block), tuple(shape))).astype(np.float32)


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
    """A full token-packed prefill batch.  Sequence n draws from block n."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    fields = {n: [] for n in ("q", "k", "v", "a", "beta")}
    for n, L in enumerate(lengths):
        t = token_inputs(wid, n, (L,), H, dk, dv, dtype, g_min)
        for f in fields:
            fields[f].append(t[f])
    out = {f: np.concatenate(x, axis=0) for f, x in fields.items()}
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
