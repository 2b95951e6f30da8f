"""Tolerances of the GPU-vs-oracle parity tests.

fp32 inputs and outputs: max |got - want| <= 1e-4 * max |want| (outputs and
states).  bf16 inputs with an fp32 state: relative Frobenius error
||got - want|| / ||want|| <= 1e-2.  The oracle always reads the inputs exactly
as the GPU does (bf16 values rounded once by the input generator).
"""
import numpy as np
import torch

FP32_MAXABS_REL = 1e-4
BF16_FROB_REL = 1e-2


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def max_abs_rel(got, want):
    got, want = to_np(got), to_np(want)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / scale) if scale > 0 else float(np.max(np.abs(got)))


def frob_rel(got, want):
    got, want = to_np(got), to_np(want)
    n = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / n) if n > 0 else float(np.linalg.norm(got))


def assert_parity(got, want, dtype, what=""):
    if dtype == "fp32":
        e = max_abs_rel(got, want)
        assert e <= FP32_MAXABS_REL, f"{what}: max-abs error {e:.3e} x max|want| > {FP32_MAXABS_REL}"
    else:
        e = frob_rel(got, want)
        assert e <= BF16_FROB_REL, f"{what}: relative Frobenius error {e:.3e} > {BF16_FROB_REL}"
    return e


def dev_tensor(x, dtype, device="cuda"):
    """float32 numpy -> device tensor of the run dtype ("fp32" or "bf16"; exact for
    values the input generator already rounded to bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


def assert_parity_blocks(got, want, dtype, block, what=""):
    """The bar applied to every run of `block` rows (the first axis) on its own,
    so that an error confined to one chunk cannot hide in a long sequence's
    norm.  A tail shorter than half a block joins the block before it (a
    relative Frobenius error over a handful of rows measures the rounding of
    those rows, not the kernel: single output rows of the bf16 path differ
    from the float64 oracle by up to about 2 %, the same on every chunk
    size).  Returns the largest per-block error."""
    got, want = to_np(got), to_np(want)
    n = want.shape[0]
    starts = list(range(0, n, block))
    if len(starts) > 1 and n - starts[-1] < block // 2:
        starts.pop()
    worst = 0.0
    for i, r in enumerate(starts):
        e = starts[i + 1] if i + 1 < len(starts) else n
        worst = max(worst, assert_parity(got[r:e], want[r:e], dtype, f"{what} rows {r}..{e - 1}"))
    return worst
