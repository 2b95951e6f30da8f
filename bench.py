#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

A timed step is one pass of the prefill path over the variable-length
workload (16 sequences with log-uniform lengths in [1024, 32768], H=32,
dk=dv=128, bf16 inputs, fp32 states from nonzero committed S0, 32-token
chunks (the fused kernel), checkpoints at every 4096 tokens plus the exact
tail written into page slots) followed by packing the 16 final states into
page slots.  `value` is that step's whole-job throughput in tokens/s with
inputs resident in HBM.  Outside the timed steps, that part also reports
("settled") the same calls timed again after --settled more untimed ones:
after idle time the GPU's clocks ramp over the first twenty or so calls.

In the same run, and reported under "parts": the same varlen prefill on the
two-kernel path at chunk 64, the single-sequence prefill (T=8192, chunk 64,
checkpoints every 512), the same sequence as 8 segments through
segment summaries, composition and per-segment prefill (context-parallel
prefill on one GPU), the front end (convolution, SiLU, L2Norm, gates) over the
varlen workload's sequences, 64 in-place decode steps (B=256 sessions),
verify-and-replay (B=64, H=16, d=32, 8 drafts), one speculative round's
rollback through the raw-input ring against full state snapshots, and
pack/unpack of the
decode batch's 256 states (537 MB, past the 256 MB Infinity Cache), each
with its algorithmic bytes or flops against the MI355X peaks, plus the
float64 CPU oracle timed on a bounded sample on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only a,b] [--no-cpu] [--settled N]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (MFMA %) + decode/replay state GB/s (HBM %), H=32 d=128"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_recurrence_kda_amd", "csrc")
# The prefill kernels' sources (a traffic figure is stamped with their hash).
PREFILL_SRC = [os.path.join(CSRC, f) for f in
               ("kda_prefill_kernels.hpp", "kda_prefill.hip", "kda_prefill_slab.hpp", "kda_slab.hip")]
# (the fused path: its kernel, the correction of split sequences, and the
# host plan that decides the split and the tile widths)
FUSED_SRC = [os.path.join(CSRC, f) for f in ("kda_prefill_kernels.hpp", "kda_prefill_slab.hpp", "kda_fused.hip",
                                             "kda_cp.hpp", "kda_api_prefill.cpp")]
HEAD_CHUNK = 32  # the headline prefill's chunk (the fused kernel)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work counts
def prefill_flops(tokens, H, dk, dv, C):
    """Algorithmic flops of the WY chunk form per token-head (dense tiles):
    Gram products 4C*dk, W 2C*dk, Ut 2C*dv, U, QS and state update 6*dk*dv,
    A_qk U 2C*dv, triangular inverse C^2/3.  (The kernels apply T to the
    residual and skip W, so they execute 2C*dk fewer; the count is kept as the
    fixed yardstick.)"""
    return tokens * H * (6 * C * dk + 4 * C * dv + 6 * dk * dv + C * C / 3.0)


def prefill_bytes(tokens, H, dk, dv, n_seqs, n_ckpt, in_bytes=2, s0=True, final=True):
    """Compulsory HBM bytes: q, k, a, v, beta read and o written once, S0
    read, checkpoints and final states written (fp32)."""
    state = H * dk * dv * 4
    b = tokens * H * ((3 * dk + dv + 1) * in_bytes + dv * in_bytes)
    b += n_ckpt * state + (n_seqs * state if s0 else 0) + (n_seqs * state if final else 0)
    return b


def segment_flops(tokens, H, dk, dv, C):
    """Algorithmic flops of the segment summaries per token-head: the k Gram
    product 2C*dk and the triangular inverse C^2/3 (per chunk, shared by both
    maps), then for each of the dv columns of B and the dk columns of A:
    Z = V - (k g) S (2 dk), U = T Z (2C) and the state update (2 dk)."""
    return tokens * H * (2 * C * dk + C * C / 3.0 + (dv + dk) * (4 * dk + 2 * C))


def front_end_bytes(T, H, dk, dv, K, n_seqs, n_windows_out, in_bytes=2):
    """Compulsory bytes of the front end: x, z_a, z_b, the weights and the
    carried windows read once; q, k, v, a, beta and the windows written once."""
    C = H * (2 * dk + dv)
    read = T * C + T * H * dk + T * H + C * K + n_seqs * (K - 1) * C
    write = T * H * (3 * dk + dv + 1) + n_windows_out * (K - 1) * C
    return (read + write) * in_bytes


def decode_bytes(B, H, dk, dv, in_bytes=2, state_bytes=4):
    return (2 * B * H * dk * dv * state_bytes + B * H * (3 * dk + dv + 1) * in_bytes
            + B * H * dv * in_bytes)


def replay_bytes(B, H, dk, dv, t_draft, n_acc, in_bytes=4, state_bytes=4):
    return (2 * B * H * dk * dv * state_bytes + int(np.sum(n_acc)) * H * (3 * dk + dv + 1) * in_bytes
            + B * H * t_draft * dv * in_bytes)


# ---------------------------------------------------------------- helpers
class Timer:
    """Wall clock around K steps plus HIP events around one kernel call per
    step, all on torch's current stream (the stream the library launches on)."""

    def __init__(self, torch, steps):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]

    def kernel_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.ev]))


def run_steps(torch, fn, steps, warmup, kernel_fn=None):
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    t0 = time.perf_counter()
    for i in range(steps):
        fn(tm.ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps * 1e3, tm.kernel_ms()


def src_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(name, kernel_src):
    """HBM bytes per launch from a committed rocprofv3 counter summary, valid
    only while the kernel source is unchanged (else None)."""
    p = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_src_sha256_16") != src_hash(kernel_src):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- parts
def bench_prefill(torch, kda, inputs, w, steps, warmup, pack_final, label, gate=False, chunk=64, settled=0):
    d = {n: torch.from_numpy(w[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "a", "beta")}
    g_min = None
    if gate:
        # Gate logits in place of a and beta (z ~ N(0, 1), the distribution a
        # and beta were drawn from), applied inside the prefill.
        g = torch.Generator(device="cuda").manual_seed(6)
        for n in ("a", "beta"):
            d[n] = torch.randn(d[n].shape, generator=g, device="cuda").to(torch.bfloat16)
        g_min = -1.0
    H, dk = w["k"].shape[1:]
    dv = w["v"].shape[2]
    cu = w["cu_seqlens"]
    N = len(cu) - 1
    T = int(cu[-1])
    s0 = None if w["s0"] is None else torch.from_numpy(w["s0"]).cuda()
    ck = w["checkpoints"]
    n_ck = sum(len(c) for c in ck)
    slots, i = [], 0
    for c in ck:
        slots.append(list(range(i, i + len(c))))
        i += len(c)
    page = H * dk * dv
    pool = torch.zeros((n_ck + N, page), dtype=torch.float32, device="cuda")
    final_slots = torch.arange(n_ck, n_ck + N, dtype=torch.int32, device="cuda")
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.prefill_workspace_size(N, T, H, dk, dv, chunk, n_ck), dtype=torch.uint8,
                     device="cuda")
    _, kernels = kda.prefill_plan(cu, H, dk, dv, chunk, ck)

    def step(ev):
        if ev is not None:
            ev[0].record()
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], cu, s0=s0, chunk=chunk,
                          checkpoints=ck, ckpt_slots=slots, page_pool=pool, o=o, s_final=sf,
                          workspace=ws, gate_g_min=g_min)
        if ev is not None:
            ev[1].record()
        if pack_final:
            kda.pack_heads(sf, final_slots, pool)

    ms, kms = run_steps(torch, step, steps, warmup)
    flops = prefill_flops(T, H, dk, dv, chunk)
    byts = prefill_bytes(T, H, dk, dv, N, n_ck, s0=s0 is not None)
    # (informational, outside the timed steps: the same call again after
    # `settled` more untimed calls, once the clocks have left their ramp)
    settled_res = None
    if settled > 0:
        _, kms2 = run_steps(torch, step, steps, settled)
        settled_res = {"after_calls": warmup + steps + settled, "kernel_ms": kms2,
                       "hbm_frac": byts / (kms2 * 1e-3) / 1e9 / HBM_PEAK_GBS}
    res = {
        "workload": label, "kernels": kernels, "chunk": chunk, "tokens": T, "n_seqs": N, "n_ckpt": n_ck,
        "ms_per_step": ms, "kernel_ms": kms,
        "tokens_per_s": T / (ms * 1e-3),
        "kernel_tokens_per_s": T / (kms * 1e-3),
        "algo_gflop": flops / 1e9, "algo_gbytes": byts / 1e9,
        "mfma_tflops": flops / (kms * 1e-3) / 1e12,
        "mfma_frac": flops / (kms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "hbm_gbs": byts / (kms * 1e-3) / 1e9,
        "hbm_frac": byts / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    # roofline: min(peak MFMA, I * BW) with I = flops / bytes
    t_roof = max(flops / (BF16_PEAK_TFLOPS * 1e12), byts / (HBM_PEAK_GBS * 1e9))
    res["roofline_frac"] = t_roof / (kms * 1e-3)
    if settled_res is not None:
        res["settled"] = settled_res
    del d, pool, o, sf, ws
    return res


def bench_segments(torch, kda, inputs, w, steps, warmup, n_seg=8, decay="g_min=-1"):
    """Context-parallel prefill of one long sequence on one GPU: the sequence
    cut into n_seg equal segments (the shares of n_seg ranks), then segment
    summaries, their composition into start states, and the prefill of every
    segment from its start (with the one-pass run's checkpoints, shifted into
    segment coordinates).  The one-pass prefill is timed beside it."""
    d = {n: torch.from_numpy(w[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "a", "beta")}
    H, dk = w["k"].shape[1:]
    dv = w["v"].shape[2]
    T = int(w["cu_seqlens"][-1])
    L = T // n_seg
    cut = [i * L for i in range(n_seg)] + [T]
    ck_all = w["checkpoints"][0]
    ck = [[p - cut[i] for p in ck_all if cut[i] < p <= cut[i + 1]] for i in range(n_seg)]
    n_ck = len(ck_all)
    slots, j = [], 0
    for c in ck:
        slots.append(list(range(j, j + len(c))))
        j += len(c)
    pool = torch.zeros((n_ck, H * dk * dv), dtype=torch.float32, device="cuda")
    A = torch.empty((n_seg, H, dk, dk), dtype=torch.float32, device="cuda")
    B = torch.empty((n_seg, H, dk, dv), dtype=torch.float32, device="cuda")
    starts = torch.empty((n_seg, H, dk, dv), dtype=torch.float32, device="cuda")
    s_end = torch.empty((H, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((n_seg, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kda.segment_summary_workspace_size(n_seg, T, H, dk, dv, 64),
                         kda.prefill_workspace_size(n_seg, T, H, dk, dv, 64, n_ck),
                         kda.prefill_workspace_size(1, T, H, dk, dv, 64, n_ck)),
                     dtype=torch.uint8, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(e):
        if e is not None:
            e[0].record()
        kda.segment_summary(d["k"], d["v"], d["a"], d["beta"], cut, chunk=64, A=A, B=B, workspace=ws)
        if e is not None:
            e[1].record()
        kda.compose_segments(A, B, None, starts=starts, s_end=s_end)
        if e is not None:
            e[2].record()
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], cut, s0=starts, chunk=64,
                          checkpoints=ck, ckpt_slots=slots, page_pool=pool, o=o, s_final=sf,
                          workspace=ws)
        if e is not None:
            e[3].record()

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    ph = np.mean([[e[k].elapsed_time(e[k + 1]) for k in range(3)] for e in ev], axis=0)

    o1 = torch.empty_like(o)
    sf1 = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")

    def one_pass(e):
        if e is not None:
            e[0].record()
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["a"], d["beta"], [0, T], chunk=64,
                          checkpoints=[ck_all], ckpt_slots=[list(range(n_ck))], page_pool=pool,
                          o=o1, s_final=sf1, workspace=ws)
        if e is not None:
            e[1].record()

    _, ms1 = run_steps(torch, one_pass, steps, warmup)
    # Agreement of the two paths on this workload (relative Frobenius).
    rel = lambda x, y: float(torch.linalg.vector_norm((x - y).float()) / torch.linalg.vector_norm(y.float()))
    flops = segment_flops(T, H, dk, dv, 64)
    summ_ms = float(ph[0])
    res = {"workload": f"context-parallel prefill on one GPU: T={T} (one sequence) in {n_seg} "
                       f"segments of {L}, H={H}, dk=dv={dk}, bf16, S0=0, chunk 64, "
                       f"ckpt every 512, {decay}",
           "ms_per_step": ms, "summary_ms": summ_ms, "compose_ms": float(ph[1]),
           "rerun_ms": float(ph[2]), "one_pass_kernel_ms": ms1,
           "tokens_per_s": T / (ms * 1e-3), "one_pass_tokens_per_s": T / (ms1 * 1e-3),
           "summary_algo_gflop": flops / 1e9,
           "summary_mfma_tflops": flops / (summ_ms * 1e-3) / 1e12,
           "summary_mfma_frac": flops / (summ_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
           "o_rel_vs_one_pass": rel(o, o1), "s_end_rel_vs_one_pass": rel(s_end, sf1[0])}
    del d, pool, A, B, starts, o, o1, sf, ws
    return res


def bench_front_end(torch, kda, inputs, steps, warmup):
    """The front end over the varlen workload's sequences (16 sequences,
    108,886 tokens, H=32, dk=dv=128, K=4, bf16), carried windows in, end
    windows out and the windows of the same checkpoints as the prefill into a
    window pool.  Inputs are drawn on the device from a seeded generator."""
    lengths = inputs.prefill_lengths(4)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T, N = int(cu[-1]), len(lengths)
    H, dk, dv, K = 32, 128, 128, 4
    C = H * (2 * dk + dv)
    g = torch.Generator(device="cuda").manual_seed(5)
    bf = torch.bfloat16
    rnd = lambda *shape: torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(bf)
    x, z_a, z_b = rnd(T, C), rnd(T, H, dk), rnd(T, H)
    w = (rnd(C, K).float() * 0.5).to(bf)
    win = rnd(N, K - 1, C)
    ck = inputs.prefill_checkpoints(lengths, 4096, True)
    n_ck = sum(len(c) for c in ck)
    slots, i = [], 0
    for c in ck:
        slots.append(list(range(i, i + len(c))))
        i += len(c)
    pool = torch.zeros((n_ck, (K - 1) * C), dtype=bf, device="cuda")
    out = {"q": torch.empty((T, H, dk), dtype=bf, device="cuda"),
           "k": torch.empty((T, H, dk), dtype=bf, device="cuda"),
           "v": torch.empty((T, H, dv), dtype=bf, device="cuda"),
           "a": torch.empty((T, H, dk), dtype=bf, device="cuda"),
           "beta": torch.empty((T, H), dtype=bf, device="cuda"),
           "window": torch.empty((N, K - 1, C), dtype=bf, device="cuda")}
    ws = torch.empty(kda.front_end_workspace_size(N, T, n_ck), dtype=torch.uint8, device="cuda")

    def step(ev):
        if ev is not None:
            ev[0].record()
        kda.front_end(x, z_a, z_b, w, H, dk, dv, -1.0, cu, win_in=win, checkpoints=ck,
                      ckpt_slots=slots, conv_pool=pool, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    ms, kms = run_steps(torch, step, steps, warmup)
    byts = front_end_bytes(T, H, dk, dv, K, N, N + n_ck)
    res = {"workload": f"front end: 16 seqs ({T} tokens, the varlen prefill's lengths), H=32, "
                       f"dk=dv=128, K=4, bf16, windows carried in and out, {n_ck} checkpoint windows",
           "tokens": T, "ms_per_step": ms, "kernel_ms": kms, "tokens_per_s": T / (kms * 1e-3),
           "algo_gbytes": byts / 1e9, "hbm_gbs": byts / (kms * 1e-3) / 1e9,
           "hbm_frac": byts / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del x, z_a, z_b, w, win, pool, out, ws
    return res


def bench_ring(torch, kda, inputs, steps, warmup):
    """Rollback machinery of one speculative round at the large replay shape
    (B=256, H=32, dk=dv=128, 8 draft steps, bf16 inputs, fp32 states, ragged
    acceptance).  Route B, the raw-input ring: one push per draft step, then
    window, verify-and-replay of the accepted prefix and reset.  Route A, full
    snapshots: the state packed into a snapshot slot after every draft step,
    then the accepted one unpacked.  The verification forward that produces
    the per-step states is the same for both and is not part of either."""
    w = inputs.replay_workload(wid=11, B=256, H=32, dk=128, dv=128, t_draft=8, dtype="bf16")
    Td, B, H, dk = w["q"].shape
    dv = w["v"].shape[-1]
    bf = torch.bfloat16
    d = {f: torch.from_numpy(w[f]).to(bf).cuda() for f in ("q", "k", "v", "a", "beta")}
    steps_in = [{f: d[f][t].contiguous() for f in d} for t in range(Td)]
    committed = torch.from_numpy(w["committed"]).cuda()
    n = torch.from_numpy(w["n_accepted"]).cuda()
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    ring = kda.RawInputRing(B, Td, H, dk, dv, bf)
    win = {f: torch.empty((Td,) + tuple(d[f].shape[1:]), dtype=bf, device="cuda") for f in d}
    win["n_valid"] = torch.empty(B, dtype=torch.int32, device="cuda")
    s_new = torch.empty_like(committed)
    o = torch.empty((B, H, Td, dv), dtype=bf, device="cuda")

    def route_b(ev):
        if ev is not None:
            ev[0].record()
        for st in steps_in:
            ring.push(slots, st["q"], st["k"], st["v"], st["a"], st["beta"])
        ring.window(slots, out=win)
        kda.verify_and_replay(committed, win["q"], win["k"], win["v"], win["a"], win["beta"], n,
                              s_new, o)
        ring.reset(slots)
        if ev is not None:
            ev[1].record()

    page = H * dk * dv
    pool = torch.empty((B * Td, page), dtype=torch.float32, device="cuda")
    snap_slots = [torch.arange(B, dtype=torch.int32, device="cuda") * Td + t for t in range(Td)]
    keep = (torch.arange(B, device="cuda") * Td + (n.long() - 1).clamp(min=0)).to(torch.int32)
    restored = torch.empty_like(committed)

    def route_a(ev):
        if ev is not None:
            ev[0].record()
        for t in range(Td):
            kda.pack_heads(committed, snap_slots[t], pool)  # the state after step t (same bytes)
        kda.unpack_heads(pool, keep, H, dk, dv, state=restored)
        if ev is not None:
            ev[1].record()

    _, ms_b = run_steps(torch, route_b, steps, warmup)
    _, ms_a = run_steps(torch, route_a, steps, warmup)
    n_sum = int(np.sum(w["n_accepted"]))
    proj = B * H * (3 * dk + dv + 1) * 2       # one step's raw inputs, bf16
    state = B * H * dk * dv * 4                # all sessions' states, fp32
    bytes_b = Td * 2 * proj + 2 * Td * proj + replay_bytes(B, H, dk, dv, Td, w["n_accepted"], 2)
    bytes_a = Td * 2 * state + 2 * state
    res = {"workload": "speculative round: B=256, H=32, dk=dv=128, 8 draft steps, bf16 inputs, "
                       f"fp32 states, {n_sum} accepted steps in all",
           "route_b_ring_ms": ms_b, "route_a_snapshot_ms": ms_a, "time_ratio_a_over_b": ms_a / ms_b,
           "route_b_gbytes": bytes_b / 1e9, "route_a_gbytes": bytes_a / 1e9,
           "bytes_ratio_a_over_b": bytes_a / bytes_b,
           "per_step_bytes_ratio": kda.snapshot_cost_ratio(H, dk, dv) * 4 / 2,
           "route_b_hbm_gbs": bytes_b / (ms_b * 1e-3) / 1e9,
           "route_a_hbm_gbs": bytes_a / (ms_a * 1e-3) / 1e9}
    del d, steps_in, committed, ring, win, s_new, o, pool, restored
    return res


def bench_decode(torch, kda, inputs, steps, warmup, state_dtype="fp32"):
    B, H, dk, dv, n_tok = 256, 32, 128, 128, 64
    state = torch.from_numpy(inputs.decode_state(2, B, H, dk, dv, 0.05)).cuda()
    sb = 4
    if state_dtype == "bf16":
        state = state.to(torch.bfloat16)
        sb = 2
    toks = []
    for s in range(n_tok):
        t = inputs.decode_step_inputs(s, 2, B, H, dk, dv, "bf16")
        toks.append({n: torch.from_numpy(x).to(torch.bfloat16).cuda() for n, x in t.items()})
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")

    # One timed step = the 64 in-place decode steps; events bracket the 64 launches.
    def step(ev):
        if ev is not None:
            ev[0].record()
        for t in toks:
            kda.decode_step(t["q"], t["k"], t["v"], t["a"], t["beta"], state, o)
        if ev is not None:
            ev[1].record()

    ms, kms = run_steps(torch, step, max(2, steps // 2), max(1, warmup // 2))
    per_launch_ms = kms / n_tok
    byts = decode_bytes(B, H, dk, dv, 2, sb)
    res = {"workload": f"decode: B=256, H=32, dk=dv=128, bf16 in, {state_dtype} state, 64 in-place steps",
           "us_per_decode_step": per_launch_ms * 1e3, "algo_gbytes_per_step": byts / 1e9,
           "hbm_gbs": byts / (per_launch_ms * 1e-3) / 1e9,
           "hbm_frac": byts / (per_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "tokens_per_s": B / (per_launch_ms * 1e-3)}
    del state, toks
    return res


def bench_replay(torch, kda, inputs, steps, warmup, shape="pages", state_dtype="fp32"):
    if shape == "pages":
        w = inputs.replay_workload()
        dt, tdt, label = "fp32", torch.float32, "replay: B=64, H=16, dk=dv=32, 8 drafts, fp32"
    else:
        w = inputs.replay_workload(wid=11, B=256, H=32, dk=128, dv=128, t_draft=8, dtype="bf16")
        dt, tdt, label = "bf16", torch.bfloat16, "replay: B=256, H=32, dk=dv=128, 8 drafts, bf16"
    d = {n: torch.from_numpy(w[n]).to(tdt).cuda() for n in ("q", "k", "v", "a", "beta")}
    committed = torch.from_numpy(w["committed"]).cuda()
    sb = 4
    if state_dtype == "bf16":
        committed = committed.to(torch.bfloat16)
        sb = 2
        label += ", bf16 state"
    n = torch.from_numpy(w["n_accepted"]).cuda()
    s_new = torch.empty_like(committed)
    Td, B, H, dk = w["q"].shape
    dv = w["v"].shape[-1]
    o = torch.empty((B, H, Td, dv), dtype=tdt, device="cuda")

    reps = 20  # back-to-back calls between one event pair

    def step(ev):
        if ev is not None:
            ev[0].record()
        for _ in range(reps):
            kda.verify_and_replay(committed, d["q"], d["k"], d["v"], d["a"], d["beta"], n, s_new, o)
        if ev is not None:
            ev[1].record()

    ms, kms = run_steps(torch, step, steps, warmup)
    kms /= reps
    byts = replay_bytes(B, H, dk, dv, Td, w["n_accepted"], 4 if dt == "fp32" else 2, sb)
    return {"workload": label, "us_per_call": kms * 1e3, "algo_mbytes": byts / 1e6,
            "hbm_gbs": byts / (kms * 1e-3) / 1e9,
            "hbm_frac": byts / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_pack(torch, kda, steps, warmup):
    """Pack the decode batch's 256 fp32 states (H=32, dk=dv=128: 537 MB, past
    the 256 MB Infinity Cache) into 256 page slots in a shuffled order, and
    unpack them back, timed apart."""
    B, H, d = 256, 32, 128
    g = torch.Generator(device="cuda").manual_seed(3)
    state = torch.randn((B, H, d, d), device="cuda", generator=g)
    pool = torch.zeros((B, H * d * d), device="cuda")
    slots = torch.randperm(B, generator=g, device="cuda").to(torch.int32)
    back = torch.empty_like(state)
    ev_p = Timer(torch, steps)
    ev_u = Timer(torch, steps)
    for i in range(warmup + steps):
        j = i - warmup
        if j >= 0:
            ev_p.ev[j][0].record()
        kda.pack_heads(state, slots, pool)
        if j >= 0:
            ev_p.ev[j][1].record()
            ev_u.ev[j][0].record()
        kda.unpack_heads(pool, slots, H, d, d, state=back)
        if j >= 0:
            ev_u.ev[j][1].record()
    torch.cuda.synchronize()
    assert torch.equal(back, state)
    byts = 2 * B * H * d * d * 4  # one pass reads and writes 256 states
    res = {"workload": "pack / unpack: 256 states of H=32, dk=dv=128 fp32 (537 MB) into 2 MiB page slots, "
                       "shuffled slot order"}
    for name, t in (("pack", ev_p), ("unpack", ev_u)):
        ms = t.kernel_ms()
        res[name] = {"us": ms * 1e3, "hbm_gbs": byts / (ms * 1e-3) / 1e9,
                     "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del state, pool, back
    return res


def copy_calibration(torch):
    """A plain 1 GiB device copy of known size (the scale for HBM counters)."""
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    y.copy_(x)
    torch.cuda.synchronize()
    return {"bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}


_CPU_W = None  # the workload the baseline's worker processes read (inherited by fork)


def _oracle_unit(u):
    """One unit of the CPU baseline: the float64 oracle, untouched, over the
    first L tokens of sequence n for heads h0 .. h0 + HG - 1, on one thread."""
    import oracle
    from threadpoolctl import threadpool_limits

    n, h0, L, HG = u
    w = _CPU_W
    lo = int(w["cu_seqlens"][n])
    hi = min(int(w["cu_seqlens"][n + 1]), lo + L)
    sl = [w[f][lo:hi, h0:h0 + HG] for f in ("q", "k", "v", "a", "beta")]
    with threadpool_limits(1):
        oracle.kda_recurrent(*sl, w["s0"][n, h0:h0 + HG])
    return (hi - lo) * HG


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, L=2048, HG=8):
    """The float64 oracle on a bounded sample of the varlen workload: the first
    L tokens of each of its 16 sequences, all 32 heads, as (sequence, group
    of HG heads) units over the host's cores (one forked process per core, one
    thread each; at most 16, the host share of one GPU).  The value is the
    sample's token-heads per second over the wall time, divided by H: tokens
    per second of the whole-head workload.  Runs before the GPU is touched."""
    import multiprocessing as mp

    global _CPU_W
    _CPU_W = w
    cores = min(len(os.sched_getaffinity(0)), 16)
    H = w["q"].shape[1]
    units = [(n, h0, L, HG) for n in range(len(w["cu_seqlens"]) - 1) for h0 in range(0, H, HG)]
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_oracle_unit, [(0, 0, 2, 1)] * cores)  # worker start-up and imports, untimed
        t0 = time.perf_counter()
        token_heads = sum(pool.map(_oracle_unit, units, chunksize=1))
        dt = time.perf_counter() - t0
    _CPU_W = None
    return {"value": token_heads / H / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"float64 oracle kda_recurrent over the first {L} tokens of each of the "
                      f"{len(w['cu_seqlens']) - 1} sequences of the same workload, all {H} heads "
                      f"(dk=dv=128), as {len(units)} (sequence, {HG}-head) units on {cores} processes; "
                      f"{token_heads / H:.0f} tokens in {dt:.1f} s wall, {dt * cores:.0f} core-s"}


def write_traffic(fetch_csv, write_csv, name="prefill_varlen"):
    """Turn two rocprofv3 counter passes into a traffic figure.

    fetch_csv / write_csv: counter_collection CSVs of a FETCH_SIZE pass and a
    WRITE_SIZE pass (KiB per dispatch) over `bench.py --only prefill4,copycal
    --steps 1 --warmup 0 --no-cpu` (name prefill_varlen: the bytes of one
    prefill call, its kernel dispatches summed) or `--only pack,copycal`
    (name pack: the bytes of each pack / unpack dispatch).  The calibration
    copy of that run (torch's copy of 1 GiB, the runtime's copyBuffer kernel)
    scales the counters to bytes.
    Writes profiles/<name>_traffic.json, stamped with the kernel source hash."""
    import csv

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    # (torch's device-to-device copy runs as the HIP runtime's blit kernel)
    f_cp = max(v for k, vals in fetch.items() if "copyBuffer" in k for v in vals)
    w_cp = max(v for k, vals in write.items() if "copyBuffer" in k for v in vals)
    copy_bytes = float(1 << 30)
    fs, ws = copy_bytes / f_cp, copy_bytes / w_cp
    cmd = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o fetch -- python3 "
           "<repo>/bench.py --only {},copycal --steps 1 --warmup 0 --no-cpu (then the same with WRITE_SIZE); "
           "python3 bench.py --traffic <fetch csv> <write csv> {}")
    res = {"copy_fetch_bytes_raw": f_cp, "copy_write_bytes_raw": w_cp, "fetch_scale": fs, "write_scale": ws}
    if name == "prefill_varlen":
        # One prefill call = one fused_kernel dispatch (bf16, chunk 32, dk 128),
        # or one local_kernel and one propagation dispatch (slab_mixed_kernel or
        # slab_kernel for bf16 at chunk 64, else prop_kernel).
        prop = lambda k: any(n in k for n in ("fused_kernel", "local_kernel", "prop_kernel", "slab_kernel",
                                              "slab_mixed_kernel"))
        knames = sorted(k for k in fetch if prop(k))
        f_pre = sum(float(np.mean(fetch[k])) for k in knames)
        w_pre = sum(float(np.mean(write[k])) for k in knames)
        fused = any("fused_kernel" in k for k in knames)
        res.update({"kernel": " + ".join(knames), "fetch_bytes_raw": f_pre, "write_bytes_raw": w_pre,
                    "hbm_bytes_per_launch": f_pre * fs + w_pre * ws,
                    "unit": "one prefill call (its kernel dispatches)",
                    "kernel_src_sha256_16": src_hash(FUSED_SRC if fused else PREFILL_SRC),
                    "command": cmd.format("prefill4", name)})
    else:
        per = {}
        for k in sorted(k for k in fetch if "kda::" in k):
            short = k.split("::")[-1].split("(")[0]
            f, w = float(np.mean(fetch[k])) * fs, float(np.mean(write.get(k, [0.0]))) * ws
            per[short] = {"dispatches": len(fetch[k]), "fetch_bytes": f, "write_bytes": w, "hbm_bytes": f + w}
        res.update({"kernels": per, "unit": "one dispatch",
                    "kernel_src_sha256_16": src_hash([os.path.join(CSRC, "kda_pack.hip")]),
                    "command": cmd.format("pack", name)})
    out = os.path.join(PROFILES, f"{name}_traffic.json")
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settled", type=int, default=100,
                    help="after the timed steps of the headline prefill, this many more untimed calls, then the "
                         "same steps timed again and reported beside them as 'settled' (informational; skipped "
                         "for runs of fewer than 10 steps, such as the profiler's)")
    ap.add_argument("--only", default="", help="comma list of: prefill4, prefill4_c64, prefill4_gated, prefill3, "
                                               "prefill3_c32, segments, front_end, decode, decode_bf16, replay, replay_big, "
                                               "replay_big_bf16, ring, pack, copycal")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--json-out", default="")
    ap.add_argument("--traffic", nargs="+", metavar="ARG",
                    help="FETCH_CSV WRITE_CSV [prefill_varlen|pack]: write profiles/<name>_traffic.json from "
                         "two counter passes")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(*args.traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA hot path here has no multi-GPU step "
              "(how it would shard is described with the design); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    from linear_attention_recurrence_kda_amd import inputs

    only = set(x for x in args.only.split(",") if x)
    want = (lambda p: not only or p in only)
    w4 = None
    if want("prefill4") or want("prefill4_c64") or (not only and not args.no_cpu):
        log("generating the varlen prefill workload ...")
        w4 = inputs.workload4()
    cpu = None
    if not args.no_cpu and w4 is not None and not only:
        # (before anything touches the GPU: the worker processes are spawned)
        log("cpu baseline (float64 oracle) ...")
        cpu = cpu_baseline(w4)

    import torch
    from linear_attention_recurrence_kda_amd import kda

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kda.lib()  # fails loudly if the HIP library is not built

    parts = {}
    varlen = ("varlen prefill: 16 seqs, len~logU[1024,32768], H=32, dk=dv=128, bf16, S0~N(0,0.1^2), "
              "chunk {}, ckpt every 4096 + tail, final states packed")
    if want("prefill4"):
        log("prefill (varlen) ...")
        parts["prefill_varlen"] = bench_prefill(torch, kda, inputs, w4, args.steps, args.warmup, True,
                                                varlen.format(HEAD_CHUNK), chunk=HEAD_CHUNK,
                                                settled=args.settled if args.steps >= 10 else 0)
    if want("prefill4_c64"):
        log("prefill (varlen, chunk 64) ...")
        parts["prefill_varlen_chunk64"] = bench_prefill(torch, kda, inputs, w4, args.steps, args.warmup, True,
                                                        varlen.format(64), chunk=64)
    if want("prefill4_gated"):
        if w4 is None:
            log("generating the varlen prefill workload ...")
            w4 = inputs.workload4()
        log("prefill (varlen, fused gate) ...")
        parts["prefill_varlen_gated"] = bench_prefill(
            torch, kda, inputs, w4, args.steps, args.warmup, True,
            "varlen prefill as above (chunk {}) with the gate fused in: a = -sigmoid(z_a), "
            "beta = sigmoid(z_b) computed from bf16 logits inside the prefill".format(HEAD_CHUNK),
            gate=True, chunk=HEAD_CHUNK)
    if want("prefill3"):
        log("prefill (single sequence) ...")
        parts["prefill_single"] = bench_prefill(
            torch, kda, inputs, inputs.workload3(), args.steps, args.warmup, False,
            "single-sequence prefill: T=8192, H=32, dk=dv=128, bf16, S0=0, chunk 64, ckpt every 512")
    if want("prefill3_c32"):
        # The same workload on the fused kernel (chunk 32), where the one
        # sequence is cut into segments whose chains run side by side and the
        # launch's tail composes and corrects them.
        log("prefill (single sequence, chunk 32) ...")
        parts["prefill_single_c32"] = bench_prefill(
            torch, kda, inputs, inputs.workload3(), args.steps, args.warmup, False,
            "single-sequence prefill: T=8192, H=32, dk=dv=128, bf16, S0=0, chunk 32 (fused kernel, the "
            "sequence in segments), ckpt every 512", chunk=HEAD_CHUNK)
    if want("segments"):
        log("segments (context-parallel prefill on one GPU) ...")
        parts["segments"] = bench_segments(torch, kda, inputs, inputs.workload3(), args.steps,
                                           args.warmup)
        # The same with weak decay (a in [-0.001, 0]): the segments' start
        # states then carry over, so the composed path's agreement with the
        # one pass measures the composition rather than a decayed-away state.
        log("segments, weak decay ...")
        ww = inputs.prefill_workload(3, [8192], H=32, dk=128, dv=128, dtype="bf16", ckpt_every=512,
                                     ckpt_tail=False, g_min=-0.001)
        parts["segments_weak_decay"] = bench_segments(torch, kda, inputs, ww, args.steps, args.warmup,
                                                      decay="g_min=-0.001")
        del ww
    if want("front_end"):
        log("front end ...")
        parts["front_end"] = bench_front_end(torch, kda, inputs, args.steps, args.warmup)
    if want("decode"):
        log("decode ...")
        parts["decode"] = bench_decode(torch, kda, inputs, args.steps, args.warmup)
    if want("decode_bf16"):
        log("decode (bf16 state) ...")
        parts["decode_bf16_state"] = bench_decode(torch, kda, inputs, args.steps, args.warmup, "bf16")
    if want("replay"):
        log("replay ...")
        parts["replay"] = bench_replay(torch, kda, inputs, args.steps, args.warmup)
    if want("replay_big"):
        log("replay (large) ...")
        parts["replay_large"] = bench_replay(torch, kda, inputs, args.steps, args.warmup, "big")
    if want("replay_big_bf16"):
        log("replay (large, bf16 state) ...")
        parts["replay_large_bf16_state"] = bench_replay(torch, kda, inputs, args.steps, args.warmup,
                                                        "big", "bf16")
    if want("ring"):
        log("raw-input ring vs snapshots ...")
        parts["ring"] = bench_ring(torch, kda, inputs, args.steps, args.warmup)
    if want("pack"):
        log("pack ...")
        parts["pack"] = bench_pack(torch, kda, args.steps, args.warmup)
    if "copycal" in only:
        parts["copy_calibration"] = copy_calibration(torch)

    head = parts.get("prefill_varlen")
    line = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    if head is not None:
        line["value"] = head["tokens_per_s"]
        line["ms_per_step"] = head["ms_per_step"]
        line["config"] = {"workload": head["workload"], "tokens": head["tokens"],
                          "n_seqs": head["n_seqs"], "H": 32, "dk": 128, "dv": 128, "chunk": head["chunk"],
                          "n_ckpt": head["n_ckpt"], "parallelism": "single GPU"}
        kbytes = head["algo_gbytes"] * 1e9
        line["roofline"] = {
            "kernel": "prefill call: " + head["kernels"],
            "bound": "hbm",
            "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": head["hbm_frac"],
            "traffic": committed_traffic("prefill_varlen", FUSED_SRC if head["chunk"] == 32 else PREFILL_SRC),
            "algo_bytes_per_launch": kbytes, "kernel_ms": head["kernel_ms"],
            "mfma_tflops": head["mfma_tflops"], "mfma_frac": head["mfma_frac"],
            "roofline_frac": head["roofline_frac"]}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    line["parts"] = parts
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
