"""bench.py on the CPU: the algorithmic byte counts behind its roofline
fractions equal the sizes of the tensors each call must read and write
(counted here from arrays of the workloads' shapes), and a run asked for more
than one GPU stops with a message."""
import os
import subprocess
import sys

import numpy as np

import bench
from linear_attention_recurrence_kda_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _nbytes(shape, itemsize):
    return int(np.prod(shape)) * itemsize


def test_decode_bytes_are_the_state_and_token_tensors():
    B, H, d = 256, 32, 128
    for state_bytes in (4, 2):
        want = (2 * _nbytes((B, H, d, d), state_bytes)                 # state read and written
                + 3 * _nbytes((B, H, d), 2) + _nbytes((B, H, d), 2)    # q, k, a and v in
                + _nbytes((B, H), 2)                                   # beta in
                + _nbytes((B, H, d), 2))                               # o out
        assert bench.decode_bytes(B, H, d, d, 2, state_bytes) == want
    assert bench.decode_bytes(B, H, d, d) == 1_084_243_968


def test_replay_bytes_count_only_accepted_inputs():
    B, H, dk, dv, td = 64, 16, 32, 32, 8
    n_acc = np.array([0, 8, 3] + [5] * (B - 3))
    want = (2 * _nbytes((B, H, dk, dv), 4)
            + int(n_acc.sum()) * (_nbytes((H, dk), 4) * 3 + _nbytes((H, dv), 4) + _nbytes((H,), 4))
            + _nbytes((B, H, td, dv), 4))
    assert bench.replay_bytes(B, H, dk, dv, td, n_acc) == want


def test_prefill_bytes_of_the_varlen_workload():
    lengths = inputs.prefill_lengths(4)
    T, N, H, d = int(sum(lengths)), len(lengths), 32, 128
    n_ck = sum(len(c) for c in inputs.prefill_checkpoints(lengths, 4096, True))
    state = _nbytes((H, d, d), 4)
    want = (3 * _nbytes((T, H, d), 2) + _nbytes((T, H, d), 2) + _nbytes((T, H), 2)  # q, k, a, v, beta
            + _nbytes((T, H, d), 2)                                                 # o
            + N * state + n_ck * state + N * state)                                 # S0, checkpoints, final
    assert bench.prefill_bytes(T, H, d, d, N, n_ck) == want
    assert T == 108_886 and n_ck == 35


def test_front_end_bytes_are_its_tensors():
    T, H, dk, dv, K, N, W = 1000, 4, 64, 32, 4, 3, 5
    C = H * (2 * dk + dv)
    read = _nbytes((T, C), 2) + _nbytes((T, H, dk), 2) + _nbytes((T, H), 2) \
        + _nbytes((C, K), 2) + _nbytes((N, K - 1, C), 2)
    write = 3 * _nbytes((T, H, dk), 2) + _nbytes((T, H, dv), 2) \
        + _nbytes((T, H), 2) + _nbytes((W, K - 1, C), 2)  # q, k, a; v; beta; windows
    assert bench.front_end_bytes(T, H, dk, dv, K, N, W) == read + write


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_stamps_name_existing_sources():
    """The sources a traffic figure is stamped with exist (a missing one would
    stop the bench before its line is printed), and the committed figures
    parse."""
    for p in bench.FUSED_SRC + bench.PREFILL_SRC:
        assert os.path.exists(p), p
    assert bench.src_hash(bench.FUSED_SRC) and bench.src_hash(bench.PREFILL_SRC)
    for name in ("prefill_varlen", "pack"):
        bench.committed_traffic(name, bench.FUSED_SRC)
