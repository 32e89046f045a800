"""bench.py on the CPU: its byte accounting and its command-line contract.

The algorithmic bytes behind the reported GB/s and roofline are checked on a
hand-counted step, and the routed-pair count against the oracle's own
placement of the DeepSeek-V3-shaped workload.  No GPU is used.
"""

from __future__ import annotations

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

import bench
import oracle
from synth import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_hand_counted():
    # 2 ranks, top_k 2, 100-byte rows, 8-byte scales, 10-element bf16 output
    # rows; 3 real tokens reaching 1, 2 and 0 ranks (3 routed pairs); tpr 2.
    w = SimpleNamespace(top_k=2, hidden_row_bytes=100, scale_row_bytes=8, hidden_size=10,
                        combine_elem_bytes=2, ep_size=2)
    b_d, b_c, N, P, R = bench.algorithmic_bytes(w, [2, 1], [0b01, 0b11, 0b00], 2, True)
    assert (N, P, R) == (3, 3, 8)
    reads = 3 * (4 * 2 * 2 + 100 + 8)       # ids + weights + hidden + scale of each real token
    writes = 3 * (100 + 8 + 4 * 2) + 8 * 4 * 2  # routed rows with their weights + the ids slot of every receive row
    assert b_d == reads + writes
    assert b_c == 3 * 4 * 2 + 3 * 20 + 3 * 20   # where each token went (K ids), routed expert rows in, outputs out
    # without weights: no weight bytes read or written
    b_d0, b_c0, *_ = bench.algorithmic_bytes(w, [2, 1], [0b01, 0b11, 0b00], 2, False)
    assert b_d0 == 3 * (4 * 2 + 100 + 8) + 3 * (100 + 8) + 8 * 4 * 2
    assert b_c0 == b_c


def test_event_overhead_is_solved_out():
    """Groups of n launches timed with one event each: t = n * D + m.  The
    alternating pass gives D + C; the solve recovers D, C and m exactly,
    also for a short last group."""
    D, C, m = 15.9, 17.0, 3.3
    n = np.array([8, 8, 4])
    td, tc = n * D + m, n * C + m
    d, c, mm = bench.solve_kernel_times(td, tc, n, D + C)
    np.testing.assert_allclose(d, D)
    np.testing.assert_allclose(c, C)
    assert abs(mm - m) < 1e-12
    # no event overhead at all: nothing subtracted
    d, c, mm = bench.solve_kernel_times(n * D, n * C, n, D + C)
    assert mm == 0.0
    np.testing.assert_allclose(d, D)


def test_routed_pairs_match_the_oracle():
    w = wl.BY_NAME["dsv3"]
    inp = wl.make_inputs(w)
    masks = bench.destination_masks(w, inp)
    p = oracle.Params(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
                      w.hidden_row_bytes)
    res = oracle.OracleMoEEp(p).dispatch(inp.hidden, inp.topk_ids, inp.topk_weights)
    routed = sum(int(r.valid.sum()) for r in res)
    assert sum(bin(m).count("1") for m in masks) == routed


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
