"""bench.py's metric arithmetic and contract, on the CPU: the visible-pair
count and FLOP formulas against closed forms, and the refusal of more
than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_visible_pairs_closed_forms():
    # dense causal, positions 0..S-1 over S keys: S (S + 1) / 2
    for s in (1, 7, 4096):
        assert bench.visible_pairs(np.arange(s), s) == s * (s + 1) // 2
    # the CP4 rank of a 32768-token sequence: chunks 0 and 7 of 4096 rows
    qpos = np.concatenate([np.arange(0, 4096), np.arange(28672, 32768)])
    first = 4096 * 4097 // 2
    second = sum(range(28673, 32769))
    assert bench.visible_pairs(qpos, 32768) == first + second == 134221824
    # positions past the keys see all of them, negative ones none
    assert bench.visible_pairs([-3, 10], 5) == 0 + 5


def test_flop_formulas():
    n, h = 134221824, 32
    fwd, bwd = bench.flops(n, h, 192, 128)
    # forward S = Q K^T and O = P V; backward S, dP, dV, dK, dQ
    assert fwd == 2.0 * n * h * (192 + 128)
    assert bwd == 2.0 * n * h * (192 + 128 + 128 + 192 + 192)
    assert abs((fwd + bwd) / 1e12 - 9.896) < 1e-3
    assert bench.kv_kernel_flops(n, h, 192, 128) == bwd - 2.0 * n * h * 192


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_is_tied_to_the_sources():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()
    t = bench.measured_traffic()
    assert t is None or t > 0
