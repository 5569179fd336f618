"""Host-side checks of bench.py, on the CPU: the one-GPU contract and the
FLOP and byte conventions of the measured workloads."""
import importlib.util
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("cid,gflop", [(1, 0.016777216), (2, 68.719476736), (3, 2199.023255552),
                                       (5, 549.755813888)])
def test_flop_convention(cid, gflop):
    """4 B H N^2 d, halved for causal masking (single-head: 2 * 2 * 256^2 * 64
    for the two products without a mask)."""
    b = _bench()
    assert abs(b.flops(W.workload(cid)) / 1e9 - gflop) < 1e-9


def test_packed_flop_convention():
    """Sum over documents of 2 H L^2 d for the seeded packed lengths."""
    b = _bench()
    w = W.workload(4)
    lengths = W.varlen_lengths(W.tensor_seed(4, "lengths"))
    assert abs(b.flops(w, lengths) - sum(2 * 16 * int(L) ** 2 * 128 for L in lengths)) < 1
    assert abs(b.flops(w, lengths) / 1e9 - 313.46) < 0.01


def test_algorithmic_bytes():
    """Q, K, V read once and O, LSE written once: the long-context workload
    moves 539.0 MB."""
    b = _bench()
    assert abs(b.algorithmic_bytes(W.workload(3)) / 1e6 - 538.97) < 0.01


def test_exact_pairs_below_dense_count():
    b = _bench()
    for cid in (2, 3):
        w = W.workload(cid)
        assert b.flops(w) < b.exact_pair_flops(w) <= b.tile_flops(w)
