"""Host logic that runs without a GPU: the benchmark's one-GPU contract and the seeded
workload generator the tests, the benchmark and the oracle's baseline all read."""
import os
import subprocess
import sys

import numpy as np
import pytest

from workloads import build, random_pair, reverse_complement_ascii

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    # the path needs no exchange between GPUs, so bench.py produces no multi-GPU figure
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_workloads_are_seeded_and_sized():
    # every config draws its bytes from its own seed: two builds are identical
    a, b = build(0), build(0)
    assert np.array_equal(a.ref, b.ref) and np.array_equal(a.query, b.query)
    assert a.ref.size == 20_000 and a.query.size == 20_000
    assert set(np.unique(a.ref).tolist()) <= set(b"ACGT")
    c1 = build(1)
    assert c1.ref.size == 2_000_000 and c1.query.size == 2_000_000
    n_frac = float(np.mean(c1.ref == ord("N")))
    assert 0.02 < n_frac < 0.08  # 5% N runs
    gc = float(np.mean((c1.ref == ord("G")) | (c1.ref == ord("C")))) / (1 - n_frac)
    assert abs(gc - 0.41) < 0.03


def test_random_pair_is_seeded_and_reverse_complement_involutes():
    r1, q1 = random_pair(9, 5_000, 4_000, plant=5, plant_len=(100, 300), identity=0.9)
    r2, q2 = random_pair(9, 5_000, 4_000, plant=5, plant_len=(100, 300), identity=0.9)
    assert np.array_equal(r1, r2) and np.array_equal(q1, q2)
    assert np.array_equal(reverse_complement_ascii(reverse_complement_ascii(q1)), q1)
