"""hspz_score_gate_noalloc: the gate for callers that cannot allocate device memory.

Through the C ABI, its flags must equal hspz_score_gate's byte for byte (and the
oracle's, to which hspz_score_gate is tied), on two calls in a row with the second
smaller, so that what the first call left in the shared static scratch cannot leak into
the second; at the largest size it takes; in every gate mode that runs a window stage;
and it must refuse what it cannot do without allocating.
"""
import numpy as np
import pytest

import oracle
from gpu_util import engine, oracle_pass, params_of, require_gpu
from workloads import random_pair

pytestmark = pytest.mark.gpu
MAX_N = 1 << 23


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _anchors(rng, ref, qry, o, k):
    """Pass anchors (long walks on planted homologs) plus random ones, edges included."""
    r = rng.integers(0, ref.size + 1, size=k, dtype=np.uint64)
    q = rng.integers(0, qry.size + 1, size=k, dtype=np.uint64)
    edge_r = np.asarray([0, 1, 7, 8, ref.size - 1, ref.size, 0, ref.size], np.uint64)
    edge_q = np.asarray([0, 1, 9, 8, qry.size, qry.size - 1, qry.size, 0], np.uint64)
    a = np.concatenate([r, edge_r]) | (np.concatenate([q, edge_q]) << np.uint64(32))
    return np.concatenate([a] + [c["anchors"] for c in o["chunks"]])


def _both(eng, a, torch):
    at = torch.from_numpy(a.view(np.int64)).cuda()
    f_ref = torch.full((a.size,), 0xAB, dtype=torch.uint8, device="cuda")
    f_na = torch.full((a.size,), 0xCD, dtype=torch.uint8, device="cuda")
    eng.score_gate(at, a.size, f_ref)
    eng.score_gate_noalloc(at, a.size, f_na)
    return f_ref.cpu().numpy(), f_na.cpu().numpy()


@pytest.mark.parametrize("gate_mode", [0, 1, 3])
def test_noalloc_gate_equals_score_gate_on_two_calls(gate_mode):
    import torch
    rng = np.random.default_rng(7 + gate_mode)
    ref, qry = random_pair(70 + gate_mode, 40_000, 35_000, n_frac=0.03, plant=30,
                           plant_len=(100, 1500), identity=0.92, gc=0.41)
    p = params_of("1101011", K=600)
    o, R, qc = oracle_pass(ref, qry, p)
    eng = engine(p, gate_mode=gate_mode)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    T = oracle.keep_threshold(p["hsp_threshold"])
    a = _anchors(rng, ref, qry, o, 200_000)
    # first call: every anchor; second call: a smaller, reordered subset
    for call, sub in enumerate((a, rng.permutation(a)[: a.size // 3])):
        want = oracle.gate(sub, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
        f_ref, f_na = _both(eng, sub, torch)
        assert np.array_equal(f_ref, want), f"call {call}: hspz_score_gate differs from oracle"
        bad = np.flatnonzero(f_na != f_ref)
        assert bad.size == 0, f"call {call}: {bad.size} flags differ, first at {bad[:5]}"
        assert 0 < int(want.sum()) < sub.size


def test_noalloc_gate_at_its_largest_size_then_smaller():
    # 2^23 anchors, many of them on the diagonal of a sequence against itself (every walk
    # outlives both window stages and goes to the exact list), then a call of 1,000
    import torch
    rng = np.random.default_rng(11)
    ref, _ = random_pair(12, 60_000, 1, gc=0.41)
    p = params_of("1101011", K=50_000)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(ref)
    d = rng.integers(0, ref.size + 1, size=MAX_N // 4, dtype=np.uint64)
    r = rng.integers(0, ref.size + 1, size=MAX_N - d.size, dtype=np.uint64)
    q = rng.integers(0, ref.size + 1, size=MAX_N - d.size, dtype=np.uint64)
    a = np.concatenate([d | (d << np.uint64(32)), r | (q << np.uint64(32))])
    a = rng.permutation(a)
    assert a.size == MAX_N
    f_ref, f_na = _both(eng, a, torch)
    assert np.array_equal(f_na, f_ref)
    codes = oracle.encode(ref)
    samp = rng.choice(a.size, size=20_000, replace=False)
    want = oracle.gate(a[samp], codes, codes, p["sub"], p["n_score"], p["xdrop"],
                       oracle.keep_threshold(p["hsp_threshold"]))
    assert np.array_equal(f_na[samp], want)
    assert int(f_na.sum()) > 0
    small = a[:1000]
    f_ref, f_na = _both(eng, small, torch)
    assert np.array_equal(f_na, f_ref)
    want = oracle.gate(small, codes, codes, p["sub"], p["n_score"], p["xdrop"],
                       oracle.keep_threshold(p["hsp_threshold"]))
    assert np.array_equal(f_na, want)


def test_noalloc_gate_refusals():
    import torch

    import ungapped_drop_hsp_amd as h
    ref, qry = random_pair(3, 5_000, 5_000)
    p = params_of("1101011")
    eng = engine(p)
    at = torch.zeros(8, dtype=torch.int64, device="cuda")
    f = torch.zeros(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(h.HspzError) as ei:  # before any upload
        eng.score_gate_noalloc(at, 8, f)
    assert ei.value.name == "HSPZ_E_STATE"
    eng.upload_reference(ref)
    eng.upload_query(qry)
    with pytest.raises(h.HspzError) as ei:  # beyond the static scratch (host-side check)
        eng.score_gate_noalloc(at, MAX_N + 1, f)
    assert ei.value.name == "HSPZ_E_CAPACITY"
    eng4 = engine(p, gate_mode=4)
    eng4.upload_reference(ref)
    eng4.upload_query(qry)
    with pytest.raises(h.HspzError) as ei:
        eng4.score_gate_noalloc(at, 8, f)
    assert ei.value.name == "HSPZ_E_INVALID"
    eng.score_gate_noalloc(at, 0, f)  # an empty call is fine
