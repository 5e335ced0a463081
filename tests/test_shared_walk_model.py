"""The diagonal-shared walks' correctness argument, checked on the CPU.

The engine can materialize many survivors of one diagonal by walking each stretch of the
diagonal once ("E. X-drop materialization", E.2-E.3, with the walks' order taken from
the sorted survivors): a walk stops at its drop, or at its first strictly new best at or
past the next survivor's start on its diagonal, and takes the rest of its result from
that neighbour.  This file models that rule in plain Python (independently of the HIP
kernels) and checks that it gives exactly the oracle's independently walked records on
inputs full of shared diagonals.  It pins the argument itself, so that a mistake in it
(the score kept at the neighbour's start, the strictness of the merge test, which side
a duplicate anchor merges into) fails here, on any machine.
"""
import numpy as np
import pytest

import oracle
from gpu_util import params_of
from workloads import SEED_PATTERN as SEED, random_pair


def _model(a, rc, qc, sub, n_score, X, merge=True):
    """Records by the merge rule (each walk alone with merge=False): (ref_start,
    query_start, len, score) per anchor, and the number of bases walked."""
    sub = np.asarray(sub, np.int64).reshape(4, 4)
    nr, nq = rc.size, qc.size

    def sigma(x, y):
        if x < 0 or y < 0 or x >= nr or y >= nq:
            return -(X + 1)  # outside a sequence: the walk drops there
        r, q = int(rc[x]), int(qc[y])
        return n_score if r > 3 or q > 3 else int(sub[r, q])

    def walk(r, q, d, wm):
        """(best, ext, merged, ds): best and earliest extent, or the score at index wm
        if the walk sets a strictly new best at an index >= wm before it drops."""
        s = best = ext = ds = 0
        i = 0
        while True:
            x, y = (r + i, q + i) if d > 0 else (r - 1 - i, q - 1 - i)
            s += sigma(x, y)
            if i == wm:
                ds = s
            if s > best:
                if i >= wm:
                    return 0, 0, True, ds, i + 1
                best, ext = s, i + 1
            elif best - s > X:
                return best, ext, False, 0, i + 1
            i += 1

    r = (a & 0xFFFFFFFF).astype(np.int64)
    q = (a >> 32).astype(np.int64)
    order = np.lexsort((r, r - q))  # by diagonal, then reference end
    rs, qs, ds_ = r[order], q[order], (r - q)[order]
    n = a.size
    INF = 1 << 62
    R = np.zeros(n, np.int64)
    K = np.zeros(n, np.int64)
    L = np.zeros(n, np.int64)
    M = np.zeros(n, np.int64)
    steps = 0
    # right walks, resolved from the end of each diagonal backwards
    for s in range(n - 1, -1, -1):
        wm = INF
        if merge and s + 1 < n and ds_[s + 1] == ds_[s] and rs[s + 1] > rs[s]:
            wm = int(rs[s + 1] - 1 - rs[s])
        best, ext, merged, dsv, w = walk(int(rs[s]), int(qs[s]), +1, wm)
        steps += w
        if merged:
            R[s], K[s] = R[s + 1] + dsv, K[s + 1] + (rs[s + 1] - rs[s])
        else:
            R[s], K[s] = best, ext
    # left walks, resolved from the start of each diagonal forwards
    for s in range(n):
        wm = INF
        if merge and s > 0 and ds_[s - 1] == ds_[s] and rs[s - 1] < rs[s]:
            wm = int(rs[s] - 1 - rs[s - 1])
        best, ext, merged, dsv, w = walk(int(rs[s]), int(qs[s]), -1, wm)
        steps += w
        if merged:
            L[s], M[s] = L[s - 1] + dsv, M[s - 1] + (rs[s] - rs[s - 1])
        else:
            L[s], M[s] = best, ext
    rec = np.zeros(n, oracle.HSP_DTYPE)
    rec["ref_start"][order] = rs - M
    rec["query_start"][order] = qs - M
    rec["len"][order] = M + K - 1
    rec["score"][order] = L + R
    return rec, steps


def _tandem(rng, unit_len, copies, mut):
    acgt = np.frombuffer(b"ACGT", np.uint8)
    unit = acgt[rng.integers(0, 4, unit_len)]
    arr = np.concatenate([unit] * copies).copy()
    flip = rng.random(arr.size) < mut
    arr[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    return arr


def _check(ref, qry, a, p):
    """The model with and without merging against the oracle; the bases each walked."""
    R = oracle.Reference(ref, p["seed_pattern"])
    qc = oracle.strand_codes(qry, "+")
    T = oracle.keep_threshold(p["hsp_threshold"])
    ids = np.arange(a.size, dtype=np.uint32)
    want, _ = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    alone, steps_alone = _model(a, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], merge=False)
    assert np.array_equal(alone, want), "the model's own walk differs from the oracle's"
    got, steps = _model(a, R.codes, qc, p["sub"], p["n_score"], p["xdrop"])
    assert np.array_equal(got, want), "the merge rule changed a record"
    return steps, steps_alone


@pytest.mark.parametrize("seed", range(3))
def test_merge_rule_on_tandem_repeats(seed):
    # every gate survivor of a tandem array against a shifted copy of it: hundreds of
    # survivors share each diagonal, spaced a few bases apart; plus every survivor again
    # (equal anchors never merge)
    rng = np.random.default_rng(700 + seed)
    acgt = np.frombuffer(b"ACGT", np.uint8)
    arr = _tandem(rng, 37 + 11 * seed, 25, 0.03 + 0.02 * seed)
    ref = np.concatenate([acgt[rng.integers(0, 4, 400)], arr, acgt[rng.integers(0, 4, 300)]])
    qry = np.concatenate([acgt[rng.integers(0, 4, 200)], arr[90:], acgt[rng.integers(0, 4, 250)]])
    p = params_of(SEED)
    o = oracle.run_pass(oracle.Reference(ref, p["seed_pattern"]), oracle.strand_codes(qry, "+"),
                        p)
    surv = np.concatenate([c["anchors"][c["ids"]] for c in o["chunks"]])
    assert surv.size > 300
    a = np.concatenate([surv, surv[::5]])
    steps, steps_alone = _check(ref, qry, a, p)
    # the point of the rule: far fewer bases walked than walking every survivor alone
    assert steps * 3 < steps_alone


@pytest.mark.parametrize("gap", [1, 2, 5, 63, 64, 65, 127, 128, 129])
def test_merge_rule_at_fixed_spacings(gap):
    # survivors at a fixed spacing on the main diagonal of a sequence and a 6% substituted
    # copy, plus anchors at and next to both sequence ends
    rng = np.random.default_rng(gap)
    ref, _ = random_pair(40 + gap, 3_000, 1)
    qry = ref.copy()
    acgt = np.frombuffer(b"ACGT", np.uint8)
    flip = rng.random(qry.size) < 0.06
    qry[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    pos = np.arange(100, 2_900, gap, dtype=np.uint64)[:400]
    edge = np.asarray([0, 1, ref.size - 1, ref.size], np.uint64)
    a = np.concatenate([pos | (pos << np.uint64(32)), edge | (edge << np.uint64(32)),
                        (pos[::7] + np.uint64(3)) | (pos[::7] << np.uint64(32))])
    _check(ref, qry, a, params_of(SEED))


@pytest.mark.parametrize("gap", [1, 3, 9, 30])
def test_merge_rule_with_tied_scores(gap):
    # match +1, mismatch -1 and a small X: running scores tie their best all the time, so
    # a merge at a best that is not strictly new would report a later extent than the
    # earliest one
    rng = np.random.default_rng(500 + gap)
    ref, _ = random_pair(60 + gap, 2_000, 1)
    qry = ref.copy()
    acgt = np.frombuffer(b"ACGT", np.uint8)
    flip = rng.random(qry.size) < 0.3
    qry[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    sub = np.where(np.eye(4, dtype=bool), 1, -1).astype(np.int32)
    p = params_of(SEED, sub=sub, xdrop=6, K=10, n_score=-1)
    pos = np.arange(50, 1_950, gap, dtype=np.uint64)[:500]
    a = np.concatenate([pos | (pos << np.uint64(32)),
                        (pos[::4] + np.uint64(1)) | (pos[::4] << np.uint64(32))])
    _check(ref, qry, a, p)

