"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small seeded inputs span several scan blocks, gate tiles and compaction blocks with
ragged tails; every byte of seeds, counts, prefix, chunks, anchors, flags, ids, status
and accepted records is compared.
"""
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import (assert_pass_equal, engine, gpu_full_pass, oracle_pass, params_of,
                      require_gpu)
from workloads import HOXD70, SEED_PATTERN, build, random_pair

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_worked_example_through_the_abi():
    # one-base seed: buckets A:0 C:3 G:1 T:5 give the page's counts 0 3 1 0 5
    g = json.load(open(os.path.join(GOLD, "hit_discovery_worked_example.json")))
    p = params_of("1")
    eng = engine(p)
    r = gpu_full_pass(eng, b"CCCGTTTTT", b"ACGAT")
    cnt, pre = r["plan_arrays"]
    assert cnt.tolist() == g["counts"] and pre.tolist() == g["inclusive_prefix"]
    a = r["chunks"][0]["anchors"]
    q_end_of = {1: 2, 2: 3, 4: 5}  # seed s covers query base s, exclusive end s + 1
    for s, slots in g["slots_by_seed_in_occurrence_order"].items():
        qe = q_end_of[int(s)]
        assert [int(a[x] >> 32) for x in slots] == [qe] * len(slots)
        # occurrences ascend in reference end along j, so slots descend
        refs = [int(a[x] & 0xFFFFFFFF) for x in slots]
        assert refs == sorted(refs)
    o, _, _ = oracle_pass(b"CCCGTTTTT", b"ACGAT", p)
    assert_pass_equal(r, o)


def test_plan_counts_follow_each_plan():
    # The plan keeps only the prefix ("C. Hit discovery", C.1-C.2); the per-seed counts are
    # looked up again on first use.  Each new plan, a real one or injected counts, must
    # replace them, also when no expansion ran in between.
    ref, qry = random_pair(31, 20_000, 20_000, plant=10, plant_len=(50, 300), identity=0.9,
                           n_frac=0.01)
    p = params_of(SEED_PATTERN)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry, strand=0)
    o, _, _ = oracle_pass(ref, qry, p)
    n = eng.num_seeds()
    assert n == o["count"].size and n > 100
    for lo, hi in [(0, n // 2), (n // 2, n), (n // 3, n // 3 + 77), (0, n)]:
        eng.plan(lo, hi)
        cnt, pre = eng.get_plan_arrays(hi - lo)
        want = np.asarray(o["count"][lo:hi], np.uint64)
        assert np.array_equal(cnt.astype(np.uint64), want), (lo, hi)
        assert np.array_equal(pre.astype(np.uint64), np.cumsum(want)), (lo, hi)
    inj = np.arange(7, dtype=np.uint32)
    eng.debug_plan_counts(inj)
    cnt, pre = eng.get_plan_arrays(inj.size)
    assert cnt.tolist() == inj.tolist() and pre.tolist() == np.cumsum(inj).tolist()
    eng.plan(0, n)
    cnt, _ = eng.get_plan_arrays(n)
    assert np.array_equal(cnt.astype(np.uint64), np.asarray(o["count"], np.uint64))


@pytest.mark.parametrize("walk", [0, 1])
def test_chunk_cuts_from_injected_counts(walk):
    gold = json.load(open(os.path.join(GOLD, "chunk_cuts_worked_example.json")))
    for case in gold["cases"]:
        eng = engine(params_of(SEED_PATTERN), chunk_walk=walk, max_hits=case["max_hits"])
        tot, nch = eng.debug_plan_counts(np.asarray([0, 3, 1, 0, 5], np.uint32))
        got = [[c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]]
               for c in (eng.get_chunk(i) for i in range(nch))]
        assert tot == 9 and got == case["chunks"]
        cnt, pre = eng.get_plan_arrays(5)
        assert pre.tolist() == [0, 3, 4, 4, 9]


@pytest.mark.parametrize("walk", [0, 1])
@pytest.mark.parametrize("seed", range(3))
def test_chunk_walk_on_many_blocks(walk, seed):
    rng = np.random.default_rng(seed)
    counts = rng.choice([0, 0, 1, 2, 5, 40, 300], size=50_000).astype(np.uint32)
    P, _ = oracle.prefix(counts)
    for mx in (1, 3, 16, 1000, 77_777, int(P[-1]) - 1, 0):
        eng = engine(params_of(SEED_PATTERN), chunk_walk=walk, max_hits=mx)
        tot, nch = eng.debug_plan_counts(counts)
        got = [eng.get_chunk(i) for i in range(nch)]
        want = oracle.chunks(P, mx)
        assert tot == int(P[-1])
        assert [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in got] == \
            [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in want]
        _, pre = eng.get_plan_arrays(counts.size)
        assert np.array_equal(pre.astype(np.uint64), P)


@pytest.mark.parametrize("walk", [0, 1])
def test_chunk_walk_edges(walk):
    # the device walk returns at most 1,024 chunks and the host walks longer lists;
    # a cut landing on the total leaves a trailing chunk of zero hits
    cases = [
        (np.ones(1024, np.uint32), 1),              # exactly 1,024 chunks
        (np.ones(1025, np.uint32), 1),              # one more: the host walks
        (np.asarray([1, 5, 0, 0], np.uint32), 2),   # [0, 1] 6 hits, then [2, 3] 0 hits
        (np.asarray([0, 0, 7, 0], np.uint32), 3),   # one non-empty seed among empty ones
        (np.zeros(3000, np.uint32), 5),             # no hits: no chunks
    ]
    for counts, mx in cases:
        P, _ = oracle.prefix(counts)
        eng = engine(params_of(SEED_PATTERN), chunk_walk=walk, max_hits=mx)
        tot, nch = eng.debug_plan_counts(counts)
        got = [eng.get_chunk(i) for i in range(nch)]
        want = oracle.chunks(P, mx)
        assert tot == int(P[-1])
        assert [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in got] == \
            [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in want]


CASES = [
    # (seed, n_ref, n_qry, pattern, max_hits, n_frac, plant, identity, gc)
    (0, 30_000, 30_000, "1101011", 0, 0.0, 20, 0.92, 0.5),
    (1, 25_000, 31_000, "1101011", 5_000, 0.03, 15, 0.85, 0.41),
    (2, 40_000, 20_000, SEED_PATTERN, 0, 0.02, 30, 0.9, 0.41),
    (3, 12_345, 23_456, "11011", 2_000, 0.05, 10, 0.95, 0.5),
    (4, 8_000, 8_000, "111", 7, 0.0, 5, 0.8, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{c[3]}-max{c[4]}")
@pytest.mark.parametrize("expand_mode,gate_mode,mat", [(0, 0, 0), (1, 1, 0), (2, 2, 0), (0, 3, 0),
                                                        (0, 4, 0), (0, 0, 2), (0, 5, 0)],
                         ids=["auto", "sparse-exact", "dense-window", "auto-window2",
                              "bucketed", "shared-walks", "key-grouped"])
def test_random_pass_parity(case, expand_mode, gate_mode, mat):
    seed, nr, nq, pat, mx, nf, plant, ident, gc = case
    ref, qry = random_pair(seed, nr, nq, n_frac=nf, plant=plant, plant_len=(60, 600),
                           identity=ident, gc=gc, alphabet_noise=True)
    p = params_of(pat, max_hits=mx)
    o, _, _ = oracle_pass(ref, qry, p)
    # the bucketed gate over 16 reference slices (the automatic width is one slice here)
    eng = engine(p, expand_mode=expand_mode, gate_mode=gate_mode,
                 ref_buckets=16 if gate_mode == 4 else 0, materialize_mode=mat)
    r = gpu_full_pass(eng, ref, qry)
    assert_pass_equal(r, o)


def _edge_anchors(rng, nr, nq, k):
    """Anchors at and next to both ends of both sequences, plus random interior ones."""
    r = list(rng.integers(0, nr + 1, size=k)) + [0, 1, 7, 8, 71, 72, 73, nr - 1, nr, nr - 48,
                                                    nr - 47, nr - 8, 0, nr, 5, nr - 5]
    q = list(rng.integers(0, nq + 1, size=k)) + [0, 1, 9, 8, 72, 71, 80, nq, nq - 1, nq - 47,
                                                    nq - 48, nq - 9, nq, 0, nq - 5, 5]
    return np.asarray([(a & 0xFFFFFFFF) | (b << 32) for a, b in zip(r, q)], np.uint64)


@pytest.mark.parametrize("gate_mode", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", range(3))
def test_gate_on_arbitrary_anchors(gate_mode, seed):
    # anchors need not come from seeds: walks from every offset near both sequence ends,
    # through N runs, and on planted homologs (long walks past the window)
    import torch
    rng = np.random.default_rng(100 + seed)
    ref, qry = random_pair(200 + seed, 3_000 + 500 * seed, 2_500 + 700 * seed, n_frac=0.05,
                           plant=12, plant_len=(100, 900), identity=0.93)
    p = params_of("11011", K=300 + 200 * seed)
    eng = engine(p, gate_mode=gate_mode, ref_buckets=7 + 60 * seed)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    a = _edge_anchors(rng, ref.size, qry.size, 30_000)
    # plus the diagonals of the planted homologs, where walks are long
    o, R, qc = oracle_pass(ref, qry, p)
    a = np.concatenate([a] + [c["anchors"] for c in o["chunks"]])
    T = oracle.keep_threshold(p["hsp_threshold"])
    want = oracle.gate(a, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    assert 0 < int(want.sum()) < a.size
    at = torch.from_numpy(a.view(np.int64)).cuda()
    f = torch.full((a.size,), 0xAB, dtype=torch.uint8, device="cuda")
    eng.score_gate(at, a.size, f)
    got = f.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} flags differ, first anchors {a[bad[:5]]}"
    if gate_mode >= 2:
        n2, nx = eng.debug_gate_deferred()
        assert 0 < n2 < a.size and 0 < nx <= n2


@pytest.mark.parametrize("gate_mode,mat", [(0, 0), (1, 1), (2, 0), (3, 0), (4, 2)])
def test_keep_threshold_equal_to_exact_totals(gate_mode, mat):
    # "D. Score gate", D.3: kept when the total is at least the threshold.  K is set to
    # totals that anchors of the pass reach exactly (ties at the boundary), to one above
    # and to one below; flags, ids, status and records must match the oracle's, which
    # is pinned at the same boundary by hand-worked totals.
    ref, qry = random_pair(31, 20_000, 20_000, n_frac=0.02, plant=25, plant_len=(40, 400),
                           identity=0.85, gc=0.41)
    p0 = params_of("1101011")
    o, R, qc = oracle_pass(ref, qry, p0)
    a = np.concatenate([c["anchors"] for c in o["chunks"]])
    tot, _ = oracle.gate_totals(a, R.codes, qc, p0["sub"], p0["n_score"], p0["xdrop"])
    vals, cnt = np.unique(tot[tot >= 200], return_counts=True)
    picks = [int(vals[np.argmax(cnt)]), int(vals[-1]), int(vals[vals.size // 2])]
    for K0 in picks:
        assert (tot == K0).any()
        for K in (K0, K0 + 1, K0 - 1):
            p = params_of("1101011", K=K)
            ok, _, _ = oracle_pass(ref, qry, p)
            kept = sum(int(c["flags"].sum()) for c in ok["chunks"])
            assert kept == int((tot >= K).sum())
            eng = engine(p, gate_mode=gate_mode, materialize_mode=mat,
                         ref_buckets=5 if gate_mode == 4 else 0)
            assert_pass_equal(gpu_full_pass(eng, ref, qry), ok)


@pytest.mark.parametrize("gate_mode", [2, 3, 4])
def test_window_gate_defers_long_walks(gate_mode):
    # a sequence against itself: every anchor on the main diagonal walks to both ends
    ref, _ = random_pair(15, 20_000, 1, gc=0.41)
    p = params_of("1101011", K=10**6)
    eng = engine(p, gate_mode=gate_mode, ref_buckets=32)
    eng.upload_reference(ref)
    eng.upload_query(ref)
    import torch
    diag = np.arange(0, ref.size + 1, 97, dtype=np.uint64)
    a = diag | (diag << np.uint64(32))
    at = torch.from_numpy(a.view(np.int64)).cuda()
    f = torch.empty(a.size, dtype=torch.uint8, device="cuda")
    eng.score_gate(at, a.size, f)
    codes = oracle.encode(ref)
    want = oracle.gate(a, codes, codes, p["sub"], p["n_score"], p["xdrop"],
                       oracle.keep_threshold(p["hsp_threshold"]))
    assert np.array_equal(f.cpu().numpy(), want)
    # every anchor walks past both windows (none sits within a window of both ends)
    n2, nx = eng.debug_gate_deferred()
    assert n2 == a.size and nx == a.size


@pytest.mark.parametrize("strand", ["+", "-"])
def test_reverse_strand_parity(strand):
    ref, qry = random_pair(7, 20_000, 20_000, plant=20, plant_len=(100, 800), identity=0.9)
    from workloads import reverse_complement_ascii
    qry = np.concatenate([qry[:10_000], reverse_complement_ascii(ref[5_000:15_000])])
    p = params_of("1101011", max_hits=30_000)
    o, _, _ = oracle_pass(ref, qry, p, strand=strand)
    assert o["total"] > 0 and sum(c["ids"].size for c in o["chunks"]) > 0
    assert_pass_equal(gpu_full_pass(engine(p), ref, qry, strand=strand), o)


def test_query_batches_parity():
    ref, qry = random_pair(8, 20_000, 30_000, plant=25, plant_len=(100, 500), identity=0.9,
                           n_frac=0.02)
    p = params_of("1101011", max_hits=4_000)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    from ungapped_drop_hsp_amd.pipeline import batches
    bs = batches(eng, 7_000, qry.size)
    assert len(bs) == 5
    for lo, hi in bs:
        o, _, _ = oracle_pass(ref, qry, p, seed_range=(lo, hi))
        assert_pass_equal(gpu_full_pass(eng, ref, qry, seed_range=(lo, hi)), o)


@pytest.mark.parametrize("mat", [0, 2], ids=["default-walks", "shared-walks"])
@pytest.mark.parametrize("xdrop,n_score", [(910, -100), (400, -100), (150, 30), (60, -20),
                                           (0, -100)])
def test_block_sizes_and_scores(xdrop, n_score, mat):
    # small X forces 4-, 2- and 1-base gate blocks (and shared walks without their
    # eight-base lane stage); a positive N score is allowed too
    sub = np.asarray(HOXD70, np.int32).copy()
    sub[0, 1], sub[1, 0] = 40, -90  # asymmetric: ref row, query column
    ref, qry = random_pair(9, 15_000, 15_000, plant=30, plant_len=(50, 400), identity=0.9,
                           n_frac=0.03)
    p = params_of("11011", sub=sub, xdrop=xdrop, K=400, n_score=n_score)
    o, _, _ = oracle_pass(ref, qry, p)
    assert_pass_equal(gpu_full_pass(engine(p, materialize_mode=mat), ref, qry), o)


@pytest.mark.parametrize("mat", [1, 2], ids=["own-walks", "shared-walks"])
def test_identical_sequences_long_walks(mat):
    # every anchor of the main diagonal walks to both sequence ends; with shared walks
    # each one merges into its neighbour's
    ref, _ = random_pair(10, 30_000, 1, gc=0.41)
    p = params_of(SEED_PATTERN, max_hits=100_000)
    o, _, _ = oracle_pass(ref, ref, p)
    r = gpu_full_pass(engine(p, materialize_mode=mat), ref, ref)
    assert_pass_equal(r, o)
    # the main diagonal's records span the whole sequence
    acc = np.concatenate([c["accepted"] for c in r["chunks"]])
    full = acc[(acc["ref_start"] == 0) & (acc["len"] == ref.size - 1)]
    assert full.size > 0


@pytest.mark.parametrize("qry", [b"", b"ACGT", b"N" * 5000, b"ACGTACGTAC" * 3],
                         ids=["empty", "short", "all-N", "repeat"])
def test_degenerate_queries(qry):
    ref, _ = random_pair(11, 5_000, 1)
    p = params_of("1101011")
    o, _, _ = oracle_pass(ref, np.frombuffer(qry, np.uint8), p)
    r = gpu_full_pass(engine(p), ref, np.frombuffer(qry, np.uint8))
    assert_pass_equal(r, o)


def test_empty_reference():
    p = params_of("11011")
    eng = engine(p)
    eng.upload_reference(b"")
    eng.upload_query(b"ACGTACGTACGT")
    assert eng.plan(0, eng.num_seeds()) == (0, 0)


def test_overflow_is_refused():
    # 70,000 x A against itself: 69,982 seeds x 69,982 hits > 2^32 - 1
    p = params_of(SEED_PATTERN)
    eng = engine(p)
    eng.upload_reference(b"A" * 70_000)
    eng.upload_query(b"A" * 70_000)
    import ungapped_drop_hsp_amd as h
    with pytest.raises(h.HspzError) as ei:
        eng.plan(0, eng.num_seeds())
    assert ei.value.name == "HSPZ_E_OVERFLOW"
    with pytest.raises(h.HspzError) as ei:
        eng.find_hits(0, 0, cap=0)
    assert ei.value.name == "HSPZ_E_STATE"
    # a smaller batch of the same query fits
    tot, nch = eng.plan(0, 1000)
    assert tot == 1000 * 69_982 and nch == 1


def test_errors_and_capacity():
    import torch
    import ungapped_drop_hsp_amd as h
    ref, qry = random_pair(12, 5_000, 5_000, plant=5, identity=0.95)
    p = params_of("11011")
    eng = engine(p)
    with pytest.raises(h.HspzError) as ei:
        eng.plan(0, 0)
    assert ei.value.name == "HSPZ_E_STATE"
    eng.upload_reference(ref)
    eng.upload_query(qry)
    with pytest.raises(h.HspzError) as ei:
        eng.plan(0, eng.num_seeds() + 1)
    assert ei.value.name == "HSPZ_E_INVALID"
    tot, nch = eng.plan(0, eng.num_seeds())
    small = torch.empty(tot - 1, dtype=torch.int64, device="cuda")
    with pytest.raises(h.HspzError) as ei:
        eng.find_hits(0, small)
    assert ei.value.name == "HSPZ_E_CAPACITY"
    a = torch.empty(tot, dtype=torch.int64, device="cuda")
    eng.find_hits(0, a)
    f = torch.empty(tot, dtype=torch.uint8, device="cuda")
    eng.score_gate(a, tot, f)
    n_keep = int((f != 0).sum())
    assert n_keep > 1
    ids = torch.empty(n_keep - 1, dtype=torch.int32, device="cuda")
    with pytest.raises(h.HspzError) as ei:
        eng.compact(f, tot, ids)
    assert ei.value.name == "HSPZ_E_CAPACITY"
    with pytest.raises(h.HspzError):
        eng.get_chunk(nch)


def test_poisoned_outputs_are_overwritten():
    import torch
    ref, qry = random_pair(13, 20_000, 20_000, plant=20, plant_len=(80, 500), identity=0.9)
    p = params_of("1101011")
    o, _, _ = oracle_pass(ref, qry, p)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    tot, _ = eng.plan(0, eng.num_seeds())
    a = torch.full((tot + 7,), -0x5454545454545455, dtype=torch.int64, device="cuda")
    f = torch.full((tot + 7,), 0xAB, dtype=torch.uint8, device="cuda")
    eng.find_hits(0, a)
    eng.score_gate(a, tot, f)
    ah = a.cpu().numpy().view(np.uint64)
    assert np.array_equal(ah[:tot], o["chunks"][0]["anchors"])
    fh = f.cpu().numpy()
    assert np.array_equal(fh[:tot], o["chunks"][0]["flags"])
    assert (fh[tot:] == 0xAB).all()  # nothing past n is touched
    ids = torch.full((tot,), -1, dtype=torch.int32, device="cuda")
    ns = eng.compact(f, tot, ids)
    hsp = torch.full((ns + 3, 4), 0x2B2B2B2B, dtype=torch.int32, device="cuda")
    st = torch.full((ns + 3,), 0xAB, dtype=torch.uint8, device="cuda")
    eng.materialize(a, ids, ns, hsp, st)
    sh = st.cpu().numpy()
    assert set(np.unique(sh[:ns]).tolist()) <= {0, 1} and (sh[ns:] == 0xAB).all()
    assert np.array_equal(sh[:ns], o["chunks"][0]["status"])


def test_unaligned_buffers_and_out_of_range_anchors():
    import torch
    ref, qry = random_pair(14, 10_000, 10_000, plant=10, plant_len=(100, 400), identity=0.92)
    p = params_of("11011")
    o, R, qc = oracle_pass(ref, qry, p)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    want = o["chunks"][0]
    n = want["anchors"].size
    extra = np.asarray([(ref.size + 5) | (3 << 32), 7 | ((qry.size + 1) << 32),
                        ref.size | (qry.size << 32), 0], np.uint64)
    anchors = np.concatenate([want["anchors"], extra])
    a = torch.from_numpy(anchors.view(np.int64)).cuda()
    base = torch.zeros(anchors.size + 9, dtype=torch.uint8, device="cuda")
    f = base[1:1 + anchors.size]  # 1-byte offset: unaligned flag buffer
    eng.score_gate(a, anchors.size, f)
    fo = oracle.gate(anchors, R.codes, qc, p["sub"], p["n_score"], p["xdrop"],
                     oracle.keep_threshold(p["hsp_threshold"]))
    assert np.array_equal(f.cpu().numpy(), fo)
    ids = torch.empty(anchors.size, dtype=torch.int32, device="cuda")
    ns = eng.compact(f, anchors.size, ids)
    assert np.array_equal(ids[:ns].cpu().numpy().view(np.uint32), oracle.compact(fo))
    # materialize out-of-range anchors directly: empty walks on both sides
    bad_ids = torch.arange(n, n + 4, dtype=torch.int32, device="cuda")
    hsp = torch.empty((4, 4), dtype=torch.int32, device="cuda")
    st = torch.empty(4, dtype=torch.uint8, device="cuda")
    eng.materialize(a, bad_ids, 4, hsp, st)
    oh, ost = oracle.materialize(anchors, np.arange(n, n + 4, dtype=np.uint32), R.codes, qc,
                                 p["sub"], p["n_score"], p["xdrop"],
                                 oracle.keep_threshold(p["hsp_threshold"]))
    assert np.array_equal(st.cpu().numpy(), ost)
    gh = hsp.cpu().numpy().view(oracle.HSP_DTYPE).reshape(-1)
    assert np.array_equal(gh[:3], oh[:3])


@pytest.mark.parametrize("mat", [0, 2], ids=["auto", "shared-walks"])
@pytest.mark.parametrize("cfg", [0, 1])
def test_config_full_parity(cfg, mat):
    w = build(cfg)
    p = w.params()
    o, _, _ = oracle_pass(w.ref, w.query, p)
    r = gpu_full_pass(engine(p, materialize_mode=mat), w.ref, w.query)
    assert_pass_equal(r, o)
    print(f"config {cfg}: anchors {r['total']} survivors {r['n_surv']} accepted {r['n_acc']}")


@pytest.mark.parametrize("mat", [1, 2], ids=["own-walks", "shared-walks"])
@pytest.mark.parametrize("seed", range(3))
def test_entropy_mode_parity(seed, mat):
    # planted homologs plus low-complexity copies, which the entropy-adjusted decision
    # rejects although their scores pass T
    ref, qry = random_pair(30 + seed, 20_000, 20_000, plant=40, plant_len=(60, 500),
                           identity=0.95, n_frac=0.01)
    ref[1000:1120] = np.frombuffer(b"AT" * 60, np.uint8)
    qry[5000:5120] = np.frombuffer(b"AT" * 60, np.uint8)
    ref[3000:3090] = np.frombuffer(b"A" * 90, np.uint8)
    qry[8000:8090] = np.frombuffer(b"A" * 90, np.uint8)
    ref[9000:9200] = np.frombuffer(b"AAGAAG" * 33 + b"AA", np.uint8)
    qry[12000:12200] = np.frombuffer(b"AAGAAG" * 33 + b"AA", np.uint8)
    p = params_of("1101011", K=600, entropy_mode=1)
    o, _, _ = oracle_pass(ref, qry, p)
    n_surv = sum(c["ids"].size for c in o["chunks"])
    n_acc = sum(c["accepted"].size for c in o["chunks"])
    assert 0 < n_acc < n_surv
    assert_pass_equal(gpu_full_pass(engine(p, materialize_mode=mat), ref, qry), o)


def test_entropy_mode_config1():
    w = build(1)
    p = dict(w.params(), entropy_mode=1)
    o, _, _ = oracle_pass(w.ref, w.query, p)
    assert_pass_equal(gpu_full_pass(engine(p), w.ref, w.query), o)


def _oracle_batch(o):
    recs = [c["accepted"] for c in o["chunks"]]
    acc = np.concatenate(recs) if recs else np.zeros(0, oracle.HSP_DTYPE)
    return dict(n_anchors=o["total"], n_chunks=len(o["chunks"]),
                n_survivors=sum(int(c["ids"].size) for c in o["chunks"]),
                n_accepted=int(acc.size)), acc


@pytest.mark.parametrize("gate_mode", [0, 5], ids=["auto", "key-grouped"])
@pytest.mark.parametrize("mat", [0, 2], ids=["default-walks", "shared-walks"])
@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: f"s{c[0]}-{c[3]}-max{c[4]}")
def test_run_batch_matches_the_oracle(case, mat, gate_mode):
    # the native whole-batch driver against the oracle's pass: counts and every accepted
    # record, in chunk order, over the whole strand and over sub-batches (with shared
    # walks the driver sorts its own survivors by diagonal alone)
    seed, nr, nq, pat, mx, nf, plant, ident, gc = case
    ref, qry = random_pair(seed, nr, nq, n_frac=nf, plant=plant, plant_len=(60, 600),
                           identity=ident, gc=gc, alphabet_noise=True)
    p = params_of(pat, max_hits=mx)
    eng = engine(p, materialize_mode=mat, gate_mode=gate_mode)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    n = eng.num_seeds()
    for lo, hi in [(0, n), (0, n // 3), (n // 3, n), (n // 2, n // 2)]:
        o, _, _ = oracle_pass(ref, qry, p, seed_range=(lo, hi))
        want, acc = _oracle_batch(o)
        st = eng.run_batch(lo, hi, time_gate=True)
        assert {k: st[k] for k in want} == want
        # one gate call over every chunk where the key-grouped stage serves a batch of
        # large chunks, else one per chunk (these chunks are small)
        assert st["whole_batch_gate"] == 0
        assert st["gate_calls"] == (1 if st["whole_batch_gate"] else st["n_chunks"])
        assert (st["gate_ms"] > 0) == (st["n_chunks"] > 0)
        got = eng.batch_records()
        assert np.array_equal(got.view(np.uint8), acc.astype(oracle.HSP_DTYPE).view(np.uint8))


@pytest.mark.timeout(600)
def test_whole_batch_gate_matches_the_oracle():
    # hspz_run_batch gates a batch of large chunks (2^22 anchors or more on average) in one
    # key-grouped call over every chunk's slots, then compacts and materializes each chunk
    # from its slice.  A 1 Mb x 1 Mb pair with an 8-of-11 seed (about 1.6e7 anchors) cut
    # into two and into three chunks, in gate modes 0 and 5 and with the shared walks, and
    # a sub-batch of small chunks (one call per chunk), against the oracle's pass.
    ref, qry = random_pair(23, 1_000_000, 1_000_000, n_frac=0.01, plant=60,
                           plant_len=(200, 3000), identity=0.9, gc=0.45)
    pat = "11011011011"
    for mx in (1 << 23, 6_000_000):
        p = params_of(pat, max_hits=mx)
        o, _, _ = oracle_pass(ref, qry, p)
        want, acc = _oracle_batch(o)
        assert want["n_chunks"] in (2, 3) and want["n_anchors"] >= (1 << 22) * want["n_chunks"]
        for gm, mat in ((0, 0), (5, 0), (0, 2)):
            eng = engine(p, gate_mode=gm, materialize_mode=mat)
            eng.upload_reference(ref)
            eng.upload_query(qry)
            st = eng.run_batch(0, eng.num_seeds(), time_gate=True)
            assert {k: st[k] for k in want} == want, (mx, gm, mat)
            assert st["whole_batch_gate"] == 1 and st["gate_calls"] == 1
            assert np.array_equal(eng.batch_records().view(np.uint8),
                                  acc.astype(oracle.HSP_DTYPE).view(np.uint8)), (mx, gm, mat)
            print(f"max_hits {mx} gate_mode {gm} materialize_mode {mat}: {want}", flush=True)
    # a sub-batch whose chunks average under 2^22 anchors: one gate call per chunk
    p = params_of(pat, max_hits=1 << 21)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    lo, hi = 0, eng.num_seeds() // 4
    o, _, _ = oracle_pass(ref, qry, p, seed_range=(lo, hi))
    want, acc = _oracle_batch(o)
    st = eng.run_batch(lo, hi, time_gate=True)
    assert {k: st[k] for k in want} == want and want["n_chunks"] > 1
    assert st["whole_batch_gate"] == 0 and st["gate_calls"] == st["n_chunks"]
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc.astype(oracle.HSP_DTYPE).view(np.uint8))


def _unit_copies(unit_seed, spacer_seed, unit_len, copies, spacer):
    """Copies of one random unit, each followed by its own random spacer."""
    bases = np.frombuffer(b"ACGT", np.uint8)
    unit = bases[np.random.default_rng(unit_seed).integers(0, 4, unit_len)]
    rs = np.random.default_rng(spacer_seed)
    parts = []
    for _ in range(copies):
        parts += [unit, bases[rs.integers(0, 4, spacer)]]
    return np.concatenate(parts)


def test_whole_batch_with_most_anchors_deferred():
    # The whole-batch gate (flag bits) when most walks outlive the first window: copies of
    # a 90-base unit (150 in each sequence, totals near 8,600: kept at K = 7,000) and of a
    # 60-base unit (420 in each, totals near 5,700: dropped), different spacers on the two
    # sides, about 9e6 anchors in two chunks.  The waves' LDS segments fill, so deferred
    # anchors also go through the global list with their slots formed from the prefix, and
    # the exact walks overflow the workgroups' pools into the exact list.
    ref = np.concatenate([_unit_copies(61, 1, 90, 150, 70), _unit_copies(62, 2, 60, 420, 70)])
    qry = np.concatenate([_unit_copies(61, 3, 90, 150, 70), _unit_copies(62, 4, 60, 420, 70)])
    p = params_of(SEED_PATTERN, max_hits=5_000_000, K=7000)
    o, _, _ = oracle_pass(ref, qry, p)
    want, acc = _oracle_batch(o)
    assert want["n_chunks"] == 2 and want["n_anchors"] >= (1 << 22) * 2
    assert 0 < want["n_accepted"] < want["n_anchors"] // 2
    for gm in (0, 5):
        eng = engine(p, gate_mode=gm)
        eng.upload_reference(ref)
        eng.upload_query(qry)
        st = eng.run_batch(0, eng.num_seeds(), time_gate=True)
        assert {k: st[k] for k in want} == want, gm
        assert st["whole_batch_gate"] == 1
        n2, nx = eng.debug_gate_deferred()
        print(f"gate_mode {gm}: {want}, second stage {n2}, exact {nx}", flush=True)
        assert n2 > want["n_anchors"] // 10 and nx > 0
        assert np.array_equal(eng.batch_records().view(np.uint8),
                              acc.astype(oracle.HSP_DTYPE).view(np.uint8)), gm


@pytest.mark.parametrize("mat", [0, 2], ids=["default-walks", "shared-walks"])
def test_run_batch_reverse_strand_and_entropy(mat):
    ref, qry = random_pair(11, 30_000, 25_000, n_frac=0.02, plant=25, plant_len=(80, 900),
                           identity=0.9, gc=0.41, alphabet_noise=True)
    for mode in (0, 1):
        p = params_of(SEED_PATTERN, max_hits=3_000, entropy_mode=mode)
        eng = engine(p, materialize_mode=mat)
        eng.upload_reference(ref)
        eng.upload_query(qry, strand=1)
        o, _, _ = oracle_pass(ref, qry, p, strand="-")
        want, acc = _oracle_batch(o)
        st = eng.run_batch(0, eng.num_seeds())
        assert {k: st[k] for k in want} == want and st["gate_calls"] == 0
        assert np.array_equal(eng.batch_records().view(np.uint8),
                              acc.astype(oracle.HSP_DTYPE).view(np.uint8))


@pytest.mark.parametrize("mat", [0, 2], ids=["default-walks", "shared-walks"])
def test_run_batch_survivors_grow_mid_batch(mat):
    # run_batch queues chunk c + 1's gate and survivor compaction before it reads chunk
    # c's counts.  Here the early chunks keep nothing and the last ones keep thousands of
    # anchors (the query ends with copies of reference stretches), so the survivor buffers
    # grow between chunks; the chunks are of uneven size.  Run twice on one engine: the
    # second call starts with grown buffers.
    rng = np.random.default_rng(21)
    acgt = np.frombuffer(b"ACGT", np.uint8)
    ref = acgt[rng.integers(0, 4, 24_000)].copy()
    qry = np.concatenate([acgt[rng.integers(0, 4, 18_000)], ref[2_000:7_000],
                          acgt[rng.integers(0, 4, 3_000)], ref[15_000:16_500]])
    # a weight-6 seed fills the first chunks with random anchors that all fail the gate
    p = params_of("11101101", max_hits=20_000)
    eng = engine(p, materialize_mode=mat)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    o, _, _ = oracle_pass(ref, qry, p)
    want, acc = _oracle_batch(o)
    kept = [int(c["ids"].size) for c in o["chunks"]]
    assert want["n_chunks"] > 5 and kept[0] == 0 and max(kept) > 2_048
    assert len({c["chunk"]["n_hits"] for c in o["chunks"]}) > 1
    for _ in range(2):
        st = eng.run_batch(0, eng.num_seeds(), time_gate=True)
        assert {k: st[k] for k in want} == want
        assert st["gate_calls"] == (1 if st["whole_batch_gate"] else st["n_chunks"])
        assert np.array_equal(eng.batch_records().view(np.uint8),
                              acc.astype(oracle.HSP_DTYPE).view(np.uint8))


@pytest.mark.parametrize("gate_mode", [0, 1, 3, 4])
def test_run_batch_shared_walks_on_tandem_repeats(gate_mode):
    # the batch driver with shared walks (its survivors sorted by diagonal alone) behind
    # every gate: windowed (0; 3 with a narrower first window), per-base (1) and bucketed
    # (4); a tandem array gives long chains of merges in each of 17 chunks; counts and
    # every accepted record against the oracle
    rng = np.random.default_rng(53)
    acgt = np.frombuffer(b"ACGT", np.uint8)
    unit = acgt[rng.integers(0, 4, 61)]
    arr = np.concatenate([unit] * 60).copy()
    flip = rng.random(arr.size) < 0.04
    arr[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    ref = np.concatenate([acgt[rng.integers(0, 4, 5_000)], arr, acgt[rng.integers(0, 4, 3_000)]])
    qry = np.concatenate([acgt[rng.integers(0, 4, 2_000)], arr[300:], acgt[rng.integers(0, 4, 1_500)]])
    p = params_of(SEED_PATTERN, max_hits=6_000)
    eng = engine(p, gate_mode=gate_mode, ref_buckets=8 if gate_mode == 4 else 0,
                 materialize_mode=2)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    o, _, _ = oracle_pass(ref, qry, p)
    want, acc = _oracle_batch(o)
    assert want["n_chunks"] > 2 and want["n_survivors"] > 2_000
    st = eng.run_batch(0, eng.num_seeds())
    assert {k: st[k] for k in want} == want
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc.astype(oracle.HSP_DTYPE).view(np.uint8))


def test_upload_seeds_replaces_the_seeder():
    # caller seeds in place of the device seeder's ("C. Hit discovery", C.1): every second
    # seed of the strand, a tenth of them with another k-mer, and some seeds listed twice;
    # the pass through the per-call ABI and through hspz_run_batch against the oracle's
    # pass over the same seeds, and the batch ranges over their window starts
    from ungapped_drop_hsp_amd.pipeline import PassBuffers, run_pass
    ref, qry = random_pair(83, 40_000, 30_000, plant=40, plant_len=(80, 900), identity=0.9,
                           n_frac=0.02)
    p = params_of(SEED_PATTERN, max_hits=20_000)
    span = len(SEED_PATTERN)
    R = oracle.Reference(ref, p["seed_pattern"])
    qc = oracle.strand_codes(qry, "+")
    kmer, q_end, _ = oracle.query_seeds(qc, p["seed_pattern"])
    rng = np.random.default_rng(83)
    k, q = kmer[::2].copy(), q_end[::2].copy()
    swap = rng.random(k.size) < 0.1
    k[swap] = rng.integers(0, 4 ** SEED_PATTERN.count("1"), int(swap.sum()))
    rep = np.sort(rng.choice(k.size, 50, replace=False))
    k, q = np.insert(k, rep, k[rep]).astype(np.uint32), np.insert(q, rep, q[rep]).astype(np.uint32)
    o = oracle.run_pass(R, qc, p, seeds=(k, q, q - span))
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    eng.upload_seeds(k, q)
    assert eng.num_seeds() == k.size
    g = run_pass(eng, 0, k.size, PassBuffers(), collect=True)
    g["seeds"] = eng.get_seeds(0, k.size)
    g["plan_arrays"] = eng.get_plan_arrays(k.size)
    g["lo"] = 0
    assert_pass_equal(g, o)
    assert sum(c["ids"].size for c in o["chunks"]) > 0
    want, acc = _oracle_batch(o)
    st = eng.run_batch(0, k.size)
    assert {kk: st[kk] for kk in want} == want
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc.astype(oracle.HSP_DTYPE).view(np.uint8))
    starts = (q - span).astype(np.int64)
    for lo, hi in [(0, qry.size), (1_000, 20_000), (5, 6)]:
        assert eng.seed_range(lo, hi) == (int(np.searchsorted(starts, lo)),
                                          int(np.searchsorted(starts, hi)))


def test_upload_seeds_errors():
    import ungapped_drop_hsp_amd as h
    ref, qry = random_pair(84, 5_000, 4_000)
    p = params_of(SEED_PATTERN)
    span = len(SEED_PATTERN)
    eng = engine(p)
    eng.upload_reference(ref)
    with pytest.raises(h.HspzError) as ei:
        eng.upload_seeds([1], [span])  # no query strand yet
    assert ei.value.code == -6
    eng.upload_query(qry)
    n = eng.num_seeds()
    for k, q in (([4 ** SEED_PATTERN.count("1")], [span]),  # k-mer out of range
                 ([1], [span - 1]), ([1], [qry.size + 1]),  # window outside the query
                 ([1, 2], [span + 9, span + 8])):           # query ends decrease
        with pytest.raises(h.HspzError) as ei:
            eng.upload_seeds(k, q)
        assert ei.value.code == -1
        assert eng.num_seeds() == n  # left as they were
    eng.upload_seeds([], [])
    assert eng.num_seeds() == 0 and eng.plan(0, 0) == (0, 0)
    eng.upload_seeds([5, 5], [qry.size, qry.size])  # the last window, twice
    assert eng.num_seeds() == 2


def test_run_batch_errors():
    p = params_of(SEED_PATTERN)
    eng = engine(p)
    import ungapped_drop_hsp_amd as h
    with pytest.raises(h.HspzError):
        eng.run_batch(0, 0)  # no reference or query yet
    ref, qry = random_pair(3, 5_000, 5_000, plant=3, plant_len=(200, 400), identity=0.95)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    with pytest.raises(h.HspzError):
        eng.run_batch(0, eng.num_seeds() + 1)
    st = eng.run_batch(0, eng.num_seeds())
    assert st["n_accepted"] == eng.batch_records().size


def _fused_vs_calls(eng, n_seeds):
    """Every chunk through find_hits + score_gate and through find_hits_gate: identical
    flags, and the fused call's anchors equal at every kept slot."""
    import torch
    tot, nch = eng.plan(0, n_seeds)
    checked = 0
    for c in range(nch):
        n = eng.get_chunk(c)["n_hits"]
        a1 = torch.empty(max(n, 1), dtype=torch.int64, device="cuda")
        f1 = torch.empty(max(n, 1) + 16, dtype=torch.uint8, device="cuda")
        a2 = torch.full((max(n, 1),), -1, dtype=torch.int64, device="cuda")
        f2 = torch.full((max(n, 1) + 16,), 7, dtype=torch.uint8, device="cuda")
        eng.find_hits(c, a1)
        eng.score_gate(a1, n, f1)
        eng.find_hits_gate(c, a2, f2)
        g1 = f1[:n].cpu().numpy()
        g2 = f2[:n].cpu().numpy()
        assert np.array_equal(g1, g2), f"chunk {c}: flags differ"
        keep = np.flatnonzero(g1)
        assert np.array_equal(a1[:n].cpu().numpy()[keep], a2[:n].cpu().numpy()[keep])
        checked += n
    return tot, checked


@pytest.mark.parametrize("gate_mode", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{c[3]}-max{c[4]}")
def test_find_hits_gate_matches_the_calls(case, gate_mode):
    seed, nr, nq, pat, mx, nf, plant, ident, gc = case
    ref, qry = random_pair(seed, nr, nq, n_frac=nf, plant=plant, plant_len=(60, 600),
                           identity=ident, gc=gc, alphabet_noise=True)
    eng = engine(params_of(pat, max_hits=mx), gate_mode=gate_mode)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    tot, checked = _fused_vs_calls(eng, eng.num_seeds())
    assert checked == tot


@pytest.mark.parametrize("slices", [1, 2, 3, 64, 256])
def test_bucketed_gate_slice_counts(slices):
    # the bucketed gate ("D. Score gate", D.5) against the oracle for 1 to 256 reference
    # slices, with anchors at both ends, past the ends (they fall in the last slice) and on
    # planted homologs; then shrinking calls on the same engine, down to none
    import torch
    rng = np.random.default_rng(slices)
    ref, qry = random_pair(40 + slices, 24_000, 9_000, n_frac=0.03, plant=20,
                           plant_len=(100, 900), identity=0.92)
    p = params_of("1101011", K=1_500)
    eng = engine(p, gate_mode=4, ref_buckets=slices)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    o, R, qc = oracle_pass(ref, qry, p)
    past = np.asarray([(ref.size + 1 + i) | (int(rng.integers(0, qry.size)) << 32)
                       for i in range(40)], np.uint64)
    a = np.concatenate([_edge_anchors(rng, ref.size, qry.size, 20_000), past] +
                       [c["anchors"] for c in o["chunks"]])
    a = a[rng.permutation(a.size)]
    want = oracle.gate(a, R.codes, qc, p["sub"], p["n_score"], p["xdrop"],
                       oracle.keep_threshold(p["hsp_threshold"]))
    assert 0 < int(want.sum()) < a.size
    at = torch.from_numpy(a.view(np.int64)).cuda()
    for n in (a.size, a.size // 3, 1, 0):
        f = torch.full((max(n, 1),), 0xAB, dtype=torch.uint8, device="cuda")
        eng.score_gate(at, n, f)
        assert np.array_equal(f[:n].cpu().numpy(), want[:n]), f"n={n}"


def _copies_with_spacers(seed, unit_len, copies, spacer):
    """Copies of one random unit separated by random spacers: anchors between copies walk
    to the end of their copy, then drop within the spacer."""
    rng = np.random.default_rng(seed)
    bases = np.frombuffer(b"ACGT", np.uint8)
    unit = bases[rng.integers(0, 4, unit_len)]
    parts = []
    for _ in range(copies):
        parts += [unit, bases[rng.integers(0, 4, spacer)]]
    return np.concatenate(parts)


@pytest.mark.parametrize("gate_mode", [0, 2, 3, 5])
def test_find_hits_gate_defers_most_anchors(gate_mode):
    # "D. Score gate", D.2: the first window stage defers every walk that outlives its
    # window; here most anchors do, more than a wave's LDS segment holds, so deferred
    # anchors reach the second stage both through the global list (segments flushed on
    # the way) and through the second stage the first stage's workgroups run themselves.
    # K is set below and at the median total, so the second stage decides both flags, and
    # out of reach, so that no walk stops early at the threshold and deferrals peak.
    # Flags and kept anchors against the oracle's, chunk by chunk.
    import torch
    seq = _copies_with_spacers(21, 90, 48, 70)
    p0 = params_of("1101011")
    o0, R, qc = oracle_pass(seq, seq, p0)
    a = np.concatenate([c["anchors"] for c in o0["chunks"]])
    tot, _ = oracle.gate_totals(a, R.codes, qc, p0["sub"], p0["n_score"], p0["xdrop"])
    for K in (3000, int(np.median(tot)), 10**6):
        p = params_of("1101011", K=K, max_hits=70_000)
        o, _, _ = oracle_pass(seq, seq, p)
        eng = engine(p, gate_mode=gate_mode)
        eng.upload_reference(seq)
        eng.upload_query(seq)
        total, nch = eng.plan(0, eng.num_seeds())
        assert nch == len(o["chunks"]) > 2 and total == o["total"] > 200_000
        kept = n2_all = 0
        for c in range(nch):
            n = eng.get_chunk(c)["n_hits"]
            at = torch.full((max(n, 1),), -1, dtype=torch.int64, device="cuda")
            f = torch.full((max(n, 1) + 16,), 7, dtype=torch.uint8, device="cuda")
            eng.find_hits_gate(c, at, f)
            want = o["chunks"][c]["flags"]
            got = f[:n].cpu().numpy()
            assert np.array_equal(got, want), f"K={K} chunk {c}: flags differ"
            keep = np.flatnonzero(want)
            got_a = at[:n].cpu().numpy().view(np.uint64)
            assert np.array_equal(got_a[keep], o["chunks"][c]["anchors"][keep])
            n2, nx = eng.debug_gate_deferred()
            assert nx <= n2 <= n
            n2_all += n2
            kept += keep.size
        if K < 10**6:
            assert 0 < kept < total
        else:
            assert kept == 0 and n2_all > total // 4


def test_find_hits_gate_huge_bucket_and_sparse_seeds():
    # one k-mer owning thousands of slots (a poly-A block on both sides), chunked so that
    # chunks start and end inside its bucket's seeds; and a reference sharing almost no
    # k-mers with the query, where most seeds own no slot
    rng = np.random.default_rng(8)
    bases = np.frombuffer(b"ACGT", np.uint8)
    ref = np.concatenate([bases[rng.integers(0, 4, 20_000)], np.full(700, ord("A"), np.uint8),
                          bases[rng.integers(0, 4, 20_000)]])
    qry = np.concatenate([bases[rng.integers(0, 4, 9_000)], np.full(300, ord("A"), np.uint8),
                          bases[rng.integers(0, 4, 9_000)]])
    for gm in (0, 5):  # 5: every chunk key-grouped, also chunks cut inside the bucket
        for mx in (0, 50_000, 3_000):
            eng = engine(params_of(SEED_PATTERN, max_hits=mx), gate_mode=gm)
            eng.upload_reference(ref)
            eng.upload_query(qry)
            tot, checked = _fused_vs_calls(eng, eng.num_seeds())
            assert checked == tot and tot > 100_000
        ref2 = bases[rng.integers(0, 4, 60_000)]
        qry2 = bases[rng.integers(0, 4, 60_000)]
        eng = engine(params_of("11111111111", max_hits=7), gate_mode=gm)
        eng.upload_reference(ref2)
        eng.upload_query(qry2)
        tot, checked = _fused_vs_calls(eng, eng.num_seeds())
        assert checked == tot


@pytest.mark.parametrize("max_hits", [0, 9_000])
def test_key_grouped_runs_of_both_shapes(max_hits):
    # The key-grouped stage enumerates each run of c bucket entries and m seeds with the
    # smaller of the two varying fastest.  One unit is in the reference 3 times and in the
    # query 120 times (c < m), another the other way round (c > m); their runs of 360
    # anchors span several 64-anchor steps and steps start inside them, and the copies are
    # homologous, so walks run long and many anchors are kept.  Everything against the
    # oracle, gated key-grouped (gate_mode 5) and chosen automatically (0).
    rng = np.random.default_rng(41)
    bases = np.frombuffer(b"ACGT", np.uint8)
    a3 = _copies_with_spacers(51, 45, 3, 30)
    a120 = _copies_with_spacers(51, 45, 120, 30)
    b120 = _copies_with_spacers(52, 45, 120, 30)
    b3 = _copies_with_spacers(52, 45, 3, 30)
    ref = np.concatenate([bases[rng.integers(0, 4, 4_000)], a3, bases[rng.integers(0, 4, 3_000)],
                          b120, bases[rng.integers(0, 4, 4_000)]])
    qry = np.concatenate([bases[rng.integers(0, 4, 3_000)], a120, bases[rng.integers(0, 4, 4_000)],
                          b3, bases[rng.integers(0, 4, 3_000)]])
    p = params_of(SEED_PATTERN, max_hits=max_hits)
    o, _, _ = oracle_pass(ref, qry, p)
    assert o["total"] > 20_000
    for gm in (5, 0):
        assert_pass_equal(gpu_full_pass(engine(p, gate_mode=gm), ref, qry), o)


def test_dedup_records_matches_the_oracle():
    # the library's host dedup against the oracle's: random record arrays with heavy
    # repetition, in place through the C ABI, the capacity error, and an empty array
    import ctypes
    import ungapped_drop_hsp_amd as h
    rng = np.random.default_rng(8)
    for n in (0, 1, 7, 5_000):
        rows = rng.integers(0, 5, size=(n, 4))
        rec = np.array([tuple(r) for r in rows], dtype=oracle.HSP_DTYPE)
        want = oracle.dedup_records(rec)
        got = h.dedup_records(rec.view(h.SEGMENT_PAIR))
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
        if n == 0:
            continue
        buf = rec.view(h.SEGMENT_PAIR).copy()
        m = ctypes.c_uint64()
        assert h.lib().hspz_dedup_records(buf.ctypes.data, n, buf.ctypes.data, n,
                                          ctypes.byref(m)) == 0
        assert np.array_equal(buf[:m.value].view(np.uint8), want.view(np.uint8))
        if want.size > 1:
            out = np.zeros(want.size, h.SEGMENT_PAIR)
            rc = h.lib().hspz_dedup_records(rec.ctypes.data, n, out.ctypes.data,
                                            want.size - 1, ctypes.byref(m))
            assert rc == -3 and m.value == want.size and not out.view(np.uint8).any()


def test_dedup_of_run_batch_records():
    # the accepted records of a batch, deduplicated, against the oracle's pass and dedup
    import ungapped_drop_hsp_amd as h
    ref, qry = random_pair(4, 20_000, 20_000, plant=12, plant_len=(300, 900),
                           identity=0.93)
    p = params_of(SEED_PATTERN, max_hits=4_000)
    eng = engine(p)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    o, _, _ = oracle_pass(ref, qry, p)
    _, acc = _oracle_batch(o)
    eng.run_batch(0, eng.num_seeds())
    got = h.dedup_records(eng.batch_records())
    want = oracle.dedup_records(acc)
    assert 0 < want.size < acc.size
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("mat", [1, 2], ids=["own-walks", "shared-walks"])
@pytest.mark.parametrize("seed", range(3))
def test_materialize_every_anchor_near_the_ends(seed, mat):
    # the exact walks read the 4-bit copies with their edge padding: materialize every
    # anchor (no gate) at and next to both ends of both sequences, past the ends, and on
    # planted homologs (walks of hundreds of bases to both sides), and compare every
    # record and status byte with the oracle
    import torch
    rng = np.random.default_rng(300 + seed)
    ref, qry = random_pair(310 + seed, 2_000 + 900 * seed, 1_500 + 1_300 * seed, n_frac=0.04,
                           plant=8, plant_len=(200, 900), identity=0.95)
    p = params_of("11011", K=150)
    eng = engine(p, materialize_mode=mat)
    eng.upload_reference(ref)
    eng.upload_query(qry)
    o, R, qc = oracle_pass(ref, qry, p)
    past = np.asarray([(ref.size + 1) | (5 << 32), 9 | ((qry.size + 3) << 32)], np.uint64)
    a = np.concatenate([_edge_anchors(rng, ref.size, qry.size, 3_000), past] +
                       [c["anchors"][:2_000] for c in o["chunks"]])
    ids = np.arange(a.size, dtype=np.uint32)
    T = oracle.keep_threshold(p["hsp_threshold"])
    oh, ost = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    assert 0 < int(ost.sum()) < a.size
    at = torch.from_numpy(a.view(np.int64)).cuda()
    it = torch.from_numpy(ids.view(np.int32)).cuda()
    hsp = torch.empty((a.size, 4), dtype=torch.int32, device="cuda")
    st = torch.empty(a.size, dtype=torch.uint8, device="cuda")
    eng.materialize(at, it, a.size, hsp, st)
    gs = st.cpu().numpy()
    gh = hsp.cpu().numpy().view(oracle.HSP_DTYPE).reshape(-1)
    assert np.array_equal(gs, ost)
    ok = ost == 1
    bad = np.flatnonzero(gh[ok] != oh[ok])
    assert bad.size == 0, f"{bad.size} records differ, first anchors {a[ok][bad[:5]]}"


@pytest.mark.parametrize("identity", [1.0, 0.93], ids=["identical", "mutated"])
def test_shared_walks_at_the_lane_window_edges(identity):
    # survivors on the main diagonal of a sequence and a copy of it, spaced so that a walk
    # merges into its neighbour on the last bases of the lane stage's first phase (32
    # bases) or on the first bases after it (the walk moves to a packed wave), on the last
    # bases of the lane stage's window, on the first bases past it (the walk goes to the
    # one-wave list), and around the 64- and 512-base tile edges; on identical sequences
    # every walk merges exactly at its neighbour's start
    import torch
    rng = np.random.default_rng(91)
    acgt = np.frombuffer(b"ACGT", np.uint8)
    ref = acgt[rng.integers(0, 4, 24_000)].copy()
    qry = ref.copy()
    if identity < 1.0:  # substitutions, each to one of the three other bases
        code = np.zeros(256, np.int64)
        code[acgt] = np.arange(4)
        flip = rng.random(qry.size) > identity
        qry[flip] = acgt[(code[qry[flip]] + rng.integers(1, 4, int(flip.sum()))) % 4]
    gaps = [1, 2, 7, 8, 9, 24, 25, 31, 32, 33, 40, 41, 63, 64, 65, 127, 128, 129, 130, 136,
            255, 256, 257, 511, 512, 513]
    pos = 200 + np.cumsum(np.tile(gaps, 8))
    pos = pos[pos < ref.size - 200]
    # the main diagonal, plus every third position again on an unrelated diagonal
    r = np.concatenate([pos, pos[::3] + 5_000])
    q = np.concatenate([pos, pos[::3]])
    keep = (r < ref.size) & (q < qry.size)
    a = (r[keep].astype(np.uint64) | (q[keep].astype(np.uint64) << np.uint64(32)))
    a = a[rng.permutation(a.size)]
    p = params_of(SEED_PATTERN)
    T = oracle.keep_threshold(p["hsp_threshold"])
    R = oracle.Reference(ref, p["seed_pattern"])
    qc = oracle.strand_codes(qry, "+")
    ids = np.arange(a.size, dtype=np.uint32)
    oh, ost = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    assert ost.sum() > 0
    for mat in (1, 2):
        eng = engine(p, materialize_mode=mat)
        eng.upload_reference(ref)
        eng.upload_query(qry)
        at = torch.from_numpy(a.view(np.int64)).cuda()
        it = torch.from_numpy(ids.view(np.int32)).cuda()
        hsp = torch.empty((a.size, 4), dtype=torch.int32, device="cuda")
        st = torch.empty(a.size, dtype=torch.uint8, device="cuda")
        eng.materialize(at, it, a.size, hsp, st)
        gs = st.cpu().numpy()
        gh = hsp.cpu().numpy().view(oracle.HSP_DTYPE).reshape(-1)
        assert np.array_equal(gs, ost), f"mode {mat}: status differs"
        ok = ost == 1
        assert np.array_equal(gh[ok], oh[ok]), f"mode {mat}: records differ"


@pytest.mark.parametrize("xdrop", [6, 8], ids=["one-wave-walks", "lane-stage"])
@pytest.mark.parametrize("gap", [1, 3, 9, 30, 150, 600])
def test_shared_walks_with_tied_scores(gap, xdrop):
    # match +1, mismatch -1 and a small X: running scores tie their best all the time, so
    # a walk may merge only at a strictly new best (a tie would move the earliest extent);
    # X = 6 leaves eight-base blocks inexact (one wave per survivor), X = 8 runs the lane
    # stage, and gaps of 150 and 600 bases send the merges to the 512-base tile walks of
    # the listed walks; records and status in both walk modes against the oracle
    import torch
    rng = np.random.default_rng(500 + gap)
    ref, _ = random_pair(60 + gap, 2_000 if gap < 100 else 8_000, 1)
    qry = ref.copy()
    acgt = np.frombuffer(b"ACGT", np.uint8)
    flip = rng.random(qry.size) < 0.3
    qry[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    sub = np.where(np.eye(4, dtype=bool), 1, -1).astype(np.int32)
    p = params_of(SEED_PATTERN, sub=sub, xdrop=xdrop, K=10, n_score=-1)
    pos = np.arange(50, ref.size - 50, gap, dtype=np.uint64)[:500]
    a = np.concatenate([pos | (pos << np.uint64(32)),
                        (pos[::4] + np.uint64(1)) | (pos[::4] << np.uint64(32))])
    T = oracle.keep_threshold(p["hsp_threshold"])
    R = oracle.Reference(ref, p["seed_pattern"])
    qc = oracle.strand_codes(qry, "+")
    ids = np.arange(a.size, dtype=np.uint32)
    oh, ost = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    assert 0 < ost.sum() < a.size
    for mat in (1, 2):
        eng = engine(p, materialize_mode=mat)
        eng.upload_reference(ref)
        eng.upload_query(qry)
        at = torch.from_numpy(a.view(np.int64)).cuda()
        it = torch.from_numpy(ids.view(np.int32)).cuda()
        hsp = torch.empty((a.size, 4), dtype=torch.int32, device="cuda")
        st = torch.empty(a.size, dtype=torch.uint8, device="cuda")
        eng.materialize(at, it, a.size, hsp, st)
        gs = st.cpu().numpy()
        gh = hsp.cpu().numpy().view(oracle.HSP_DTYPE).reshape(-1)
        assert np.array_equal(gs, ost), f"mode {mat}: status differs"
        ok = ost == 1
        assert np.array_equal(gh[ok], oh[ok]), f"mode {mat}: records differ"


def test_shared_walks_on_tandem_repeats_and_duplicates():
    # shared walks where they pay: a tandem array (thousands of survivors on a few
    # diagonals, long chains of merges), plus every survivor listed twice (equal anchors
    # never merge) and anchors in an arbitrary order; records against the oracle
    import torch
    rng = np.random.default_rng(77)
    acgt = np.frombuffer(b"ACGT", np.uint8)
    unit = acgt[rng.integers(0, 4, 97)]
    arr = np.concatenate([unit] * 40).copy()
    flip = rng.random(arr.size) < 0.05
    arr[flip] = acgt[rng.integers(0, 4, int(flip.sum()))]
    ref = np.concatenate([acgt[rng.integers(0, 4, 3_000)], arr, acgt[rng.integers(0, 4, 2_000)]])
    qry = np.concatenate([acgt[rng.integers(0, 4, 1_000)], arr[500:], acgt[rng.integers(0, 4, 900)]])
    p = params_of(SEED_PATTERN)
    o, R, qc = oracle_pass(ref, qry, p)
    a = np.concatenate([c["anchors"][c["ids"]] for c in o["chunks"]])
    assert a.size > 2_000
    a = np.concatenate([a, a[: a.size // 3]])
    a = a[rng.permutation(a.size)]
    T = oracle.keep_threshold(p["hsp_threshold"])
    ids = np.arange(a.size, dtype=np.uint32)
    oh, ost = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    for mat in (1, 2):
        eng = engine(p, materialize_mode=mat)
        eng.upload_reference(ref)
        eng.upload_query(qry)
        at = torch.from_numpy(a.view(np.int64)).cuda()
        it = torch.from_numpy(ids.view(np.int32)).cuda()
        hsp = torch.empty((a.size, 4), dtype=torch.int32, device="cuda")
        st = torch.empty(a.size, dtype=torch.uint8, device="cuda")
        eng.materialize(at, it, a.size, hsp, st)
        gs = st.cpu().numpy()
        gh = hsp.cpu().numpy().view(oracle.HSP_DTYPE).reshape(-1)
        assert np.array_equal(gs, ost), f"mode {mat}: status differs"
        ok = ost == 1
        assert np.array_equal(gh[ok], oh[ok]), f"mode {mat}: records differ"


@pytest.mark.parametrize("pat", ["1", "11", "111111", "1101011"])
def test_plan_counts_from_the_packed_table(pat):
    # The plan reads hit counts and bucket starts from records of 28 keys (a start and a
    # count byte per key); a record holding a count over 254 is read from the full table
    # instead.  Tandem copies of ACGT give a few keys hundreds of hits (marked records)
    # beside ordinary ones; every key of a record is queried, at every offset in it.
    rng = np.random.default_rng(5)
    bases = np.frombuffer(b"ACGT", np.uint8)
    ref = np.concatenate([bases[rng.integers(0, 4, 120_000)],
                          np.frombuffer(b"ACGT" * 400, np.uint8),
                          bases[rng.integers(0, 4, 30_000)]])
    qry = np.concatenate([bases[rng.integers(0, 4, 40_000)], ref[119_000:123_000]])
    p = params_of(pat)
    o, _, _ = oracle_pass(ref, qry, p)
    assert int(o["count"].max()) > 254
    eng = engine(p)
    assert_pass_equal(gpu_full_pass(eng, ref, qry), o)


def test_key_grouped_stage_upload_orders_and_caller_seeds():
    # the key-grouped first stage needs the grouped seeds and their buckets: the
    # reference uploaded after the query, uploaded again, and caller seeds (some k-mers
    # repeated, others absent from the reference) must each give the oracle's records
    ref, qry = random_pair(41, 30_000, 25_000, n_frac=0.02, plant=20, plant_len=(80, 700),
                           identity=0.9, gc=0.41)
    p = params_of("1101011", max_hits=20_000)
    o, R, qc = oracle_pass(ref, qry, p)
    want, acc = _oracle_batch(o)
    eng = engine(p, gate_mode=5)
    eng.upload_query(qry)
    eng.upload_reference(ref)  # after the query
    st = eng.run_batch(0, eng.num_seeds())
    assert {k: st[k] for k in want} == want
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc.astype(oracle.HSP_DTYPE).view(np.uint8))
    ref_b, _ = random_pair(42, 30_000, 1, gc=0.41)
    eng.upload_reference(ref_b)  # a different reference: new buckets for the same runs
    ob, _, _ = oracle_pass(ref_b, qry, p)
    want_b, acc_b = _oracle_batch(ob)
    st = eng.run_batch(0, eng.num_seeds())
    assert {k: st[k] for k in want_b} == want_b
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc_b.astype(oracle.HSP_DTYPE).view(np.uint8))
    # caller seeds: every third seed, with a run of one repeated k-mer
    kmer, q_end, _ = oracle.query_seeds(qc, p["seed_pattern"])
    k2, q2 = kmer[::3].copy(), q_end[::3].copy()
    k2[100:400] = k2[100]
    eng.upload_reference(ref)
    eng.upload_seeds(k2, q2)
    oc = oracle.run_pass(R, qc, p, seeds=(k2, q2, q2 - 7))
    want_c, acc_c = _oracle_batch(oc)
    st = eng.run_batch(0, eng.num_seeds())
    assert {k: st[k] for k in want_c} == want_c
    assert np.array_equal(eng.batch_records().view(np.uint8),
                          acc_c.astype(oracle.HSP_DTYPE).view(np.uint8))
