"""Pins for the CPU oracle: page values, closed forms, brute force and invariants.

None of these re-run the oracle's own formula; each fixes a value by another route
(the pages' worked example, IEEE-754 rounding, hand arithmetic, brute-force
enumeration or a prefix-array restatement of the stopping rule).
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import HOXD70, SEED_PATTERN, random_pair

GOLD = os.path.join(os.path.dirname(__file__), "golden")
SUB = np.asarray(HOXD70, np.int32)
X, K, NS = 910, 3000, -100


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ hit discovery

def test_worked_example_prefix_and_slots():
    g = _gold("hit_discovery_worked_example.json")
    counts = np.asarray(g["counts"], np.uint32)
    P, ok = oracle.prefix(counts)
    assert ok and P.tolist() == g["inclusive_prefix"]
    # occurrence j of seed s carries the marker 100*s + j so its slot can be read back
    first = np.zeros(counts.size, np.int64)
    ends = []
    for s, c in enumerate(counts):
        first[s] = len(ends)
        ends.extend(100 * s + j for j in range(c))
    ends = np.asarray(ends, np.uint32)
    q_end = np.arange(counts.size, dtype=np.uint32)
    ch = oracle.chunks(P, 0)
    assert len(ch) == 1
    a = oracle.anchors(P, counts, first, ends, q_end, ch[0])
    slot_of = {int(v & 0xFFFFFFFF): i for i, v in enumerate(a)}
    for s, slots in g["slots_by_seed_in_occurrence_order"].items():
        s = int(s)
        got = [slot_of[100 * s + j] for j in range(len(slots))]
        assert got == slots
        assert all(int(a[x] >> 32) == s for x in got)


@pytest.mark.parametrize("case", _gold("chunk_cuts_worked_example.json")["cases"],
                         ids=lambda c: f"max{c['max_hits']}")
def test_chunk_cuts_worked_example(case):
    P, _ = oracle.prefix(np.asarray([0, 3, 1, 0, 5], np.uint32))
    got = [[c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]]
           for c in oracle.chunks(P, case["max_hits"])]
    assert got == case["chunks"]


def test_chunk_local_slots_of_worked_example_under_max4():
    # seed 4 lands in the second chunk (base 4): local slots 9-1-4-j = 4..0
    counts = np.asarray([0, 3, 1, 0, 5], np.uint32)
    P, _ = oracle.prefix(counts)
    first = np.asarray([0, 0, 3, 4, 4], np.int64)
    ends = np.asarray([10, 11, 12, 20, 40, 41, 42, 43, 44], np.uint32)
    ch = oracle.chunks(P, 4)
    a = oracle.anchors(P, counts, first, ends, np.arange(5, dtype=np.uint32), ch[1])
    assert [int(v & 0xFFFFFFFF) for v in a] == [44, 43, 42, 41, 40]


def test_zero_total_gives_no_chunks():
    P, ok = oracle.prefix(np.zeros(7, np.uint32))
    assert ok and oracle.chunks(P, 0) == [] and oracle.chunks(P, 3) == []


def test_refusal_beyond_32_bit_total():
    P, ok = oracle.prefix(np.asarray([0xFFFFFFFF, 1], np.uint32))
    assert not ok and int(P[-1]) == 1 << 32
    P, ok = oracle.prefix(np.asarray([0xFFFFFFFE, 1], np.uint32))
    assert ok and int(P[-1]) == 0xFFFFFFFF


@pytest.mark.parametrize("seed", range(6))
def test_chunk_invariants_random(seed):
    rng = np.random.default_rng(seed)
    counts = rng.choice([0, 0, 1, 2, 3, 17, 40], size=400).astype(np.uint32)
    P, _ = oracle.prefix(counts)
    total = int(P[-1])
    for mx in (1, 2, 3, 16, 50, 333, total, total + 1, 0):
        ch = oracle.chunks(P, mx)
        # contiguous, covering every seed, no seed split
        assert ch[0]["seed_lo"] == 0 and ch[-1]["seed_hi"] == counts.size - 1
        for a, b in zip(ch, ch[1:]):
            assert b["seed_lo"] == a["seed_hi"] + 1
        assert sum(c["n_hits"] for c in ch) == total
        for c in ch:
            assert c["n_hits"] == int(counts[c["seed_lo"]:c["seed_hi"] + 1].sum())
            if mx:
                # at most one seed bucket over the cap
                assert c["n_hits"] < mx + int(counts[c["seed_hi"]]) or c is ch[-1]
                if c is not ch[-1]:
                    assert c["n_hits"] >= mx


# ------------------------------------------------------------------ seeds and index

def test_pattern_weight_and_span():
    care, span = oracle.pattern(SEED_PATTERN)
    assert span == 19 and care.tolist() == [0, 1, 2, 4, 7, 8, 11, 13, 15, 16, 17, 18]
    for bad in ("", "0111", "1110", "11x1", "1" * 17):
        with pytest.raises(ValueError):
            oracle.pattern(bad)


def test_encode_rules():
    c = oracle.encode(b"ACGTacgtNnRY-*")
    assert c.tolist() == [0, 1, 2, 3, 0, 1, 2, 3, 4, 4, 4, 4, 4, 4]
    assert oracle.revcomp(oracle.encode(b"AACGTN")).tolist() == [4, 0, 1, 2, 3, 3]


def test_window_validity_and_key():
    # 19-base window: care positions hold A,C,G,T,... ; don't-care positions may be N
    pat = "1101"
    base = b"ACNG"  # care at 0,1,3 -> A,C,G ; position 2 is don't-care
    kmer, q_end, pos = oracle.query_seeds(oracle.encode(base), pat)
    assert pos.tolist() == [0] and q_end.tolist() == [4]
    assert kmer.tolist() == [(0 << 4) | (1 << 2) | 2]
    kmer, _, _ = oracle.query_seeds(oracle.encode(b"ANCG"), pat)
    assert kmer.size == 0
    kmer, _, pos = oracle.query_seeds(oracle.encode(b"TTTTT"), "11")
    assert pos.tolist() == [0, 1, 2, 3] and set(kmer.tolist()) == {15}


@pytest.mark.parametrize("seed", range(8))
def test_index_matches_brute_force(seed):
    ref, qry = random_pair(seed, 700, 600, n_frac=0.05, plant=4, plant_len=(30, 120),
                           identity=0.95, gc=0.5, alphabet_noise=True)
    pat = "1101011" if seed % 2 else "11011"
    rc, qc = oracle.encode(ref), oracle.encode(qry)
    ref_o = oracle.Reference(ref, pat)
    kmer, q_end, _ = oracle.query_seeds(qc, pat)
    cnt, first = oracle.counts_indexed(ref_o.keys, ref_o.ends, kmer)
    assert np.array_equal(cnt, oracle.counts_brute(rc, pat, kmer))
    P, ok = oracle.prefix(cnt)
    assert ok
    for mx in (0, 7, 64):
        for ch in oracle.chunks(P, mx):
            a = oracle.anchors(P, cnt, first, ref_o.ends, q_end, ch)
            b = oracle.anchors_brute(rc, pat, P, kmer, q_end, ch)
            assert np.array_equal(a, b)


def test_brute_force_anchor_set_is_all_equal_key_pairs():
    ref, qry = random_pair(99, 300, 300, plant=3, plant_len=(40, 80), identity=1.0)
    pat = "111"
    rc, qc = oracle.encode(ref), oracle.encode(qry)
    kmer, q_end, qpos = oracle.query_seeds(qc, pat)
    cnt = oracle.counts_brute(rc, pat, kmer)
    P, _ = oracle.prefix(cnt)
    ch = oracle.chunks(P, 0)[0]
    a = oracle.anchors_brute(rc, pat, P, kmer, q_end, ch)
    want = set()
    for i in range(len(rc) - 2):
        for j in range(len(qc) - 2):
            if rc[i:i + 3].max() < 4 and (rc[i:i + 3] == qc[j:j + 3]).all():
                want.add((i + 3, j + 3))
    assert {(int(v & 0xFFFFFFFF), int(v >> 32)) for v in a} == want
    assert len(want) == len(a)


# ------------------------------------------------------------------ threshold

def test_keep_threshold_closed_forms():
    assert oracle.keep_threshold(3000) == 3000
    assert oracle.keep_threshold(1) == 1
    # float32 has a 24-bit significand: 2^24 + 1 rounds to 2^24 (ties-to-even)
    assert oracle.keep_threshold((1 << 24) + 1) == 1 << 24
    # 2^24 + 3 rounds up to 2^24 + 4, which 2^24 + 3 itself reaches
    assert oracle.keep_threshold((1 << 24) + 3) == (1 << 24) + 3
    # 2^25 + 1 rounds to 2^25 (spacing 4 above 2^25); 2^25 - 1 sits halfway between
    # 2^25 - 2 and 2^25 (spacing 2 below) and ties to the even 2^25, so it is kept
    assert oracle.keep_threshold((1 << 25) + 1) == (1 << 25) - 1
    for k in (2, 17, 4095, 1 << 20, (1 << 24) - 1, 1 << 24):
        assert oracle.keep_threshold(k) == k


def test_keep_threshold_is_least_kept_total():
    for k in (3000, (1 << 24) + 1, (1 << 25) + 5, 123456789):
        t = oracle.keep_threshold(k)
        fk = np.float32(k)
        assert np.float32(t) >= fk and np.float32(t - 1) < fk


# ------------------------------------------------------------------ X-drop

def test_xdrop_hand_worked_case():
    g = _gold("xdrop_hand_worked.json")
    rc, qc = oracle.encode(g["ref"].encode()), oracle.encode(g["query"].encode())
    # the listed running scores are the matrix entries summed by hand
    sig = [int(SUB[a, b]) for a, b in zip(rc, qc)]
    assert np.cumsum(sig)[:19].tolist() == g["running_scores"]
    best, ext = oracle.xdrop(rc, qc, 0, 0, +1, SUB, NS, g["xdrop"])
    assert (best, ext) == (g["right_best"], g["right_extent"])
    anchor = np.asarray([0], np.uint64)  # r = q = 0: no left walk
    tot, steps = oracle.gate_totals(anchor, rc, qc, SUB, NS, g["xdrop"])
    assert tot.tolist() == [91] and steps.tolist() == [g["bases_scored"]]


def test_xdrop_uses_ref_row_query_column():
    # asymmetric matrix: sub[A][C] = 50, sub[C][A] = -50
    sub = np.full((4, 4), -10, np.int32)
    sub[0, 1], sub[1, 0] = 50, -50
    rc, qc = oracle.encode(b"A"), oracle.encode(b"C")
    assert oracle.xdrop(rc, qc, 0, 0, +1, sub, NS, 100) == (50, 1)
    assert oracle.xdrop(qc, rc, 0, 0, +1, sub, NS, 100) == (0, 0)
    # left walk scores the base before the anchor
    assert oracle.xdrop(rc, qc, 1, 1, -1, sub, NS, 100) == (50, 1)
    assert oracle.xdrop(rc, qc, 0, 0, -1, sub, NS, 100) == (0, 0)


def test_xdrop_identical_sequences_closed_form():
    ref, _ = random_pair(5, 400, 1)
    rc = oracle.encode(ref)
    diag = SUB[rc, rc].astype(np.int64)
    for r in (0, 1, 57, 399, 400):
        R, k = oracle.xdrop(rc, rc, r, r, +1, SUB, NS, X)
        L, m = oracle.xdrop(rc, rc, r, r, -1, SUB, NS, X)
        assert (R, k) == (int(diag[r:].sum()), 400 - r)
        assert (L, m) == (int(diag[:r].sum()), r)
    a = np.asarray([57 | (57 << 32)], np.uint64)
    ids = np.asarray([0], np.uint32)
    hsp, st = oracle.materialize(a, ids, rc, rc, SUB, NS, X, 1)
    assert (int(hsp[0]["ref_start"]), int(hsp[0]["query_start"]), int(hsp[0]["len"]),
            int(hsp[0]["score"])) == (0, 0, 399, int(diag.sum()))
    assert st.tolist() == [1]


def test_xdrop_all_mismatch_and_edges():
    rc = oracle.encode(b"A" * 50)
    qc = oracle.encode(b"T" * 50)
    assert oracle.xdrop(rc, qc, 10, 10, +1, SUB, NS, X) == (0, 0)
    assert oracle.xdrop(rc, qc, 10, 10, -1, SUB, NS, X) == (0, 0)
    # N pairs score n_score
    rn, qn = oracle.encode(b"NA"), oracle.encode(b"AA")
    assert oracle.xdrop(rn, qn, 0, 0, +1, SUB, NS, X) == (0, 0)
    assert oracle.xdrop(rn, qn, 0, 0, +1, SUB, 30, X) == (121, 2)
    # walks stop at the end of the shorter side
    assert oracle.xdrop(oracle.encode(b"AAAA"), oracle.encode(b"AA"), 0, 0, +1, SUB, NS,
                        X) == (182, 2)
    assert oracle.xdrop(oracle.encode(b"AAAA"), oracle.encode(b"AA"), 4, 2, -1, SUB, NS,
                        X) == (182, 2)


def _walk_by_prefix_arrays(sig, X):
    """The stopping rule restated on whole prefix arrays (no running loop state)."""
    if len(sig) == 0:
        return 0, 0, 0
    s = np.concatenate(([0], np.cumsum(sig)))          # s[0] = 0 is the empty prefix
    run_max = np.maximum.accumulate(s)
    dropped = np.nonzero(run_max[1:] - s[1:] > X)[0]
    n = (dropped[0] + 1) if dropped.size else len(sig)  # bases scored
    best = int(run_max[n])
    ext = int(np.argmax(s[: n + 1] == best))            # first prefix attaining best
    return best, ext, n


@pytest.mark.parametrize("seed", range(10))
def test_xdrop_matches_prefix_array_definition(seed):
    rng = np.random.default_rng(seed)
    for trial in range(60):
        n = int(rng.integers(0, 80))
        rc = rng.integers(0, 5, size=n).astype(np.uint8)
        qc = np.where(rng.random(n) < 0.6, rc, rng.integers(0, 5, size=n)).astype(np.uint8)
        x = int(rng.choice([0, 1, 50, 200, 910]))
        ns = int(rng.choice([-100, 0, 40]))
        sig = np.where((rc > 3) | (qc > 3), ns, SUB[np.minimum(rc, 3), np.minimum(qc, 3)])
        want = _walk_by_prefix_arrays(sig.astype(np.int64), x)
        got = oracle.xdrop(rc, qc, 0, 0, +1, SUB, ns, x)
        assert got == want[:2]
        # the left walk is the same rule on the reversed bases before the anchor
        gotl = oracle.xdrop(rc, qc, n, n, -1, SUB, ns, x)
        assert gotl == _walk_by_prefix_arrays(sig[::-1].astype(np.int64), x)[:2]


# ------------------------------------------------------------------ gate + materialize

def _small_pass(seed, max_hits=0, pat=SEED_PATTERN):
    ref, qry = random_pair(seed, 3000, 3000, n_frac=0.02, plant=6, plant_len=(80, 400),
                           identity=0.9, gc=0.41)
    params = dict(seed_pattern=pat, sub=HOXD70, n_score=NS, xdrop=X, hsp_threshold=K,
                  max_hits=max_hits)
    r = oracle.Reference(ref, pat)
    qc = oracle.strand_codes(qry, "+")
    return r, qc, params, oracle.run_pass(r, qc, params)


@pytest.mark.parametrize("seed", range(4))
def test_gate_flags_agree_with_exact_totals(seed):
    r, qc, params, out = _small_pass(seed)
    for ch in out["chunks"]:
        tot, _ = oracle.gate_totals(ch["anchors"], r.codes, qc, SUB, NS, X)
        assert np.array_equal(ch["flags"], (tot >= K).astype(np.uint8))
        assert np.array_equal(ch["ids"], np.nonzero(ch["flags"])[0].astype(np.uint32))
        # materializer's score equals the gate's total for every survivor
        assert np.array_equal(ch["hsp"]["score"].astype(np.int64), tot[ch["ids"]])
        assert ch["status"].all()  # integer decision: accepted == survivors
        assert np.array_equal(ch["accepted"], ch["hsp"][ch["status"] == 1])


@pytest.mark.parametrize("seed", range(4))
def test_segment_pair_is_interval_sum_with_earliest_ends(seed):
    r, qc, params, out = _small_pass(seed)
    rc = r.codes
    for ch in out["chunks"]:
        for rec, aid in zip(ch["hsp"], ch["ids"]):
            a = int(ch["anchors"][aid])
            ar, aq = a & 0xFFFFFFFF, a >> 32
            rs, qs, ln = int(rec["ref_start"]), int(rec["query_start"]), int(rec["len"])
            assert ar - rs == aq - qs  # same diagonal as the anchor
            seg_r, seg_q = rc[rs:rs + ln + 1], qc[qs:qs + ln + 1]
            sig = np.where((seg_r > 3) | (seg_q > 3), NS,
                           SUB[np.minimum(seg_r, 3), np.minimum(seg_q, 3)])
            assert int(sig.sum()) == int(rec["score"])
            # earliest endpoints: the right part's best is first reached at its end
            right = np.cumsum(sig[ar - rs:])
            if right.size:
                assert right.argmax() == right.size - 1
                assert (right[:-1] < right[-1]).all()


def test_gate_monotone_in_x_and_k():
    ref, qry = random_pair(11, 4000, 4000, plant=8, plant_len=(40, 300), identity=0.8)
    pat = "11011011"
    r = oracle.Reference(ref, pat)
    qc = oracle.strand_codes(qry, "+")
    kmer, q_end, _ = oracle.query_seeds(qc, pat)
    cnt, first = oracle.counts_indexed(r.keys, r.ends, kmer)
    P, _ = oracle.prefix(cnt)
    a = oracle.anchors(P, cnt, first, r.ends, q_end, oracle.chunks(P, 0)[0])
    prev = None
    for x in (0, 100, 400, 910, 2000):
        f = oracle.gate(a, r.codes, qc, SUB, NS, x, 1500)
        if prev is not None:
            assert (f >= prev).all()
        prev = f
    prev = None
    for k in (500, 1000, 1500, 3000):
        f = oracle.gate(a, r.codes, qc, SUB, NS, 910, oracle.keep_threshold(k))
        if prev is not None:
            assert (f <= prev).all()
        prev = f


def test_random_background_anchors_do_not_survive():
    # no planted homology at 41% GC: the pages' funnel has almost every hit rejected
    ref, qry = random_pair(21, 60000, 60000, gc=0.41)
    r = oracle.Reference(ref, SEED_PATTERN)
    qc = oracle.strand_codes(qry, "+")
    params = dict(seed_pattern=SEED_PATTERN, sub=HOXD70, n_score=NS, xdrop=X,
                  hsp_threshold=K, max_hits=0)
    out = oracle.run_pass(r, qc, params)
    n = sum(ch["anchors"].size for ch in out["chunks"])
    s = sum(ch["ids"].size for ch in out["chunks"])
    assert n > 100 and s == 0


# ------------------------------------------------------------------ entropy-adjusted accept

def _shannon_bits(codes):
    """Entropy in bits of the A/C/G/T composition, from -sum p log2 p (N dropped)."""
    c = np.bincount(codes[codes < 4], minlength=4).astype(np.float64)
    n = c.sum()
    p = c[c > 0] / n
    return float(-(p * np.log2(p)).sum())


def test_entropy_closed_forms():
    enc = oracle.encode
    assert oracle.entropy_bits(enc(b"AAAAAAAAAA"), 0, 9) == 0.0          # one letter: 0 bits
    assert oracle.entropy_bits(enc(b"ACGT" * 16), 0, 63) == 2.0          # uniform, n = 64: 2 bits
    assert oracle.entropy_bits(enc(b"AC" * 32), 0, 63) == 1.0            # two letters: 1 bit
    assert oracle.entropy_bits(enc(b"NNNNN"), 0, 4) == -1.0              # nothing to count
    # N inside the interval is excluded; the interval is closed (len + 1 bases)
    assert oracle.entropy_bits(enc(b"ANCNGNT"), 0, 6) == 2.0
    assert oracle.entropy_bits(enc(b"ACGTA"), 0, 3) == 2.0
    assert oracle.entropy_bits(enc(b"ACGTA"), 1, 3) == 2.0


@pytest.mark.parametrize("seed", range(4))
def test_entropy_matches_shannon_definition(seed):
    rng = np.random.default_rng(seed)
    ref, _ = random_pair(seed, 3000, 1, n_frac=0.05, gc=0.2 + 0.15 * seed)
    rc = oracle.encode(ref)
    for _ in range(200):
        s = int(rng.integers(0, rc.size - 1))
        l = int(rng.integers(0, min(400, rc.size - s - 1)))
        want = _shannon_bits(rc[s:s + l + 1])
        got = oracle.entropy_bits(rc, s, l)
        if (rc[s:s + l + 1] < 4).any():
            assert abs(got - want) < 1e-12
        else:
            assert got == -1.0


def test_entropy_mode_decision():
    # records from planted homologs; mode 1 keeps a record iff score * H >= 2K as well
    ref, qry = random_pair(21, 20_000, 20_000, plant=40, plant_len=(60, 500), identity=0.95,
                           gc=0.5)
    # low-complexity planted copies too, so that the entropy test rejects some records
    ref[1000:1120] = np.frombuffer(b"AT" * 60, np.uint8)
    qry[5000:5120] = np.frombuffer(b"AT" * 60, np.uint8)
    ref[3000:3090] = np.frombuffer(b"A" * 90, np.uint8)
    qry[8000:8090] = np.frombuffer(b"A" * 90, np.uint8)
    K = 600
    p = dict(seed_pattern="1101011", sub=SUB, n_score=NS, xdrop=X, hsp_threshold=K,
             max_hits=0)
    R = oracle.Reference(ref, p["seed_pattern"])
    qc = oracle.encode(qry)
    o0 = oracle.run_pass(R, qc, p)
    o1 = oracle.run_pass(R, qc, dict(p, entropy_mode=1))
    T = oracle.keep_threshold(K)
    n_rej = 0
    for c0, c1 in zip(o0["chunks"], o1["chunks"]):
        assert np.array_equal(c0["hsp"], c1["hsp"])  # the records do not depend on the mode
        for h, s0, s1 in zip(c0["hsp"], c0["status"], c1["status"]):
            H = _shannon_bits(R.codes[h["ref_start"]:h["ref_start"] + h["len"] + 1])
            margin = float(h["score"]) * H - 2.0 * K
            if abs(margin) < 1e-6 * K:
                continue
            assert s0 == (h["score"] >= T)
            assert s1 == (s0 and margin > 0)
            n_rej += int(s0 and not s1)
        assert set(map(bytes, c1["accepted"])) <= set(map(bytes, c0["accepted"]))
    assert n_rej > 0


# ------------------------------------------------------------------ host dedup

def _records(rows):
    return np.array([tuple(r) for r in rows], dtype=oracle.HSP_DTYPE)


def test_dedup_special_cases():
    assert oracle.dedup_records(_records([])).size == 0
    same = _records([(5, 7, 30, 3100)] * 6)
    assert oracle.dedup_records(same).tolist() == [(5, 7, 30, 3100)]
    distinct = _records([(i, 2 * i, 10 + i, 3000 + i) for i in range(9)])
    assert oracle.dedup_records(distinct).tolist() == distinct.tolist()
    # records that differ in one field only are all kept, in their order
    one_off = _records([(1, 1, 1, 1), (2, 1, 1, 1), (1, 2, 1, 1), (1, 1, 2, 1),
                        (1, 1, 1, 2), (1, 1, 1, 1)])
    assert oracle.dedup_records(one_off).tolist() == one_off[:5].tolist()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dedup_against_brute_force(seed):
    # record i is kept iff no earlier record equals it in all four fields
    rng = np.random.default_rng(seed)
    n = 400
    rows = rng.integers(0, 4, size=(n, 4))
    rows[:, 3] += 2999  # scores near the threshold
    rec = _records(rows)
    keep = [i for i in range(n) if not any((rows[j] == rows[i]).all() for j in range(i))]
    got = oracle.dedup_records(rec)
    assert got.tolist() == rec[keep].tolist()
    assert oracle.dedup_records(got).tolist() == got.tolist()  # idempotent


def test_dedup_of_a_pass_removes_repeated_records_only():
    # anchors on the diagonal of one planted homolog materialize the same interval, so a
    # pass's accepted records repeat; dedup keeps each distinct record once, in order
    ref, qry = random_pair(4, 20_000, 20_000, plant=12, plant_len=(300, 900),
                           identity=0.93)
    p = dict(seed_pattern=SEED_PATTERN, sub=HOXD70, n_score=NS, xdrop=X, hsp_threshold=K,
             max_hits=0, entropy_mode=0)
    R = oracle.Reference(ref, SEED_PATTERN)
    o = oracle.run_pass(R, oracle.strand_codes(qry, "+"), p)
    acc = np.concatenate([c["accepted"] for c in o["chunks"]])
    d = oracle.dedup_records(acc)
    assert 0 < d.size < acc.size
    assert len(set(d.tolist())) == d.size and set(d.tolist()) == set(acc.tolist())
    first = [acc.tolist().index(r) for r in d.tolist()]
    assert first == sorted(first)


# ------------------------------------------------------------------ keep boundary

def test_keep_boundary_hand_worked():
    # "D. Score gate", D.3: kept when the total is at least the threshold.  The totals
    # are worked by hand in the golden file; a threshold equal to the total keeps the
    # anchor and one above drops it, in the gate and in the materializer's decision.
    g = _gold("keep_boundary_hand_worked.json")
    for case in g["cases"]:
        rc, qc = oracle.encode(case["ref"].encode()), oracle.encode(case["query"].encode())
        r, q = case["r"], case["q"]
        assert oracle.xdrop(rc, qc, r, q, +1, SUB, NS, g["xdrop"]) == \
            (case["right_best"], case["right_extent"])
        assert oracle.xdrop(rc, qc, r, q, -1, SUB, NS, g["xdrop"]) == \
            (case["left_best"], case["left_extent"])
        a = np.asarray([r | (q << 32)], np.uint64)
        ids = np.zeros(1, np.uint32)
        tot = case["total"]
        for K, keep in ((tot, 1), (tot + 1, 0), (tot - 1, 1)):
            T = oracle.keep_threshold(K)
            assert T == K  # |K| <= 2^24: the single-precision threshold is K itself
            assert oracle.gate(a, rc, qc, SUB, NS, g["xdrop"], T).tolist() == [keep]
            hsp, st = oracle.materialize(a, ids, rc, qc, SUB, NS, g["xdrop"], T, K=K)
            assert st.tolist() == [keep]
            assert [int(hsp[0][f]) for f in ("ref_start", "query_start", "len", "score")] \
                == case["record"]


# ------------------------------------------------------------------ score width

def test_score_width_refusal_at_the_int32_limit():
    # identical all-C sequences: every pair scores HOXD70 C/C = 100, so neither walk ever
    # drops and the total of an anchor is 100 times the sequence length.  21,474,836
    # bases give 2,147,483,600 <= 2^31 - 1 and the record is stored; one base more gives
    # 2,147,483,700, which does not fit in int32, and the oracle refuses the call.
    for n, fits in ((21_474_836, True), (21_474_837, False)):
        c = oracle.encode(b"C" * n)
        a = np.asarray([(n // 2) | ((n // 2) << 32)], np.uint64)
        ids = np.zeros(1, np.uint32)
        tot, _ = oracle.gate_totals(a, c, c, SUB, NS, X)
        assert tot.tolist() == [100 * n]
        if fits:
            hsp, st = oracle.materialize(a, ids, c, c, SUB, NS, X, 3000)
            assert int(hsp[0]["score"]) == 100 * n == 2_147_483_600
            assert (int(hsp[0]["ref_start"]), int(hsp[0]["len"])) == (0, n - 1)
            assert st.tolist() == [1]
        else:
            with pytest.raises(OverflowError):
                oracle.materialize(a, ids, c, c, SUB, NS, X, 3000)
