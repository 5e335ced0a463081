"""Device seeder and reference indexer against the oracle ("C. Hit discovery", C.1).

The index table is compared whole: the cumulative bucket-end table (leading 0, one entry
per packed k-mer) against the oracle's sorted key list, and the bucket array of reference
end coordinates element by element (the order inside a bucket is ascending, so it is
unique).  Seeds are compared whole too: packed k-mer, query end, and the window start
behind hspz_seed_range.  Inputs mix case, N runs and bytes that are not bases; lengths
sit around the seed span and across the radix sort's 2,048-pair blocks (one, two and
three blocks); seed weights
1, 4, 12 and 13 take one to four 8-bit radix passes.
"""
import numpy as np
import pytest

import oracle
from gpu_util import engine, params_of, require_gpu

pytestmark = pytest.mark.gpu

PAT12 = "1110100110010101111"
PAT13 = "1111111111111"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _messy(rng, n, gc=0.45):
    """Random bases with N runs, lower case and a sprinkle of other bytes."""
    p = np.array([(1 - gc) / 2, gc / 2, gc / 2, (1 - gc) / 2])
    s = np.frombuffer(b"ACGT", np.uint8)[rng.choice(4, size=n, p=p)].copy()
    if n == 0:
        return s
    low = rng.random(n) < 0.2
    s[low] = s[low] + 32
    for _ in range(max(1, n // 20000)):
        a = int(rng.integers(0, n))
        s[a:a + int(rng.integers(1, 60))] = ord("N")
    odd = rng.random(n) < 0.002
    s[odd] = np.frombuffer(b"RYnKM-\n*", np.uint8)[rng.integers(0, 8, size=int(odd.sum()))]
    return s


def _check_index(eng, R, pat):
    end, pos = eng.get_index()
    w = pat.count("1")
    nb = 1 << (2 * w)
    assert end.size == nb + 1
    want_end = np.searchsorted(R.keys, np.arange(nb + 1, dtype=np.uint64), side="left")
    assert end[0] == 0
    assert np.array_equal(end.astype(np.int64), want_end.astype(np.int64)), "bucket ends differ"
    assert np.array_equal(pos, R.ends), "bucket contents differ"


def _check_seeds(eng, qc, pat):
    kmer, q_end, spos = oracle.query_seeds(qc, pat)
    assert eng.num_seeds() == kmer.size
    gk, gq = eng.get_seeds(0, kmer.size)
    assert np.array_equal(gk, kmer) and np.array_equal(gq, q_end), "seeds differ"
    n = qc.size
    for lo, hi in [(0, n), (0, 0), (n // 3, n // 2), (n // 2, n + 5), (1, 2)]:
        want = (int(np.searchsorted(spos, lo)), int(np.searchsorted(spos, hi)))
        assert eng.seed_range(lo, hi) == want


LENGTHS = [0, 1, 18, 19, 20, 2047 + 18, 2048 + 18, 2049 + 18, 4095 + 18, 4096 + 18,
           4097 + 18, 70_001, 1_000_003]


@pytest.mark.parametrize("n", LENGTHS)
def test_index_and_seeds_lengths(n):
    rng = np.random.default_rng(n)
    ref = _messy(rng, n)
    qry = _messy(rng, n // 2 + 7)
    p = params_of(PAT12)
    eng = engine(p)
    eng.upload_reference(ref)
    R = oracle.Reference(ref, PAT12)
    _check_index(eng, R, PAT12)
    for strand in ("+", "-"):
        eng.upload_query(qry, strand=1 if strand == "-" else 0)
        _check_seeds(eng, oracle.strand_codes(qry, strand), PAT12)


@pytest.mark.parametrize("pat", ["1", "1101", PAT12, PAT13])
def test_index_seed_weights(pat):
    rng = np.random.default_rng(len(pat))
    ref = _messy(rng, 300_017)
    qry = _messy(rng, 50_003)
    eng = engine(params_of(pat))
    eng.upload_reference(ref)
    _check_index(eng, oracle.Reference(ref, pat), pat)
    eng.upload_query(qry, strand=1)
    _check_seeds(eng, oracle.strand_codes(qry, "-"), pat)


def test_single_bucket_keeps_position_order():
    # every window has the same key: one bucket of 69,982 ends spanning 35 radix blocks,
    # which must stay in ascending order through every stable pass
    ref = np.frombuffer(b"A" * 70_000, np.uint8)
    eng = engine(params_of(PAT12))
    eng.upload_reference(ref)
    R = oracle.Reference(ref, PAT12)
    _check_index(eng, R, PAT12)
    end, pos = eng.get_index()
    assert pos.size == 70_000 - len(PAT12) + 1
    assert np.all(np.diff(pos.astype(np.int64)) == 1)


def test_reupload_replaces_index():
    rng = np.random.default_rng(5)
    eng = engine(params_of(PAT12))
    for n in (200_000, 30_000, 0, 90_000):
        ref = _messy(rng, n)
        eng.upload_reference(ref)
        _check_index(eng, oracle.Reference(ref, PAT12), PAT12)
