"""Parity at the workloads' full sizes (c2 5 Mb, c3 50 Mb, c4 200 Mb both strands).

The HIP path runs exactly as bench.py runs it (whole query batches, the workload's
MAX_HITS, default modes).  Every output byte of every strand, batch and chunk is
compared with the CPU oracle's through SHA-256 digests that
``tests/golden/make_full_size_digests.py`` wrote by running the oracle over the whole
pass (``tests/golden/full_size_c<N>.json``):
  - the whole reference index (bucket starts and contents) and every seed;
  - every hit count and the whole global prefix of each batch, and its chunk list;
  - per chunk, through the per-call ABI: every anchor, every gate flag, every survivor
    id, the status of every survivor and every accepted record;
  - per batch, through hspz_run_batch (the timed path, expansion fused into the gate):
    every accepted record, chunk by chunk.
Nothing is sampled.  When a digest differs, the test recomputes that chunk with the
oracle and names the first element that differs.
"""
import collections
import concurrent.futures as cf
import hashlib
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import engine, require_gpu
from workloads import build

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).hexdigest()


def _gold(cfg):
    with open(os.path.join(GOLD, f"full_size_c{cfg}.json")) as fh:
        return json.load(fh)


class _Diagnose:
    """On a digest mismatch: the oracle's own arrays for one chunk, element by element."""

    def __init__(self, w, p, strand):
        self.w, self.p, self.strand = w, p, strand
        self._R = None

    def first_difference(self, lo, hi, ci, field, got):
        p = self.p
        if self._R is None:
            self._R = oracle.Reference(self.w.ref, p["seed_pattern"])
            self._qc = oracle.strand_codes(self.w.query, self.strand)
            self._seeds = oracle.query_seeds(self._qc, p["seed_pattern"])
        R, qc = self._R, self._qc
        kmer, q_end, _ = self._seeds
        count, first = oracle.counts_indexed(R.keys, R.ends, kmer[lo:hi])
        P, _ = oracle.prefix(count)
        ch = oracle.chunks(P, p["max_hits"])[ci]
        T = oracle.keep_threshold(p["hsp_threshold"])
        want = {}
        want["anchors"] = oracle.anchors(P, count, first, R.ends, q_end[lo:hi], ch)
        if field != "anchors":
            want["flags"] = oracle.gate(want["anchors"], R.codes, qc, p["sub"], p["n_score"],
                                        p["xdrop"], T)
            want["ids"] = oracle.compact(want["flags"])
            hsp, want["status"] = oracle.materialize(want["anchors"], want["ids"], R.codes,
                                                     qc, p["sub"], p["n_score"], p["xdrop"],
                                                     T, K=p["hsp_threshold"])
            want["accepted"] = oracle.compact_hsps(hsp, want["status"])
        w_ = want[field].reshape(-1)
        g_ = got.reshape(-1)
        if w_.dtype != g_.dtype:
            g_ = g_.view(w_.dtype)
        if w_.size != g_.size:
            return f"{field}: {g_.size} elements against the oracle's {w_.size}"
        bad = np.flatnonzero(w_ != g_)
        i = int(bad[0]) if bad.size else -1
        return (f"{field}: {bad.size} elements differ, first at {i}: "
                f"gpu {g_[i]!r} oracle {w_[i]!r}" if bad.size else f"{field}: equal?")


def _run_config(cfg):
    from ungapped_drop_hsp_amd.pipeline import PassBuffers, batches
    d = _gold(cfg)
    w = build(cfg)
    p = w.params()
    assert d["workload"] == w.name and d["params"]["max_hits"] == p["max_hits"]
    eng = engine(p)
    eng.upload_reference(w.ref)
    end, pos = eng.get_index()
    assert pos.size >= d["index"]["n_windows"]
    assert sha(end) == d["index"]["end"], "bucket starts differ"
    assert sha(pos[: d["index"]["n_windows"]]) == d["index"]["pos"], "bucket contents differ"
    del end, pos
    bufs = PassBuffers()
    pool = cf.ThreadPoolExecutor(max_workers=8)
    stats = []
    try:
        for strand, so in d["strands"].items():
            eng.upload_query(w.query, strand=1 if strand == "-" else 0)
            assert eng.num_seeds() == so["n_seeds"]
            gk, gq = eng.get_seeds(0, so["n_seeds"])
            assert sha(gk) == so["kmer"] and sha(gq) == so["q_end"], "seeds differ"
            del gk, gq
            bs = batches(eng, w.batch_len, w.query.size)
            assert bs == [(b["seed_lo"], b["seed_hi"]) for b in so["batches"]], \
                "batch ranges differ"
            diag = _Diagnose(w, p, strand)
            for bi, bo in enumerate(so["batches"]):
                stats.append(_check_batch(eng, bufs, pool, diag, strand, bi, bo))
    finally:
        pool.shutdown(wait=True)
    return stats


def _check_batch(eng, bufs, pool, diag, strand, bi, bo):
    lo, hi = bo["seed_lo"], bo["seed_hi"]
    tot, nch = eng.plan(lo, hi)
    assert tot == bo["total"] and nch == len(bo["chunks"])
    gc, gp = eng.get_plan_arrays(hi - lo)
    assert sha(gc) == bo["count"], "hit counts differ"
    assert sha(gp) == bo["prefix"], "global prefix differs"
    got_ch = [eng.get_chunk(i) for i in range(nch)]
    assert [(c["seed_lo"] - lo, c["seed_hi"] - lo, c["hit_lo"], c["n_hits"])
            for c in got_ch] == [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"])
                                 for c in bo["chunks"]], "chunk lists differ"
    pending = collections.deque()
    bad = []

    def settle(limit):
        while len(pending) > limit:
            ci, arrays, futs = pending.popleft()
            for field, fut in futs.items():
                if fut.result() != bo["chunks"][ci][field]:
                    bad.append(f"strand {strand} batch {bi} chunk {ci}: " +
                               diag.first_difference(lo, hi, ci, field, arrays[field]))
                    return

    for ci, co in enumerate(bo["chunks"]):
        n = co["n_hits"]
        bufs.ensure(n)
        eng.find_hits(ci, bufs.anchors)
        eng.score_gate(bufs.anchors, n, bufs.flags)
        ns = eng.compact(bufs.flags, n, bufs.ids, cap=n)
        bufs.ensure(n, ns)
        eng.materialize(bufs.anchors, bufs.ids, ns, bufs.hsp, bufs.status)
        na = eng.compact_hsps(bufs.hsp, bufs.status, ns, bufs.out)
        assert (ns, na) == (co["n_surv"], co["n_acc"]), \
            f"strand {strand} batch {bi} chunk {ci}: survivor or accepted counts differ"
        arrays = dict(anchors=bufs.anchors[:n].cpu().numpy(),
                      flags=bufs.flags[:n].cpu().numpy(),
                      ids=bufs.ids[:ns].cpu().numpy(),
                      status=bufs.status[:ns].cpu().numpy(),
                      accepted=bufs.out[:na].cpu().numpy())
        pending.append((ci, arrays, {k: pool.submit(sha, v) for k, v in arrays.items()}))
        settle(3)
        assert not bad, bad[0]
    settle(0)
    assert not bad, bad[0]
    # the timed path: the whole batch in one native call, against every chunk's digest
    sb = eng.run_batch(lo, hi)
    assert (sb["n_chunks"], sb["n_survivors"], sb["n_accepted"]) == \
        (nch, bo["n_surv"], bo["n_acc"]), "run_batch counts differ"
    rec = eng.batch_records().view(np.uint8).reshape(-1)
    off = 0
    for ci, co in enumerate(bo["chunks"]):
        part = rec[off: off + 16 * co["n_acc"]]
        off += 16 * co["n_acc"]
        assert sha(part) == co["accepted"], \
            f"strand {strand} batch {bi} chunk {ci}: run_batch records differ"
    assert off == rec.size
    st = dict(strand=strand, batch=bi, total=tot, chunks=nch, surv=bo["n_surv"],
              acc=bo["n_acc"])
    print(f"strand {strand} batch {bi}: {st} every digest equal", flush=True)
    return st


@pytest.mark.timeout(600)
def test_c2_dense_tandem_full_size():
    # 5 Mb x 5 Mb, MAX_HITS 2^20: 58 chunks; dense buckets in the tandem region
    st = _run_config(2)
    assert st[0]["chunks"] > 40 and st[0]["surv"] > 0


@pytest.mark.timeout(600)
def test_c3_50mb_full_size():
    st = _run_config(3)
    assert st[0]["chunks"] == 2 and 1.2e8 < st[0]["total"] < 2.6e8


@pytest.mark.timeout(1100)
def test_c4_200mb_both_strands_batches():
    # 200 Mb x 200 Mb, both strands, 50 Mb query batches, MAX_HITS 2^26
    st = _run_config(4)
    assert len(st) == 8 and all(s["chunks"] > 1 for s in st)


@pytest.mark.timeout(600)
def test_c3_bucketed_gate_full_size():
    # the bucketed gate (gate_mode 4, automatic slices: 12 of 2^22 bases) on every c3
    # chunk: every flag byte against the oracle's digest; then the whole batch through
    # run_batch, record for record against the default gate's
    import torch
    d = _gold(3)
    w = build(3)
    p = w.params()
    eng0, eng4 = engine(p), engine(p, gate_mode=4)
    for e in (eng0, eng4):
        e.upload_reference(w.ref)
        e.upload_query(w.query)
    n_seeds = eng0.num_seeds()
    _, nch = eng0.plan(0, n_seeds)
    assert eng4.plan(0, n_seeds)[1] == nch == 2
    gold = d["strands"]["+"]["batches"][0]["chunks"]
    for c in range(nch):
        n = eng0.get_chunk(c)["n_hits"]
        a = torch.empty(n, dtype=torch.int64, device="cuda")
        f4 = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
        eng0.find_hits(c, a)
        eng4.score_gate(a, n, f4)
        assert sha(f4.cpu().numpy()) == gold[c]["flags"], f"chunk {c}: bucketed flags differ"
        print(f"chunk {c}: {n} anchors, {int(f4.sum())} kept", flush=True)
        del a, f4
    s0, s4 = eng0.run_batch(0, n_seeds), eng4.run_batch(0, n_seeds)
    assert (s0["n_survivors"], s0["n_accepted"]) == (s4["n_survivors"], s4["n_accepted"])
    assert np.array_equal(eng0.batch_records().view(np.uint8),
                          eng4.batch_records().view(np.uint8))
