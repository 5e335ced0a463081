"""Write the oracle's full-size digests for the 5 Mb, 50 Mb and 200 Mb workloads.

    python tests/golden/make_full_size_digests.py [--configs 2 3 4] [--workers N]

For every strand, query batch and MAX_HITS chunk of each workload this runs the CPU
oracle over the whole pass -- the reference index, the query seeds, hit counts and
global prefix ("C. Hit discovery", C.1-C.3), every anchor in the pages' backward raw
order (C.5), every gate flag and survivor id ("D. Score gate", D.2-D.4), and every
record, status byte and accepted record ("E. X-drop materialization", E.1-E.5) -- and
stores a SHA-256 digest of each array in ``full_size_c<N>.json`` beside this script.
The GPU full-size tests hash their own outputs the same way and compare every digest.

Only ``oracle/`` and ``workloads/`` are called.  The oracle stays single-threaded: the
work is split over worker processes by seed shards (hit counts) and by chunks (all
later steps), and each worker runs the unchanged oracle functions on its share.

Canonical bytes (little-endian, no header; one digest per array):
  index.end   u32[4^weight + 1]  bucket starts with a leading 0 (= windows with a smaller key)
  index.pos   u32[windows]       reference ends grouped by key, ascending within a key
  seeds       u32 k-mer and u32 query end of every seed of the strand
  batch       u32 hit count and u32 inclusive prefix of every seed of the batch
  chunk       u64 anchors, u8 flags, u32 survivor ids, u8 status of every survivor,
              16-byte accepted records (ref_start, query_start, len, score)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import mmap
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import build  # noqa: E402

SHARD = 1 << 21  # seeds per hit-count task

# State shared with forked workers (set before each pool is created).
G = {}


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).hexdigest()


def _shared(n: int, dtype) -> np.ndarray:
    """An array in anonymous shared memory: a forked worker's writes reach the parent."""
    dt = np.dtype(dtype)
    buf = mmap.mmap(-1, max(n, 1) * dt.itemsize)
    return np.frombuffer(buf, dtype=dt, count=n)


def _counts_task(span):
    lo, hi = span
    c, f = oracle.counts_indexed(G["keys"], G["ends"], G["kmer"][lo:hi])
    G["count"][lo:hi] = c
    G["first"][lo:hi] = f
    return hi - lo


def _chunk_task(ci):
    ch = G["chunks"][ci]
    p = G["params"]
    a = oracle.anchors(G["P"], G["count"], G["first"], G["ends"], G["q_end"], ch)
    f = oracle.gate(a, G["rcodes"], G["qcodes"], p["sub"], p["n_score"], p["xdrop"], G["T"])
    ids = oracle.compact(f)
    hsp, st = oracle.materialize(a, ids, G["rcodes"], G["qcodes"], p["sub"], p["n_score"],
                                 p["xdrop"], G["T"], K=p["hsp_threshold"])
    acc = oracle.compact_hsps(hsp, st)
    return ci, dict(seed_lo=ch["seed_lo"], seed_hi=ch["seed_hi"], hit_lo=ch["hit_lo"],
                    n_hits=ch["n_hits"], n_surv=int(ids.size), n_acc=int(acc.size),
                    anchors=sha(a), flags=sha(f), ids=sha(ids), status=sha(st),
                    accepted=sha(acc))


def _batches(w, pos):
    """Query batches as seed ranges: the seeds whose window starts in each slice of
    ``batch_len`` query positions (the whole strand when batch_len is 0)."""
    if not w.batch_len:
        return [(0, int(pos.size))]
    edges = np.searchsorted(pos, np.arange(0, w.query.size + w.batch_len, w.batch_len))
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def run_config(cfg: int, workers: int, log) -> dict:
    t0 = time.time()
    w = build(cfg)
    p = w.params()
    R = oracle.Reference(w.ref, p["seed_pattern"])
    weight = len(oracle.pattern(p["seed_pattern"])[0])
    end = np.searchsorted(R.keys, np.arange((1 << (2 * weight)) + 1, dtype=np.uint64))
    out = dict(workload=w.name, hash="sha256", generator="tests/golden/make_full_size_digests.py",
               params=dict(seed_pattern=p["seed_pattern"], xdrop=p["xdrop"],
                           hsp_threshold=p["hsp_threshold"], n_score=p["n_score"],
                           max_hits=p["max_hits"]),
               index=dict(n_windows=int(R.ends.size), end=sha(end.astype(np.uint32)),
                          pos=sha(R.ends.astype(np.uint32))),
               strands={})
    del end
    T = oracle.keep_threshold(p["hsp_threshold"])
    log(f"{w.name}: index of {R.ends.size} windows in {time.time() - t0:.0f} s")
    for strand in w.strands:
        qc = oracle.strand_codes(w.query, strand)
        kmer, q_end, pos = oracle.query_seeds(qc, p["seed_pattern"])
        so = dict(n_seeds=int(kmer.size), kmer=sha(kmer), q_end=sha(q_end), batches=[])
        for bi, (lo, hi) in enumerate(_batches(w, pos)):
            n = hi - lo
            G.clear()
            G.update(keys=R.keys, ends=R.ends, kmer=kmer[lo:hi], q_end=q_end[lo:hi],
                     count=_shared(n, np.uint32), first=_shared(n, np.int64),
                     rcodes=R.codes, qcodes=qc, params=p, T=T)
            ctx = mp.get_context("fork")
            with ctx.Pool(workers) as pool:
                spans = [(s, min(s + SHARD, n)) for s in range(0, n, SHARD)]
                assert sum(pool.map(_counts_task, spans)) == n
            P, ok = oracle.prefix(G["count"])
            assert ok, "the batch total does not fit the 32-bit hit index"
            chunks = oracle.chunks(P, p["max_hits"])
            G.update(P=P, chunks=chunks)
            bo = dict(seed_lo=lo, seed_hi=hi, total=int(P[-1]) if n else 0,
                      count=sha(G["count"]), prefix=sha(P.astype(np.uint32)),
                      chunks=[None] * len(chunks))
            t1 = time.time()
            with ctx.Pool(workers) as pool:
                for ci, rec in pool.imap_unordered(_chunk_task, range(len(chunks))):
                    bo["chunks"][ci] = rec
            bo["n_surv"] = sum(c["n_surv"] for c in bo["chunks"])
            bo["n_acc"] = sum(c["n_acc"] for c in bo["chunks"])
            so["batches"].append(bo)
            log(f"{w.name} strand {strand} batch {bi}: {n} seeds, {bo['total']} anchors, "
                f"{len(chunks)} chunks, {bo['n_surv']} survivors, {bo['n_acc']} accepted "
                f"({time.time() - t1:.0f} s)")
            G.clear()
        out["strands"][strand] = so
    log(f"{w.name}: done in {time.time() - t0:.0f} s")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--configs", type=int, nargs="+", default=[2, 3, 4])
    ap.add_argument("--workers", type=int, default=max(1, (os.cpu_count() or 2) - 1))
    ap.add_argument("--out-dir", default=HERE)
    args = ap.parse_args()
    oracle.build()

    def log(msg):
        print(msg, flush=True)

    for cfg in args.configs:
        d = run_config(cfg, args.workers, log)
        path = os.path.join(args.out_dir, f"full_size_c{cfg}.json")
        with open(path + ".tmp", "w") as fh:
            json.dump(d, fh, indent=1)
            fh.write("\n")
        os.replace(path + ".tmp", path)
        log(f"wrote {path}")


if __name__ == "__main__":
    main()
