"""The committed full-size digests (tests/golden/full_size_c<N>.json) are the oracle's.

Recomputed here on the CPU, with the oracle alone and independently of the script that
wrote them, for the 5 Mb workload: the reference index, every seed, the batch's hit
counts, prefix and chunk list, and every array of its last chunk.  The GPU full-size
tests compare the HIP path's outputs with these digests.
"""
import hashlib
import json
import os

import numpy as np

import oracle
from workloads import CONFIGS, build

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).hexdigest()


def test_every_workload_has_digests_of_its_shape():
    for cfg, strands, batches in ((2, "+", 1), (3, "+", 1), (4, "+-", 4)):
        d = json.load(open(os.path.join(GOLD, f"full_size_c{cfg}.json")))
        spec = CONFIGS[cfg]
        assert d["hash"] == "sha256" and d["workload"] == spec["name"]
        assert d["params"]["max_hits"] == spec["max_hits"]
        assert "".join(d["strands"]) == strands == spec["strands"]
        for so in d["strands"].values():
            assert len(so["batches"]) == batches
            for b in so["batches"]:
                assert b["total"] == sum(c["n_hits"] for c in b["chunks"])
                assert b["n_surv"] == sum(c["n_surv"] for c in b["chunks"])
                for c in b["chunks"]:
                    assert c["n_acc"] <= c["n_surv"] <= c["n_hits"]
                    assert all(len(c[k]) == 64 for k in
                               ("anchors", "flags", "ids", "status", "accepted"))


def test_c2_digests_are_the_oracles():
    d = json.load(open(os.path.join(GOLD, "full_size_c2.json")))
    w = build(2)
    p = w.params()
    R = oracle.Reference(w.ref, p["seed_pattern"])
    weight = len(oracle.pattern(p["seed_pattern"])[0])
    end = np.searchsorted(R.keys, np.arange((1 << (2 * weight)) + 1, dtype=np.uint64))
    assert sha(end.astype(np.uint32)) == d["index"]["end"]
    assert sha(R.ends) == d["index"]["pos"] and R.ends.size == d["index"]["n_windows"]
    qc = oracle.strand_codes(w.query, "+")
    kmer, q_end, _ = oracle.query_seeds(qc, p["seed_pattern"])
    so = d["strands"]["+"]
    assert (sha(kmer), sha(q_end), kmer.size) == (so["kmer"], so["q_end"], so["n_seeds"])
    b = so["batches"][0]
    count, first = oracle.counts_indexed(R.keys, R.ends, kmer)
    P, ok = oracle.prefix(count)
    assert ok and (sha(count), sha(P.astype(np.uint32))) == (b["count"], b["prefix"])
    ch = oracle.chunks(P, p["max_hits"])
    assert [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in ch] == \
        [(c["seed_lo"], c["seed_hi"], c["hit_lo"], c["n_hits"]) for c in b["chunks"]]
    T = oracle.keep_threshold(p["hsp_threshold"])
    c = ch[-1]
    a = oracle.anchors(P, count, first, R.ends, q_end, c)
    f = oracle.gate(a, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T)
    ids = oracle.compact(f)
    hsp, st = oracle.materialize(a, ids, R.codes, qc, p["sub"], p["n_score"], p["xdrop"], T,
                                 K=p["hsp_threshold"])
    acc = oracle.compact_hsps(hsp, st)
    want = b["chunks"][-1]
    assert (sha(a), sha(f), sha(ids), sha(st), sha(acc)) == \
        (want["anchors"], want["flags"], want["ids"], want["status"], want["accepted"])
