"""Helpers shared by the GPU parity tests: run one pass on both sides and compare."""
from __future__ import annotations

import numpy as np

import oracle


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "gpu-marked tests need an MI355X"
    return torch


def engine(params, expand_mode=0, chunk_walk=0, max_hits=None, gate_mode=0, ref_buckets=0,
           materialize_mode=0):
    import ungapped_drop_hsp_amd as h
    return h.Engine(seed_pattern=params["seed_pattern"], sub=params["sub"],
                    n_score=params["n_score"], xdrop=params["xdrop"],
                    hsp_threshold=params["hsp_threshold"],
                    max_hits=params["max_hits"] if max_hits is None else max_hits,
                    expand_mode=expand_mode, chunk_walk=chunk_walk, gate_mode=gate_mode,
                    entropy_mode=params.get("entropy_mode", 0), ref_buckets=ref_buckets,
                    materialize_mode=materialize_mode)


def params_of(pattern, max_hits=0, sub=None, xdrop=910, K=3000, n_score=-100, entropy_mode=0):
    from workloads import HOXD70
    return dict(seed_pattern=pattern, sub=HOXD70 if sub is None else sub, n_score=n_score,
                xdrop=xdrop, hsp_threshold=K, max_hits=max_hits, entropy_mode=entropy_mode)


def gpu_full_pass(eng, ref, qry, strand="+", seed_range=None, bufs=None):
    from ungapped_drop_hsp_amd.pipeline import PassBuffers, run_pass
    eng.upload_reference(ref)
    eng.upload_query(qry, strand=1 if strand == "-" else 0)
    lo, hi = seed_range if seed_range is not None else (0, eng.num_seeds())
    bufs = bufs or PassBuffers()
    g = run_pass(eng, lo, hi, bufs, collect=True)
    g["seeds"] = eng.get_seeds(lo, hi)
    g["plan_arrays"] = eng.get_plan_arrays(hi - lo)
    g["lo"] = lo
    return g


def assert_pass_equal(g, o, check_gate=True):
    """Element-by-element equality of a GPU pass and an oracle pass (same batch)."""
    kmer, q_end = g["seeds"]
    assert np.array_equal(kmer, o["kmer"]), "seed k-mers differ"
    assert np.array_equal(q_end, o["q_end"]), "seed query ends differ"
    assert g["total"] == o["total"]
    cnt, pre = g["plan_arrays"]
    assert np.array_equal(cnt, o["count"]), "hit counts differ"
    assert np.array_equal(pre.astype(np.uint64), o["P"]), "global prefix differs"
    gc = [(c["chunk"]["seed_lo"] - g["lo"], c["chunk"]["seed_hi"] - g["lo"],
           c["chunk"]["hit_lo"], c["chunk"]["n_hits"]) for c in g["chunks"]]
    oc = [(c["chunk"]["seed_lo"], c["chunk"]["seed_hi"], c["chunk"]["hit_lo"],
           c["chunk"]["n_hits"]) for c in o["chunks"]]
    assert gc == oc, "chunk lists differ"
    for gch, och in zip(g["chunks"], o["chunks"]):
        assert np.array_equal(gch["anchors"], och["anchors"]), "anchors differ"
        if not check_gate:
            continue
        bad = np.nonzero(gch["flags"] != och["flags"])[0]
        assert bad.size == 0, f"{bad.size} flags differ, first at {bad[:5]}"
        assert np.array_equal(gch["ids"], och["ids"]), "survivor ids differ"
        assert np.array_equal(gch["status"], och["status"]), "status differs"
        acc = och["status"] == 1
        assert np.array_equal(gch["hsp"][acc], och["hsp"][acc]), "accepted records differ"
        assert np.array_equal(gch["accepted"], och["accepted"]), "compacted records differ"


def oracle_pass(ref, qry, params, strand="+", seed_range=None):
    R = oracle.Reference(ref, params["seed_pattern"])
    qc = oracle.strand_codes(qry, strand)
    return oracle.run_pass(R, qc, params, seed_range=seed_range), R, qc
