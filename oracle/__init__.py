"""CPU oracle for the hspZ seed-and-extend path -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper around ``oracle.c`` (plain C, single-threaded) plus ``run_pass``,
which chains the oracle's steps for one strand and one query batch in the order the
hspZ pages give them ("C. Hit discovery", "D. Score gate", "E. X-drop
materialization").  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

HSP_DTYPE = np.dtype([("ref_start", "<u4"), ("query_start", "<u4"), ("len", "<u4"),
                      ("score", "<i4")])

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (plain gcc)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC,
           "-o", _SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    sig = {
        "orc_encode": (None, [_P, _I64, _P]),
        "orc_revcomp_codes": (None, [_P, _I64, _P]),
        "orc_pattern": (ctypes.c_int, [ctypes.c_char_p, _P, _P]),
        "orc_query_seeds": (_I64, [_P, _I64, ctypes.c_char_p, _P, _P, _P]),
        "orc_ref_index": (_I64, [_P, _I64, ctypes.c_char_p, _P, _P]),
        "orc_counts_indexed": (None, [_P, _P, _I64, _P, _I64, _P, _P]),
        "orc_counts_brute": (None, [_P, _I64, ctypes.c_char_p, _P, _I64, _P]),
        "orc_prefix": (ctypes.c_int, [_P, _I64, _P]),
        "orc_chunks": (_I64, [_P, _I64, ctypes.c_uint64, _P, _P, _P, _P]),
        "orc_anchors": (None, [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_uint64, _P]),
        "orc_anchors_brute": (None, [_P, _I64, ctypes.c_char_p, _P, _P, _P, _I64, _I64,
                                     ctypes.c_uint64, _P]),
        "orc_keep_threshold": (_I32, [_I32]),
        "orc_xdrop": (None, [_P, _I64, _P, _I64, _I64, _I64, ctypes.c_int, _P, _I32, _I32,
                             _P, _P]),
        "orc_gate": (None, [_P, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _P]),
        "orc_gate_totals": (None, [_P, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _P, _P]),
        "orc_compact": (_I64, [_P, _I64, _P]),
        "orc_entropy_bits": (ctypes.c_double, [_P, _I64, _I64, _I64]),
        "orc_materialize": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _I64, _P, _I32,
                                           _I32, _I32, _I32, _I32, _P, _P]),
        "orc_compact_hsps": (_I64, [_P, _P, _I64, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _sub(sub) -> np.ndarray:
    m = _c(sub, np.int32).reshape(-1)
    assert m.size == 16
    return m


# ----------------------------------------------------------------------------- steps

def encode(ascii) -> np.ndarray:
    a = _c(np.frombuffer(ascii, np.uint8) if isinstance(ascii, (bytes, bytearray)) else ascii,
           np.uint8)
    out = np.empty(a.size, np.uint8)
    _load().orc_encode(_ptr(a), a.size, _ptr(out))
    return out


def revcomp(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.size, np.uint8)
    _load().orc_revcomp_codes(_ptr(c), c.size, _ptr(out))
    return out


def pattern(p: str):
    care = np.zeros(64, np.int32)
    span = np.zeros(1, np.int32)
    w = _load().orc_pattern(p.encode(), _ptr(care), _ptr(span))
    if w < 0:
        raise ValueError(f"malformed seed pattern {p!r}")
    return care[:w].copy(), int(span[0])


def query_seeds(codes, pat: str):
    c = _c(codes, np.uint8)
    n = max(c.size, 1)
    kmer = np.empty(n, np.uint32)
    q_end = np.empty(n, np.uint32)
    pos = np.empty(n, np.int64)
    m = _load().orc_query_seeds(_ptr(c), c.size, pat.encode(), _ptr(kmer), _ptr(q_end),
                                _ptr(pos))
    if m < 0:
        raise ValueError("malformed seed pattern")
    return kmer[:m].copy(), q_end[:m].copy(), pos[:m].copy()


def ref_index(codes, pat: str):
    c = _c(codes, np.uint8)
    n = max(c.size, 1)
    keys = np.empty(n, np.uint32)
    ends = np.empty(n, np.uint32)
    m = _load().orc_ref_index(_ptr(c), c.size, pat.encode(), _ptr(keys), _ptr(ends))
    if m < 0:
        raise ValueError("malformed seed pattern or out of memory")
    return keys[:m].copy(), ends[:m].copy()


def counts_indexed(keys, ends, kmer):
    kmer = _c(kmer, np.uint32)
    count = np.empty(kmer.size, np.uint32)
    first = np.empty(kmer.size, np.int64)
    _load().orc_counts_indexed(_ptr(keys), _ptr(ends), keys.size, _ptr(kmer), kmer.size,
                               _ptr(count), _ptr(first))
    return count, first


def counts_brute(rcodes, pat: str, kmer):
    rc = _c(rcodes, np.uint8)
    kmer = _c(kmer, np.uint32)
    count = np.empty(kmer.size, np.uint32)
    _load().orc_counts_brute(_ptr(rc), rc.size, pat.encode(), _ptr(kmer), kmer.size,
                             _ptr(count))
    return count


def prefix(count):
    count = _c(count, np.uint32)
    P = np.empty(count.size, np.uint64)
    rc = _load().orc_prefix(_ptr(count), count.size, _ptr(P))
    return P, rc == 0


def chunks(P, max_hits: int) -> List[Dict]:
    P = _c(P, np.uint64)
    n = max(P.size, 1)
    lo = np.empty(n, np.int64)
    hi = np.empty(n, np.int64)
    hl = np.empty(n, np.uint64)
    nh = np.empty(n, np.uint64)
    c = _load().orc_chunks(_ptr(P), P.size, max_hits, _ptr(lo), _ptr(hi), _ptr(hl),
                           _ptr(nh))
    return [dict(seed_lo=int(lo[i]), seed_hi=int(hi[i]), hit_lo=int(hl[i]),
                 n_hits=int(nh[i])) for i in range(c)]


def anchors(P, count, first, ends, q_end, chunk) -> np.ndarray:
    out = np.empty(max(chunk["n_hits"], 1), np.uint64)
    _load().orc_anchors(_ptr(_c(P, np.uint64)), _ptr(_c(count, np.uint32)),
                        _ptr(_c(first, np.int64)), _ptr(_c(ends, np.uint32)),
                        _ptr(_c(q_end, np.uint32)), chunk["seed_lo"], chunk["seed_hi"],
                        chunk["hit_lo"], _ptr(out))
    return out[: chunk["n_hits"]]


def anchors_brute(rcodes, pat, P, kmer, q_end, chunk) -> np.ndarray:
    out = np.empty(max(chunk["n_hits"], 1), np.uint64)
    rc = _c(rcodes, np.uint8)
    _load().orc_anchors_brute(_ptr(rc), rc.size, pat.encode(), _ptr(_c(P, np.uint64)),
                              _ptr(_c(kmer, np.uint32)), _ptr(_c(q_end, np.uint32)),
                              chunk["seed_lo"], chunk["seed_hi"], chunk["hit_lo"],
                              _ptr(out))
    return out[: chunk["n_hits"]]


def keep_threshold(K: int) -> int:
    return int(_load().orc_keep_threshold(int(K)))


def xdrop(rcodes, qcodes, r: int, q: int, direction: int, sub, n_score: int, X: int):
    rc = _c(rcodes, np.uint8)
    qc = _c(qcodes, np.uint8)
    best = np.zeros(1, np.int64)
    ext = np.zeros(1, np.int64)
    _load().orc_xdrop(_ptr(rc), rc.size, _ptr(qc), qc.size, r, q, direction,
                      _ptr(_sub(sub)), n_score, X, _ptr(best), _ptr(ext))
    return int(best[0]), int(ext[0])


def gate(anchors_, rcodes, qcodes, sub, n_score, X, T) -> np.ndarray:
    a = _c(anchors_, np.uint64)
    rc = _c(rcodes, np.uint8)
    qc = _c(qcodes, np.uint8)
    flags = np.empty(a.size, np.uint8)
    _load().orc_gate(_ptr(a), a.size, _ptr(rc), rc.size, _ptr(qc), qc.size,
                     _ptr(_sub(sub)), n_score, X, T, _ptr(flags))
    return flags


def gate_totals(anchors_, rcodes, qcodes, sub, n_score, X):
    a = _c(anchors_, np.uint64)
    rc = _c(rcodes, np.uint8)
    qc = _c(qcodes, np.uint8)
    tot = np.empty(a.size, np.int64)
    steps = np.empty(a.size, np.int64)
    _load().orc_gate_totals(_ptr(a), a.size, _ptr(rc), rc.size, _ptr(qc), qc.size,
                            _ptr(_sub(sub)), n_score, X, _ptr(tot), _ptr(steps))
    return tot, steps


def compact(flags) -> np.ndarray:
    f = _c(flags, np.uint8)
    ids = np.empty(max(f.size, 1), np.uint32)
    m = _load().orc_compact(_ptr(f), f.size, _ptr(ids))
    return ids[:m].copy()


def entropy_bits(rcodes, ref_start: int, length: int) -> float:
    rc = _c(rcodes, np.uint8)
    return float(_load().orc_entropy_bits(_ptr(rc), rc.size, ref_start, length))


def materialize(anchors_, ids, rcodes, qcodes, sub, n_score, X, T, K=None, entropy_mode=0):
    a = _c(anchors_, np.uint64)
    ids = _c(ids, np.uint32)
    rc = _c(rcodes, np.uint8)
    qc = _c(qcodes, np.uint8)
    hsp = np.zeros(max(ids.size, 1), HSP_DTYPE)
    status = np.zeros(max(ids.size, 1), np.uint8)
    rc_ = _load().orc_materialize(_ptr(a), _ptr(ids), ids.size, _ptr(rc), rc.size,
                                  _ptr(qc), qc.size, _ptr(_sub(sub)), n_score, X, T,
                                  T if K is None else K, entropy_mode, _ptr(hsp),
                                  _ptr(status))
    if rc_ != 0:
        raise OverflowError("a record's score L* + R* does not fit in int32: refused")
    return hsp[: ids.size], status[: ids.size]


def compact_hsps(hsp, status) -> np.ndarray:
    hsp = np.ascontiguousarray(hsp, dtype=HSP_DTYPE)
    st = _c(status, np.uint8)
    out = np.zeros(max(hsp.size, 1), HSP_DTYPE)
    m = _load().orc_compact_hsps(_ptr(hsp), _ptr(st), hsp.size, _ptr(out))
    return out[:m].copy()


def dedup_records(hsp) -> np.ndarray:
    """Host dedup after acceptance ("D. Score gate", introduction: accepted raw HSPs,
    then fewer final HSPs after host dedup; the order it depends on is fixed in
    "C. Hit discovery", C.5).  The pages give no rule; the reading taken: a record is a
    duplicate when an earlier record of the array has the same four fields, and the
    records that are not duplicates are kept in their order."""
    hsp = np.ascontiguousarray(hsp, dtype=HSP_DTYPE).reshape(-1)
    seen = set()
    keep = []
    for i, r in enumerate(hsp.tolist()):
        if r not in seen:
            seen.add(r)
            keep.append(i)
    return hsp[np.array(keep, dtype=np.int64)].copy()


# ----------------------------------------------------------------------------- a pass

class Reference:
    """Encoded reference plus the oracle's sorted (key, end) index."""

    def __init__(self, ascii, pat: str):
        self.codes = encode(ascii)
        self.pattern = pat
        self.keys, self.ends = ref_index(self.codes, pat)


def strand_codes(query_ascii, strand: str) -> np.ndarray:
    c = encode(query_ascii)
    return revcomp(c) if strand == "-" else c


def run_pass(ref: Reference, qcodes: np.ndarray, params: Dict, *, seed_range=None,
             stages=("anchors", "gate", "materialize"), seeds=None) -> Dict:
    """All oracle steps for one strand and one batch of query seeds.

    ``seed_range`` = (lo, hi) half-open indices into the strand's seed list (all seeds by
    default).  ``seeds`` = the (kmer, q_end, pos) triple that ``query_seeds`` returns for
    ``qcodes``, when the caller already has it.  Returns the seeds, counts, prefix,
    chunks and, per chunk, anchors, flags, survivor ids, records, status and accepted
    records.
    """
    pat = params["seed_pattern"]
    kmer, q_end, pos = seeds if seeds is not None else query_seeds(qcodes, pat)
    if seed_range is not None:
        lo, hi = seed_range
        kmer, q_end, pos = kmer[lo:hi], q_end[lo:hi], pos[lo:hi]
    count, first = counts_indexed(ref.keys, ref.ends, kmer)
    P, ok = prefix(count)
    out = dict(kmer=kmer, q_end=q_end, pos=pos, count=count, first=first, P=P,
               total=int(P[-1]) if P.size else 0, ok=ok, chunks=[])
    if not ok:
        return out
    T = keep_threshold(params["hsp_threshold"])
    out["T"] = T
    sub, ns, X = params["sub"], params["n_score"], params["xdrop"]
    for ch in chunks(P, params["max_hits"]):
        rec = dict(chunk=ch)
        if "anchors" in stages:
            a = anchors(P, count, first, ref.ends, q_end, ch)
            rec["anchors"] = a
            if "gate" in stages:
                f = gate(a, ref.codes, qcodes, sub, ns, X, T)
                rec["flags"] = f
                ids = compact(f)
                rec["ids"] = ids
                if "materialize" in stages:
                    h, st = materialize(a, ids, ref.codes, qcodes, sub, ns, X, T,
                                        K=params["hsp_threshold"],
                                        entropy_mode=params.get("entropy_mode", 0))
                    rec["hsp"], rec["status"] = h, st
                    rec["accepted"] = compact_hsps(h, st)
        out["chunks"].append(rec)
    return out
