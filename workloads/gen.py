"""Synthetic DNA pairs shaped like the hspZ workloads (five configurations, c0..c4).

Every draw comes from ``numpy.random.Generator(PCG64(1000 + config index))`` so a
configuration is the same bytes on every machine.  The recipe per configuration is
listed in ``CONFIGS`` and restated in the design doc.  Homologs are substitution-only: a
planted copy keeps each base with probability ``u`` and otherwise replaces it with one
of the other three bases uniformly.  Planted intervals never overlap within one
sequence; N runs are written last and may cover planted material.

Scoring parameters (seed pattern, HOXD70 matrix, X-drop, K, MAX_HITS) travel with the
workload as plain data; nothing here evaluates them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

SEED_PATTERN = "1110100110010101111"  # 12-of-19 spaced seed
# HOXD70, rows = reference base, columns = query base, order A, C, G, T.
HOXD70 = (
    (91, -114, -31, -123),
    (-114, 100, -125, -31),
    (-31, -125, 100, -114),
    (-123, -31, -114, 91),
)
XDROP = 910
HSP_K = 3000
N_SCORE = -100

_ASCII = np.frombuffer(b"ACGT", dtype=np.uint8)
_GC41 = (0.295, 0.205, 0.205, 0.295)
_UNIFORM = (0.25, 0.25, 0.25, 0.25)


@dataclasses.dataclass
class Workload:
    name: str
    ref: np.ndarray            # uint8 ASCII
    query: np.ndarray          # uint8 ASCII (forward strand)
    seed_pattern: str
    sub: Tuple[Tuple[int, ...], ...]
    n_score: int
    xdrop: int
    hsp_threshold: int
    max_hits: int              # 0 = unlimited
    strands: str               # "+" or "+-"
    batch_len: int             # query positions per batch; 0 = whole query
    info: Dict

    def params(self) -> Dict:
        return dict(seed_pattern=self.seed_pattern, sub=self.sub, n_score=self.n_score,
                    xdrop=self.xdrop, hsp_threshold=self.hsp_threshold,
                    max_hits=self.max_hits)


# --------------------------------------------------------------------------- helpers

def _background(rng: np.random.Generator, n: int, probs) -> np.ndarray:
    return rng.choice(4, size=n, p=np.asarray(probs, dtype=np.float64)).astype(np.uint8)


def _mutate(rng: np.random.Generator, codes: np.ndarray, identity: float) -> np.ndarray:
    out = codes.copy()
    hit = rng.random(out.size) >= identity
    k = int(hit.sum())
    if k:
        out[hit] = (out[hit] + rng.integers(1, 4, size=k, dtype=np.uint8)) & 3
    return out


def _revcomp_codes(codes: np.ndarray) -> np.ndarray:
    return (3 - codes[::-1]).astype(np.uint8)


def _place(rng: np.random.Generator, n_total: int, lengths: np.ndarray) -> np.ndarray:
    """Random non-overlapping start positions for intervals of the given lengths."""
    k = lengths.size
    free = n_total - int(lengths.sum())
    if free < 0:
        raise ValueError("planted material longer than the sequence")
    cuts = np.sort(rng.integers(0, free + 1, size=k))
    order = rng.permutation(k)
    starts = np.empty(k, dtype=np.int64)
    starts[order] = cuts + np.concatenate(([0], np.cumsum(lengths[order])[:-1]))
    return starts


def _n_runs(rng: np.random.Generator, seq: np.ndarray, frac: float, lo: int, hi: int) -> int:
    if frac <= 0:
        return 0
    target = int(frac * seq.size)
    covered = np.zeros(seq.size, dtype=bool)
    runs, have = 0, 0
    while have < target:
        # draw about half of what is missing at a time, so the overshoot stays small
        batch = max(1, (target - have) // (lo + hi) + 1)
        lens = rng.integers(lo, hi + 1, size=batch)
        starts = rng.integers(0, max(1, seq.size - hi), size=batch)
        for s, l in zip(starts, lens):
            covered[s:s + l] = True
        runs += batch
        have = int(covered.sum())
    seq[covered] = ord("N")
    return runs


def _to_ascii(codes: np.ndarray) -> np.ndarray:
    return _ASCII[codes]


def reverse_complement_ascii(seq: np.ndarray) -> np.ndarray:
    """Reverse complement of an ASCII sequence; A<->T, C<->G, anything else -> N."""
    lut = np.full(256, ord("N"), dtype=np.uint8)
    for a, b in (("A", "T"), ("C", "G"), ("G", "C"), ("T", "A"),
                 ("a", "T"), ("c", "G"), ("g", "C"), ("t", "A")):
        lut[ord(a)] = ord(b)
    return lut[seq[::-1]]


# --------------------------------------------------------------------------- recipes

def _homologs(rng, ref, qry, n, len_draw, id_draw, rc_frac=0.0, extra_ref=(), extra_qry=()):
    """Plant n homolog pairs plus already-drawn extra intervals, all non-overlapping.

    ``extra_ref``/``extra_qry`` are lists of code arrays (repeat fragments) placed
    together with the homologs so nothing overlaps.
    """
    lens = np.asarray([len_draw(rng) for _ in range(n)], dtype=np.int64)
    ids = np.asarray([id_draw(rng) for _ in range(n)], dtype=np.float64)
    rc = rng.random(n) < rc_frac
    ex_r = np.asarray([e.size for e in extra_ref], dtype=np.int64)
    ex_q = np.asarray([e.size for e in extra_qry], dtype=np.int64)
    st_r = _place(rng, ref.size, np.concatenate((lens, ex_r)))
    st_q = _place(rng, qry.size, np.concatenate((lens, ex_q)))
    for i in range(n):
        a, b, l = st_r[i], st_q[i], lens[i]
        seg = _mutate(rng, ref[a:a + l], ids[i])
        qry[b:b + l] = _revcomp_codes(seg) if rc[i] else seg
    for j, e in enumerate(extra_ref):
        a = st_r[n + j]
        ref[a:a + e.size] = e
    for j, e in enumerate(extra_qry):
        b = st_q[n + j]
        qry[b:b + e.size] = e
    return dict(n_homologs=n, homolog_bp=int(lens.sum()), rc=int(rc.sum()),
                mean_identity=float(ids.mean()) if n else 0.0)


def _fragments(rng, families: List[np.ndarray], total_bp: int, flen: Tuple[int, int],
               identity: float) -> List[np.ndarray]:
    out, acc = [], 0
    while acc < total_bp:
        f = families[int(rng.integers(0, len(families)))]
        l = int(rng.integers(flen[0], min(flen[1], f.size) + 1))
        s = int(rng.integers(0, f.size - l + 1))
        out.append(_mutate(rng, f[s:s + l], identity))
        acc += l
    return out


def _c0(rng):
    n = 20_000
    ref = _background(rng, n, _UNIFORM)
    qry = _background(rng, n, _UNIFORM)
    info = _homologs(rng, ref, qry, 10, lambda r: int(r.integers(200, 801)), lambda r: 0.85)
    return _to_ascii(ref), _to_ascii(qry), info


def _c1(rng):
    n = 2_000_000
    ref = _background(rng, n, _GC41)
    qry = _background(rng, n, _GC41)
    info = _homologs(rng, ref, qry, 500, lambda r: int(r.integers(100, 5001)),
                     lambda r: float(r.uniform(0.70, 0.95)))
    ref, qry = _to_ascii(ref), _to_ascii(qry)
    info["n_runs_ref"] = _n_runs(rng, ref, 0.05, 10, 1000)
    info["n_runs_qry"] = _n_runs(rng, qry, 0.05, 10, 1000)
    return ref, qry, info


def _tandem_region(rng, units, n_bp):
    parts, acc = [], 0
    while acc < n_bp:
        u = units[int(rng.integers(0, len(units)))]
        copies = int(rng.integers(10, 101))
        arr = np.concatenate([_mutate(rng, u, 0.90) for _ in range(copies)])
        parts.append(arr)
        acc += arr.size
    return np.concatenate(parts)[:n_bp]


def _c2(rng):
    n = 5_000_000
    units = [_background(rng, int(rng.integers(50, 301)), _UNIFORM) for _ in range(20)]
    ref = _background(rng, n, _UNIFORM)
    qry = _background(rng, n, _UNIFORM)
    span = int(0.30 * n)
    for seq in (ref, qry):  # arrays kept clustered in one region per sequence
        start = int(rng.integers(0, n - span + 1))
        seq[start:start + span] = _tandem_region(rng, units, span)
    return _to_ascii(ref), _to_ascii(qry), dict(units=len(units), tandem_bp=span)


# Mix for the 50 Mb workload.  The literal homolog list (20,000 segments of
# 50-10,000 bp at 65-95 % identity) would make about 6 % of raw anchors survive; the
# configuration asks for the mix to be tuned to the funnel shape the pages report
# (~0.02 % survivors), so lengths are log-uniform and identities skewed low.  The
# numbers below were chosen by measuring the funnel (the design doc records the result).
C3_MIX = dict(
    n_homologs=20_000, len_lo=50, len_hi=10_000, len_shape=8.0,
    id_lo=0.65, id_hi=0.95, id_shape=30.0,
    repeat_frac=0.15, families=2_000, fam_len=(300, 3000), frag_len=(30, 60),
    repeat_identity=0.80, n_frac=0.03,
)


def _skewed_len(r, lo, hi, shape):
    # log-uniform on [lo, hi] raised to ``shape`` toward the short end
    t = float(r.random()) ** shape
    return int(round(np.exp(np.log(lo) + t * (np.log(hi) - np.log(lo)))))


def _skewed_id(r, lo, hi, shape):
    return lo + (hi - lo) * float(r.random()) ** shape


def _c3_like(rng, n, scale, rc_frac):
    m = C3_MIX
    ref = _background(rng, n, _GC41)
    qry = _background(rng, n, _GC41)
    fams = [_background(rng, int(rng.integers(m["fam_len"][0], m["fam_len"][1] + 1)), _GC41)
            for _ in range(int(m["families"] * scale))]
    rep_bp = int(m["repeat_frac"] * n)
    ex_r = _fragments(rng, fams, rep_bp, m["frag_len"], m["repeat_identity"])
    ex_q = _fragments(rng, fams, rep_bp, m["frag_len"], m["repeat_identity"])
    info = _homologs(
        rng, ref, qry, int(m["n_homologs"] * scale),
        lambda r: _skewed_len(r, m["len_lo"], m["len_hi"], m["len_shape"]),
        lambda r: _skewed_id(r, m["id_lo"], m["id_hi"], m["id_shape"]),
        rc_frac=rc_frac, extra_ref=ex_r, extra_qry=ex_q)
    ref, qry = _to_ascii(ref), _to_ascii(qry)
    info["repeat_fragments"] = (len(ex_r), len(ex_q))
    info["n_runs_ref"] = _n_runs(rng, ref, m["n_frac"], 10, 1000)
    info["n_runs_qry"] = _n_runs(rng, qry, m["n_frac"], 10, 1000)
    return ref, qry, info


def _c3(rng):
    return _c3_like(rng, 50_000_000, 1.0, 0.0)


def _c4(rng):
    return _c3_like(rng, 200_000_000, 4.0, 0.5)


CONFIGS = {
    0: dict(name="c0-20kb-uniform", make=_c0, max_hits=0, strands="+", batch_len=0),
    1: dict(name="c1-2Mb-gc41-N5", make=_c1, max_hits=0, strands="+", batch_len=0),
    2: dict(name="c2-5Mb-tandem30", make=_c2, max_hits=1 << 20, strands="+", batch_len=0),
    3: dict(name="c3-50Mb-gc41-N3", make=_c3, max_hits=1 << 27, strands="+", batch_len=0),
    4: dict(name="c4-200Mb-both-strands", make=_c4, max_hits=1 << 26, strands="+-",
            batch_len=50_000_000),
}


def build(index: int) -> Workload:
    """Draw configuration ``index`` (0..4) from its fixed seed."""
    spec = CONFIGS[index]
    rng = np.random.Generator(np.random.PCG64(1000 + index))
    ref, qry, info = spec["make"](rng)
    return Workload(name=spec["name"], ref=ref, query=qry, seed_pattern=SEED_PATTERN,
                    sub=HOXD70, n_score=N_SCORE, xdrop=XDROP, hsp_threshold=HSP_K,
                    max_hits=spec["max_hits"], strands=spec["strands"],
                    batch_len=spec["batch_len"], info=info)


def random_pair(seed: int, n_ref: int, n_qry: int, *, n_frac: float = 0.0,
                plant: int = 0, plant_len: Tuple[int, int] = (30, 200),
                identity: float = 0.9, gc: float = 0.5,
                alphabet_noise: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Small random pair for property tests: optional planted homologs and N runs.

    ``alphabet_noise`` sprinkles lowercase bases and IUPAC letters so that encoding
    rules get exercised.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    p = ((1 - gc) / 2, gc / 2, gc / 2, (1 - gc) / 2)
    ref = _background(rng, n_ref, p)
    qry = _background(rng, n_qry, p)
    for _ in range(plant):
        hi = min(plant_len[1], n_ref, n_qry)
        lo = min(plant_len[0], hi)
        if hi < 1:
            break
        l = int(rng.integers(lo, hi + 1))
        a = int(rng.integers(0, n_ref - l + 1))
        b = int(rng.integers(0, n_qry - l + 1))
        qry[b:b + l] = _mutate(rng, ref[a:a + l], identity)
    ref, qry = _to_ascii(ref), _to_ascii(qry)
    for seq in (ref, qry):
        if n_frac > 0 and seq.size > 0:
            k = max(1, int(n_frac * seq.size / 8))
            for _ in range(k):
                s = int(rng.integers(0, seq.size))
                seq[s:s + int(rng.integers(1, 16))] = ord("N")
        if alphabet_noise and seq.size > 0:
            k = max(1, seq.size // 50)
            idx = rng.integers(0, seq.size, size=k)
            seq[idx[: k // 2]] = np.frombuffer(b"acgt", np.uint8)[rng.integers(0, 4, k // 2)]
            seq[idx[k // 2:]] = np.frombuffer(b"RYKMSWn-", np.uint8)[
                rng.integers(0, 8, k - k // 2)]
    return ref, qry
