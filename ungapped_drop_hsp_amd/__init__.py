"""Python binding of libhspz, the MI355X seed-and-extend hot path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared
in ``include/hspz.h``.  PyTorch supplies device memory (tensors) and streams.  Importing
this package raises if ``libhspz.so`` has not been built -- there is no fallback.

Names follow the C ABI without the ``hspz_`` prefix.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhspz.so")

HSPZ_OK = 0
ERRORS = {-1: "HSPZ_E_INVALID", -2: "HSPZ_E_OVERFLOW", -3: "HSPZ_E_CAPACITY",
          -4: "HSPZ_E_NOMEM", -5: "HSPZ_E_HIP", -6: "HSPZ_E_STATE"}

SEGMENT_PAIR = np.dtype([("ref_start", "<u4"), ("query_start", "<u4"), ("len", "<u4"),
                         ("score", "<i4")])

# Every symbol include/hspz.h declares.
ABI_SYMBOLS = (
    "hspz_engine_create", "hspz_engine_destroy", "hspz_keep_threshold", "hspz_last_error",
    "hspz_upload_reference", "hspz_upload_query", "hspz_num_seeds", "hspz_seed_range",
    "hspz_plan", "hspz_get_chunk", "hspz_find_hits", "hspz_score_gate", "hspz_compact",
    "hspz_materialize", "hspz_compact_hsps", "hspz_get_seeds", "hspz_get_plan_arrays",
    "hspz_get_index", "hspz_debug_plan_counts", "hspz_debug_walk_steps",
    "hspz_debug_gate_deferred", "hspz_run_batch", "hspz_get_batch_records",
    "hspz_find_hits_gate", "hspz_dedup_records", "hspz_upload_seeds",
    "hspz_score_gate_noalloc", "hspz_debug_line_probe",
)


class HspzError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class Params(ctypes.Structure):
    _fields_ = [("seed_pattern", ctypes.c_char_p), ("sub", ctypes.c_int32 * 16),
                ("n_score", ctypes.c_int32), ("xdrop", ctypes.c_int32),
                ("hsp_threshold", ctypes.c_int32), ("expand_mode", ctypes.c_int32),
                ("max_hits", ctypes.c_uint64), ("chunk_walk", ctypes.c_int32),
                ("device", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("entropy_mode", ctypes.c_int32), ("ref_buckets", ctypes.c_int32),
                ("materialize_mode", ctypes.c_int32)]


class Chunk(ctypes.Structure):
    _fields_ = [("seed_lo", ctypes.c_uint64), ("seed_hi", ctypes.c_uint64),
                ("hit_lo", ctypes.c_uint64), ("n_hits", ctypes.c_uint64)]


class BatchStats(ctypes.Structure):
    _fields_ = [("n_anchors", ctypes.c_uint64), ("n_chunks", ctypes.c_uint64),
                ("n_survivors", ctypes.c_uint64), ("n_accepted", ctypes.c_uint64),
                ("gate_calls", ctypes.c_uint64), ("gate_ms", ctypes.c_double),
                ("whole_batch_gate", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python ungapped_drop_hsp_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, U64, I32, U32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32
    PU64, PU32 = ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint32)
    sig = {
        "hspz_engine_create": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.POINTER(P)]),
        "hspz_engine_destroy": (ctypes.c_int, [P]),
        "hspz_keep_threshold": (I32, [P]),
        "hspz_last_error": (ctypes.c_char_p, [P]),
        "hspz_upload_reference": (ctypes.c_int, [P, P, U64, P]),
        "hspz_upload_query": (ctypes.c_int, [P, P, U64, I32, P]),
        "hspz_upload_seeds": (ctypes.c_int, [P, P, P, U64, P]),
        "hspz_num_seeds": (U64, [P]),
        "hspz_seed_range": (ctypes.c_int, [P, U64, U64, PU64, PU64]),
        "hspz_plan": (ctypes.c_int, [P, U64, U64, P, PU64, PU32]),
        "hspz_get_chunk": (ctypes.c_int, [P, U32, ctypes.POINTER(Chunk)]),
        "hspz_find_hits": (ctypes.c_int, [P, U32, P, U64, P]),
        "hspz_score_gate": (ctypes.c_int, [P, P, U64, P, P]),
        "hspz_score_gate_noalloc": (ctypes.c_int, [P, P, U64, P, P]),
        "hspz_debug_line_probe": (ctypes.c_int, [P, U64, ctypes.c_uint32, ctypes.c_uint32,
                                                 ctypes.c_uint32, ctypes.c_uint32,
                                                 ctypes.c_uint32, ctypes.c_uint32, P, P]),
        "hspz_compact": (ctypes.c_int, [P, P, U64, P, U64, PU64, P]),
        "hspz_materialize": (ctypes.c_int, [P, P, P, U64, P, P, P]),
        "hspz_compact_hsps": (ctypes.c_int, [P, P, P, U64, P, U64, PU64, P]),
        "hspz_get_seeds": (ctypes.c_int, [P, U64, U64, P, P]),
        "hspz_get_plan_arrays": (ctypes.c_int, [P, P, P]),
        "hspz_get_index": (ctypes.c_int, [P, P, P, PU64, PU64]),
        "hspz_run_batch": (ctypes.c_int, [P, U64, U64, ctypes.c_int32,
                                          ctypes.POINTER(BatchStats), P]),
        "hspz_get_batch_records": (ctypes.c_int, [P, P, U64, PU64]),
        "hspz_find_hits_gate": (ctypes.c_int, [P, ctypes.c_uint32, P, U64, P, P]),
        "hspz_dedup_records": (ctypes.c_int, [P, U64, P, U64, PU64]),
        "hspz_debug_plan_counts": (ctypes.c_int, [P, P, U64, P, PU64, PU32]),
        "hspz_debug_walk_steps": (ctypes.c_int, [P, P, U64, PU64, P]),
        "hspz_debug_gate_deferred": (ctypes.c_int, [P, PU64, PU64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor, or a raw integer address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("expected a device tensor")
        if not x.is_contiguous():
            raise ValueError("expected a contiguous tensor")
        return x.data_ptr()
    raise TypeError(f"cannot take a device pointer of {type(x)}")


def _nbytes(x) -> Optional[int]:
    if hasattr(x, "data_ptr"):
        return x.numel() * x.element_size()
    return None


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host_bytes(seq) -> np.ndarray:
    if isinstance(seq, (bytes, bytearray)):
        return np.frombuffer(bytes(seq), dtype=np.uint8)
    a = np.ascontiguousarray(seq)
    if a.dtype != np.uint8:
        raise TypeError("sequence must be bytes or a uint8 array")
    return a


def dedup_records(records: np.ndarray) -> np.ndarray:
    """Exact-duplicate removal of accepted records (host): the first of equal records is
    kept, in input order."""
    rec = np.ascontiguousarray(records, dtype=SEGMENT_PAIR).reshape(-1)
    out = np.empty(max(rec.size, 1), SEGMENT_PAIR)
    n = ctypes.c_uint64()
    rc = _lib.hspz_dedup_records(rec.ctypes.data if rec.size else None, rec.size,
                                 out.ctypes.data, out.size, ctypes.byref(n))
    if rc != 0:
        raise HspzError(rc, _lib.hspz_last_error(None).decode())
    return out[:n.value].copy()


def debug_line_probe(region, region_bytes: int, window_dwords: int, in_flight: int,
                     blocks: int, iters: int, seed: int, key: int, sink, stream=None):
    """Launch the random-line probe (test-only; the caller times it on ``stream``)."""
    rc = _lib.hspz_debug_line_probe(_ptr(region), region_bytes, window_dwords, in_flight,
                                    blocks, iters, seed, key, _ptr(sink), _stream(stream))
    if rc != 0:
        raise HspzError(rc, "line probe rejected its arguments or failed to launch")


class Engine:
    """One engine: a reference index and one query strand on one device."""

    def __init__(self, seed_pattern: str, sub, n_score: int, xdrop: int, hsp_threshold: int,
                 max_hits: int = 0, expand_mode: int = 0, chunk_walk: int = 0,
                 device: int = 0, gate_mode: int = 0, entropy_mode: int = 0,
                 ref_buckets: int = 0, materialize_mode: int = 0):
        self._pat = seed_pattern.encode()
        m = np.asarray(sub, dtype=np.int32).reshape(-1)
        if m.size != 16:
            raise ValueError("sub must hold 16 entries (4x4, ref row, query column)")
        p = Params(self._pat, (ctypes.c_int32 * 16)(*m.tolist()), n_score, xdrop,
                   hsp_threshold, expand_mode, max_hits, chunk_walk, device, gate_mode,
                   entropy_mode, ref_buckets, materialize_mode)
        h = ctypes.c_void_p()
        rc = _lib.hspz_engine_create(ctypes.byref(p), ctypes.byref(h))
        if rc != HSPZ_OK:
            raise HspzError(rc, _lib.hspz_last_error(None).decode())
        self._h = h
        self.device = device

    # -- plumbing
    def _check(self, rc: int):
        if rc != HSPZ_OK:
            raise HspzError(rc, _lib.hspz_last_error(self._h).decode())

    def close(self):
        if getattr(self, "_h", None):
            _lib.hspz_engine_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- ABI
    @property
    def keep_threshold(self) -> int:
        return int(_lib.hspz_keep_threshold(self._h))

    def last_error(self) -> str:
        return _lib.hspz_last_error(self._h).decode()

    def upload_reference(self, seq, stream=None):
        a = _host_bytes(seq)
        self._check(_lib.hspz_upload_reference(self._h, a.ctypes.data, a.size, _stream(stream)))

    def upload_query(self, seq, strand: int = 0, stream=None):
        a = _host_bytes(seq)
        self._check(_lib.hspz_upload_query(self._h, a.ctypes.data, a.size, strand,
                                           _stream(stream)))

    def upload_seeds(self, kmer, q_end, stream=None):
        """The caller's seeds (packed k-mers, query ends) in place of the seeder's."""
        k = np.ascontiguousarray(kmer, dtype=np.uint32)
        q = np.ascontiguousarray(q_end, dtype=np.uint32)
        if k.shape != q.shape or k.ndim != 1:
            raise ValueError("kmer and q_end must be 1-D arrays of one length")
        self._check(_lib.hspz_upload_seeds(self._h, k.ctypes.data, q.ctypes.data, k.size,
                                           _stream(stream)))

    def num_seeds(self) -> int:
        return int(_lib.hspz_num_seeds(self._h))

    def seed_range(self, pos_lo: int, pos_hi: int) -> Tuple[int, int]:
        lo, hi = ctypes.c_uint64(), ctypes.c_uint64()
        self._check(_lib.hspz_seed_range(self._h, pos_lo, pos_hi, ctypes.byref(lo),
                                         ctypes.byref(hi)))
        return lo.value, hi.value

    def plan(self, seed_lo: int, seed_hi: int, stream=None) -> Tuple[int, int]:
        tot, nch = ctypes.c_uint64(), ctypes.c_uint32()
        self._check(_lib.hspz_plan(self._h, seed_lo, seed_hi, _stream(stream),
                                   ctypes.byref(tot), ctypes.byref(nch)))
        return tot.value, nch.value

    def get_chunk(self, i: int) -> Dict[str, int]:
        c = Chunk()
        self._check(_lib.hspz_get_chunk(self._h, i, ctypes.byref(c)))
        return dict(seed_lo=c.seed_lo, seed_hi=c.seed_hi, hit_lo=c.hit_lo, n_hits=c.n_hits)

    def find_hits(self, chunk: int, anchors, cap: Optional[int] = None, stream=None):
        if cap is None:
            cap = _nbytes(anchors) // 8
        self._check(_lib.hspz_find_hits(self._h, chunk, _ptr(anchors), cap, _stream(stream)))

    def find_hits_gate(self, chunk: int, anchors, flags, cap: Optional[int] = None,
                       stream=None):
        """find_hits + score_gate fused: all flags; anchors only where the flag is 1."""
        if cap is None:
            cap = _nbytes(anchors) // 8
        self._check(_lib.hspz_find_hits_gate(self._h, chunk, _ptr(anchors), cap, _ptr(flags),
                                             _stream(stream)))

    def score_gate(self, anchors, n: int, flags, stream=None):
        self._check(_lib.hspz_score_gate(self._h, _ptr(anchors), n, _ptr(flags),
                                         _stream(stream)))

    def score_gate_noalloc(self, anchors, n: int, flags, stream=None):
        self._check(_lib.hspz_score_gate_noalloc(self._h, _ptr(anchors), n, _ptr(flags),
                                                 _stream(stream)))

    def compact(self, flags, n: int, ids, cap: Optional[int] = None, stream=None) -> int:
        if cap is None:
            cap = _nbytes(ids) // 4 if ids is not None else 0
        out = ctypes.c_uint64()
        self._check(_lib.hspz_compact(self._h, _ptr(flags), n, _ptr(ids), cap, ctypes.byref(out),
                                      _stream(stream)))
        return out.value

    def materialize(self, anchors, ids, n_surv: int, hsp, status, stream=None):
        self._check(_lib.hspz_materialize(self._h, _ptr(anchors), _ptr(ids), n_surv, _ptr(hsp),
                                          _ptr(status), _stream(stream)))

    def compact_hsps(self, hsp, status, n: int, out, cap: Optional[int] = None,
                     stream=None) -> int:
        if cap is None:
            cap = _nbytes(out) // 16 if out is not None else 0
        res = ctypes.c_uint64()
        self._check(_lib.hspz_compact_hsps(self._h, _ptr(hsp), _ptr(status), n, _ptr(out), cap,
                                           ctypes.byref(res), _stream(stream)))
        return res.value

    def get_seeds(self, lo: int, hi: int) -> Tuple[np.ndarray, np.ndarray]:
        k = np.empty(max(hi - lo, 0), np.uint32)
        q = np.empty(max(hi - lo, 0), np.uint32)
        self._check(_lib.hspz_get_seeds(self._h, lo, hi, k.ctypes.data, q.ctypes.data))
        return k, q

    def run_batch(self, seed_lo: int, seed_hi: int, time_gate: bool = False,
                  stream=None) -> Dict:
        """The whole pass over seeds [seed_lo, seed_hi) in one native call; the accepted
        records stay in the engine's pinned staging (``batch_records``)."""
        st = BatchStats()
        self._check(_lib.hspz_run_batch(self._h, seed_lo, seed_hi, 1 if time_gate else 0,
                                        ctypes.byref(st), _stream(stream)))
        return {f: getattr(st, f) for f, _ in BatchStats._fields_}

    def batch_records(self) -> np.ndarray:
        """Accepted records of the last run_batch, in chunk order."""
        n = ctypes.c_uint64()
        self._check(_lib.hspz_get_batch_records(self._h, None, 0, ctypes.byref(n)))
        out = np.empty(max(n.value, 1), SEGMENT_PAIR)
        self._check(_lib.hspz_get_batch_records(self._h, out.ctypes.data, n.value,
                                                ctypes.byref(n)))
        return out[:n.value]

    def get_index(self) -> Tuple[np.ndarray, np.ndarray]:
        """(bucket ends with the leading 0, reference ends grouped by k-mer)."""
        nb, npos = ctypes.c_uint64(), ctypes.c_uint64()
        self._check(_lib.hspz_get_index(self._h, None, None, ctypes.byref(nb),
                                        ctypes.byref(npos)))
        end = np.empty(nb.value + 1, np.uint32)
        pos = np.empty(max(npos.value, 1), np.uint32)
        self._check(_lib.hspz_get_index(self._h, end.ctypes.data, pos.ctypes.data,
                                        ctypes.byref(nb), ctypes.byref(npos)))
        return end, pos[:npos.value]

    def get_plan_arrays(self, n: int) -> Tuple[np.ndarray, np.ndarray]:
        c = np.empty(max(n, 1), np.uint32)
        p = np.empty(max(n, 1), np.uint32)
        self._check(_lib.hspz_get_plan_arrays(self._h, c.ctypes.data, p.ctypes.data))
        return c[:n], p[:n]

    def debug_plan_counts(self, counts, stream=None) -> Tuple[int, int]:
        c = np.ascontiguousarray(counts, dtype=np.uint32)
        tot, nch = ctypes.c_uint64(), ctypes.c_uint32()
        self._check(_lib.hspz_debug_plan_counts(self._h, c.ctypes.data, c.size, _stream(stream),
                                                ctypes.byref(tot), ctypes.byref(nch)))
        return tot.value, nch.value

    def debug_walk_steps(self, anchors, n: int, stream=None) -> int:
        tot = ctypes.c_uint64()
        self._check(_lib.hspz_debug_walk_steps(self._h, _ptr(anchors), n, ctypes.byref(tot),
                                               _stream(stream)))
        return tot.value

    def debug_gate_deferred(self, stream=None) -> Tuple[int, int]:
        """(anchors sent to the second window stage, anchors decided by the exact walk)."""
        a, b = ctypes.c_uint64(), ctypes.c_uint64()
        self._check(_lib.hspz_debug_gate_deferred(self._h, ctypes.byref(a), ctypes.byref(b),
                                                  _stream(stream)))
        return a.value, b.value
