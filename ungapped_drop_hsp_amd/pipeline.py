"""Sequencing of one pass over a query batch through the C ABI.

Host orchestration only (which call follows which, buffer sizing); every step of the
path runs in libhspz's kernels.  The order is the pages': plan (C.1-C.3), then per chunk
find_hits (C.4-C.5), score_gate (D.1-D.3), compact (D.4), materialize and compact_hsps
(E.1-E.5).
"""
from __future__ import annotations

from collections import defaultdict
from typing import Dict, List, Optional

import numpy as np

from . import SEGMENT_PAIR, Engine


class PassBuffers:
    """Caller-owned device buffers for one chunk at a time, grown on demand.

    Growth is geometric (at least a quarter more each time), so chunks that differ by a
    few anchors do not reallocate the buffers pass after pass.
    """

    def __init__(self, device: int = 0, anchors: int = 0, survivors: int = 0):
        import torch
        self.torch = torch
        self.dev = torch.device("cuda", device)
        self.cap_a = 0
        self.cap_s = 0
        self.ensure(anchors, survivors)

    def ensure(self, n_anchors: int, n_surv: int = 0):
        t = self.torch
        if n_anchors > self.cap_a or self.cap_a == 0:
            cap = max(int(n_anchors), 1024, self.cap_a + self.cap_a // 4)
            self.anchors = t.empty(cap, dtype=t.int64, device=self.dev)
            self.flags = t.empty(cap + 16, dtype=t.uint8, device=self.dev)
            self.ids = t.empty(cap, dtype=t.int32, device=self.dev)
            self.cap_a = cap
        if n_surv > self.cap_s or self.cap_s == 0:
            cap = max(int(n_surv), 1024, self.cap_s + self.cap_s // 4)
            self.hsp = t.empty((cap, 4), dtype=t.int32, device=self.dev)
            self.status = t.empty(cap + 16, dtype=t.uint8, device=self.dev)
            self.out = t.empty((cap, 4), dtype=t.int32, device=self.dev)
            self.cap_s = cap


class StageTimer:
    """HIP events around each ABI call, recorded on the stream the call launches on.

    ``spans[name]`` collects (start, end) event pairs; ``elapsed_ms()`` sums them per
    stage after a synchronisation.  ``units[name]`` holds what each launch processed
    (anchors for the gate), so per-launch averages can be formed.  ``only`` limits the
    events to the named stages (each event costs host time between launches).
    """

    def __init__(self, only=None):
        import torch
        self.torch = torch
        self.only = None if only is None else frozenset(only)  # stages to time (None: all)
        self.spans = defaultdict(list)
        self.units = defaultdict(list)

    def start(self, name: str, stream=None):
        if self.only is not None and name not in self.only:
            return None
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        return ev

    def stop(self, name: str, ev0, units: int = 0, stream=None):
        if ev0 is None:
            return
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev1.record(stream)
        self.spans[name].append((ev0, ev1))
        self.units[name].append(int(units))

    def elapsed_ms(self) -> Dict[str, List[float]]:
        self.torch.cuda.synchronize()
        return {k: [a.elapsed_time(b) for a, b in v] for k, v in self.spans.items()}

    def reset(self):
        self.spans.clear()
        self.units.clear()


def _host_records(t, n: int) -> np.ndarray:
    if n == 0:
        return np.zeros(0, SEGMENT_PAIR)
    return t[:n].cpu().numpy().view(SEGMENT_PAIR).reshape(-1)


def run_pass(eng: Engine, seed_lo: int, seed_hi: int, bufs: PassBuffers, *,
             collect: bool = False, stream=None, timer: Optional[StageTimer] = None) -> Dict:
    """Plan seeds [seed_lo, seed_hi) and run every chunk to accepted records.

    The accepted records of every chunk are copied to the host (the pass's output).  With
    ``collect`` the anchors, flags, ids, records and status of each chunk are copied too.
    With ``timer`` every call is bracketed by events on the launch stream.
    """
    tm = timer

    def t0(name):
        return tm.start(name, stream) if tm else None

    def t1(name, ev, units=0):
        if tm:
            tm.stop(name, ev, units, stream)

    ev = t0("plan")
    total, nch = eng.plan(seed_lo, seed_hi, stream=stream)
    t1("plan", ev, seed_hi - seed_lo)
    out: Dict = dict(total=total, n_chunks=nch, chunks=[], n_surv=0, n_acc=0)
    for c in range(nch):
        ch = eng.get_chunk(c)
        n = ch["n_hits"]
        bufs.ensure(n)
        ev = t0("find_hits")
        eng.find_hits(c, bufs.anchors, stream=stream)
        t1("find_hits", ev, n)
        ev = t0("score_gate")
        eng.score_gate(bufs.anchors, n, bufs.flags, stream=stream)
        t1("score_gate", ev, n)
        ev = t0("compact")
        ns = eng.compact(bufs.flags, n, bufs.ids, cap=n, stream=stream)
        t1("compact", ev, n)
        bufs.ensure(n, ns)
        ev = t0("materialize")
        eng.materialize(bufs.anchors, bufs.ids, ns, bufs.hsp, bufs.status, stream=stream)
        t1("materialize", ev, ns)
        ev = t0("compact_hsps")
        na = eng.compact_hsps(bufs.hsp, bufs.status, ns, bufs.out, stream=stream)
        t1("compact_hsps", ev, ns)
        rec: Dict = dict(chunk=ch, n_anchors=n, n_surv=ns, n_acc=na,
                         accepted=_host_records(bufs.out, na))
        if collect:
            rec["anchors"] = bufs.anchors[:n].cpu().numpy().view(np.uint64)
            rec["flags"] = bufs.flags[:n].cpu().numpy()
            rec["ids"] = bufs.ids[:ns].cpu().numpy().view(np.uint32)
            rec["hsp"] = _host_records(bufs.hsp, ns)
            rec["status"] = bufs.status[:ns].cpu().numpy()
        out["chunks"].append(rec)
        out["n_surv"] += ns
        out["n_acc"] += na
    return out


def batches(eng: Engine, batch_len: int, query_len: int) -> List[tuple]:
    """Seed ranges of consecutive query-position slices of batch_len (0 = whole query)."""
    if batch_len <= 0:
        return [(0, eng.num_seeds())]
    out = []
    for pos in range(0, max(query_len, 1), batch_len):
        a, b = eng.seed_range(pos, pos + batch_len)
        if b > a:
            out.append((a, b))
    return out
