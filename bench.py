"""Benchmark of the seed-and-extend hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--cpu-seconds S]

A step is one whole pass over the workload's query seeds, for every strand and query
batch it names: plan (hit counts, global prefix, MAX_HITS chunk cut), then for every
chunk the backward expansion, the score gate, survivor compaction, exact materialization
and accepted-record compaction, with the accepted records copied to the host.  Each batch
is one call of the library's native driver (hspz_run_batch).  The
reference index, the query seeds and the encoded sequences are resident in HBM before the
timed region starts (the engine holds one strand at a time, so each strand is uploaded
before its own timed passes and the step time sums the strands).

Prints one JSON line: raw anchors/s through the whole pass (``value``), HSPs/s, per-stage
times from HIP events on the launch stream (one extra step instrumented throughout, after
the timed ones), the score gate's roofline figures (its launches timed inside the timed
steps) and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "raw anchors/s through gate+materialize at 1 GPU; gate HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
CUS, LANES, CLOCK_GHZ = 256, 64, 2.4
# One base step of an X-drop walk needs at least three 32-bit vector operations on
# CDNA4: forming the substitution-table address, the drawdown update (one saturating add
# on the drawdown's complement) and, shared between two bases through three-input
# min/add, the running extreme and the running score.  The ALU peak in base steps per
# second follows from the lane count.
OPS_PER_BASE_STEP = 3
ALU_PEAK_GSTEPS = CUS * LANES * CLOCK_GHZ / OPS_PER_BASE_STEP   # G base steps/s
# Compulsory bytes of one hspz_find_hits_gate call (expansion fused into the gate): per
# anchor its 4-byte bucket entry read and its 1-byte flag written; per seed its 4-byte
# inclusive prefix, bucket start and query end read.
GATE_BYTES_PER_ANCHOR = 5
GATE_BYTES_PER_SEED = 12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index (3 = 50 Mb x 50 Mb, the one the metric is quoted on)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle sample budget in seconds (0 skips the CPU leg)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--gate-mode", type=int, default=0, choices=[0, 1, 2, 3, 4, 5],
                    help="score gate variant (0 auto, 1 exact walk, 2 window, 3 narrow window, "
                         "4 reference-bucketed window, 5 key-grouped window)")
    return ap.parse_args()


def line_ceiling(torch, h, region_bytes: int, window_dwords: int):
    """Random-line rate of the memory fabric, from the library's probe kernel.

    The probe reads windows of ``window_dwords`` dwords at the start of random 128-byte
    lines of a region of ``region_bytes`` (each window one line), with 1, 2 or 4 windows in
    flight per lane; the best rate is the ceiling for a kernel whose traffic is one random
    line per unit of work in a footprint of that size.  Returns (lines/s, per-variant).
    """
    nbytes = max(128, (region_bytes + 127) // 128 * 128)
    region = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    blocks = 4096
    rates = {}
    for k in (1, 2, 4):
        iters = max(1, (1 << 26) // (blocks * 256 * k))
        args = (region, nbytes, window_dwords, k, blocks, iters, 12345, 0x5EED5EED, sink)
        h.debug_line_probe(*args, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            h.debug_line_probe(*args, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rates[k] = blocks * 256 * k * iters / (e0.elapsed_time(e1) / 3 / 1000.0)
    del region
    return max(rates.values()), {f"in_flight_{k}": v for k, v in rates.items()}


# The sources the hspz_find_hits_gate call is compiled from (its kernels, and the block scan
# and byte fill it launches); the committed counter summary holds their combined SHA-256.
GATE_SOURCES = ("k_gate.hip", "walk.h", "wave.h", "hspz_internal.h", "k_plan.hip",
                "k_bucket.hip")


def gate_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in GATE_SOURCES:
        with open(os.path.join(ROOT, "ungapped_drop_hsp_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gate_traffic(workload: str, gate_mode: int, anchors_per_call: float):
    """Measured fabric bytes per timed gate call from the committed counter summary.

    The summary was taken with rocprofv3 FETCH_SIZE / WRITE_SIZE runs and calibrated
    against a plain device copy.  It applies only to the sources it was measured on, to
    the same workload and gate mode, and to calls of the same size; otherwise None.
    """
    path = os.path.join(ROOT, "profiles", "find_hits_gate_traffic_c3_50Mb.json")
    try:
        rec = json.load(open(path))
        sha = gate_sources_sha()
    except OSError:
        return None
    if (rec.get("gate_sources_sha256") != sha or not rec["workload"].startswith(workload)
            or rec.get("gate_mode", 0) != gate_mode
            or abs(rec.get("anchors_per_call", 0) - anchors_per_call) > 1e-3 * anchors_per_call):
        return None
    return rec["hbm_bytes_per_call"]


# State of the CPU oracle leg, built before any GPU call and inherited by the forked
# worker processes of the all-core timing.
_ORC = {}
_BLOCK = 20_000


def cpu_setup(w, workers: int):
    """Untimed oracle setup (encoding, the reference index, the query's seed list: the
    GPU side also does these outside its timed region), then a pool of worker processes
    forked before this process touches the GPU; they never use it."""
    import multiprocessing as mp

    import oracle
    p = w.params()
    R = oracle.Reference(w.ref, p["seed_pattern"])
    qc = oracle.strand_codes(w.query, "+")
    seeds = oracle.query_seeds(qc, p["seed_pattern"])
    n = seeds[0].size
    _ORC.update(R=R, qc=qc, seeds=seeds, p=p, n=n,
                order=np.random.default_rng(0).permutation(max(n // _BLOCK, 1)))
    return mp.get_context("fork").Pool(workers) if workers > 1 else None


def _oracle_blocks(blocks, deadline=None, budget=None):
    """The oracle's whole pass (counts, prefix, chunks, anchors, gate, compaction,
    materialization) over contiguous blocks of query seeds, until the time is up."""
    import oracle
    o_ = _ORC
    anchors = surv = acc = seeds_done = 0
    t0 = time.perf_counter()
    for b in blocks:
        lo, hi = int(b) * _BLOCK, min(o_["n"], int(b) * _BLOCK + _BLOCK)
        o = oracle.run_pass(o_["R"], o_["qc"], o_["p"], seed_range=(lo, hi), seeds=o_["seeds"])
        anchors += o["total"]
        seeds_done += hi - lo
        for ch in o["chunks"]:
            surv += ch["ids"].size
            acc += ch["accepted"].size
        now = time.perf_counter()
        if (budget is not None and now - t0 >= budget) or \
                (deadline is not None and time.time() >= deadline):
            break
    return dict(anchors=anchors, surv=surv, acc=acc, seeds=seeds_done,
                seconds=time.perf_counter() - t0)


def _oracle_worker(args):
    rank, workers, deadline = args
    return _oracle_blocks(_ORC["order"][rank::workers], deadline=deadline)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pool, workers: int, budget_s: float):
    """The CPU oracle, as it stands, on a bounded sample of the same pass.

    Contiguous blocks of 20,000 query seeds, spread evenly over the query in a fixed
    shuffled order, go through the oracle's whole pass.  Timed twice: in this process on
    one core for the budget, then in ``workers`` forked processes at once (worker w takes
    blocks w, w + workers, ... of the same order) for the same budget.  The oracle itself
    is single-threaded and unchanged; the all-core figure is the summed raw anchors over
    the longest worker's time.
    """
    one = _oracle_blocks(_ORC["order"], budget=budget_s)
    n = _ORC["n"]
    single = dict(value=one["anchors"] / one["seconds"], unit="anchors/s", cores=1,
                  seconds=one["seconds"],
                  sample=f"{one['seeds']} of {n} query seeds: {one['anchors']} raw anchors, "
                         f"{one['surv']} survivors, {one['acc']} accepted")
    out = dict(value=single["value"], unit="anchors/s", cores=1, kind="oracle",
               sample=f"blocks of {_BLOCK} query seeds spread over the query; single "
                      f"thread: {single['sample']} in {one['seconds']:.1f} s",
               seconds=one["seconds"], single_thread=single, nproc=os.cpu_count(),
               cpu_model=_cpu_model())
    if pool is None:
        return out
    deadline = time.time() + budget_s
    t0 = time.perf_counter()
    parts = pool.map(_oracle_worker, [(r, workers, deadline) for r in range(workers)])
    el = max(max(p_["seconds"] for p_ in parts), time.perf_counter() - t0)
    tot = {k: sum(p_[k] for p_ in parts) for k in ("anchors", "surv", "acc", "seeds")}
    out.update(value=tot["anchors"] / el, cores=workers, seconds=el,
               sample=f"blocks of {_BLOCK} query seeds spread over the query, one oracle per "
                      f"worker process on {workers} cores: {tot['seeds']} of {n} query seeds, "
                      f"{tot['anchors']} raw anchors, {tot['surv']} survivors, {tot['acc']} "
                      f"accepted in {el:.1f} s; single thread: {single['value']:.4g} "
                      f"anchors/s")
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path needs no exchange between GPUs, so "
              "no multi-GPU figure is produced (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    from workloads import build

    t = time.perf_counter()
    w = build(args.config)
    gen_s = time.perf_counter() - t
    p = w.params()
    print(f"[bench] workload {w.name} generated in {gen_s:.1f} s", file=sys.stderr, flush=True)
    # The CPU oracle leg's setup and worker processes come first: the workers are forked
    # before this process initialises the GPU.  Workers: the cores this process may run
    # on, at most 16 (one GPU's share of the host).
    pool = None
    workers = min(len(os.sched_getaffinity(0)), 16)
    if args.cpu_seconds > 0:
        t = time.perf_counter()
        pool = cpu_setup(w, workers)
        print(f"[bench] oracle setup and {workers} worker processes in "
              f"{time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    import ungapped_drop_hsp_amd as h
    from ungapped_drop_hsp_amd.pipeline import PassBuffers, StageTimer, batches, run_pass

    eng = h.Engine(seed_pattern=p["seed_pattern"], sub=p["sub"], n_score=p["n_score"],
                   xdrop=p["xdrop"], hsp_threshold=p["hsp_threshold"], max_hits=p["max_hits"],
                   gate_mode=args.gate_mode)
    t = time.perf_counter()
    eng.upload_reference(w.ref)
    torch.cuda.synchronize()
    upload_s = time.perf_counter() - t
    print(f"[bench] reference index uploaded in {upload_s:.1f} s", file=sys.stderr, flush=True)

    # A step covers every strand and every query batch of the workload.  The engine holds
    # one query strand at a time, so each strand's seeds are uploaded before its own
    # warmup and timed passes; the step time is the sum over strands.
    # The timed passes run each batch through the native driver (hspz_run_batch: plan and
    # every chunk in one call, records to pinned host memory), which brackets each
    # score-gate call with HIP events on the launch stream for the roofline.  The
    # per-stage breakdown comes from one more step per strand through the per-call ABI,
    # with events around every call, after the timed ones.
    bufs = PassBuffers(0)
    stages = StageTimer()
    wall = 0.0
    gate_ms_sum = 0.0
    gate_calls = gate_anchors = whole_batches = 0
    anchors = surv = acc = chunks = seeds = 0
    chunk_list = []  # (strand, lo, hi) batches of the last step, for the walk statistics
    # Python's cyclic collector stays off over the passes: a collection inside the timed
    # loop stalls the launching thread (tens of ms on the 200 Mb workload) and shows up
    # as idle GPU time in whichever stage it lands.
    gc.collect()
    gc.disable()
    for strand in w.strands:
        t = time.perf_counter()
        eng.upload_query(w.query, strand=1 if strand == "-" else 0)
        torch.cuda.synchronize()
        upload_s += time.perf_counter() - t
        bs = batches(eng, w.batch_len, w.query.size)
        seeds += eng.num_seeds()
        print(f"[bench] strand {strand}: {eng.num_seeds()} seeds in {len(bs)} batch(es)",
              file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            for lo, hi in bs:
                eng.run_batch(lo, hi)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            res = [eng.run_batch(lo, hi, time_gate=True) for lo, hi in bs]
            for r in res:
                gate_ms_sum += r["gate_ms"]
                gate_calls += r["gate_calls"]
                gate_anchors += r["n_anchors"]
                whole_batches += r["whole_batch_gate"]
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        for lo, hi in bs:
            run_pass(eng, lo, hi, bufs, timer=stages)
        anchors += sum(r["n_anchors"] for r in res)
        surv += sum(r["n_survivors"] for r in res)
        acc += sum(r["n_accepted"] for r in res)
        chunks += sum(r["n_chunks"] for r in res)
        # the walk statistics below run on the current strand's last batches
        chunk_list = [(strand, lo, hi) for lo, hi in bs]
    gc.enable()
    print(f"[bench] {args.steps} timed steps in {wall:.3f} s", file=sys.stderr, flush=True)

    ms_per_step = 1000.0 * wall / args.steps
    value = anchors / (ms_per_step / 1000.0)
    stage_ms = {k: sum(v) for k, v in stages.elapsed_ms().items()}

    # Gate roofline: compulsory bytes and exact base steps of the launches timed above.
    gate_launches = gate_calls
    gate_ms_avg = gate_ms_sum / gate_launches
    units_avg = gate_anchors / gate_launches
    gate_bytes_avg = (GATE_BYTES_PER_ANCHOR * gate_anchors
                      + GATE_BYTES_PER_SEED * seeds * args.steps) / gate_launches
    gate_gbs = gate_bytes_avg / (gate_ms_avg * 1e6)
    # base steps per anchor and the gate's stage split, over the last strand's batches
    steps_total = walked = 0
    deferred = [0, 0]
    for _, lo, hi in chunk_list:
        _, nch = eng.plan(lo, hi)
        for c in range(nch):
            ch = eng.get_chunk(c)
            bufs.ensure(ch["n_hits"])
            eng.find_hits(c, bufs.anchors)
            steps_total += eng.debug_walk_steps(bufs.anchors, ch["n_hits"])
            walked += ch["n_hits"]
            eng.score_gate(bufs.anchors, ch["n_hits"], bufs.flags)
            try:
                d2, dx = eng.debug_gate_deferred()
                deferred = [deferred[0] + d2, deferred[1] + dx]
            except h.HspzError:
                deferred = None
    steps_per_anchor = steps_total / max(walked, 1)
    gate_gsteps = steps_per_anchor * units_avg / (gate_ms_avg * 1e6)

    traffic = gate_traffic(w.name, args.gate_mode, units_avg)
    # The gate's reference windows are 64-byte reads from the 4-bit reference copy and its
    # line-split twin (about one byte per reference base in all); the plan's lookups read
    # one dword of the 4-bit count table (eight keys' counts) per seed.
    ceiling, ceiling_runs = line_ceiling(torch, h, int(w.ref.size), 16)
    gate_lines = None if traffic is None else traffic / 128.0 / (gate_ms_avg / 1000.0)
    ct_bytes = 4 * -(-(4 ** len([c for c in p["seed_pattern"] if c == "1"])) // 8)
    plan_ceiling, plan_runs = line_ceiling(torch, h, ct_bytes, 1)
    plan_ms = stage_ms.get("plan", 0.0)  # every seed of the step planned once

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    out = dict(
        metric=METRIC, value=value, unit="anchors/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="int32", data="synthetic",
        config=dict(workload=w.name, ref_bp=int(w.ref.size), query_bp=int(w.query.size),
                    strands=w.strands, batch_bp=w.batch_len or int(w.query.size),
                    seed_pattern=p["seed_pattern"], xdrop=p["xdrop"],
                    hsp_threshold=p["hsp_threshold"], max_hits=p["max_hits"], seeds=seeds,
                    raw_anchors=anchors, chunks=chunks, survivors=surv, accepted=acc,
                    gate_mode=args.gate_mode),
        hsps_per_s=acc / (ms_per_step / 1000.0),
        stage_ms=stage_ms,
        roofline=dict(bound="alu", achieved=gate_gsteps, peak=ALU_PEAK_GSTEPS,
                      unit="G base-steps/s", frac=gate_gsteps / ALU_PEAK_GSTEPS,
                      traffic=traffic,
                      kernel=("the gate over the whole batch at once (key-grouped first "
                              "window stage forming its own anchors, its workgroups then "
                              "running the second stage and exact walks of their deferred "
                              "anchors)"
                              if whole_batches else
                              "find_hits_gate per chunk (first window stage forming its own "
                              "anchors, key-grouped when a chunk holds enough seeds; second "
                              "stage; exact list)"),
                      launches_per_step=gate_launches // args.steps,
                      avg_launch_ms=gate_ms_avg, anchors_per_launch=units_avg,
                      base_steps_per_anchor=steps_per_anchor),
        gate_hbm=dict(achieved=gate_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=gate_gbs / HBM_PEAK_GBS, bytes_per_anchor=GATE_BYTES_PER_ANCHOR,
                      bytes_per_seed=GATE_BYTES_PER_SEED, bytes_per_launch=gate_bytes_avg),
        gate_anchors_per_s=units_avg / (gate_ms_avg / 1000.0),
        # the gate's measured fabric traffic in 128-byte lines/s against the random-line
        # rate of a plain gather kernel, measured in this run
        gate_lines=dict(achieved=gate_lines, ceiling=ceiling, unit="lines/s",
                        frac=None if gate_lines is None else gate_lines / ceiling,
                        ceiling_probe=dict(region_bytes=int(w.ref.size), window_bytes=64,
                                           **ceiling_runs)),
        # the plan's random lines: one count-table dword per seed, over the plan stage's
        # time (hit counts, block scan, offsets, chunk walk) in the instrumented pass
        plan_lines=dict(achieved=seeds / (plan_ms / 1000.0) if plan_ms > 0 else None,
                        ceiling=plan_ceiling, unit="lines/s",
                        frac=seeds / (plan_ms / 1000.0) / plan_ceiling if plan_ms > 0 else None,
                        ceiling_probe=dict(region_bytes=ct_bytes, window_bytes=4,
                                           **plan_runs)),
        gate_stage2_fraction=None if deferred is None else deferred[0] / max(walked, 1),
        gate_exact_fraction=None if deferred is None else deferred[1] / max(walked, 1),
        setup_s=dict(generate=gen_s, upload=upload_s),
    )
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(pool, workers, args.cpu_seconds)
        if pool is not None:
            pool.close()
            pool.join()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
