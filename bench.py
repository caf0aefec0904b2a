#!/usr/bin/env python3
"""Benchmark: batched DMA-descriptor building on one MI355X.

One step = the whole hot path over one batch: page-rounded MR lookup, PRP
build (PRP1/PRP2 + chained lists; packed lists by default, --layout page for
one run of list pages per request) and stable split by queue, three calls on
one stream, over the 16,777,216-request Mixed workload (256 GiB heap of
4,194,304 GPU pages, 4,096 regions, log-uniform 512 B - 1 MiB requests,
Zipf(1.1) over 64 queues). Inputs are resident in HBM before timing starts.

Prints ONE JSON line:
  value        requests per second (millions) over the K timed steps (wall
               clock between two synchronizations)
  step         median/min/p95 of one step from HIP events around each of
               >= 20 further steps; algorithmic bytes with every column
               counted once (and the per-call sum beside it)
  roofline     the dominant call (the PRP build of the step's layout):
               algorithmic bytes of one launch / its mean duration from HIP
               events recorded on its stream around every call of >= 10
               sampled timed steps (per_call_ms likewise)
  batch_call   dmadesc_build_batch (lookup, PRP build and split in one call
               that reads the request columns once) on the same batch
  graph_step   the step's calls captured once in a HIP graph and replayed
               (median/min/p95 of replays): the device time without the
               host's per-call launch cost
  per_config   Tiny, Small-I/O, Large/chaining and MR-heavy, each with its own
               functions, median/min/p95 over >= 20 iterations (>= 200 for
               Tiny and Small), eager and as graph replays
  split_alone  dmadesc_partition_by_queue alone over 64 and 256 Zipf queues
               (the two rankings)
  emit_sqe, registry, build_put, cq_mirror: the stages beside the path,
               timed after the steps
  cpu_baseline the single-threaded oracle, per function and end to end,
               median of 3 runs on one pinned core

Profiler passes use --quick (the warm-up and timed steps only),
--stage-emit-sqe (the submission-entry stage alone), --stage-registry (the
registry's two batches alone), --copy-calibration (a 1 GiB device copy, for
counter scales) and --list-write-floor.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD public specification
PRP_SOURCES = ["build_prp.hip", "dd_device.hpp", "dd_lookback.hpp"]


def traffic_file(layout: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_build_prp_{layout}_{workload}.json")


def recorded_traffic(layout: str, workload: str):
    """HBM bytes per launch of the PRP build from the counter record in
    profiles/, or None when there is none or the kernel sources changed
    since the counters were taken."""
    tf = traffic_file(layout, workload)
    if not os.path.exists(tf):
        return None
    with open(tf) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != prp_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed",
                    choices=["tiny", "small", "large", "mrheavy", "mixed"])
    ap.add_argument("--layout", default="packed", choices=["packed", "page"],
                    help="PRP list layout of the timed step: lists back to back "
                         "(dmadesc_build_prp_packed) or one run of list pages per request "
                         "(dmadesc_build_prp); the other layout's PRP build is timed too")
    ap.add_argument("--cpu-sample", type=int, default=1 << 24,
                    help="requests of the workload the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sampled-steps", type=int, default=10,
                    help="timed steps that carry per-call HIP events (at least 10; each "
                         "event record is a queue marker that costs a few microseconds)")
    ap.add_argument("--dist-steps", type=int, default=30,
                    help="steps timed one by one with HIP events for median/min/p95")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config lines of the other workloads")
    ap.add_argument("--quick", action="store_true",
                    help="warm-up and timed steps only (for profiler passes): no other "
                         "layout, step distribution, batch call, configs, stages or CPU baseline")
    ap.add_argument("--emit-reps", type=int, default=20,
                    help="launches of the submission-entry stage timed after the steps "
                         "(0 = skip it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for counter scaling) and exit")
    ap.add_argument("--list-write-floor", action="store_true",
                    help="time a library scatter that writes the same 128-byte list lines "
                         "as the PRP build (its layout's write floor) and exit")
    ap.add_argument("--stage-emit-sqe", action="store_true",
                    help="run the step's calls once, then time only the submission-entry "
                         "stage on their outputs (--emit-reps launches; for profiler passes) "
                         "and exit")
    ap.add_argument("--stage-registry", action="store_true",
                    help="time only the registry's register and deregister batches "
                         "(10 calls each; for profiler passes) and exit")
    return ap.parse_args()


def prp_source_hash() -> str:
    h = hashlib.sha256()
    for f in PRP_SOURCES:
        with open(os.path.join(ROOT, "memory_dma_descriptor_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(d, np):
    """Bytes each call must move, each column once (per request: lookup 16
    read + 25 written; PRP 16 read + 8 per GPU page touched, 17 written + 8
    per list word; split 4 read + 4 written; the region table 20 per region).
    List words: page layout m + L - 1 per request (entries and chain
    pointers); packed layout the whole dense range, E + floor(E / 511) words
    for E entries in all. `step_*` count every column of the step once: off
    and len are read once although both the lookup and the PRP build take
    them."""
    off, ln = d["off"], d["len"]
    n = off.shape[0]
    heap = np.uint64(d["lut_entries"]) * np.uint64(65536)
    valid = (ln > 0) & (off % 4 == 0) & (off + ln <= heap) & (off + ln >= off)
    pages = np.where(valid, ((off & np.uint64(4095)) + ln + np.uint64(4095)) >> np.uint64(12), 0)
    frames = np.where(valid, ((off + ln - np.uint64(1)) >> np.uint64(16)) - (off >> np.uint64(16)) + np.uint64(1), 0)
    lists = pages >= 3
    m = np.where(lists, pages - 1, 0).astype(np.float64)
    lp = np.where(lists, (pages - 2 + 510) // 511, 0).astype(np.float64)
    entries = float((m + lp - np.where(lists, 1.0, 0.0)).sum())
    e_total = int(m.sum())
    packed_words = float(e_total + e_total // 511)
    lookup = n * (16 + 25) + d["regions"] * 20
    prp_base = n * (16 + 17) + 8 * float(frames.sum())
    split = n * 8
    out = dict(lookup=float(lookup), build_prp=prp_base + 8 * entries,
               build_prp_packed=prp_base + 8 * packed_words, partition=float(split),
               list_entries=entries, prp_entries=float(pages.astype(np.float64).sum()))
    # The step, each column once: off/len read once, whatever reads them.
    for layout, key in (("page", "build_prp"), ("packed", "build_prp_packed")):
        b = 0.0
        if d["regions"]:
            b += out["lookup"]
        if d["lut_entries"]:
            b += out[key] - (n * 16 if d["regions"] else 0)
        if d["nqueues"]:
            b += split
        out[f"step_{layout}"] = b
        out[f"step_sum_{layout}"] = (out["lookup"] if d["regions"] else 0) + \
            (out[key] if d["lut_entries"] else 0) + (split if d["nqueues"] else 0)
    return out


def dist(np, ms):
    """median, min and p95 of a list of milliseconds."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 5), "min_ms": round(float(a.min()), 5),
            "p95_ms": round(float(np.percentile(a, 95)), 5), "iterations": int(a.size)}


def timed_iters(torch, np, fn, reps, warm=3):
    """Runs fn warm + reps times, each bracketed by HIP events on the current
    stream; returns the reps durations in ms."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


class Step:
    """The path's calls over one uploaded workload: lookup (if it has
    regions), PRP build (if it has a heap) and split (if it has queues), in
    that order on the current stream, with outputs and workspaces reused."""

    def __init__(self, dd, torch, np, d, packed):
        self.dd, self.torch, self.d, self.packed = dd, torch, d, packed
        dev = torch.device("cuda:0")
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        self.n, self.nq, self.bus = d["n"], d["nqueues"], d["list_bus_base"]
        self.rs, self.re, self.rk = up(d["rstart"]), up(d["rend"]), up(d["rlkey"])
        self.off, self.ln, self.qid, self.lut = up(d["off"]), up(d["len"]), up(d["qid"]), up(d["lut"])
        self.lk = self.pr = self.sp = self.bt = None
        self.pool = self.pool_pages = None
        need = dd.workspace_bytes(dd.OP_MR_LOOKUP, self.n, d["regions"])
        self.ws_lk = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        if d["lut_entries"]:
            self.pool, self.pool_pages = self.pool_for(packed)
            self.ws_prp = torch.empty(max(dd.workspace_bytes(dd.OP_BUILD_PRP, self.n), 1),
                                      dtype=torch.uint8, device=dev)
        if self.nq:
            self.ws_sp = torch.empty(max(dd.workspace_bytes(dd.OP_PARTITION, self.n, self.nq), 1),
                                     dtype=torch.uint8, device=dev)

    def pool_for(self, packed):
        """A pool of exactly the pages the batch needs (asked of the library
        itself: with an empty pool the call still reports them)."""
        torch, dev = self.torch, self.torch.device("cuda:0")
        empty = torch.empty((0, 512), dtype=torch.uint64, device=dev)
        probe = self.dd.build_prp(self.lut, self.off, self.ln, self.bus, empty, packed=packed)
        pages = int(probe["total_pages"].cpu()[0])
        return torch.empty((max(pages, 1), 512), dtype=torch.uint64, device=dev), pages

    def calls(self):
        out = []
        if self.d["regions"]:
            out.append("mr_lookup")
        if self.d["lut_entries"]:
            out.append("build_prp_packed" if self.packed else "build_prp")
        if self.nq:
            out.append("partition_by_queue")
        return out

    def run(self, ev=None):
        """One step; with `ev` (a list of len(calls) + 1 events) each call is
        bracketed on the stream it runs on."""
        dd, d = self.dd, self.d
        k = 0
        if ev:
            ev[0].record()
        if d["regions"]:
            self.lk = dd.mr_lookup(self.rs, self.re, self.rk, self.off, self.ln,
                                   va_base=d["va_base"], out=self.lk, ws=self.ws_lk)
            k += 1
            if ev:
                ev[k].record()
        if d["lut_entries"]:
            self.pr = dd.build_prp(self.lut, self.off, self.ln, self.bus, self.pool, out=self.pr,
                                   ws=self.ws_prp, packed=self.packed, check=False)
            k += 1
            if ev:
                ev[k].record()
        if self.nq:
            self.sp = dd.partition_by_queue(self.qid, self.nq, out=self.sp, ws=self.ws_sp,
                                            check=False)
            k += 1
            if ev:
                ev[k].record()

    def batch(self):
        """The same step as one dmadesc_build_batch call."""
        d = self.d
        if self.bt is None:
            self.ws_bt = self.torch.empty(
                self.dd.batch_workspace_bytes(self.n, self.nq, d["regions"]),
                dtype=self.torch.uint8, device=self.torch.device("cuda:0"))
        self.bt = self.dd.build_batch(self.lut, self.off, self.ln, self.qid, self.nq, self.bus,
                                      self.pool, self.rs, self.re, self.rk, va_base=d["va_base"],
                                      packed=self.packed, lookup=bool(d["regions"]), out=self.bt,
                                      ws=self.ws_bt, check=False)

    def check_outputs(self, np):
        """After the timed work: no refused requests beyond those the
        workload itself makes, no expired slot-scan wait, no overflow ids."""
        res = {}
        if self.pr is not None:
            st = self.pr["status"].cpu().numpy()
            res["refused_requests"] = int((st != 0).sum())
            res["expired_waits"] = int(self.ws_prp[4:8].view(self.torch.int32).item())
            if res["expired_waits"] or (st == self.dd.PRP_EBUSY).any():
                raise RuntimeError("a slot-scan wait expired during the benchmark")
        if self.sp is not None:
            res["overflow_ids"] = int(self.sp["n_invalid"].view(self.torch.int64)[0].item())
        return res


def graph_step(torch, np, st, reps):
    """The step's calls captured once in a HIP graph and replayed reps times
    (each replay bracketed by events): the device time of the step without
    the host's per-call launch cost, which dominates small batches."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st.run()
    ms = timed_iters(torch, np, g.replay, reps)
    return g, ms


def run_config(dd, torch, np, name, reps, packed=True):
    """One workload with its own functions (lookup, PRP build, split as it
    has them): median/min/p95 of reps steps, per-call medians, rates."""
    import synth
    d = synth.generate(name)
    ab = algorithmic_bytes(d, np)
    st = Step(dd, torch, np, d, packed)
    layout = "packed" if packed else "page"
    step_ms = timed_iters(torch, np, st.run, reps)
    calls = st.calls()
    ev_ms = {c: [] for c in calls}
    for _ in range(min(reps, 50)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        st.run(ev)
        torch.cuda.synchronize()
        for k, c in enumerate(calls):
            ev_ms[c].append(ev[k].elapsed_time(ev[k + 1]))
    med = float(np.median(step_ms))
    nbytes = ab[f"step_{layout}"]
    out = {"workload": name, "requests": d["n"], "functions": calls,
           "requests_per_s": round(d["n"] / (med * 1e-3), 1),
           "step": dist(np, step_ms),
           "step_algorithmic_bytes": nbytes,
           "step_algorithmic_gbs": round(nbytes / (med * 1e-3) / 1e9, 1),
           "step_frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "per_call_median_ms": {c: round(float(np.median(v)), 5) for c, v in ev_ms.items()}}
    if d["lut_entries"]:
        key = "build_prp_packed" if packed else "build_prp"
        pm = float(np.median(ev_ms[key]))
        out.update(prp_layout=layout, list_pages=st.pool_pages,
                   prp_entries_per_s=round(ab["prp_entries"] / (med * 1e-3), 1),
                   prp_call={"algorithmic_bytes": ab[key],
                             "gbs": round(ab[key] / (pm * 1e-3) / 1e9, 1),
                             "frac": round(ab[key] / (pm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
    if d["regions"]:
        lm = float(np.median(ev_ms["mr_lookup"]))
        out["lookup_call"] = {"regions": d["regions"], "algorithmic_bytes": ab["lookup"],
                              "gbs": round(ab["lookup"] / (lm * 1e-3) / 1e9, 1),
                              "frac": round(ab["lookup"] / (lm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if d["lut_entries"] and d["nqueues"]:
        # The same step as one dmadesc_build_batch call (four kernels
        # instead of six: the difference that matters for small batches).
        bms = timed_iters(torch, np, st.batch, reps)
        bmed = float(np.median(bms))
        out["batch_call"] = {**dist(np, bms), "requests_per_s": round(d["n"] / (bmed * 1e-3), 1),
                             "algorithmic_gbs": round(nbytes / (bmed * 1e-3) / 1e9, 1),
                             "frac_of_peak": round(nbytes / (bmed * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    g, gms = graph_step(torch, np, st, reps)
    gmed = float(np.median(gms))
    out["graph_step"] = {**dist(np, gms), "requests_per_s": round(d["n"] / (gmed * 1e-3), 1),
                         "algorithmic_gbs": round(nbytes / (gmed * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(nbytes / (gmed * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del g
    out.update(st.check_outputs(np))
    return out


def emit_stage(dd, d, np, torch, prp_out, sp_out, ln, reps):
    """Times dmadesc_emit_sqe on the step's PRP and split outputs: every queue
    gets a ring of 65536 entries with all but one slot free, tails from a
    seeded draw, cursors at 0, so each launch consumes the first window of
    every bucket. Algorithmic bytes: per consumed entry 4 (perm) + 1 (status)
    + 8 (len); per placed entry 24 (slba, prp1, prp2) + 64 (the entry) + 4
    (request map); per queue 48."""
    import synth
    dev = torch.device("cuda:0")
    n, nq = d["n"], d["nqueues"]
    depth = 65536
    rings = torch.empty((nq, depth * 64), dtype=torch.uint8, device=dev)
    ring = torch.tensor([rings[q].data_ptr() for q in range(nq)],
                        dtype=torch.int64).view(torch.uint64).to(dev)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    depth_t = up(np.full(nq, depth, np.uint32))
    free_t = up(np.full(nq, depth - 1, np.uint32))
    tail0 = up(np.random.default_rng(1).integers(0, depth, nq).astype(np.uint32))
    cursor0 = torch.zeros(nq, dtype=torch.uint64, device=dev)
    tail, cursor = tail0.clone(), cursor0.clone()
    placed = torch.empty(nq, dtype=torch.uint32, device=dev)
    rid = torch.empty(nq * depth, dtype=torch.uint32, device=dev)
    slba = up(synth.slba(d["name"], n))
    ws = torch.empty(dd.workspace_bytes(dd.OP_EMIT_SQE, n, nq), dtype=torch.uint8, device=dev)

    def call():
        tail.copy_(tail0)
        cursor.copy_(cursor0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dd.emit_sqe(sp_out["perm"], sp_out["qoff"], prp_out["status"], ln, slba,
                    prp_out["prp1"], prp_out["prp2"], ring, depth_t, free_t, tail, cursor,
                    placed=placed, req_of_slot=rid, ws=ws)
        e1.record()
        return e0, e1

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = [call() for _ in range(reps)]
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    consumed = int(cursor.cpu().numpy().astype(np.int64).sum())
    n_placed = int(placed.cpu().numpy().astype(np.int64).sum())
    nbytes = consumed * 13 + n_placed * (24 + 64 + 4) + nq * 48
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernels": "k_sqe_order + k_sqe_count + k_sqe_emit + k_sqe_finish", "ring_depth": depth,
            "consumed": consumed, "placed": n_placed, "mean_launch_ms": round(ms, 4),
            "algorithmic_bytes_per_launch": nbytes, "achieved_gbs": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "entries_per_s": round(n_placed / (ms * 1e-3), 1)}


def split_stage(dd, np, torch, n, reps):
    """Times dmadesc_partition_by_queue alone on n requests with Zipf(1.1)
    queue ids over 64 queues (LDS-counter ranking, as in the step) and over
    256 queues (ballot ranking); algorithmic bytes: qid read, perm written,
    the offsets."""
    import synth
    out = {}
    for nq in (64, 256):
        qid = torch.from_numpy(synth.queue_ids(n, nq, seed=nq)).to("cuda")
        ws = torch.empty(dd.workspace_bytes(dd.OP_PARTITION, n, nq), dtype=torch.uint8,
                         device="cuda")
        res = {"o": None}

        def call():
            res["o"] = dd.partition_by_queue(qid, nq, out=res["o"], ws=ws, check=False)
        ms = timed_iters(torch, np, call, reps)
        d = dist(np, ms)
        nbytes = 8 * n + 8 * (nq + 2)
        out[f"nq{nq}"] = {"ranking": "lds_counters" if nq <= 70 else "ballots",
                          "requests": n, **d,
                          "requests_per_s": round(n / (d["median_ms"] * 1e-3), 1),
                          "algorithmic_bytes": nbytes,
                          "achieved_gbs": round(nbytes / (d["median_ms"] * 1e-3) / 1e9, 1),
                          "frac": round(nbytes / (d["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del qid, ws
    return out


def put_stage(dd, np, torch, n, reps):
    """Times dmadesc_build_put on n seeded puts against a 256 GiB VMM heap of
    2 MiB chunks on 8 PEs (lengths as the Mixed requests). Algorithmic bytes:
    per put 28 read (src, dst, bytes, pe) + 13 written (first, count, status);
    per descriptor 32 written + 8 of keys read."""
    import synth
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    b = synth.put_batch(n)
    args = [up(b["src"]), up(b["dst"]), up(b["len"]), up(b["pe"]), b["local_base"], b["heap"],
            b["chunk_shift"], up(b["lkeys"]), up(b["peer_base"]), up(b["rkeys"])]
    probe = dd.build_put(*args, torch.empty((0, 4), dtype=torch.uint64, device=dev))
    torch.cuda.synchronize()
    total = int(probe["total"].cpu()[0])
    desc = torch.empty((total, 4), dtype=torch.uint64, device=dev)
    ws = torch.empty(max(dd.workspace_bytes(dd.OP_BUILD_PUT, n), 1), dtype=torch.uint8, device=dev)
    out, ms = None, []
    for r in range(reps + 3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = dd.build_put(*args, desc, out=out, ws=ws, check=False)
        e1.record()
        if r >= 3:
            ms.append((e0, e1))
    torch.cuda.synchronize()
    mean = float(np.mean([a.elapsed_time(c) for a, c in ms]))
    nbytes = n * (28 + 13) + total * (32 + 8)
    gbs = nbytes / (mean * 1e-3) / 1e9
    return {"kernels": "k_ws_clear + k_put_build", "puts": n, "descriptors": total,
            "heap": "256 GiB, 2 MiB chunks, 8 PEs", "mean_launch_ms": round(mean, 4),
            "puts_per_s": round(n / (mean * 1e-3), 1),
            "descriptors_per_s": round(total / (mean * 1e-3), 1),
            "algorithmic_bytes_per_launch": nbytes, "achieved_gbs": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def cq_stage(dd, np, torch, reps):
    """Times dmadesc_cq_mirror draining 64 device-memory completion queues of
    65,536 entries, each holding one full pass of completions when the call
    starts (stop flag already set, so every wave leaves after its queue is
    empty), into mirror queues in device memory and then in pinned host
    memory (the host completion queues of the method). Slots are reset from a
    copy before each timed call. Algorithmic bytes: per entry 16 read + 16
    written."""
    dev = torch.device("cuda:0")
    nq, depth = dd.CQ_MAX_SLOTS, 65536
    rng = np.random.default_rng(9)
    e = rng.integers(0, 1 << 32, (nq, depth, 4), dtype=np.uint64).astype(np.uint32)
    e[..., 3] |= np.uint32(1 << 16)                    # first pass: phase tag 1
    src = torch.from_numpy(e.view(np.int32)).to(dev)
    stop = torch.ones(1, dtype=torch.int32, device=dev).view(torch.uint32)
    n = nq * depth
    out = {"kernel": "k_cq_mirror", "queues": nq, "depth": depth, "entries_per_launch": n,
           "algorithmic_bytes_per_launch": n * 32}
    for where in ("device", "host"):
        dst = (torch.zeros_like(src) if where == "device"
               else torch.zeros(src.shape, dtype=torch.int32).pin_memory())
        slots = dd.cq_slots(nq, dev)
        for q in range(nq):
            dd.cq_attach(slots, q, src[q], dst[q], depth, 1)
        saved = slots.clone()
        ms = []
        for r in range(reps + 2):
            slots.copy_(saved)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dd.cq_mirror(slots, stop, idle_polls=1)
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ms.append(e0.elapsed_time(e1))
        st = dd.cq_slot_state(slots)
        ok = bool((st["copied"] == depth).all() and torch.equal(src.cpu(), dst.cpu()))
        mean = float(np.mean(ms))
        gbs = n * 32 / (mean * 1e-3) / 1e9
        out[f"{where}_mirror"] = {
            "mirrored_exactly": ok, "mean_launch_ms": round(mean, 4),
            "entries_per_s": round(n / (mean * 1e-3), 1),
            "us_per_poll": round(mean * 1e3 / (depth / 256), 3),
            "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del dst
    return out


def registry_stage(dd, d, np, torch, reps):
    """Times one register batch (65,536 calls) and one deregister batch on a
    device registration table that starts as the workload's 4,096 regions:
    half the calls fall inside a region (hit), a quarter are new ranges and a
    quarter repeat those (hit on a record of the same batch); the deregister
    batch names handles of the table, some beyond their references (stale).
    The table is restored from a copy before each timed call."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    reg = dd.DeviceRegistry(0)
    rs, re_ = d["rstart"], d["rend"]
    reg.register(up(rs), up(re_ - rs))
    n = dd.REG_MAX_BATCH
    pick = rng.integers(0, len(rs), n)
    span = (re_ - rs)[pick]
    off = rng.integers(0, 1 << 62, n).astype(np.uint64) % np.maximum(span // np.uint64(2), 1)
    addr = rs[pick] + off
    size = np.maximum((span - off) // np.uint64(4), np.uint64(1))
    fresh = np.arange(n // 4, dtype=np.uint64)
    addr[n // 2: 3 * n // 4] = np.uint64(1 << 46) + fresh * np.uint64(1 << 21)
    size[n // 2: 3 * n // 4] = np.uint64(1 << 20)
    addr[3 * n // 4:] = addr[n // 2: 3 * n // 4] + np.uint64(4096)
    size[3 * n // 4:] = np.uint64(4096)
    g_addr, g_size = up(addr), up(size)
    reg.grow(32768)                                     # room for the batch's inserts
    saved = {k: getattr(reg, k).clone() for k in ("start", "end", "id", "refs", "by_start",
                                                  "state")}

    def restore():
        for k, t in saved.items():
            getattr(reg, k).copy_(t)

    def timed(fn):
        out, ms = None, []
        for r in range(reps + 2):
            restore()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = fn()
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ms.append(e0.elapsed_time(e1))
        return out, float(np.mean(ms))

    out, reg_ms = timed(lambda: reg.register(g_addr, g_size, grow=False))
    kinds = np.bincount(out["kind"].cpu().numpy(), minlength=5)
    handles = saved["id"][:len(rs)].cpu().numpy()
    dh = up(rng.choice(handles, n))
    st, dereg_ms = timed(lambda: reg.deregister(dh))
    sts = np.bincount(st.cpu().numpy(), minlength=3)
    return {"table_records": int(len(rs)), "batch": n,
            "register_batch_ms": round(reg_ms, 4), "deregister_batch_ms": round(dereg_ms, 4),
            "registrations_per_s": round(n / (reg_ms * 1e-3), 1),
            "deregistrations_per_s": round(n / (dereg_ms * 1e-3), 1),
            "register_kinds": {"hit": int(kinds[1]), "new": int(kinds[2]),
                               "hit_new": int(kinds[3]), "invalid": int(kinds[0])},
            "deregister_status": {"ok": int(sts[0]), "removed": int(sts[1]),
                                  "stale": int(sts[2])},
            "note": "register timing includes the binding's read of the needed capacity"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, sample, layout):
    """The single-threaded oracle (lookup, PRP build of the step's layout
    with lists into a pre-faulted host pool, split) on the first `sample`
    requests of the workload, pinned to one core: each function timed 3
    times (1 if a run passes 20 s), medians reported; end to end = the sum
    of the medians."""
    import numpy as np

    import oracle
    import synth
    d = synth.generate(name, n=sample)
    n, bus = d["n"], d["list_bus_base"]
    build = oracle.build_prp_packed if layout == "packed" else oracle.build_prp
    fns = {}
    if d["regions"]:
        fns["mr_lookup"] = lambda: oracle.mr_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"],
                                                    d["len"], va_base=d["va_base"])
    pool = None
    if d["lut_entries"]:
        total = build(d["lut"], d["off"], d["len"], bus, 0)["total"]
        pool = np.ones((max(total, 1), 512), dtype=np.uint64)      # pre-faulted, reused
        fns["build_prp"] = lambda: build(d["lut"], d["off"], d["len"], bus, total, pool=pool)
    if d["nqueues"]:
        fns["partition_by_queue"] = lambda: oracle.partition(d["qid"], d["nqueues"])
    old = os.sched_getaffinity(0)
    cpu = min(old)
    os.sched_setaffinity(0, {cpu})
    times = {k: [] for k in fns}
    try:
        for r in range(3):
            for k, fn in fns.items():
                t0 = time.perf_counter()
                fn()
                times[k].append(time.perf_counter() - t0)
            if max(v[-1] for v in times.values()) > 20.0:
                break
    finally:
        os.sched_setaffinity(0, old)
    med = {k: float(np.median(v)) for k, v in times.items()}
    e2e = sum(med.values())
    ab = algorithmic_bytes(d, np)
    per = {k: {"median_s": round(v, 4), "requests_per_s": round(n / v, 1), "runs": len(times[k])}
           for k, v in med.items()}
    if "build_prp" in per:
        per["build_prp"]["prp_entries_per_s"] = round(ab["prp_entries"] / med["build_prp"], 1)
    return {"value": round(n / e2e / 1e6, 4), "unit": "M req/s", "cores": 1, "kind": "oracle",
            "sample": (f"first {n:,} requests of the {name} workload: "
                       + " + ".join(fns) + f" ({layout} lists into a pre-faulted host pool), "
                       "single thread pinned to one core, median of 3 runs per function, "
                       f"{sum(sum(v) for v in times.values()):.1f} s in all"),
            "per_function": per,
            "prp_entries_per_s": round(ab["prp_entries"] / e2e, 1) if pool is not None else None,
            "host_cores": os.cpu_count(), "cpu_model": cpu_model()}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def list_write_floor(name, steps):
    """Writes exactly the 128-byte lines the PRP build writes for `name` (each
    list run padded to whole lines at the head of its list pages) with
    torch's index_fill_, a plain library scatter, and reports its rate. This
    bounds what any kernel can reach for the list writes of that layout."""
    import numpy as np
    import torch

    import synth
    d = synth.generate(name)
    off, ln = d["off"], d["len"]
    heap = np.uint64(d["lut_entries"]) * np.uint64(65536)
    valid = (ln > 0) & (off % 4 == 0) & (off + ln <= heap)
    pages = np.where(valid, ((off & np.uint64(4095)) + ln + np.uint64(4095)) >> np.uint64(12), 0)
    lists = pages >= 3
    lp = np.where(lists, (pages - 2 + 510) // 511, 0).astype(np.int64)
    ent = np.where(lists, pages - 1 + lp - 1, 0).astype(np.int64)
    slot = np.cumsum(lp) - lp
    nl = (ent + 15) // 16
    first = np.repeat(slot * 32, nl)
    within = np.arange(int(nl.sum())) - np.repeat(np.cumsum(nl) - nl, nl)
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(first + within).to(dev)
    pool = torch.empty((int(lp.sum()) * 32, 16), dtype=torch.int64, device=dev)
    pool.index_fill_(0, idx, 7)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        pool.index_fill_(0, idx, 7)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = int(nl.sum()) * 128
    print(json.dumps({"list_write_floor": {"workload": name, "lines": int(nl.sum()),
                                           "bytes": nbytes, "ms": round(ms, 4),
                                           "gbs": round(nbytes / ms / 1e6, 1),
                                           "method": "torch index_fill_ of the 128-byte list lines"}}),
          flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on one GPU only (requests are independent, so "
              "a batch would shard by index range with no exchange); use --gpus 1",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.list_write_floor:
        list_write_floor(args.workload, min(args.steps, 20))
        return

    import memory_dma_descriptor_amd as dd
    import synth

    if args.stage_emit_sqe:
        d = synth.generate(args.workload)
        if not (d["lut_entries"] and d["nqueues"]):
            raise SystemExit("bench.py: the submission-entry stage needs a workload with a "
                             "heap and queues")
        st = Step(dd, torch, np, d, args.layout == "packed")
        st.run()
        torch.cuda.synchronize()
        r = emit_stage(dd, d, np, torch, st.pr, st.sp, st.ln, max(args.emit_reps, 1))
        print(json.dumps({"emit_sqe": r, "workload": args.workload}), flush=True)
        return
    if args.stage_registry:
        d = synth.generate(args.workload)
        if not d["regions"]:
            raise SystemExit("bench.py: the registry stage needs a workload with regions")
        r = registry_stage(dd, d, np, torch, 10)
        print(json.dumps({"registry": r, "workload": args.workload}), flush=True)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.generate(args.workload)
    n, nq = d["n"], d["nqueues"]
    packed = args.layout == "packed"
    layout = args.layout
    ab = algorithmic_bytes(d, np)
    st = Step(dd, torch, np, d, packed)
    calls = st.calls()
    prp_key = "build_prp_packed" if packed else "build_prp"
    dominant = prp_key if d["lut_entries"] else "mr_lookup"
    dom_bytes = ab[prp_key] if d["lut_entries"] else ab["lookup"]

    # The other layout's PRP build, timed alone on the same inputs. It runs
    # before the warm-up steps, so the timed steps find the GPU at its
    # steady clocks (the first few dozen steps otherwise run about 1 % slow).
    other = None
    if d["lut_entries"] and not args.quick:
        o_pool, o_pages = st.pool_for(not packed)
        o_key = "build_prp" if packed else "build_prp_packed"
        o_out = [None]

        def o_call():
            o_out[0] = dd.build_prp(st.lut, st.off, st.ln, st.bus, o_pool, out=o_out[0],
                                    ws=st.ws_prp, packed=not packed, check=False)
        o_ms = timed_iters(torch, np, o_call, max(args.steps // 2, 20))
        o_med = float(np.median(o_ms))
        o_gbs = ab[o_key] / (o_med * 1e-3) / 1e9
        other = {"list_pages": o_pages, "algorithmic_bytes_per_launch": ab[o_key],
                 **dist(np, o_ms), "achieved_gbs": round(o_gbs, 1),
                 "frac": round(o_gbs / PEAK_HBM_GBS, 4),
                 "traffic": recorded_traffic("packed" if not packed else "page", args.workload),
                 "refused_requests": int((o_out[0]["status"].cpu().numpy() != 0).sum())}
        del o_pool, o_out

    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    # Timed steps; per-call events on >= 10 of them, spread evenly.
    k_sampled = min(args.steps, max(10, args.sampled_steps))
    sampled = set(np.linspace(0, args.steps - 1, k_sampled).round().astype(int).tolist())
    events = []
    t0 = time.perf_counter()
    for s_i in range(args.steps):
        ev = None
        if s_i in sampled:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
            events.append(ev)
        st.run(ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    per_call = {c: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in events]))
                for k, c in enumerate(calls)}
    checks = st.check_outputs(np)

    # Step-time distribution: steps timed one by one.
    step_ms = timed_iters(torch, np, st.run, 3 if args.quick else max(args.dist_steps, 20),
                          warm=0)
    step_bytes, step_sum = ab[f"step_{layout}"], ab[f"step_sum_{layout}"]
    step_med = float(np.median(step_ms))

    # The same calls captured in a HIP graph and replayed.
    graph = None
    if not args.quick:
        g, gms = graph_step(torch, np, st, max(args.dist_steps, 20))
        g_med = float(np.median(gms))
        graph = {**dist(np, gms), "requests_per_s": round(n / (g_med * 1e-3), 1),
                 "algorithmic_gbs": round(step_bytes / (g_med * 1e-3) / 1e9, 1),
                 "frac_of_peak": round(step_bytes / (g_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del g

    # The same step as one dmadesc_build_batch call, checked against the
    # separate calls' outputs (which are those of the last step).
    batch = None
    if d["lut_entries"] and nq and not args.quick:
        ref = {}
        for o in (st.lk, st.pr, st.sp):
            if o:
                ref.update({k: v.clone() for k, v in o.items()})
        b_ms = timed_iters(torch, np, st.batch, 20)
        same = all(torch.equal(st.bt[k], v) for k, v in ref.items())
        b_med = float(np.median(b_ms))
        batch = {"call": "dmadesc_build_batch", **dist(np, b_ms),
                 "requests_per_s": round(n / (b_med * 1e-3), 1),
                 "algorithmic_gbs": round(step_bytes / (b_med * 1e-3) / 1e9, 1),
                 "frac": round(step_bytes / (b_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "same_outputs_as_the_calls": bool(same)}
        del ref

    dom_ms = per_call[dominant]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = recorded_traffic(layout, args.workload) if d["lut_entries"] else None
    kernel = {"build_prp_packed": "dmadesc_build_prp_packed (k_ws_clear + k_prp_build)",
              "build_prp": "dmadesc_build_prp (k_ws_clear + k_prp_build)",
              "mr_lookup": "dmadesc_mr_lookup"}[dominant]
    result = {
        "metric": "descriptor requests/sec (M/s) + achieved HBM GB/s vs MI355X peak",
        "value": round(n * args.steps / elapsed / 1e6, 3),
        "unit": "M req/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": args.workload, "requests": n, "lut_entries": d["lut_entries"],
                   "regions": d["regions"], "nqueues": nq, "prp_layout": layout,
                   "list_pages": st.pool_pages,
                   "calls": " + ".join(calls) + ", one stream"},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "mean_launch_ms": round(dom_ms, 4), "sampled_launches": len(events)},
        "step": {**dist(np, step_ms),
                 "algorithmic_bytes": step_bytes,
                 "algorithmic_bytes_per_call_sum": step_sum,
                 "algorithmic_gbs": round(step_bytes / (step_med * 1e-3) / 1e9, 1),
                 "frac_of_peak": round(step_bytes / (step_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "timed_region_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                 "timed_region_frac": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "per_call_sampled_steps": len(events),
        "prp_entries_per_s": round(ab["prp_entries"] * args.steps / elapsed, 1),
        "checks": checks,
    }
    if graph:
        result["graph_step"] = graph
    if batch:
        result["batch_call"] = batch
    if other:
        result[f"{'page' if packed else 'packed'}_layout_build_prp"] = other
    if args.quick:
        args.no_configs, args.emit_reps, args.no_cpu_baseline = True, 0, True
    if not args.no_configs:
        result["per_config"] = {}
        for name, reps in (("tiny", 200), ("small", 200), ("large", 20), ("mrheavy", 20),
                           ("mixed", 20)):
            if name == args.workload:
                continue
            result["per_config"][name] = run_config(dd, torch, np, name, reps, packed)
            torch.cuda.empty_cache()
    if nq and d["lut_entries"] and args.emit_reps > 0:
        result["emit_sqe"] = emit_stage(dd, d, np, torch, st.pr, st.sp, st.ln, args.emit_reps)
    if d["regions"] and args.emit_reps > 0:
        result["registry"] = registry_stage(dd, d, np, torch, 10)
    if nq and args.emit_reps > 0:
        result["split_alone"] = split_stage(dd, np, torch, n, max(args.emit_reps, 20))
    if args.emit_reps > 0:
        result["build_put"] = put_stage(dd, np, torch, n, args.emit_reps)
    if args.emit_reps > 0:
        result["cq_mirror"] = cq_stage(dd, np, torch, 10)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, min(args.cpu_sample, n), layout)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
