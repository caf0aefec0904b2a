#!/usr/bin/env python3
"""Benchmark: batched DMA-descriptor building on one MI355X.

One step = the whole hot path over one batch: page-rounded MR lookup, PRP
build (PRP1/PRP2 + chained lists; packed lists by default, --layout page for
one run of list pages per request) and stable split by queue, three calls on
one stream, over the 16,777,216-request Mixed workload (256 GiB heap of
4,194,304 GPU pages, 4,096 regions, log-uniform 512 B - 1 MiB requests,
Zipf(1.1) over 64 queues). Inputs are resident in HBM before timing starts.

Prints ONE JSON line. `value` is requests per second (millions) over the
timed steps; `roofline` describes the dominant call (the PRP build of the
step's layout; the other layout's build is timed alone beside it):
algorithmic bytes of one launch / its mean duration from HIP events recorded
on the stream it runs on, on every 10th timed step (`per_call_ms` likewise;
each event record is a queue marker that would add a few microseconds to
every step). `emit_sqe` times the stage after the path (NVMe
submission entries for the first window of every queue) on the step's outputs,
`registry` a batch of registrations and deregistrations on the device
registration table, `build_put` RDMA put descriptors for a VMM heap and
`cq_mirror` the completion-queue mirror draining 64 full queues, all outside
the timed steps. `cpu_baseline` times the single-threaded oracle on a
bounded sample of the same workload.
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed",
                    choices=["tiny", "small", "large", "mixed"])
    ap.add_argument("--layout", default="packed", choices=["packed", "page"],
                    help="PRP list layout of the timed step: lists back to back "
                         "(dmadesc_build_prp_packed) or one run of list pages per request "
                         "(dmadesc_build_prp); the other layout's PRP build is timed too")
    ap.add_argument("--cpu-sample", type=int, default=1 << 21,
                    help="requests of the workload the oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record per-call HIP events on every k-th timed step (each event "
                         "record is a queue marker that costs a few microseconds)")
    ap.add_argument("--emit-reps", type=int, default=20,
                    help="launches of the submission-entry stage timed after the steps "
                         "(0 = skip it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for counter scaling) and exit")
    ap.add_argument("--list-write-floor", action="store_true",
                    help="time a library scatter that writes the same 128-byte list lines "
                         "as the PRP build (its layout's write floor) and exit")
    return ap.parse_args()


def prp_source_hash() -> str:
    h = hashlib.sha256()
    for f in PRP_SOURCES:
        with open(os.path.join(ROOT, "memory_dma_descriptor_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(d, np):
    """Bytes each call must move, each column once (per-request figures:
    lookup 16 read + 25 written; PRP 16 read + 8 per GPU page touched, 17
    written + 8 per list word; split 4 read + 4 written). List words: page
    layout m + L - 1 per request (entries and chain pointers); packed layout
    the whole dense range, E + floor(E / 511) words for E entries in all."""
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
    base = n * (16 + 17) + 8 * float(frames.sum())
    split = n * 8
    return dict(lookup=float(lookup), build_prp=base + 8 * entries,
                build_prp_packed=base + 8 * packed_words, partition=float(split),
                list_entries=entries, prp_entries=float(pages.astype(np.float64).sum()))


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
    return {"kernels": "k_sqe_count + k_sqe_emit + k_sqe_finish", "ring_depth": depth,
            "consumed": consumed, "placed": n_placed, "mean_launch_ms": round(ms, 4),
            "algorithmic_bytes_per_launch": nbytes, "achieved_gbs": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "entries_per_s": round(n_placed / (ms * 1e-3), 1)}


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


def cpu_baseline(name, sample, min_seconds, layout):
    import numpy as np

    import oracle
    import synth
    d = synth.generate(name, n=sample)
    bus = d["list_bus_base"]
    build = oracle.build_prp_packed if layout == "packed" else oracle.build_prp
    total = build(d["lut"], d["off"], d["len"], bus, 0)["total"]
    pool = np.ones((max(total, 1), 512), dtype=np.uint64)      # pre-faulted, reused
    old = os.sched_getaffinity(0)
    cpu = min(old)
    os.sched_setaffinity(0, {cpu})
    try:
        reps, spent = 0, 0.0
        while spent < min_seconds:
            t0 = time.perf_counter()
            if d["regions"]:
                oracle.mr_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"], d["len"],
                                 va_base=d["va_base"])
            build(d["lut"], d["off"], d["len"], bus, total, pool=pool)
            oracle.partition(d["qid"], d["nqueues"])
            spent += time.perf_counter() - t0
            reps += 1
    finally:
        os.sched_setaffinity(0, old)
    return {"value": round(sample * reps / spent / 1e6, 4), "unit": "M req/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"first {sample:,} requests of the {name} workload, lookup + PRP build "
                       f"({layout} lists into a pre-faulted host pool) + split, single thread pinned "
                       f"to one core, {reps} repetitions, {spent:.1f} s"),
            "host_cores": os.cpu_count()}


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.generate(args.workload)
    n, nq = d["n"], d["nqueues"]
    bus = d["list_bus_base"]
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    rs, re_, rk = up(d["rstart"]), up(d["rend"]), up(d["rlkey"])
    off, ln, qid, lut = up(d["off"]), up(d["len"]), up(d["qid"]), up(d["lut"])

    # Capacity query: with an empty pool the call still reports the pages
    # the batch needs.
    packed = args.layout == "packed"
    empty = torch.empty((0, 512), dtype=torch.uint64, device=dev)

    def pool_for(pk):
        probe = dd.build_prp(lut, off, ln, bus, empty, packed=pk)
        torch.cuda.synchronize()
        pages = int(probe["total_pages"].cpu()[0])
        return torch.empty((max(pages, 1), 512), dtype=torch.uint64, device=dev), pages

    pool, pool_pages = pool_for(packed)

    lk_out = prp_out = sp_out = None
    ws_prp = torch.empty(max(dd.workspace_bytes(dd.OP_BUILD_PRP, n), 1), dtype=torch.uint8, device=dev)
    ws_sp = torch.empty(max(dd.workspace_bytes(dd.OP_PARTITION, n, max(nq, 1)), 1),
                        dtype=torch.uint8, device=dev)

    def step(timed_calls):
        # The three calls are issued back to back on the current stream; on
        # sampled steps HIP events bracket each call on that stream.
        nonlocal lk_out, prp_out, sp_out
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed_calls else None
        if ev: ev[0].record()
        if d["regions"]:
            lk_out = dd.mr_lookup(rs, re_, rk, off, ln, va_base=d["va_base"], out=lk_out)
        if ev: ev[1].record()
        prp_out = dd.build_prp(lut, off, ln, bus, pool, out=prp_out, ws=ws_prp, packed=packed,
                               check=False)
        if ev: ev[2].record()
        if nq:
            sp_out = dd.partition_by_queue(qid, nq, out=sp_out, ws=ws_sp, check=False)
        if ev: ev[3].record()
        return ev

    ab = algorithmic_bytes(d, np)
    # The other layout's PRP build, timed alone on the same inputs. It runs
    # before the warm-up steps, so the timed steps find the GPU at its
    # steady clocks (the first few dozen steps otherwise run about 1 % slow).
    other = "page" if packed else "packed"
    o_pool, o_pages = pool_for(not packed)
    o_out = None
    o_ev = []
    for r in range(max(args.steps // 2, 3) + 3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        o_out = dd.build_prp(lut, off, ln, bus, o_pool, out=o_out, ws=ws_prp, packed=not packed,
                             check=False)
        e1.record()
        if r >= 3:
            o_ev.append((e0, e1))
    torch.cuda.synchronize()
    o_ms = float(np.mean([a.elapsed_time(b) for a, b in o_ev]))
    o_key = "build_prp" if packed else "build_prp_packed"
    o_gbs = ab[o_key] / (o_ms * 1e-3) / 1e9
    o_refused = int((o_out["status"].cpu().numpy() != 0).sum())
    del o_pool, o_out

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    events = []
    every = max(args.event_every, 1)
    t0 = time.perf_counter()
    for s_i in range(args.steps):
        ev = step(s_i % every == every - 1 or (s_i == args.steps - 1 and not events))
        if ev:
            events.append(ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    calls = ["mr_lookup", "build_prp", "partition_by_queue"]
    per_call = {c: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in events]))
                for k, c in enumerate(calls)}
    status = prp_out["status"].cpu().numpy()
    prp_key = "build_prp_packed" if packed else "build_prp"
    step_bytes = ab["lookup"] * bool(d["regions"]) + ab[prp_key] + ab["partition"] * bool(nq)
    ms = elapsed / args.steps * 1e3
    prp_ms = per_call["build_prp"]
    achieved = ab[prp_key] / (prp_ms * 1e-3) / 1e9

    traffic = None
    tf = traffic_file(args.layout, args.workload)
    if os.path.exists(tf):
        with open(tf) as f:
            rec = json.load(f)
        if rec.get("source_sha256") == prp_source_hash():
            traffic = rec.get("traffic_bytes_per_launch")


    kernel = ("dmadesc_build_prp_packed" if packed else "dmadesc_build_prp") + \
        " (k_ws_clear + k_prp_build)"
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
                   "regions": d["regions"], "nqueues": nq, "prp_layout": args.layout,
                   "list_pages": pool_pages,
                   "calls": f"mr_lookup + {kernel.split()[0][8:]} + partition_by_queue, one stream"},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": ab[prp_key],
                     "mean_launch_ms": round(prp_ms, 4)},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "per_call_sampled_steps": len(events),
        "step_algorithmic_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "prp_entries_per_s": round(ab["prp_entries"] * args.steps / elapsed, 1),
        "refused_requests": int((status != 0).sum()),
        f"{other}_layout_build_prp": {
            "mean_launch_ms": round(o_ms, 4), "list_pages": o_pages,
            "algorithmic_bytes_per_launch": ab[o_key], "achieved_gbs": round(o_gbs, 1),
            "frac": round(o_gbs / PEAK_HBM_GBS, 4),
            "refused_requests": o_refused},
    }
    if nq and args.emit_reps > 0:
        result["emit_sqe"] = emit_stage(dd, d, np, torch, prp_out, sp_out, ln, args.emit_reps)
    if d["regions"] and args.emit_reps > 0:
        result["registry"] = registry_stage(dd, d, np, torch, 10)
    if args.emit_reps > 0:
        result["build_put"] = put_stage(dd, np, torch, n, args.emit_reps)
    if args.emit_reps > 0:
        result["cq_mirror"] = cq_stage(dd, np, torch, 10)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, min(args.cpu_sample, n),
                                              args.cpu_seconds, args.layout)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
