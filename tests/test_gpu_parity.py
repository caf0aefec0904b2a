"""GPU parity: the HIP library through its C ABI against the CPU oracle, bit
for bit, on the five workloads (scaled copies that span many blocks with a
ragged tail, and the full sizes) and on edge suites."""
import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import oracle
import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

BUS = synth.LIST_BUS_BASE


def _perm_lut(rng, p, base=synth.PHYS_BASE):
    return np.uint64(base) + rng.permutation(p).astype(np.uint64) * np.uint64(65536)


# ------------------------------------------------------------ workloads ---

SCALED = {"tiny": 4096, "small": 100_003, "large": 3_001, "mrheavy": 200_003,
          "mixed": 60_001}


@pytest.mark.parametrize("name", list(SCALED))
def test_workload_scaled(name):
    d = synth.generate(name, n=SCALED[name])
    gc.say(f"workload {name} n={d['n']}")
    if d["regions"]:
        gc.check_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"], d["len"],
                        va_base=d["va_base"], page_shift=d["page_shift"], ctx=name)
    if d["lut_entries"]:
        o = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, 0, pool=None)
        gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, o["total"] + 3, ctx=name)
    if d["nqueues"]:
        gc.check_split(d["qid"], d["nqueues"], ctx=name)


@pytest.mark.parametrize("name", ["small", "large", "mrheavy", "mixed"])
def test_workload_full_size(name):
    d = synth.generate(name)
    gc.say(f"workload {name} full n={d['n']}")
    if d["regions"]:
        gc.check_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"], d["len"],
                        va_base=d["va_base"], page_shift=d["page_shift"], ctx=name)
    if d["lut_entries"]:
        total = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, 0, pool=None)["total"]
        if name == "large":
            gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, total + 5, ctx=name)
        else:
            # Every list page of the full batch (46 GB of lists for Mixed),
            # compared chunk by chunk.
            _, _, pages = gc.check_prp_chunked(d["lut"], d["off"], d["len"], BUS, total + 5,
                                               ctx=name)
            assert pages == total
    if d["nqueues"]:
        gc.check_split(d["qid"], d["nqueues"], ctx=name)


def test_mixed_three_calls_one_stream():
    """Lookup, PRP build and split back to back on one non-default stream."""
    d = synth.generate("mixed", n=150_001)
    o_l = oracle.mr_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"], d["len"],
                           va_base=d["va_base"])
    o_pool_pages = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, 0, pool=None)["total"]
    o_pool = np.full((o_pool_pages, 512), gc.CANARY, dtype=np.uint64)
    o_p = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, o_pool_pages, pool=o_pool)
    o_s = oracle.partition(d["qid"], 64)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rs, re_, rk = gc.dev(d["rstart"]), gc.dev(d["rend"]), gc.dev(d["rlkey"])
        off, ln, qid, lut = gc.dev(d["off"]), gc.dev(d["len"]), gc.dev(d["qid"]), gc.dev(d["lut"])
        pool = torch.empty((o_pool_pages, 512), dtype=torch.uint64, device="cuda")
        pool.view(torch.int64).fill_(gc.CANARY_I64)
        lk = dd.mr_lookup(rs, re_, rk, off, ln, va_base=d["va_base"])
        pr = dd.build_prp(lut, off, ln, BUS, pool)
        sp = dd.partition_by_queue(qid, 64)
    s.synchronize()
    gc.assert_lookup_equal(o_l, {k: gc.host(v) for k, v in lk.items()}, "mixed/stream")
    g = {k: gc.host(v) for k, v in pr.items()}
    g["total"] = int(g.pop("total_pages")[0])
    gc.assert_prp_columns_equal(o_p, g, "mixed/stream")
    gp = gc.host(pool)
    gc.mask_padding(o_pool, gp, gc.padding_spans(o_p["prp2"], o_p["status"], d["off"], d["len"], BUS))
    assert np.array_equal(gp, o_pool)
    assert np.array_equal(gc.host(sp["perm"]), o_s["perm"])
    assert np.array_equal(gc.host(sp["qoff"]), o_s["qoff"])


def test_deterministic_repeat():
    d = synth.generate("mixed", n=80_000)
    total = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, 0, pool=None)["total"]
    a, pa = gc.gpu_prp(d["lut"], d["off"], d["len"], BUS, total)
    b, pb = gc.gpu_prp(d["lut"], d["off"], d["len"], BUS, total)
    for k in ("prp1", "prp2", "status"):
        assert np.array_equal(a[k], b[k])
    assert torch.equal(pa.view(torch.int64), pb.view(torch.int64))
    s1, s2 = gc.gpu_split(d["qid"], 64), gc.gpu_split(d["qid"], 64)
    assert np.array_equal(s1["perm"], s2["perm"])


# ------------------------------------------------------------- PRP edges ---

def test_prp_tiny_heap_boundaries():
    rng = np.random.default_rng(7)
    lut = _perm_lut(rng, 4)
    offs = sorted(set(list(range(0, 256, 4)) + list(range(4096 - 64, 4096 + 64, 4))
                      + list(range(65536 - 128, 65536 + 64, 4))
                      + list(range(2 * 65536 - 8, 2 * 65536 + 8, 4))))
    lens = [1, 3, 4, 5, 100, 4092, 4095, 4096, 4097, 8191, 8192, 8193, 12288, 12289,
            65536, 65537, 70000]
    off = np.array([o for o in offs for _ in lens], np.uint64)
    ln = np.array([l for _ in offs for l in lens], np.uint64)
    total = oracle.build_prp(lut, off, ln, BUS, 0, pool=None)["total"]
    gc.check_prp_full(lut, off, ln, BUS, total, ctx="tiny-heap")


@pytest.mark.parametrize("m", [2, 3, 510, 511, 512, 513, 1021, 1022, 1023, 1024, 1533,
                               1534, 1535, 1536, 2048, 2049, 5000])
def test_prp_chain_sizes(m):
    rng = np.random.default_rng(m)
    lut = _perm_lut(rng, 512)
    # the same list size at several sub-page offsets, plus filler requests
    off = np.array([4096 * 7, 4096 * 7 + 4, 65536 * 3 - 4, 100, 0], np.uint64)
    ln = np.array([(m + 1) * 4096, (m + 1) * 4096 - 8, m * 4096 + 8, m * 4096, 4096], np.uint64)
    total = oracle.build_prp(lut, off, ln, BUS, 0, pool=None)["total"]
    gc.check_prp_full(lut, off, ln, BUS, total + 2, ctx=f"chain m={m}")


def test_prp_status_and_enospc():
    rng = np.random.default_rng(9)
    p = 64
    lut = _perm_lut(rng, p)
    heap = p * 65536
    top = (1 << 64) - 1
    off = np.array([0, 0, 2, 4, top - 3, heap - 4096, heap - 4092, 0, 8, 4096, 12, 16, 0],
                   np.uint64)
    ln = np.array([0, 4096, 4096, 16, 8, 4096, 4096, 5 * 4096, 3 * 4096, 600 * 4096, 4096,
                   9 * 4096, 3 * 4096], np.uint64)
    for cap in (1, 2, 3, 5, 6, 7):
        gc.check_prp_full(lut, off, ln, BUS, cap, ctx=f"status cap={cap}")
    # pool_pages == 0: every list request is refused, no pool needed
    o = oracle.build_prp(lut, off, ln, BUS, 0, pool=None)
    g, _ = gc.gpu_prp(lut, off, ln, BUS, 0)
    gc.assert_prp_columns_equal(o, g, "cap=0")


def test_prp_enospc_in_many_blocks():
    d = synth.generate("large", n=2500)
    total = oracle.build_prp(d["lut"], d["off"], d["len"], BUS, 0, pool=None)["total"]
    for cap in (total // 3, total - 1):
        gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, cap, ctx=f"enospc cap={cap}")


def test_prp_empty_and_single():
    rng = np.random.default_rng(1)
    lut = _perm_lut(rng, 16)
    g, _ = gc.gpu_prp(lut, np.empty(0, np.uint64), np.empty(0, np.uint64), BUS, 4)
    assert g["total"] == 0 and g["prp1"].size == 0
    gc.check_prp_full(lut, np.array([65536 - 4], np.uint64), np.array([3 * 4096], np.uint64),
                      BUS, 1, ctx="single")
    # no heap at all: every request is past the heap
    g, _ = gc.gpu_prp(np.empty(0, np.uint64), np.array([0, 8], np.uint64),
                      np.array([4096, 4], np.uint64), BUS, 4)
    assert list(g["status"]) == [2, 2] and g["total"] == 0


def test_prp_list_longer_than_2_24_words():
    """A request whose list needs more than 2^24 words (a 64 GiB transfer)
    among small ones: such a round takes the library's 64-bit list path."""
    rng = np.random.default_rng(24)
    p = (1 << 20) + 256                                  # 64 GiB + 16 MiB heap
    lut = _perm_lut(rng, p)
    n = 700
    ln = rng.integers(1, 300 * 4096, size=n).astype(np.uint64)
    off = (rng.integers(0, 1 << 28, size=n) * 4).astype(np.uint64)
    ln[5] = ((1 << 24) + 9) * 4096 - 12                  # 2^24 + 10 pages
    off[5] = 4 * 1000
    ln[600] = ((1 << 24) + 600) * 4096
    off[600] = 65536 * 7 + 8
    total = oracle.build_prp(lut, off, ln, BUS, 0, pool=None)["total"]
    gc.check_prp_full(lut, off, ln, BUS, total + 1, ctx="huge list")


def test_prp_unaligned_table_entries():
    """Table entries need not be 64 KiB aligned: results are still the
    table value plus the in-page offset, as in the oracle."""
    rng = np.random.default_rng(11)
    lut = _perm_lut(rng, 256) + rng.integers(0, 65536, size=256).astype(np.uint64)
    off = (rng.integers(0, (256 * 65536 - 600 * 4096) // 4, size=3000) * 4).astype(np.uint64)
    ln = rng.integers(1, 600 * 4096, size=3000).astype(np.uint64)
    total = oracle.build_prp(lut, off, ln, BUS, 0, pool=None)["total"]
    gc.check_prp_full(lut, off, ln, BUS, total, ctx="unaligned lut")


# ---------------------------------------------------------- lookup edges ---

def _table(rng, count, abut_p=0.3):
    start, end = [], []
    cur = 0x7000_0000_0000
    for _ in range(count):
        if rng.random() >= abut_p:
            cur += 4096 * int(rng.integers(1, 64))
        size = 4096 * int(rng.integers(1, 256))
        start.append(cur)
        end.append(cur + size)
        cur += size
    return np.array(start, np.uint64), np.array(end, np.uint64)


def _queries(rng, start, end, n):
    lo = int(start[0]) - 3 * 4096 if len(start) else 0x7000_0000_0000
    hi = int(end[-1]) + 3 * 4096 if len(end) else lo + (1 << 20)
    c = rng.integers(0, 5, size=n)
    off = rng.integers(lo, hi, size=n).astype(np.uint64)
    ln = rng.integers(1, 1 << 20, size=n).astype(np.uint64)
    if len(start):
        r = rng.integers(0, len(start), size=n)
        s, e = start[r].astype(np.int64), end[r].astype(np.int64)
        a = s + (rng.random(n) * (e - s)).astype(np.int64)
        edge = np.where(rng.random(n) < 0.5, s, e)
        d1 = rng.integers(1, 5000, size=n)
        d2 = rng.integers(1, 5000, size=n)
        off = np.where(c == 0, s, np.where(c == 1, a, np.where(c == 2, edge - d1, off.astype(np.int64))))
        inner = np.maximum(1, (rng.random(n) * (e - a)).astype(np.int64))
        ln = np.where(c == 0, e - s, np.where(c == 1, inner, np.where(c == 2, d1 + d2, ln.astype(np.int64))))
    return np.asarray(off).astype(np.uint64), np.asarray(ln).astype(np.uint64)


@pytest.mark.parametrize("count", [0, 1, 2, 63, 64, 65, 4096, 4097, 8192, 8193, 65536, 65537,
                                   100_000, 262_147])
@pytest.mark.parametrize("page_shift", [12, 16])
def test_lookup_tables(count, page_shift):
    # Above 4,096 regions both large-table paths: the record copy in a
    # workspace (every 4th start in LDS up to 65,536 regions, then every
    # 8th, 16th ... with a global narrowing step) and no workspace.
    rng = np.random.default_rng(count * 3 + page_shift)
    start, end = _table(rng, count)
    lkey = rng.integers(1, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)
    off, ln = _queries(rng, start, end, 30_011)
    for records in ((True, False) if count > 4096 else (True,)):
        gc.check_lookup(start, end, lkey, off, ln, page_shift=page_shift, records=records,
                        ctx=f"R={count} shift={page_shift} records={records}")


@pytest.mark.parametrize("page_shift", [13, 21, 30])
def test_lookup_large_table_coarse_pages(page_shift):
    # Pages larger than most regions: many starts share a page and few are
    # page multiples, which the record path's page deltas and alignment bits
    # must resolve exactly as the plain search does.
    rng = np.random.default_rng(page_shift)
    start, end = _table(rng, 20_000)
    lkey = rng.integers(1, 1 << 32, size=20_000, dtype=np.uint64).astype(np.uint32)
    off, ln = _queries(rng, start, end, 20_011)
    p = 1 << page_shift
    # Plus ranges that round exactly onto regions whose bounds are page multiples.
    al = np.nonzero(((start % p) == 0) & ((end % p) == 0))[0]
    off = np.concatenate([off, start[al], start[al] + np.uint64(1)])
    ln = np.concatenate([ln, end[al] - start[al], np.maximum(end[al] - start[al] - 2, 1)])
    for records in (True, False):
        gc.check_lookup(start, end, lkey, off, ln, page_shift=page_shift, records=records,
                        ctx=f"shift={page_shift} records={records}")


def _spread_table(kind, count, rng):
    """Tables whose starts span very different ranges: the LDS kernel buckets
    the span between the first and the last start."""
    if kind == "wide":            # starts spread over almost the whole 2^64 range
        step = ((1 << 64) - (1 << 32)) // max(count, 1)
        start = [4096 + i * (step & ~0xFFF) for i in range(count)]
        size = [4096 * int(rng.integers(1, 64)) for _ in range(count)]
    elif kind == "skewed":        # nearly all regions in one bucket, a few far away
        start, cur = [], 0x1000
        for i in range(count):
            if i in (count // 3, 2 * count // 3, count - 1):
                cur += 1 << 44
            start.append(cur)
            cur += 4096 * int(rng.integers(1, 4))
        size = [4096] * count
    else:                         # "even": one region per equal slot
        start = [0x7000_0000_0000 + i * (1 << 26) + 4096 * int(rng.integers(0, 16))
                 for i in range(count)]
        size = [4096 * int(rng.integers(1, 1024)) for _ in range(count)]
    start = np.array(start, np.uint64)
    end = np.minimum(start.astype(object) + np.array(size, dtype=object), (1 << 64) - 4096)
    return start, np.array(end, dtype=np.uint64)


def _queries_u64(rng, start, end, n):
    """Query mix of _queries in Python integers (addresses up to 2^64): whole
    regions, ranges inside one, ranges across an edge, and ranges anywhere."""
    top = (1 << 64) - (1 << 21)
    off, ln = [], []
    for _ in range(n):
        r = int(rng.integers(0, len(start)))
        s, e = int(start[r]), int(end[r])
        c = int(rng.integers(0, 4))
        if c == 0:
            o, l = s, e - s
        elif c == 1:
            o = s + int(rng.random() * (e - s))
            l = max(1, int(rng.random() * (e - o)))
        elif c == 2:
            edge = s if rng.random() < 0.5 else e
            d1, d2 = int(rng.integers(1, 5000)), int(rng.integers(1, 5000))
            o, l = max(edge - d1, 0), d1 + d2
        else:
            o, l = int(rng.random() * top), int(rng.integers(1, 1 << 20))
        off.append(o)
        ln.append(l)
    return np.array(off, np.uint64), np.array(ln, np.uint64)


@pytest.mark.parametrize("kind", ["wide", "skewed", "even"])
@pytest.mark.parametrize("count", [1, 3, 1000, 4096, 20_001])
def test_lookup_bucket_spreads(kind, count):
    rng = np.random.default_rng(count + len(kind))
    start, end = _spread_table(kind, count, rng)
    lkey = rng.integers(1, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)
    off, ln = _queries_u64(rng, start, end, 20_011)
    # Plus: below the first start, past the last, and at every bucket edge of
    # a few regions (exact starts, one page before, the last page inside).
    extra_off, extra_ln = [0, int(start[0]) - 4096 if start[0] >= 4096 else 0,
                           int(end[-1]), (1 << 64) - 8192], [4096, 4096, 4096, 4096]
    for r in rng.integers(0, count, size=min(count, 200)):
        s, e = int(start[r]), int(end[r])
        extra_off += [s, max(s - 4096, 0), e - 4096, e]
        extra_ln += [e - s, 4096, 4096, 4096]
    off = np.concatenate([off, np.array(extra_off, np.uint64)])
    ln = np.concatenate([ln, np.array(extra_ln, np.uint64)])
    for records in ((True, False) if count > 4096 else (True,)):
        gc.check_lookup(start, end, lkey, off, ln, records=records,
                        ctx=f"{kind} R={count} records={records}")


def test_lookup_invalid_and_va_base():
    start = np.array([0x1000, 0x9000], np.uint64)
    end = np.array([0x5000, 0xA000], np.uint64)
    lkey = np.array([3, 4], np.uint32)
    top = (1 << 64) - 1
    off = np.array([0x0, 0x1000, 0x10, top - 0x100, top - 0x10, top - 0x2000, 0x8000], np.uint64)
    ln = np.array([0x10, 0x0, 0x4000, 0x10, 0x10, 0x10, 0x1000], np.uint64)
    for va in (0, 0x1000, (1 << 64) - 0x1000):
        gc.check_lookup(start, end, lkey, off, ln, va_base=va, ctx=f"va={va:#x}")
    gc.check_lookup(start, end, lkey, off, ln, page_shift=30, ctx="shift30")


@pytest.mark.parametrize("count", [1000, 20_000])
def test_lookup_unaligned_columns(count):
    """Columns that start 8 bytes (1 byte for kind) past an aligned address take
    the element-by-element path and must give the same answers (LDS table and
    record path)."""
    rng = np.random.default_rng(41)
    start, end = _table(rng, count)
    lkey = rng.integers(1, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)
    off, ln = _queries(rng, start, end, 5003)
    n = off.shape[0]
    o = oracle.mr_lookup(start, end, lkey, off, ln)
    def shift(a):
        buf = torch.empty(a.numel() + 1, dtype=a.dtype, device="cuda")
        buf[1:].copy_(a)
        return buf[1:]

    out = dict(handle=torch.empty(n + 1, dtype=torch.int32, device="cuda")[1:],
               lkey=torch.empty(n + 1, dtype=torch.uint32, device="cuda")[1:],
               kind=torch.empty(n + 1, dtype=torch.uint8, device="cuda")[1:],
               rbase=torch.empty(n + 1, dtype=torch.uint64, device="cuda")[1:],
               rend=torch.empty(n + 1, dtype=torch.uint64, device="cuda")[1:])
    dd.mr_lookup(gc.dev(start), gc.dev(end), gc.dev(lkey), shift(gc.dev(off)), shift(gc.dev(ln)),
                 out=out)
    torch.cuda.synchronize()
    gc.assert_lookup_equal(o, {k: gc.host(v) for k, v in out.items()}, "unaligned")


def test_lookup_register_sequence_table():
    base = 0x7F00_0000_0000
    reg = oracle.Registry(12)
    reg.register(base, 0x200000)
    s, e, _ = reg.table()
    off = np.array([base, base, base + 0x1000, base + 0x400000], np.uint64)
    ln = np.array([0x200000, 0x200000, 0x100000, 0x200000], np.uint64)
    o, g = gc.check_lookup(s, e, np.array([7], np.uint32), off, ln, ctx="register seq")
    assert list(g["kind"]) == [1, 1, 2, 0]


# ----------------------------------------------------------- split edges ---

# Up to 70 queues the scatter ranks by counters, from 71 on by ballots; a
# block covers 4,096 requests.
@pytest.mark.parametrize("nq", [1, 2, 3, 7, 8, 16, 64, 65, 70, 71, 255, 256])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 2047, 2048, 2049, 4096, 4097, 8191, 8192, 8193,
                               16_385, 70_001])
def test_split_sizes(nq, n):
    rng = np.random.default_rng(nq * 1000 + n)
    qid = rng.integers(0, nq + 2, size=n).astype(np.uint32)
    qid[rng.random(n) < 0.01] = np.uint32(0xFFFFFFFF)
    gc.check_split(qid, nq, ctx=f"nq={nq} n={n}")


@pytest.mark.parametrize("nq", [71, 256])
def test_split_full_size_ballot_path(nq):
    # The ballot ranking (above 70 queues) at the Mixed batch size, Zipf ids
    # (a few dense buckets, many sparse ones) and some overflow ids.
    n = synth.shape("mixed")["n"]
    qid = synth.queue_ids(n, nq, seed=nq)
    qid[::100_003] = np.uint32(nq + 5)
    gc.check_split(qid, nq, ctx=f"full size nq={nq}")


@pytest.mark.parametrize("nq", [64, 256])
def test_split_unaligned_qid(nq):
    """A queue-id column 4 bytes past a 16-byte boundary takes the scalar loads."""
    rng = np.random.default_rng(nq + 11)
    n = 3 * 4096 + 77
    qid = rng.integers(0, nq + 1, size=n).astype(np.uint32)
    buf = gc.dev(np.zeros(n + 1, np.uint32))
    buf[1:].copy_(gc.dev(qid))
    out = dd.partition_by_queue(buf[1:], nq, check=False)
    torch.cuda.synchronize()
    o = oracle.partition(qid, nq)
    assert np.array_equal(gc.host(out["perm"]), o["perm"])
    assert np.array_equal(gc.host(out["qoff"]), o["qoff"])


def test_split_skewed_and_empty():
    rng = np.random.default_rng(5)
    qid = np.zeros(100_000, np.uint32)
    qid[rng.random(100_000) < 0.001] = 7
    gc.check_split(qid, 64, ctx="skewed")
    g = gc.gpu_split(np.empty(0, np.uint32), 8)
    assert list(g["qoff"]) == [0] * 10 and g["n_invalid"] == 0


def test_binding_rejects_bad_arguments():
    q = gc.dev(np.zeros(10, np.uint32))
    with pytest.raises(dd.DmadescError):
        dd.partition_by_queue(q, 0)
    with pytest.raises(dd.DmadescError):
        dd.partition_by_queue(q, 257)
    z = gc.dev(np.zeros(4, np.uint64))
    pool = torch.empty((1, 512), dtype=torch.uint64, device="cuda")
    with pytest.raises(dd.DmadescError):
        dd.build_prp(z, z, z, 0x1008, pool)
    with pytest.raises(dd.DmadescError):
        dd.mr_lookup(z, z, gc.dev(np.zeros(4, np.uint32)), z, z, page_shift=11)
    skewed = torch.empty(2 * 512 + 1, dtype=torch.uint64, device="cuda")[1:].view(2, 512)
    with pytest.raises(dd.DmadescError):                 # pool not 16-byte aligned
        dd.build_prp(z, z, z, 0x1000, skewed)
