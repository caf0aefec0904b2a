"""GPU parity of the fused batch call (dmadesc_build_batch) with the oracle:
every lookup column against O1, PRP1/PRP2/status/total and every pool word
(canary-filled on both sides) against O2 or O2p, and perm/qoff/n_invalid
against O3, bit for bit, at scaled sizes (many blocks, ragged tails) and at
full size, in both list layouts, with the edge cases of each column group."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import oracle
import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

BUS = synth.LIST_BUS_BASE


def _oracle_pages(lut, off, ln, packed):
    build = oracle.build_prp_packed if packed else oracle.build_prp
    return build(lut, off, ln, BUS, 1 << 50)["total"]


def check_batch(d, nq, packed=True, lookup=True, pool_pages=None, ctx="", va_base=None,
                page_shift=12, qid=None):
    """Runs dmadesc_build_batch on workload dict `d` and compares every
    output with the oracle's three functions on the same inputs."""
    off, ln, lut = d["off"], d["len"], d["lut"]
    qid = d["qid"] if qid is None else qid
    va = d["va_base"] if va_base is None else va_base
    n = len(off)
    if pool_pages is None:
        pool_pages = max(_oracle_pages(lut, off, ln, packed), 1)
    gc.say(f"batch {ctx}: n={n} nq={nq} packed={packed} lookup={lookup} "
           f"regions={len(d['rstart'])} pool={pool_pages}")
    pool = torch.empty((pool_pages, 512), dtype=torch.uint64, device="cuda")
    pool.view(torch.int64).fill_(gc.CANARY_I64)
    ws = torch.full((max(dd.batch_workspace_bytes(n, nq, len(d["rstart"]) if lookup else 0), 1),),
                    0xAB, dtype=torch.uint8, device="cuda")
    g = dd.build_batch(gc.dev(lut), gc.dev(off), gc.dev(ln), gc.dev(np.asarray(qid, np.uint32)),
                       nq, BUS, pool, gc.dev(d["rstart"]), gc.dev(d["rend"]), gc.dev(d["rlkey"]),
                       va_base=va, page_shift=page_shift, packed=packed, lookup=lookup, ws=ws,
                       check=False)
    torch.cuda.synchronize()
    g = {k: gc.host(v) for k, v in g.items()}
    if n:
        blocks, expired = gc.host(ws[:8]).view(np.uint32)
        assert blocks == -(-n // gc.prp_tile(n)) and expired == 0, (ctx, blocks, expired)
    # lookup
    if lookup:
        o_l = oracle.mr_lookup(d["rstart"], d["rend"], d["rlkey"], off, ln, va_base=va,
                               page_shift=page_shift)
        gc.assert_lookup_equal(o_l, g, ctx)
    else:
        assert "handle" not in g
    # PRP columns and the whole pool
    o_pool = np.full((pool_pages, 512), gc.CANARY, dtype=np.uint64)
    build = oracle.build_prp_packed if packed else oracle.build_prp
    o_p = build(lut, off, ln, BUS, pool_pages, pool=o_pool)
    gp = dict(prp1=g["prp1"], prp2=g["prp2"], status=g["status"],
              total=int(g["total_pages"][0]))
    gc.assert_prp_columns_equal(o_p, gp, ctx)
    got = gc.host(pool)
    if not packed:
        gc.mask_padding(o_pool, got, gc.padding_spans(o_p["prp2"], o_p["status"], off, ln, BUS))
    if not np.array_equal(o_pool, got):
        bad = np.argwhere(o_pool != got)
        s, p = bad[0]
        raise AssertionError(f"{ctx} pool: {len(bad)} words differ, first page {s} word {p}")
    # split
    o_s = oracle.partition(qid, nq)
    for k in ("perm", "qoff"):
        if not np.array_equal(o_s[k], g[k]):
            bad = np.nonzero(o_s[k] != g[k])[0]
            raise AssertionError(f"{ctx} split {k}: {bad.size} differ, first at {bad[0]}")
    assert int(g["n_invalid"][0]) == o_s["n_invalid"], ctx
    return g


@pytest.mark.parametrize("packed", [True, False])
@pytest.mark.parametrize("name,n", [("tiny", None), ("small", 300_001), ("mixed", 1_000_003),
                                    ("mixed", 8191), ("small", 1025)])
def test_workloads_scaled(name, n, packed):
    d = synth.generate(name, n=n)
    check_batch(d, d["nqueues"], packed=packed, ctx=f"{name}/{n}")


@pytest.mark.parametrize("packed", [True, False])
def test_large_without_lookup(packed):
    # The Large workload names no regions: the lookup columns are not asked for.
    d = synth.generate("large", n=70_001)
    check_batch(d, d["nqueues"], packed=packed, lookup=False, ctx="large/70001")


@pytest.mark.parametrize("name", ["small", "large", "mixed"])
def test_full_size_packed(name):
    d = synth.generate(name)
    check_batch(d, d["nqueues"], packed=True, lookup=bool(d["regions"]), ctx=f"full {name}")


def test_full_size_large_page_layout():
    d = synth.generate("large")
    check_batch(d, d["nqueues"], packed=False, lookup=False, ctx="full large/page")


@pytest.mark.parametrize("nq", [1, 3, 70, 71, 256])
def test_queue_counts_and_overflow_ids(nq):
    # 70 queues is the last count ranked by LDS counters (8,192-request
    # tiles), 71 the first ranked by ballots (4,096-request tiles); ids up to
    # nq + 2 put some requests in the overflow bucket.
    rng = np.random.default_rng(nq)
    d = synth.generate("mixed", n=200_003)
    qid = rng.integers(0, nq + 3, d["n"]).astype(np.uint32)
    check_batch(d, nq, qid=qid, ctx=f"nq={nq}")


def test_many_regions_through_the_index():
    # MR-heavy's 65,536 regions (a 131,072-bucket index) with its own
    # queries; their VAs lie far past a 1 GiB heap, so every PRP is ERANGE.
    t = synth.generate("mrheavy", n=300_001)
    d = synth.generate("tiny", n=16)
    d.update(rstart=t["rstart"], rend=t["rend"], rlkey=t["rlkey"], off=t["off"], len=t["len"],
             qid=np.zeros(t["n"], np.uint32), n=t["n"])
    g = check_batch(d, 1, va_base=0, ctx="mrheavy table")
    assert (g["status"] == dd.PRP_ERANGE).any()
    assert set(np.unique(g["kind"]).tolist()) >= {dd.MISS, dd.EXACT, dd.CONTAINED}


def test_empty_table_and_edge_requests():
    rng = np.random.default_rng(9)
    d = synth.generate("mixed", n=50_000)
    off, ln = d["off"].copy(), d["len"].copy()
    heap = d["lut_entries"] << 16
    sel = rng.choice(d["n"], 600, replace=False)
    ln[sel[:100]] = 0                                   # EINVAL / INVALID
    off[sel[100:200]] |= np.uint64(2)                   # not dword aligned
    off[sel[200:300]] = np.uint64(heap - 4096)          # past the heap end
    ln[sel[200:300]] = np.uint64(8192)
    off[sel[300:400]] = np.uint64(2 ** 64 - 4096)       # wraps
    ln[sel[300:400]] = np.uint64(8192)
    d.update(off=off, len=ln)
    check_batch(d, 64, ctx="edge requests")
    e = dict(d)
    e.update(rstart=d["rstart"][:0], rend=d["rend"][:0], rlkey=d["rlkey"][:0])
    g = check_batch(e, 64, ctx="empty table")
    assert set(np.unique(g["kind"]).tolist()) <= {dd.MISS, dd.INVALID}


def test_page_shift_16():
    d = synth.generate("small", n=40_000)
    check_batch(d, 64, page_shift=16, ctx="64 KiB pages")


def test_tiny_batches():
    d = synth.generate("mixed", n=1)
    check_batch(d, 64, ctx="one request")
    z = synth.generate("mixed", n=16)
    z.update(off=z["off"][:0], len=z["len"][:0], qid=z["qid"][:0], n=0)
    g = check_batch(z, 5, ctx="empty batch")
    assert list(g["qoff"]) == [0] * 7 and int(g["total_pages"][0]) == 0


def test_enospc_suffix_in_a_small_pool():
    d = synth.generate("mixed", n=100_000)
    need = _oracle_pages(d["lut"], d["off"], d["len"], True)
    g = check_batch(d, 64, pool_pages=need // 3, ctx="packed pool a third too small")
    assert (g["status"] == dd.PRP_ENOSPC).any()


def test_checked_call_reports_overflow_ids():
    d = synth.generate("mixed", n=10_000)
    pool = torch.empty((_oracle_pages(d["lut"], d["off"], d["len"], True), 512),
                       dtype=torch.uint64, device="cuda")
    qid = d["qid"].copy()
    qid[17] = 64
    with pytest.raises(dd.DmadescRefused) as e:
        dd.build_batch(gc.dev(d["lut"]), gc.dev(d["off"]), gc.dev(d["len"]), gc.dev(qid), 64,
                       BUS, pool, gc.dev(d["rstart"]), gc.dev(d["rend"]), gc.dev(d["rlkey"]),
                       va_base=d["va_base"])
    assert int(gc.host(e.value.out["n_invalid"])[0]) == 1


def test_batch_rejects_bad_arguments():
    d = synth.generate("mixed", n=100)
    pool = torch.empty((8, 512), dtype=torch.uint64, device="cuda")
    args = (gc.dev(d["lut"]), gc.dev(d["off"]), gc.dev(d["len"]), gc.dev(d["qid"]))
    with pytest.raises(dd.DmadescError):
        dd.build_batch(*args, 0, BUS, pool)                          # nqueues 0
    with pytest.raises(dd.DmadescError):
        dd.build_batch(*args, 64, BUS + 8, pool)                     # unaligned bus base
    with pytest.raises(dd.DmadescError):
        dd.build_batch(*args, 64, BUS, pool, gc.dev(d["rstart"]), gc.dev(d["rend"]),
                       gc.dev(d["rlkey"]), page_shift=11)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        dd.build_batch(*args, 64, BUS, pool, ws=small)


def _tiled_table(rng, va, span, count):
    """`count` sorted, non-overlapping regions over [va, va + span), bounds on
    64 KiB multiples (valid for every page size tested), random gaps."""
    if count == 0:
        z = np.zeros(0, np.uint64)
        return z, z.copy(), np.zeros(0, np.uint32)
    slot = max((span // count) & ~0xFFFF, 1 << 17)
    k = np.arange(count, dtype=np.uint64)
    start = np.uint64(va) + k * np.uint64(slot) + \
        (rng.integers(0, 2, count).astype(np.uint64) << np.uint64(16))
    size = rng.integers(1, slot >> 16, count).astype(np.uint64) << np.uint64(16)
    end = np.minimum(start + size, np.uint64(va) + (k + np.uint64(1)) * np.uint64(slot))
    lkey = rng.integers(1, 1 << 32, count, dtype=np.uint64).astype(np.uint32)
    return start, end, lkey


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Seeded random batches: sizes, table sizes on both sides of the LDS
    limit, queue counts on both sides of the ranking switch, page sizes and
    both list layouts; the batch call and (for the same table) the lookup's
    record and plain paths against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    name = ("small", "mixed")[seed % 2]
    n = int(rng.integers(1, 60_000))
    d = synth.generate(name, n=n, seed=seed + 1)
    R = int(rng.choice([0, 1, 17, 1000, 4096, 4097, 9000, 20_000]))
    heap = d["lut_entries"] << 16
    rs, re_, rk = _tiled_table(rng, d["va_base"], heap, R)
    nq = int(rng.choice([1, 5, 64, 70, 71, 200, 256]))
    qid = synth.queue_ids(n, nq, seed=seed + 3)
    qid[rng.random(n) < 0.01] = np.uint32(nq + 1)
    ps = int(rng.choice([12, 13, 16]))
    packed = bool(rng.integers(0, 2))
    d.update(rstart=rs, rend=re_, rlkey=rk)
    check_batch(d, nq, packed=packed, qid=qid, page_shift=ps,
                ctx=f"seed={seed} {name} n={n} R={R} nq={nq} shift={ps} packed={packed}")
    for records in ((True, False) if R > 4096 else (True,)):
        gc.check_lookup(rs, re_, rk, d["off"], d["len"], va_base=d["va_base"], page_shift=ps,
                        records=records, ctx=f"seed={seed} lookup R={R} records={records}")
