"""Shared helpers for the GPU parity tests: run the C-ABI library through its
binding and compare with the oracle, column by column, bit for bit."""
from __future__ import annotations

import numpy as np
import torch

import memory_dma_descriptor_amd as dd
import oracle

CANARY = 0xCCCC_CCCC_CCCC_CCCC
CANARY_I64 = np.uint64(CANARY).astype(np.int64).item()
# The library may write the words after a request's last list entry, up to
# the next multiple of PAD_WORDS words inside that request's final list page
# (their contents are unspecified); every other pool word it must leave alone.
PAD_WORDS = 8


def prp_tile(n):
    """Requests per block of the PRP build's slot scan: 256 for batches of at
    most 2^16 requests, 512 up to 2^19, 2,048 up to 2^22, 1,024 above (the
    library's choice, stated in dmadesc_build_prp's header comment)."""
    if n <= (1 << 16):
        return 256
    return 512 if n <= (1 << 19) else 2048 if n <= (1 << 22) else 1024


def padding_spans(prp2, status, off, ln, bus, slot_base=0):
    """(page, first word, end word) arrays of the words after each list's last
    entry that the library may write, from the oracle's PRP2 and status."""
    off = np.asarray(off, np.uint64)
    ln = np.asarray(ln, np.uint64)
    pages = ((off & np.uint64(4095)) + ln + np.uint64(4095)) >> np.uint64(12)
    sel = np.nonzero((np.asarray(status) == 0) & (pages >= 3))[0]
    m = pages[sel].astype(np.int64) - 1
    lp = (m - 1 + 510) // 511
    final_words = m - 511 * (lp - 1)
    end = np.minimum(512, -(-final_words // PAD_WORDS) * PAD_WORDS)
    page = ((np.asarray(prp2)[sel] - np.uint64(bus)) // np.uint64(4096)).astype(np.int64) \
        + lp - 1 - slot_base
    keep = end > final_words
    return page[keep], final_words[keep], end[keep]


def mask_padding(a, b, spans):
    """Makes the padding words of both pools equal before they are compared."""
    page, lo, hi = spans
    ok = (page >= 0) & (page < a.shape[0])
    page, lo, hi = page[ok], lo[ok], hi[ok]
    width = hi - lo
    if width.size == 0:
        return
    rows = np.repeat(page, width)
    cols = np.repeat(lo, width) + (np.arange(int(width.sum())) - np.repeat(np.cumsum(width) - width, width))
    a[rows, cols] = 0
    b[rows, cols] = 0


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def say(msg: str) -> None:
    print(msg, flush=True)


# ----------------------------------------------------------------- lookup ---

def gpu_lookup(start, end, lkey, off, ln, va_base=0, page_shift=12, records=True):
    ws = None
    if records and len(start) > 4096:
        # A canary after the record workspace: the kernels stay inside it.
        need = dd.workspace_bytes(dd.OP_MR_LOOKUP, len(off), len(start))
        ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    out = dd.mr_lookup(dev(np.asarray(start, np.uint64)), dev(np.asarray(end, np.uint64)),
                       dev(np.asarray(lkey, np.uint32)), dev(np.asarray(off, np.uint64)),
                       dev(np.asarray(ln, np.uint64)), va_base=va_base, page_shift=page_shift,
                       ws=None if ws is None else ws[:need], records=records)
    torch.cuda.synchronize()
    if ws is not None:
        assert (host(ws[need:]) == 0x5A).all(), "lookup wrote past its record workspace"
    return {k: host(v) for k, v in out.items()}


def assert_lookup_equal(o, g, ctx=""):
    for k in ("handle", "lkey", "kind", "rbase", "rend"):
        if not np.array_equal(o[k], g[k]):
            bad = np.nonzero(o[k] != g[k])[0]
            raise AssertionError(f"{ctx} lookup column {k}: {bad.size} mismatches, first at "
                                 f"{bad[0]}: oracle {o[k][bad[0]]} gpu {g[k][bad[0]]}")


def check_lookup(start, end, lkey, off, ln, va_base=0, page_shift=12, ctx="", records=True):
    o = oracle.mr_lookup(start, end, lkey, off, ln, va_base=va_base, page_shift=page_shift)
    g = gpu_lookup(start, end, lkey, off, ln, va_base=va_base, page_shift=page_shift,
                   records=records)
    assert_lookup_equal(o, g, ctx)
    return o, g


# -------------------------------------------------------------------- PRP ---

def gpu_prp(lut, off, ln, bus, pool_pages, packed=False):
    """Runs dmadesc_build_prp (or its packed form) on a canary-filled pool;
    returns (outputs as numpy, the device pool)."""
    pool = torch.empty((pool_pages, 512), dtype=torch.uint64, device="cuda")
    pool.view(torch.int64).fill_(CANARY_I64)
    n = len(off)
    ws = torch.full((max(dd.workspace_bytes(dd.OP_BUILD_PRP, n), 8),), 0xAB,
                    dtype=torch.uint8, device="cuda")
    out = dd.build_prp(dev(np.asarray(lut, np.uint64)), dev(np.asarray(off, np.uint64)),
                       dev(np.asarray(ln, np.uint64)), bus, pool, ws=ws, packed=packed)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    g["total"] = int(g.pop("total_pages")[0])
    if n:
        # workspace header: blocks that ran, and bounded waits that expired
        blocks, timeouts = host(ws[:8]).view(np.uint32)
        assert 1 <= blocks <= n and timeouts == 0, (blocks, timeouts)
    return g, pool


def assert_prp_columns_equal(o, g, ctx=""):
    for k in ("prp1", "prp2", "status"):
        if not np.array_equal(o[k], g[k]):
            bad = np.nonzero(o[k] != g[k])[0]
            raise AssertionError(f"{ctx} PRP column {k}: {bad.size} mismatches, first at "
                                 f"{bad[0]}: oracle {o[k][bad[0]]:#x} gpu {g[k][bad[0]]:#x}")
    assert o["total"] == g["total"], (ctx, o["total"], g["total"])


def check_prp_full(lut, off, ln, bus, pool_pages, ctx="", packed=False):
    """Whole-pool comparison: both pools start as canary, so equal pools mean
    the GPU wrote exactly the oracle's entries and nothing else (the page
    layout's padding words aside; the packed layout has none)."""
    o_pool = np.full((pool_pages, 512), CANARY, dtype=np.uint64)
    build = oracle.build_prp_packed if packed else oracle.build_prp
    o = build(lut, off, ln, bus, pool_pages, pool=o_pool)
    g, pool = gpu_prp(lut, off, ln, bus, pool_pages, packed=packed)
    assert_prp_columns_equal(o, g, ctx)
    gp = host(pool)
    if not packed:
        mask_padding(o_pool, gp, padding_spans(o["prp2"], o["status"], off, ln, bus))
    if not np.array_equal(o_pool, gp):
        bad = np.argwhere(o_pool != gp)
        s, p = bad[0]
        raise AssertionError(f"{ctx} pool: {len(bad)} mismatching entries, first at page {s} "
                             f"entry {p}: oracle {o_pool[s, p]:#x} gpu {gp[s, p]:#x}")
    return o, g


def check_prp_chunked(lut, off, ln, bus, pool_pages, ctx="", chunk=1 << 20):
    """Full-size check of the page layout, every list page included: every
    PRP1/PRP2/status and the total against the oracle run without a pool;
    then, chunk by chunk of requests, the oracle run on the chunk alone at
    its slot offset (the oracle's own page count of the requests before it)
    writes the chunk's list pages, which must equal the GPU pool's pages at
    that offset (padding words masked); pool pages past the total untouched."""
    o = oracle.build_prp(lut, off, ln, bus, pool_pages, pool=None)
    g, pool = gpu_prp(lut, off, ln, bus, pool_pages)
    assert_prp_columns_equal(o, g, ctx)
    n = len(off)
    slot0 = 0
    compared = 0
    for i0 in range(0, n, chunk):
        i1 = min(n, i0 + chunk)
        o_off, o_ln = off[i0:i1], ln[i0:i1]
        base = bus + slot0 * 4096
        need = oracle.build_prp(lut, o_off, o_ln, base, pool_pages - slot0, pool=None)["total"]
        want = np.full((max(need, 1), 512), CANARY, dtype=np.uint64)
        part = oracle.build_prp(lut, o_off, o_ln, base, need, pool=want)
        # The chunk run places its requests exactly as the whole run does.
        for k in ("prp1", "prp2", "status"):
            assert np.array_equal(part[k], o[k][i0:i1]), (ctx, i0, k)
        if need:
            got = host(pool[slot0:slot0 + need])
            mask_padding(got, want, padding_spans(part["prp2"], part["status"], o_off, o_ln,
                                                  bus, slot_base=slot0))
            if not np.array_equal(got, want[:need]):
                bad = np.argwhere(got != want[:need])
                raise AssertionError(f"{ctx} list pages of requests [{i0}, {i1}): {len(bad)} "
                                     f"words differ, first at page {slot0 + bad[0][0]} "
                                     f"word {bad[0][1]}")
        compared += need
        slot0 += need
    assert slot0 == o["total"] == compared, (ctx, slot0, o["total"])
    tail = pool.view(torch.int64)[min(g["total"], pool_pages):]
    assert bool((tail == CANARY_I64).all()), f"{ctx}: pool pages past the total were written"
    return o, g, compared


# ------------------------------------------------------------------ split ---

def gpu_split(qid, nq, check=False):
    out = dd.partition_by_queue(dev(np.asarray(qid, np.uint32)), nq, check=check)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    g["n_invalid"] = int(g["n_invalid"][0])
    return g


def check_split(qid, nq, ctx=""):
    o = oracle.partition(qid, nq)
    g = gpu_split(qid, nq)
    for k in ("perm", "qoff"):
        if not np.array_equal(o[k], g[k]):
            bad = np.nonzero(o[k] != g[k])[0]
            raise AssertionError(f"{ctx} split column {k}: {bad.size} mismatches, first at "
                                 f"{bad[0]}: oracle {o[k][bad[0]]} gpu {g[k][bad[0]]}")
    assert o["n_invalid"] == g["n_invalid"], ctx
    if o["n_invalid"]:
        # The checked call reports the overflow bucket after synchronizing.
        try:
            gpu_split(qid, nq, check=True)
        except dd.DmadescRefused as e:
            assert np.array_equal(host(e.out["perm"]), o["perm"]), ctx
        else:
            raise AssertionError(f"{ctx}: overflow ids were not reported")
    return o, g


# ------------------------------------------------------ submission entries ---

RING_FILL = 0xEE
RID_FILL = 0xA5A5A5A5


class SqeRig:
    """Rings, request maps, tails and cursors of both sides for a series of
    dmadesc_emit_sqe calls. `refuse` queues get ring address 0 (None for the
    oracle); `misalign` queues get a ring address 16 bytes into a buffer that
    has room for a whole ring past it (so even a wrong write stays inside it)."""

    def __init__(self, depth, tail, refuse=(), misalign=(), req_map=True):
        self.depth = np.asarray(depth, np.uint32)
        nq = self.depth.size
        self.nq = nq
        # GPU buffers leave room for slots up to tail + depth, so that even a
        # queue the library should refuse for its tail could not be written
        # outside its buffer.
        rows = [max(int(d), 1) for d in self.depth]
        grow = [rows[q] + int(np.asarray(tail)[q]) for q in range(nq)]
        self.o_rings = [None if (q in refuse or q in misalign)
                        else np.full((rows[q], 64), RING_FILL, np.uint8) for q in range(nq)]
        self.g_bufs = [torch.full((grow[q] * 64 + 64,), RING_FILL, dtype=torch.uint8,
                                  device="cuda") for q in range(nq)]
        addrs = []
        for q in range(nq):
            p = self.g_bufs[q].data_ptr()
            assert p % 256 == 0
            addrs.append(0 if q in refuse else (p + 16 if q in misalign else p))
        self.g_ring = torch.tensor(addrs, dtype=torch.int64).view(torch.uint64).cuda()
        self.o_tail = np.asarray(tail, np.uint32).copy()
        self.o_cursor = np.zeros(nq, np.uint64)
        self.g_tail = dev(self.o_tail.copy())
        self.g_cursor = dev(self.o_cursor.copy())
        self.g_depth = dev(self.depth)
        self.o_rid = self.g_rid = None
        if req_map:
            self.o_rid = np.full((nq, 65536), RID_FILL, np.uint32)
            self.g_rid = dev(np.full(nq * 65536, RID_FILL, np.uint32))

    def call(self, o_in, g_in, free, lba_shift=9, opcode=0x02, nsid=1, ctx=""):
        """o_in / g_in: dict(perm, qoff, status, len, slba, prp1, prp2) as numpy
        arrays (oracle) and device tensors (GPU). Compares every output."""
        free = np.asarray(free, np.uint32)
        say(f"emit_sqe {ctx}: nq={self.nq} n={o_in['len'].size} lba_shift={lba_shift}")
        o = oracle.emit_sqe(o_in["perm"], o_in["qoff"], o_in["status"], o_in["len"],
                            o_in["slba"], o_in["prp1"], o_in["prp2"], self.o_rings,
                            self.depth, free, self.o_tail, self.o_cursor,
                            req_of_slot=self.o_rid, opcode=opcode, nsid=nsid,
                            lba_shift=lba_shift)
        g = dd.emit_sqe(g_in["perm"], g_in["qoff"], g_in["status"], g_in["len"],
                        g_in["slba"], g_in["prp1"], g_in["prp2"], self.g_ring, self.g_depth,
                        dev(free), self.g_tail, self.g_cursor, req_of_slot=self.g_rid,
                        opcode=opcode, nsid=nsid, lba_shift=lba_shift)
        torch.cuda.synchronize()
        self.o_tail, self.o_cursor = o["tail"], o["cursor"]
        for k, want, got in (("placed", o["placed"], host(g["placed"])),
                             ("tail", o["tail"], host(self.g_tail)),
                             ("cursor", o["cursor"], host(self.g_cursor))):
            if not np.array_equal(want, got):
                bad = np.nonzero(want != got)[0]
                raise AssertionError(f"{ctx} {k}: queues {bad[:8].tolist()}: oracle "
                                     f"{want[bad[:8]].tolist()} gpu {got[bad[:8]].tolist()}")
        for q in range(self.nq):
            gb = host(self.g_bufs[q])
            if self.o_rings[q] is None:
                assert (gb == RING_FILL).all(), f"{ctx} refused queue {q} was written"
                continue
            ob = self.o_rings[q].reshape(-1)
            if not np.array_equal(gb[:ob.size], ob):
                bad = np.nonzero(gb[:ob.size] != ob)[0]
                raise AssertionError(f"{ctx} ring {q}: {bad.size} bytes differ, first in "
                                     f"slot {bad[0] // 64} byte {bad[0] % 64}")
            assert (gb[ob.size:] == RING_FILL).all(), f"{ctx} ring {q} written past its end"
        if self.o_rid is not None:
            gr = host(self.g_rid).reshape(self.nq, 65536)
            if not np.array_equal(gr, self.o_rid):
                bad = np.argwhere(gr != self.o_rid)
                raise AssertionError(f"{ctx} req_of_slot: {len(bad)} differ, first {bad[0]}")
        return o


def sqe_inputs(perm, qoff, status, ln, slba, prp1, prp2):
    """The same emission inputs as numpy (oracle) and device tensors (GPU)."""
    o = dict(perm=np.asarray(perm, np.uint32), qoff=np.asarray(qoff, np.uint64),
             status=np.asarray(status, np.uint8), len=np.asarray(ln, np.uint64),
             slba=np.asarray(slba, np.uint64), prp1=np.asarray(prp1, np.uint64),
             prp2=np.asarray(prp2, np.uint64))
    return o, {k: dev(v) for k, v in o.items()}
