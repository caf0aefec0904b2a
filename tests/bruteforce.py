"""Independent brute-force definitions used to pin the oracle.

These restate what the results must be in a different form from the oracle:
integer floor/ceil instead of masks, a scan over every region instead of a
binary search, a walk over every byte of a request instead of page arithmetic,
a chain walk that follows pointers instead of slot arithmetic, and a library
stable sort instead of a counting split. Pure Python / numpy, small inputs only.
"""
from __future__ import annotations

import numpy as np

MISS, EXACT, CONTAINED, INVALID = 0, 1, 2, 3
U64_MAX = (1 << 64) - 1


def round_bounds(a: int, size: int, page: int):
    """Whole pages covering [a, a+size): floor of the start, ceiling of the end."""
    lo = (a // page) * page
    hi = -(-(a + size) // page) * page
    return lo, hi


def lookup(start, end, lkey, off, length, va_base=0, page_shift=12):
    """Containment lookup by scanning every region for one that holds the
    rounded range."""
    page = 1 << page_shift
    start = [int(x) for x in start]
    end = [int(x) for x in end]
    res = []
    for o, ln in zip(off, length):
        a, size = va_base + int(o), int(ln)
        if size == 0 or a > U64_MAX or a + size > U64_MAX:
            res.append((-1, 0, INVALID, 0, 0))
            continue
        lo, hi = round_bounds(a, size, page)
        if hi > U64_MAX:
            res.append((-1, 0, INVALID, 0, 0))
            continue
        hit = None
        for r, (s, e) in enumerate(zip(start, end)):
            if s <= lo and hi <= e:
                hit = r
                break
        if hit is None:
            res.append((-1, 0, MISS, lo, hi))
        else:
            k = EXACT if (lo == start[hit] and hi == end[hit]) else CONTAINED
            res.append((hit, int(lkey[hit]), k, lo, hi))
    return res


def phys_bytes(lut: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Physical address of heap bytes x: the 64 KiB GPU page's physical
    address plus the byte's position inside that GPU page."""
    x = x.astype(np.uint64)
    return lut[x // np.uint64(65536)] + x % np.uint64(65536)


def touched_pages(lut: np.ndarray, off: int, size: int):
    """Walks every byte of [off, off+size) and returns (physical address of the
    first byte, physical 4 KiB page addresses touched, in order, no repeats)."""
    x = np.arange(off, off + size, dtype=np.uint64)
    ph = phys_bytes(lut, x)
    pg = ph // np.uint64(4096)
    keep = np.ones(pg.shape[0], dtype=bool)
    keep[1:] = pg[1:] != pg[:-1]
    return int(ph[0]), [int(p) * 4096 for p in pg[keep]]


def chain_walk(pool: np.ndarray, bus: int, prp2: int, count: int, allow_offset=False):
    """Follows an NVMe PRP list from PRP2 and returns (the `count` data
    entries, the list slots visited). In a list page, the last entry is a
    pointer to the next list page whenever more than one entry remains. With
    allow_offset, PRP2 may point to any qword of its page (the NVMe rule for
    the list pointer in a command); chain pointers must name a page start."""
    rel = prp2 - bus
    assert rel >= 0 and rel % 8 == 0, "PRP2 is not a qword address in the pool"
    assert allow_offset or rel % 4096 == 0, "PRP2 does not name a list page"
    slot = rel // 4096
    slots = [slot]
    entries = []
    pos = (rel % 4096) // 8
    while len(entries) < count:
        if pos == 511 and count - len(entries) > 1:
            nxt = int(pool[slot, 511]) - bus
            assert nxt >= 0 and nxt % 4096 == 0, "chain pointer does not name a list page"
            slot = nxt // 4096
            slots.append(slot)
            pos = 0
            continue
        entries.append(int(pool[slot, pos]))
        pos += 1
    return entries, slots


def stable_split(qid: np.ndarray, nqueues: int):
    """Stable sort of request indices by bucket (ids >= nqueues share the
    overflow bucket) and bucket starts from a histogram."""
    b = np.minimum(qid.astype(np.int64), nqueues)
    perm = np.argsort(b, kind="stable").astype(np.uint32)
    counts = np.bincount(b, minlength=nqueues + 1)
    qoff = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint64)
    return perm, qoff, int(counts[nqueues])


# NVMe common command format, little endian: opcode, flags, command id,
# namespace id, CDW2-3, metadata pointer, PRP1, PRP2, starting LBA (CDW10-11),
# CDW12 (number of blocks minus one in bits 15:0, flags above), CDW13-15.
SQE_FORMAT = "<BBHI8s8sQQQHH12s"


def pack_sqe(opcode: int, cid: int, nsid: int, prp1: int, prp2: int, slba: int,
             nlb0: int) -> bytes:
    """One 64-byte submission entry laid out field by field."""
    import struct
    return struct.pack(SQE_FORMAT, opcode, 0, cid, nsid, bytes(8), bytes(8), prp1, prp2,
                       slba, nlb0, 0, bytes(12))


def unpack_sqe(raw: bytes) -> dict:
    import struct
    f = struct.unpack(SQE_FORMAT, bytes(raw))
    return dict(opcode=f[0], flags=f[1], cid=f[2], nsid=f[3], cdw2_3=f[4], mptr=f[5],
                prp1=f[6], prp2=f[7], slba=f[8], nlb0=f[9], cdw12_hi=f[10], rest=f[11])


def queue_feed(qid, status, length, lba_shift, q):
    """Request indices of queue q in request order, with whether each can be
    expressed as one command (PRP built, whole blocks, 1..65536 blocks)."""
    idx = np.flatnonzero(np.asarray(qid) == q)
    block = 1 << lba_shift
    out = []
    for i in idx:
        ln = int(length[i])
        ok = int(status[i]) == 0 and ln > 0 and ln % block == 0 and ln // block <= 65536
        out.append((int(i), ok))
    return out


class RecordList:
    """Registration records as a plain Python list kept in start order: a
    range is rounded to whole pages (floor / ceiling); the first record in list
    order that contains it gains a reference, else a new record goes after
    every record starting at or before it; a deregistration drops a reference
    and removes the record at zero; a handle no record holds is stale."""

    def __init__(self, page_shift=12):
        self.page = 1 << page_shift
        self.recs = []          # [start, end, handle, refs]
        self.next = 1

    def register(self, addr, size):
        if size == 0 or addr + size > U64_MAX:
            return 0, "invalid"
        lo, hi = round_bounds(addr, size, self.page)
        if hi > U64_MAX:
            return 0, "invalid"
        for r in self.recs:
            if r[0] <= lo and hi <= r[1]:
                r[3] += 1
                return r[2], "hit"
        pos = sum(1 for r in self.recs if r[0] <= lo)
        h = self.next
        self.next += 1
        self.recs.insert(pos, [lo, hi, h, 1])
        return h, "new"

    def deregister(self, handle):
        for k, r in enumerate(self.recs):
            if r[2] == handle:
                r[3] -= 1
                if r[3] == 0:
                    del self.recs[k]
                    return "removed"
                return "ok"
        return "stale"


class CqController:
    """A completion queue as the NVMe controller fills it: entries are written
    in queue order, the phase tag (dword 3 bit 16) 1 on the first pass through
    the queue and inverted on every pass after."""

    def __init__(self, depth, seed=0):
        self.depth = depth
        self.cq = np.zeros((depth, 4), np.uint32)
        self.tail = 0
        self.phase = 1
        self.rng = np.random.default_rng(seed)
        self.log = []                       # every entry written, in order

    def complete(self, count):
        for _ in range(count):
            e = self.rng.integers(0, 1 << 32, 4, dtype=np.uint64).astype(np.uint32)
            e[3] = (e[3] & np.uint32(~(1 << 16) & 0xFFFFFFFF)) | np.uint32(self.phase << 16)
            self.cq[self.tail] = e
            self.log.append(e.copy())
            self.tail += 1
            if self.tail == self.depth:
                self.tail = 0
                self.phase ^= 1
