"""Pins the CPU oracle to what the pages and the mathematics fix.

Nothing here touches the GPU library. Each test checks the oracle against a
value printed on the pages (tests/golden/), a closed form, an invariant, or an
independent brute force (tests/bruteforce.py).
"""
import os

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BUS = 0x0000_1000_0000_0000


def _rows(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# --------------------------------------------------------------------------
# O1 page rounding and containment
# --------------------------------------------------------------------------

def test_rounding_table_from_ib_mr_cache():
    rows = _rows("nccl26_ib_mr_rounding.txt")
    off = np.array([int(r[0], 16) for r in rows], np.uint64)
    ln = np.array([int(r[1]) for r in rows], np.uint64)
    out = oracle.mr_lookup(np.empty(0), np.empty(0), np.empty(0), off, ln, page_shift=12)
    for k, r in enumerate(rows):
        assert int(out["rbase"][k]) == int(r[2], 16)
        assert (int(out["rend"][k]) - int(out["rbase"][k])) // 4096 == int(r[3])
        assert out["kind"][k] == oracle.MISS and out["handle"][k] == -1


def _replay_register_sequence(base):
    reg = oracle.Registry(12)
    names = {}
    for op, s, e, want in _rows("nccl26_comm_register_sequence.txt"):
        if op == "register":
            h = reg.register(base + int(s, 16), int(e, 16) - int(s, 16))
            assert h > 0
            if want.startswith("="):
                assert h == names[want[1:]]
            elif want == "new":
                assert h != names["h1"]
                names["hdis"] = h
            else:
                names[want] = h
        elif op == "refs":
            assert reg.refs(names["h1"]) == int(want)
        elif op == "deregister":
            rc = reg.deregister(names["h1"])
            assert rc == (0 if want == "ok" else -1)
    return reg, names


def test_register_sequence_replay():
    base = 0x7F00_0000_0000
    reg, names = _replay_register_sequence(base)
    # h1 is gone after three deregisters; the disjoint record remains.
    assert reg.refs(names["h1"]) == -1
    assert reg.refs(names["hdis"]) == 1
    assert reg.count() == 1


def test_register_sequence_as_batch_lookup():
    """The four ranges of the experiment, looked up against the table that
    the first registration creates: exact, exact, contained, miss."""
    base = 0x7F00_0000_0000
    rows = [r for r in _rows("nccl26_comm_register_sequence.txt") if r[0] == "register"]
    off = np.array([base + int(r[1], 16) for r in rows], np.uint64)
    ln = np.array([int(r[2], 16) - int(r[1], 16) for r in rows], np.uint64)
    reg = oracle.Registry(12)
    reg.register(int(off[0]), int(ln[0]))
    s, e, _ = reg.table()
    out = oracle.mr_lookup(s, e, np.array([7], np.uint32), off, ln)
    assert list(out["kind"]) == [oracle.EXACT, oracle.EXACT, oracle.CONTAINED, oracle.MISS]
    assert list(out["handle"]) == [0, 0, 0, -1]
    assert list(out["lkey"]) == [7, 7, 7, 0]
    # With the disjoint range registered too, it becomes an exact hit on record 1.
    reg.register(int(off[3]), int(ln[3]))
    s, e, _ = reg.table()
    out = oracle.mr_lookup(s, e, np.array([7, 9], np.uint32), off, ln)
    assert list(out["kind"]) == [oracle.EXACT, oracle.EXACT, oracle.CONTAINED, oracle.EXACT]
    assert list(out["handle"]) == [0, 0, 0, 1]


def test_registry_partial_overlap_is_not_a_hit():
    reg = oracle.Registry(12)
    h1 = reg.register(0x10_0000, 0x20_0000)
    h2 = reg.register(0x20_0000, 0x20_0000)     # overlaps h1's second half only
    assert h2 != h1 and reg.count() == 2
    assert reg.register(0x10_0000 + 1, 4096) == h1   # contained after rounding
    assert reg.refs(h1) == 2


def test_registry_capacity_growth():
    reg = oracle.Registry(12)
    assert reg.capacity() == 0
    seen = []
    for k in range(129):
        reg.register(k * 0x10_0000, 4096)
        if reg.capacity() not in seen:
            seen.append(reg.capacity())
    assert seen == [32, 64, 128, 256]


def test_registry_unknown_handle_is_error():
    reg = oracle.Registry(12)
    assert reg.deregister(12345) == -1
    assert reg.register(0x1000, 0) == 0


def _random_table(rng, count, abut_p=0.3, gran=4096):
    start, end = [], []
    cur = 0x7000_0000_0000
    for _ in range(count):
        if rng.random() >= abut_p:
            cur += gran * int(rng.integers(1, 64))
        size = gran * int(rng.integers(1, 256))
        start.append(cur)
        end.append(cur + size)
        cur += size
    return np.array(start, np.uint64), np.array(end, np.uint64)


def _queries_for(rng, start, end, n):
    lo = int(start[0]) - 3 * 4096 if len(start) else 0x7000_0000_0000
    hi = int(end[-1]) + 3 * 4096 if len(end) else lo + (1 << 20)
    off, ln = [], []
    for _ in range(n):
        c = rng.integers(0, 5)
        if c == 0 and len(start):                        # exact region
            r = int(rng.integers(0, len(start)))
            off.append(int(start[r])); ln.append(int(end[r]) - int(start[r]))
        elif c == 1 and len(start):                      # inside a region
            r = int(rng.integers(0, len(start)))
            a = int(rng.integers(int(start[r]), int(end[r])))
            off.append(a); ln.append(int(rng.integers(1, int(end[r]) - a + 1)))
        elif c == 2 and len(start):                      # across an edge
            r = int(rng.integers(0, len(start)))
            edge = int(start[r]) if rng.random() < 0.5 else int(end[r])
            d1, d2 = int(rng.integers(1, 5000)), int(rng.integers(1, 5000))
            off.append(edge - d1); ln.append(d1 + d2)
        else:                                            # anywhere
            a = int(rng.integers(lo, hi))
            off.append(a); ln.append(int(rng.integers(1, 1 << 20)))
    return np.array(off, np.uint64), np.array(ln, np.uint64)


@pytest.mark.parametrize("count", [0, 1, 2, 64, 300])
@pytest.mark.parametrize("page_shift", [12, 16])
def test_lookup_matches_full_scan(count, page_shift):
    rng = np.random.default_rng(1000 + count + page_shift)
    start, end = _random_table(rng, count)
    lkey = rng.integers(1, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)
    off, ln = _queries_for(rng, start, end, 1500)
    out = oracle.mr_lookup(start, end, lkey, off, ln, page_shift=page_shift)
    want = bf.lookup(start, end, lkey, off, ln, page_shift=page_shift)
    for i, (h, k_, kind, lo, hi) in enumerate(want):
        got = (int(out["handle"][i]), int(out["lkey"][i]), int(out["kind"][i]),
               int(out["rbase"][i]), int(out["rend"][i]))
        assert got == (h, k_, kind, lo, hi), (i, int(off[i]), int(ln[i]))


def test_lookup_va_base_and_invalid_ranges():
    start = np.array([0x1000, 0x9000], np.uint64)
    end = np.array([0x5000, 0xA000], np.uint64)
    lkey = np.array([3, 4], np.uint32)
    top = (1 << 64) - 1
    off = np.array([0x0, 0x1000, 0x10, top - 0x100, top - 0x10], np.uint64)
    ln = np.array([0x10, 0x0, 0x4000, 0x10, 0x10], np.uint64)
    out = oracle.mr_lookup(start, end, lkey, off, ln, va_base=0x1000)
    want = bf.lookup(start, end, lkey, off, ln, va_base=0x1000)
    for i, w in enumerate(want):
        got = (int(out["handle"][i]), int(out["lkey"][i]), int(out["kind"][i]),
               int(out["rbase"][i]), int(out["rend"][i]))
        assert got == w, i
    assert list(out["kind"]) == [oracle.CONTAINED, oracle.INVALID, oracle.MISS,
                                 oracle.INVALID, oracle.INVALID]


# --------------------------------------------------------------------------
# O2 PRP construction
# --------------------------------------------------------------------------

def _perm_lut(rng, p, base=0x2000_0000_0000):
    return (np.uint64(base) + rng.permutation(p).astype(np.uint64) * np.uint64(65536))


def _check_prp_against_bytewalk(lut, off, ln, out, bus):
    """Every request: PRP1, PRP2 and the chained list against the byte walk."""
    heap = lut.shape[0] * 65536
    slots_used = []
    for i in range(off.shape[0]):
        o, size = int(off[i]), int(ln[i])
        st = int(out["status"][i])
        if size == 0 or o % 4 or o + size > (1 << 64) - 1:
            assert st == oracle.EINVAL
            continue
        if o + size > heap:
            assert st == oracle.ERANGE
            continue
        first, pages = bf.touched_pages(lut, o, size)
        p1, p2 = int(out["prp1"][i]), int(out["prp2"][i])
        if st == oracle.ENOSPC:
            assert len(pages) >= 3 and p1 == 0 and p2 == 0
            continue
        assert st == oracle.OK
        assert p1 == first
        if len(pages) == 1:
            assert p2 == 0
        elif len(pages) == 2:
            assert p2 == pages[1]
        else:
            entries, slots = bf.chain_walk(out["pool"], bus, p2, len(pages) - 1)
            assert entries == pages[1:]
            assert slots == list(range(slots[0], slots[0] + len(slots)))
            slots_used.append((i, slots))
    return slots_used


def test_prp_bytewalk_tiny_heap_boundaries():
    """4-entry heap (256 KiB): every dword offset near 4 KiB and 64 KiB
    boundaries with lengths around page multiples."""
    rng = np.random.default_rng(7)
    lut = _perm_lut(rng, 4)
    offs = sorted(set(list(range(0, 256, 4)) + list(range(4096 - 64, 4096 + 64, 4))
                      + list(range(65536 - 128, 65536 + 64, 4))
                      + list(range(2 * 65536 - 8, 2 * 65536 + 8, 4))))
    lens = [1, 3, 4, 5, 100, 4092, 4095, 4096, 4097, 8191, 8192, 8193, 12288, 12289,
            65536, 65537, 70000]
    off = np.array([o for o in offs for _ in lens], np.uint64)
    ln = np.array([l for _ in offs for l in lens], np.uint64)
    cap = 4096
    out = oracle.build_prp(lut, off, ln, BUS, cap, pool=True)
    used = _check_prp_against_bytewalk(lut, off, ln, out, BUS)
    # list pages are handed out in request order, back to back from slot 0
    nxt = 0
    for _, slots in used:
        assert slots[0] == nxt
        nxt += len(slots)
    assert out["total"] == nxt


@pytest.mark.parametrize("p", [8, 128])
def test_prp_bytewalk_random(p):
    rng = np.random.default_rng(100 + p)
    lut = _perm_lut(rng, p)
    heap = p * 65536
    n = 600
    ln = rng.integers(1, 40 * 4096, size=n).astype(np.uint64)
    off = (rng.integers(0, heap // 4, size=n) * 4).astype(np.uint64)
    off = np.minimum(off, np.uint64(heap) - ln) // np.uint64(4) * np.uint64(4)
    out = oracle.build_prp(lut, off, ln, BUS, 4096, pool=True)
    _check_prp_against_bytewalk(lut, off, ln, out, BUS)
    assert (out["status"] == 0).all()


def test_prp_identity_table_is_textbook_contiguous_list():
    """With table[i] = base + 64 KiB * i the heap is physically contiguous and
    the list must be the textbook one: base + page-aligned offset + 4 KiB*k."""
    p = 256
    base = 0x3000_0000_0000
    lut = np.uint64(base) + np.arange(p, dtype=np.uint64) * np.uint64(65536)
    rng = np.random.default_rng(3)
    n = 400
    ln = rng.integers(1, 3 * 512 * 4096, size=n).astype(np.uint64)
    off = (rng.integers(0, (p * 65536 - 3 * 512 * 4096) // 4, size=n) * 4).astype(np.uint64)
    out = oracle.build_prp(lut, off, ln, BUS, 1 << 14, pool=True)
    for i in range(n):
        o, size = int(off[i]), int(ln[i])
        npg = (o % 4096 + size + 4095) // 4096
        assert int(out["prp1"][i]) == base + o
        want = [base + (o // 4096) * 4096 + 4096 * k for k in range(1, npg)]
        if npg == 1:
            assert int(out["prp2"][i]) == 0
        elif npg == 2:
            assert int(out["prp2"][i]) == want[0]
        else:
            got, _ = bf.chain_walk(out["pool"], BUS, int(out["prp2"][i]), npg - 1)
            assert got == want


def test_single_list_page_limit():
    rows = _rows("upcie_single_list_limit.txt")
    p = 64
    rng = np.random.default_rng(5)
    lut = _perm_lut(rng, p)
    off = np.array([65536 * 3] * len(rows), np.uint64)        # page aligned
    ln = np.array([int(r[0]) * 4096 for r in rows], np.uint64)
    out = oracle.build_prp(lut, off, ln, BUS, 64, pool=True)
    nxt = 0
    for i, r in enumerate(rows):
        want_pages = int(r[1])
        if want_pages == 0:
            continue
        slot = (int(out["prp2"][i]) - BUS) // 4096
        assert slot == nxt
        _, slots = bf.chain_walk(out["pool"], BUS, int(out["prp2"][i]), int(r[0]) - 1)
        assert len(slots) == want_pages
        nxt += want_pages
    assert out["total"] == nxt


@pytest.mark.parametrize("m", [2, 3, 510, 511, 512, 513, 1021, 1022, 1023, 1024,
                               1533, 1534, 1535, 1536, 2048])
def test_chain_layout_around_page_multiples(m):
    """m list entries (m+1 pages): every non-final list page holds 511 entries
    plus a pointer, the final one at most 512, and pages are consecutive."""
    p = 256
    rng = np.random.default_rng(m)
    lut = _perm_lut(rng, p)
    o = 4096 * 7
    out = oracle.build_prp(lut, np.array([o], np.uint64), np.array([(m + 1) * 4096], np.uint64),
                           BUS, 16, pool=True)
    assert out["status"][0] == 0
    entries, slots = bf.chain_walk(out["pool"], BUS, int(out["prp2"][0]), m)
    _, pages = bf.touched_pages(lut, o, (m + 1) * 4096)
    assert entries == pages[1:]
    assert slots == list(range(len(slots)))
    assert out["total"] == len(slots)
    final = m - 511 * (len(slots) - 1)
    assert 1 <= final <= 512 and (len(slots) == 1 or final >= 2)


def test_prp_status_cases_and_enospc_suffix():
    p = 64
    rng = np.random.default_rng(9)
    lut = _perm_lut(rng, p)
    heap = p * 65536
    top = (1 << 64) - 1
    off = np.array([0, 0, 2, 4, top - 3, heap - 4096, heap - 4092,
                     0, 8, 4096, 12, 16, 0], np.uint64)
    ln = np.array([0, 4096, 4096, 16, 8, 4096, 4096,
                   5 * 4096, 3 * 4096, 600 * 4096, 4096, 9 * 4096, 3 * 4096], np.uint64)
    out = oracle.build_prp(lut, off, ln, BUS, 2, pool=True)
    st = list(out["status"])
    assert st[:7] == [1, 0, 1, 0, 1, 0, 2]
    # lists: idx 7 (1 page, fits slot 0), idx 8 (1 page, slot 1), idx 9 (2 pages
    # -> slots 2,3 > cap 2: ENOSPC), idx 11 and 12 refused too (suffix).
    assert st[7:] == [0, 0, 3, 0, 3, 3]
    assert int(out["prp2"][7]) == BUS and int(out["prp2"][8]) == BUS + 4096
    assert out["total"] == 1 + 1 + 2 + 1 + 1
    for i in (9, 11, 12):
        assert out["prp1"][i] == 0 and out["prp2"][i] == 0
    _check_prp_against_bytewalk(lut, off, ln, out, BUS)


# --------------------------------------------------------------------------
# O3 stable split
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nq,n", [(1, 1000), (16, 5000), (64, 20000), (3, 0), (200, 7000)])
def test_partition_matches_stable_sort(nq, n):
    rng = np.random.default_rng(nq * 7 + n)
    qid = rng.integers(0, nq + 3, size=n).astype(np.uint32)   # some overflow ids
    out = oracle.partition(qid, nq)
    perm, qoff, ninv = bf.stable_split(qid, nq)
    assert np.array_equal(out["perm"], perm)
    assert np.array_equal(out["qoff"], qoff)
    assert out["n_invalid"] == ninv
