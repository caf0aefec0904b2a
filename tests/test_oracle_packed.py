"""Pins of the oracle's packed-list PRP build (O2p): every list, followed as an
NVMe controller follows it (from PRP2 with its in-page offset), yields the
4 KiB pages the request's bytes touch; the lists of different requests use
disjoint words and pack the pool densely; and hand-built layouts around page
ends hold the words the NVMe chaining rule asks for."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

BUS = 0x1000_0000_0000
CANARY = np.uint64(0xDEAD_BEEF_DEAD_BEEF)


def _perm_lut(rng, p):
    return (np.uint64(0x2000_0000_0000) + rng.permutation(p).astype(np.uint64) * np.uint64(65536))


def _walk_words(pool, prp2, count):
    """Words (page, index) an NVMe controller reads for a list of `count`
    entries from prp2: data entries and chain pointers."""
    rel = prp2 - BUS
    page, pos = rel // 4096, (rel % 4096) // 8
    words, got = [], 0
    while got < count:
        if pos == 511 and count - got > 1:
            words.append((page, 511))
            page, pos = (int(pool[page, 511]) - BUS) // 4096, 0
            continue
        words.append((page, pos))
        got += 1
        pos += 1
    return words


def _aligned_pages(lut, off, size):
    """Pages of a request that starts on a 4 KiB boundary: one per 4 KiB step
    (closed form; the byte walk is too slow for the larger layouts)."""
    assert off % 4096 == 0
    return int(bf.phys_bytes(lut, np.array([off]))[0]), [
        int(bf.phys_bytes(lut, np.array([off + 4096 * k]))[0]) for k in range(-(-size // 4096))]


def _check_layout(lut, off, ln, pool_pages=1 << 20, pages_of=bf.touched_pages):
    o = oracle.build_prp_packed(lut, off, ln, BUS, pool_pages)
    pages_needed = o["total"]
    pool = np.full((max(min(pages_needed, pool_pages), 1), 512), CANARY, np.uint64)
    o = oracle.build_prp_packed(lut, off, ln, BUS, min(pages_needed, pool_pages), pool=pool)
    ref = oracle.build_prp(lut, off, ln, BUS, 1 << 40)            # page layout, pinned on its own
    owner = {}
    m_total = 0
    for i in range(off.size):
        size = int(ln[i])
        st = int(o["status"][i])
        if st in (1, 2):
            assert st == int(ref["status"][i])
            continue
        first, pages = pages_of(lut, int(off[i]), size)
        m = len(pages) - 1
        if m >= 2:
            m_total += m
        if st == 3:
            assert int(o["prp1"][i]) == 0 and int(o["prp2"][i]) == 0
            continue
        assert st == 0 and int(o["prp1"][i]) == first
        if len(pages) == 1:
            assert int(o["prp2"][i]) == 0
        elif len(pages) == 2:
            assert int(o["prp2"][i]) == pages[1]
        else:
            ent, _ = bf.chain_walk(pool, BUS, int(o["prp2"][i]), m, allow_offset=True)
            assert ent == pages[1:], f"request {i}"
            for w in _walk_words(pool, int(o["prp2"][i]), m):
                assert w not in owner, f"word {w} used by requests {owner[w]} and {i}"
                owner[w] = i
    assert pages_needed == -(-m_total // 511)
    return o, pool, owner


@pytest.mark.parametrize("seed", range(4))
def test_chain_walks_match_byte_walk(seed):
    rng = np.random.default_rng(seed)
    p = 64
    lut = _perm_lut(rng, p)
    heap = p * 65536
    n = 120
    ln = rng.choice([1, 100, 4096, 8192, 12288, 4096 * 40, 4096 * 510, 4096 * 511,
                     4096 * 512, 4096 * 513, 4096 * 1022, 4096 * 1023], n).astype(np.uint64)
    ln = ln + rng.integers(0, 3, n).astype(np.uint64) * np.uint64(4)
    off = (rng.integers(0, heap // 4, n).astype(np.uint64) * np.uint64(4))
    off = np.minimum(off, np.uint64(heap) - ln)
    off -= off % np.uint64(4)
    ln[:3] = [0, 5, heap]                               # EINVAL, EINVAL (off % 4 == 1 below)
    off[1] = 1
    _check_layout(lut, off, ln)


def test_layout_is_dense_and_zero_filled():
    rng = np.random.default_rng(11)
    m = rng.integers(2, 1500, 400)
    m[::7] = 510                                           # many lists end near page ends
    off = np.cumsum(np.concatenate([[0], (m[:-1] + 1) * 4096])).astype(np.uint64)
    ln = ((m + 1) * 4096).astype(np.uint64)
    lut = _perm_lut(rng, int(off[-1] + ln[-1]) // 65536 + 1)
    o, pool, owner = _check_layout(lut, off, ln, pages_of=_aligned_pages)
    assert (o["status"] == 0).all()
    # Every word below the end of the last list is a list word, or one of the
    # zero words the layout leaves (word 511 of a page whose last list ended in
    # word 510, word 0 of a page whose last entry moved up into word 511).
    end = int(m.sum())
    last_word = end + end // 511                         # word just past the last slot
    used = np.zeros(pool.size, bool)
    for (pg, w) in owner:
        used[pg * 512 + w] = True
    flat = pool.reshape(-1)
    rest = np.flatnonzero(~used[:last_word])
    assert (flat[rest] == 0).all()
    assert (flat[last_word + 1:] == CANARY).all() or last_word + 1 >= flat.size


def _hand(ms, pool_pages=16):
    lut = np.arange(256, dtype=np.uint64) * np.uint64(65536) + np.uint64(0x2000_0000_0000)
    ms = np.asarray(ms)
    off = np.cumsum(np.concatenate([[0], (ms[:-1] + 1) * 4096])).astype(np.uint64)
    ln = ((ms + 1) * 4096).astype(np.uint64)
    pool = np.full((pool_pages, 512), CANARY, np.uint64)
    o = oracle.build_prp_packed(lut, off, ln, BUS, pool_pages, pool=pool)
    return o, pool, off


def _phys(x):
    return 0x2000_0000_0000 + int(x)


def test_list_ending_in_word_510_leaves_511_zero():
    o, pool, off = _hand([509, 2])
    assert int(o["prp2"][1]) == BUS + 8 * 509
    assert int(pool[0, 509]) == _phys(off[1] + 4096) and int(pool[0, 510]) == _phys(off[1] + 8192)
    assert int(pool[0, 511]) == 0 and pool[1, 0] == CANARY


def test_single_remaining_entry_takes_word_511():
    o, pool, off = _hand([510, 2, 3])
    assert int(o["prp2"][1]) == BUS + 8 * 510
    assert int(pool[0, 511]) == _phys(off[1] + 8192)      # data, not a pointer
    assert int(pool[1, 0]) == 0                          # the slot it vacated
    assert int(o["prp2"][2]) == BUS + 4096 + 8           # next list: page 1, word 1
    assert o["total"] == 2


def test_two_remaining_entries_chain():
    o, pool, off = _hand([510, 3])
    assert int(pool[0, 511]) == BUS + 4096               # pointer to page 1
    assert int(pool[1, 0]) == _phys(off[1] + 8192) and int(pool[1, 1]) == _phys(off[1] + 12288)


@pytest.mark.parametrize("m,words", [(511, 511), (512, 512), (513, 514), (1022, 1023),
                                     (1023, 1024)])
def test_lists_from_a_page_start(m, words):
    o, pool, off = _hand([m])
    assert int(o["prp2"][0]) == BUS
    ent, slots = bf.chain_walk(pool, BUS, int(o["prp2"][0]), m, allow_offset=True)
    assert ent == [_phys(off[0] + 4096 * (k + 1)) for k in range(m)]
    assert len(_walk_words(pool, int(o["prp2"][0]), m)) == words


def test_enospc_is_a_suffix_and_total_counts_all():
    o, pool, off = _hand([300, 300, 300, 300], pool_pages=2)
    assert o["status"].tolist() == [0, 0, 0, 3]          # 900 slots fit in 1022, 1200 do not
    assert o["total"] == 3
    assert (pool[1, 900 - 511 + 1:] == CANARY).all()     # nothing past the last fitting list
