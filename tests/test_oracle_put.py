"""Pins of the oracle's put descriptors (O6): the closed-form piece count, a
byte walk on tiny chunks (pieces are the maximal runs of bytes that stay in
one source chunk and one destination chunk), and per-request invariants."""
from __future__ import annotations

import numpy as np
import pytest

import oracle

LB, PB = 0x7000_0000_0000, [0x1_0000_0000_0000, 0x2_0000_0000_0000, 0x3_0000_0000_0000]


def _keys(nchunks, npes, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.integers(1, 1 << 32, nchunks, dtype=np.uint64).astype(np.uint32),
            rng.integers(1, 1 << 32, npes * nchunks, dtype=np.uint64).astype(np.uint32))


def _closed_count(s, d, b, c):
    """1 + source boundaries crossed + destination boundaries crossed - shared."""
    cs = (s + b - 1) // c - s // c
    cd = (d + b - 1) // c - d // c
    common = cs if (s - d) % c == 0 else 0
    return 1 + cs + cd - common


@pytest.mark.parametrize("shift", [4, 6, 12])
def test_byte_walk_on_small_chunks(shift):
    c = 1 << shift
    heap = 64 * c
    rng = np.random.default_rng(shift)
    n = 200
    b = rng.integers(1, 6 * c, n).astype(np.uint64)
    s = (rng.integers(0, heap, n).astype(np.uint64) % (np.uint64(heap) - b))
    d = (rng.integers(0, heap, n).astype(np.uint64) % (np.uint64(heap) - b))
    d[:20] = s[:20]                                          # same phase
    pe = rng.integers(0, 3, n).astype(np.uint32)
    lk, rk = _keys(64, 3, shift)
    o = oracle.build_put(s, d, b, pe, LB, heap, shift, lk, PB, rk, 1 << 20)
    assert (o["status"] == 0).all()
    for i in range(n):
        si, di, bi, p = int(s[i]), int(d[i]), int(b[i]), int(pe[i])
        runs, x = [], 0
        while x < bi:                                        # walk byte by byte
            key = ((si + x) // c, (di + x) // c)
            y = x
            while y < bi and ((si + y) // c, (di + y) // c) == key:
                y += 1
            runs.append((x, y - x, key))
            x = y
        assert int(o["count"][i]) == len(runs) == _closed_count(si, di, bi, c)
        got = o["desc"][int(o["first"][i]): int(o["first"][i]) + len(runs)]
        for (x, ln, (sc, dc)), g in zip(runs, got):
            assert int(g["laddr"]) == LB + si + x and int(g["raddr"]) == PB[p] + di + x
            assert int(g["len"]) == ln and int(g["req"]) == i
            assert int(g["lkey"]) == int(lk[sc]) and int(g["rkey"]) == int(rk[p * 64 + dc])


def test_static_heap_splits_only_at_the_message_limit():
    heap = 1 << 40
    b = np.array([1, 1 << 31, (1 << 31) + 1, 5 * (1 << 31) + 7], np.uint64)
    s = np.array([3, 0, 100, 12345], np.uint64)
    d = np.array([0, 7, 4096, 99], np.uint64)
    pe = np.array([2, 0, 1, 2], np.uint32)
    o = oracle.build_put(s, d, b, pe, LB, heap, 0, [77], PB, [11, 22, 33], 16)
    assert o["count"].tolist() == [1, 1, 2, 6] and o["total"] == 10
    last = o["desc"][4:10]
    assert [int(x) for x in last["len"]] == [1 << 31] * 5 + [7]
    assert (last["lkey"] == 77).all() and (last["rkey"] == 33).all()
    assert int(last["raddr"][5]) == PB[2] + 99 + 5 * (1 << 31)


@pytest.mark.parametrize("seed", range(3))
def test_counts_and_invariants_on_a_large_heap(seed):
    rng = np.random.default_rng(seed)
    shift = 21
    c = 1 << shift
    heap = 1 << 30
    n = 3000
    b = np.exp(rng.uniform(0, np.log(64 * c), n)).astype(np.uint64) + np.uint64(1)
    s = rng.integers(0, heap, n).astype(np.uint64) % (np.uint64(heap) - b)
    d = rng.integers(0, heap, n).astype(np.uint64) % (np.uint64(heap) - b)
    pe = rng.integers(0, 3, n).astype(np.uint32)
    lk, rk = _keys(heap >> shift, 3, seed)
    o = oracle.build_put(s, d, b, pe, LB, heap, shift, lk, PB, rk, 1 << 22)
    want = [_closed_count(int(si), int(di), int(bi), c) for si, di, bi in zip(s, d, b)]
    assert o["count"].tolist() == want
    assert o["first"].tolist() == np.concatenate([[0], np.cumsum(want)[:-1]]).tolist()
    desc = o["desc"][:o["total"]]
    lens = np.bincount(desc["req"].astype(np.int64), weights=desc["len"].astype(np.float64),
                       minlength=n)
    assert np.array_equal(lens.astype(np.uint64), b)
    # within a request: contiguous, and each piece inside one chunk on both sides
    same = desc["req"][1:] == desc["req"][:-1]
    assert (desc["laddr"][1:][same] == desc["laddr"][:-1][same] + desc["len"][:-1][same]).all()
    lo_s = (desc["laddr"] - np.uint64(LB)) >> np.uint64(shift)
    hi_s = (desc["laddr"] - np.uint64(LB) + desc["len"] - np.uint64(1)) >> np.uint64(shift)
    assert (lo_s == hi_s).all()


def test_status_and_enospc_suffix():
    heap = 1 << 20
    s = np.array([0, 0, 0, heap - 8, 0, 100, 0, 0], np.uint64)
    d = np.array([0, 0, 0, 0, heap - 8, 100, 0, 0], np.uint64)
    b = np.array([0, 4096, 4096, 16, 16, 4096 * 3, 8192, 4096], np.uint64)
    pe = np.array([0, 3, 0, 0, 0, 0, 1, 2], np.uint32)
    lk, rk = _keys(heap >> 12, 3)
    o = oracle.build_put(s, d, b, pe, LB, heap, 12, lk, PB, rk, 5)
    assert o["status"].tolist() == [1, 1, 0, 2, 2, 0, 3, 3]
    assert o["count"].tolist() == [0, 0, 1, 0, 0, 4, 2, 1] and o["total"] == 8
    assert o["first"].tolist() == [0, 0, 0, 1, 1, 1, 5, 7]
