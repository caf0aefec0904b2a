"""Pins of the oracle's submission-entry stage (O5) against an NVMe entry
packed field by field with `struct`, and against per-queue rings replayed as
Python deques fed by `numpy.flatnonzero` (no shared code with the oracle's
counting split)."""
from __future__ import annotations

from collections import deque

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

NONE = 0xFFFFFFFF


def _batch(rng, n, nq, lba_shift=9, bad_p=0.1):
    qid = rng.integers(0, nq + 1, n).astype(np.uint32)          # nq = out of range
    blocks = rng.integers(1, 300, n)
    length = (blocks << lba_shift).astype(np.uint64)
    odd = rng.random(n) < bad_p / 2
    length[odd] += np.uint64(4)                                  # not whole blocks
    status = np.where(rng.random(n) < bad_p / 2, 3, 0).astype(np.uint8)
    prp1 = (np.uint64(0x2000_0000_0000) + np.arange(n, dtype=np.uint64) * np.uint64(4096)
            + np.uint64(8))                                      # unique per request
    prp2 = rng.integers(0, 1 << 47, n, dtype=np.uint64)
    slba = rng.integers(0, 1 << 40, n, dtype=np.uint64)
    return dict(qid=qid, length=length, status=status, prp1=prp1, prp2=prp2, slba=slba)


def _split(qid, nq):
    p = oracle.partition(qid, nq)
    return p["perm"], p["qoff"]


def test_entry_layout_matches_struct_packing():
    b = dict(qid=np.zeros(3, np.uint32),
             length=np.array([512, 4096 * 3, 512 * 65536], np.uint64),
             status=np.zeros(3, np.uint8),
             prp1=np.array([0x2000_0000_1008, 0x2000_0001_0000, 0x2000_0002_0000], np.uint64),
             prp2=np.array([0, 0x2000_0003_0000, 0x1000_0000_0000], np.uint64),
             slba=np.array([7, 0xFF_FFFF_FFFF, 0], np.uint64))
    perm, qoff = _split(b["qid"], 1)
    ring = np.full((8, 64), 0xAB, np.uint8)
    rid = np.full((1, 65536), NONE, np.uint32)
    out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                          b["prp2"], [ring], [8], [7], [6], [0], req_of_slot=rid,
                          opcode=0x02, nsid=0x11223344)
    assert rid[0, [6, 7, 0]].tolist() == [0, 1, 2]
    assert (np.delete(rid[0], [6, 7, 0]) == NONE).all()
    assert out["tail"].tolist() == [1] and out["cursor"].tolist() == [3]
    assert out["placed"].tolist() == [3]
    for i, s in enumerate([6, 7, 0]):
        nlb0 = int(b["length"][i]) // 512 - 1
        want = bf.pack_sqe(0x02, s, 0x11223344, int(b["prp1"][i]), int(b["prp2"][i]),
                           int(b["slba"][i]), nlb0)
        assert bytes(ring[s]) == want
    assert (ring[1:6] == 0xAB).all()                   # slots not written stay as they were
    f = bf.unpack_sqe(ring[0])
    assert f["nlb0"] == 65535 and f["cid"] == 0 and f["rest"] == bytes(12)


def _replay(b, nq, rings, depth, free, tail, cursor, lba_shift=9, opcode=2, nsid=1):
    """The expected result of one call, queue by queue, as deques."""
    slot = {}                                             # (queue, slot) -> request
    tail, cursor = list(tail), list(cursor)
    placed = [0] * nq
    for q in range(nq):
        d = int(depth[q])
        if rings[q] is None or d < 2 or d > 65536 or int(tail[q]) >= d:
            continue
        feed = deque(bf.queue_feed(b["qid"], b["status"], b["length"], lba_shift, q))
        for _ in range(int(cursor[q])):
            if feed:
                feed.popleft()
        room = min(int(free[q]), d - 1)
        took = 0
        while feed and took < room:
            i, ok = feed.popleft()
            took += 1
            if not ok:
                continue
            s = (int(tail[q]) + placed[q]) % d
            placed[q] += 1
            slot[(q, s)] = i
            rings[q][s] = np.frombuffer(bf.pack_sqe(
                opcode, s, nsid, int(b["prp1"][i]), int(b["prp2"][i]), int(b["slba"][i]),
                int(b["length"][i]) // (1 << lba_shift) - 1), np.uint8)
        tail[q] = (int(tail[q]) + placed[q]) % d
        cursor[q] = int(cursor[q]) + took
    return slot, tail, cursor, placed


@pytest.mark.parametrize("nq,n,seed", [(1, 50, 1), (3, 400, 2), (8, 3000, 3), (64, 5000, 4)])
def test_one_call_matches_deque_replay(nq, n, seed):
    rng = np.random.default_rng(seed)
    b = _batch(rng, n, nq)
    perm, qoff = _split(b["qid"], nq)
    depth = rng.integers(2, 200, nq).astype(np.uint32)
    depth[0] = 2                                          # one-entry queue
    free = rng.integers(0, 300, nq).astype(np.uint32)     # some above depth - 1
    tail = (rng.integers(0, 1 << 30, nq) % depth).astype(np.uint32)
    cursor = rng.integers(0, 30, nq).astype(np.uint64)
    got_rings = [np.full((int(d), 64), 0x5A, np.uint8) for d in depth]
    want_rings = [r.copy() for r in got_rings]
    if nq > 2:
        got_rings[2] = want_rings[2] = None               # refused queue
    rid = np.full((nq, 65536), NONE, np.uint32)
    out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                          b["prp2"], got_rings, depth, free, tail, cursor, req_of_slot=rid)
    slot, wtail, wcursor, wplaced = _replay(b, nq, want_rings, depth, free, tail, cursor)
    want_rid = np.full((nq, 65536), NONE, np.uint32)
    for (q, s), i in slot.items():
        want_rid[q, s] = i
    np.testing.assert_array_equal(rid, want_rid)
    assert out["tail"].tolist() == wtail
    assert out["cursor"].tolist() == wcursor
    assert out["placed"].tolist() == wplaced
    for g, w in zip(got_rings, want_rings):
        if w is not None:
            np.testing.assert_array_equal(g, w)


@pytest.mark.parametrize("lba_shift", [9, 12])
def test_refused_queues_and_block_limits(lba_shift):
    blk = 1 << lba_shift
    n = 6
    b = dict(qid=np.array([0, 1, 2, 3, 4, 4], np.uint32),
             length=np.array([blk, blk, blk, blk, blk * 65537, blk * 65536], np.uint64),
             status=np.zeros(n, np.uint8), prp1=np.arange(n, dtype=np.uint64) + np.uint64(1),
             prp2=np.zeros(n, np.uint64), slba=np.zeros(n, np.uint64))
    perm, qoff = _split(b["qid"], 5)
    depth = np.array([1, 65537, 4, 4, 65536], np.uint32)
    tail = np.array([0, 0, 4, 3, 65535], np.uint32)       # queue 2: tail == depth
    rings = [np.zeros((max(int(d), 1), 64), np.uint8) for d in depth]
    rid = np.full((5, 65536), NONE, np.uint32)
    out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                          b["prp2"], rings, depth, [9] * 5, tail, [0] * 5, req_of_slot=rid,
                          lba_shift=lba_shift)
    assert out["placed"].tolist() == [0, 0, 0, 1, 1]
    assert out["cursor"].tolist() == [0, 0, 0, 1, 2]
    assert out["tail"].tolist() == [0, 0, 4, 0, 0]
    assert (rid[:3] == NONE).all()
    assert rid[3, 3] == 3 and rid[4, 65535] == 5
    assert (rid != NONE).sum() == 2
    assert bf.unpack_sqe(rings[4][65535])["nlb0"] == 65535


def test_drain_places_every_expressible_request_once_in_order():
    rng = np.random.default_rng(9)
    nq, n = 5, 4000
    b = _batch(rng, n, nq, bad_p=0.2)
    perm, qoff = _split(b["qid"], nq)
    depth = np.array([16, 2, 33, 100, 7], np.uint32)
    tail = np.array([3, 1, 32, 0, 6], np.uint32)
    cursor = np.zeros(nq, np.uint64)
    rings = [np.zeros((int(d), 64), np.uint8) for d in depth]
    seen = [[] for _ in range(nq)]
    rid = np.full((nq, 65536), NONE, np.uint32)
    for _ in range(2000):
        prev_tail = tail.copy()
        # The controller has fetched everything: the whole ring is free.
        out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                              b["prp2"], rings, depth, depth - 1, tail, cursor,
                              req_of_slot=rid)
        for q in range(nq):
            assert out["placed"][q] <= depth[q] - 1
            for k in range(int(out["placed"][q])):
                s = (int(prev_tail[q]) + k) % int(depth[q])
                f = bf.unpack_sqe(rings[q][s])
                assert f["cid"] == s
                i = int(rid[q, s])
                assert f["prp1"] == int(b["prp1"][i])
                seen[q].append((i, f["slba"], f["nlb0"]))
        tail, cursor = out["tail"], out["cursor"]
        if (cursor == np.diff(qoff)[:nq]).all():
            break
    for q in range(nq):
        feed = bf.queue_feed(b["qid"], b["status"], b["length"], 9, q)
        want = [(i, int(b["slba"][i]), int(b["length"][i]) // 512 - 1) for i, ok in feed if ok]
        assert seen[q] == want


def test_empty_batch_and_zero_free():
    b = _batch(np.random.default_rng(1), 0, 2)
    perm, qoff = _split(b["qid"], 2)
    rings = [np.zeros((4, 64), np.uint8)] * 2
    out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                          b["prp2"], rings, [4, 4], [3, 3], [1, 2], [0, 0])
    assert out["placed"].tolist() == [0, 0] and out["tail"].tolist() == [1, 2]
    b = _batch(np.random.default_rng(2), 10, 1, bad_p=0)
    perm, qoff = _split(b["qid"], 1)
    out = oracle.emit_sqe(perm, qoff, b["status"], b["length"], b["slba"], b["prp1"],
                          b["prp2"], [np.zeros((4, 64), np.uint8)], [4], [0], [1], [0])
    assert out["placed"].tolist() == [0] and out["cursor"].tolist() == [0]
