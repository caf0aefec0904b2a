"""GPU parity of dmadesc_cq_mirror with the oracle's O7 drain: every mirrored
queue's copy (whole mirror compared, canary-filled on both sides), head,
phase, count and acknowledgement, bit for bit -- on queues filled before the
launch, over repeated calls, on detached and unusable slots, and with a
producer writing completions on another stream while the mirror runs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import oracle
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

DST_FILL = 0xA5A5A5A5


def state_at(depth, g):
    """Head and expected phase once g completions have been consumed."""
    return g % depth, 1 - (g // depth) % 2


def completions(depth, lo, hi, rng):
    """Positions and entries of completions lo..hi-1 as the controller writes
    them: random dwords, phase tag (dword 3 bit 16) 1 on even passes."""
    g = np.arange(lo, hi, dtype=np.int64)
    e = rng.integers(0, 1 << 32, (g.size, 4), dtype=np.uint64).astype(np.uint32)
    phase = (1 - (g // depth) % 2).astype(np.uint32)
    e[:, 3] = (e[:, 3] & np.uint32(0xFFFEFFFF)) | (phase << np.uint32(16))
    return (g % depth).astype(np.int64), e


class Queue:
    """One device-memory completion queue, its mirror and the host's copy of
    both."""

    def __init__(self, depth, g0, rng, garbage=False):
        self.depth, self.g = depth, g0
        self.src = np.zeros((max(depth, 1), 4), np.uint32)
        if garbage:
            self.src[:] = rng.integers(0, 1 << 32, self.src.shape, dtype=np.uint64)
        else:
            pos, e = completions(depth, max(0, g0 - depth), g0, rng)
            self.src[pos] = e
        self.dst = np.full_like(self.src, DST_FILL)
        self.head, self.phase = state_at(depth, g0) if depth else (0, 1)
        self.copied, self.ack = 0, 0
        self.d_src = gc.dev(self.src.view(np.int32))
        self.d_dst = gc.dev(self.dst.view(np.int32))

    def produce(self, count, rng):
        """count more completions (host and device copies of the queue)."""
        pos, e = completions(self.depth, self.g, self.g + count, rng)
        self.src[pos] = e
        self.g += count
        self.d_src.copy_(gc.dev(self.src.view(np.int32)))

    def oracle_drain(self, gen=1):
        c, self.head, self.phase, self.ack = oracle.cq_drain(self.src, self.dst, gen, self.head,
                                                             self.phase, self.ack)
        self.copied += c


def attach(slots, q, queue, gen=1):
    dd.cq_attach(slots, q, queue.d_src, queue.d_dst, queue.depth, gen, queue.head, queue.phase)


def run_mirror(slots, mode, idle=1):
    stop = torch.ones(1, dtype=torch.int32, device="cuda").view(torch.uint32)
    if mode == "idle":
        stop.zero_()
    dd.cq_mirror(slots, stop, idle_polls=idle if mode == "idle" else 1 << 16)
    torch.cuda.synchronize()


def check(slots, queues, ctx, gens=None):
    st = dd.cq_slot_state(slots)
    for q, v in enumerate(queues):
        where = f"{ctx} slot {q} depth {v.depth}"
        assert st["head"][q] == v.head, (where, st["head"][q], v.head)
        assert st["phase"][q] == v.phase, (where, st["phase"][q], v.phase)
        assert st["copied"][q] == v.copied, (where, st["copied"][q], v.copied)
        assert st["ack"][q] == v.ack, (where, st["ack"][q], v.ack)
        if gens is not None:
            assert st["generation"][q] == gens[q], where
        got = gc.host(v.d_dst).view(np.uint32)
        if not np.array_equal(got, v.dst):
            bad = np.nonzero((got != v.dst).any(axis=1))[0]
            raise AssertionError(f"{where}: {bad.size} mirror entries differ, first at "
                                 f"{bad[0]}: oracle {v.dst[bad[0]]} gpu {got[bad[0]]}")


# (depth, completions consumed before, completions waiting)
PREFILLED = [(2, 0, 0), (2, 0, 2), (2, 1, 1), (3, 5, 3), (64, 0, 64), (64, 10, 64),
             (65, 0, 65), (65, 60, 10), (100, 150, 99), (1024, 1000, 50), (4097, 3, 4097),
             (65536, 65000, 65536), (65536, 0, 1), (128, 7, 0),
             # runs ending in each 64-entry part of a 256-entry poll, and on its edges
             (300, 0, 130), (256, 0, 256), (257, 250, 257), (1000, 0, 192), (1000, 0, 64),
             (1000, 0, 128), (1000, 900, 255), (512, 100, 511)]


@pytest.mark.parametrize("mode", ["stop", "idle"])
def test_prefilled_queues_match_oracle(mode):
    rng = np.random.default_rng(11)
    queues = []
    for depth, g0, count in PREFILLED:
        v = Queue(depth, g0, rng)
        v.produce(count, rng)
        queues.append(v)
    garbage = Queue(777, 0, rng, garbage=True)      # random phase bits everywhere
    garbage.head, garbage.phase = 500, 1
    queues.append(garbage)
    slots = dd.cq_slots(len(queues))
    for q, v in enumerate(queues):
        attach(slots, q, v)
    gc.say(f"cq_mirror prefilled {mode}: {len(queues)} slots")
    run_mirror(slots, mode)
    for v in queues:
        v.oracle_drain()
    check(slots, queues, f"prefilled {mode}", gens=[1] * len(queues))


def test_repeated_calls_continue():
    rng = np.random.default_rng(12)
    depths = [2, 5, 64, 65, 300, 4096, 65536]
    queues = [Queue(d, int(rng.integers(0, 3 * d)), rng) for d in depths]
    slots = dd.cq_slots(len(queues))
    for q, v in enumerate(queues):
        attach(slots, q, v)
    for call in range(6):
        for v in queues:                  # at most a queue's worth between calls
            v.produce(int(rng.integers(0, v.depth + 1)), rng)
        gc.say(f"cq_mirror repeated call {call}")
        run_mirror(slots, "stop" if call % 2 else "idle", idle=3)
        for v in queues:
            v.oracle_drain()
        check(slots, queues, f"call {call}")


def test_reattach_serves_the_new_queue():
    rng = np.random.default_rng(13)
    a, b = Queue(256, 0, rng), Queue(1000, 0, rng)
    a.produce(200, rng)
    b.produce(900, rng)
    slots = dd.cq_slots(1)
    attach(slots, 0, a, gen=1)
    run_mirror(slots, "stop")
    a.oracle_drain()
    check(slots, [a], "first attachment")
    attach(slots, 0, b, gen=3)             # fresh count and position for the new queue
    a.produce(50, rng)                     # the old queue is no longer mirrored
    gc.say("cq_mirror re-attached")
    run_mirror(slots, "idle", idle=2)
    b.oracle_drain()
    check(slots, [b], "second attachment", gens=[3])
    assert np.array_equal(gc.host(a.d_dst).view(np.uint32)[:200], a.src[:200])
    assert (gc.host(a.d_dst).view(np.uint32)[200:250] == DST_FILL).all()


def test_even_generation_is_acknowledged():
    rng = np.random.default_rng(14)
    queues = [Queue(64, 0, rng) for _ in range(4)]
    for v in queues:
        v.produce(40, rng)
    slots = dd.cq_slots(4)
    gens = [0, 2, 5, 8]
    for q, v in enumerate(queues):
        attach(slots, q, v, gen=1)
        slots.view(torch.int64)[q, 2:3].fill_(64 | (gens[q] << 32))
    gc.say("cq_mirror even generations")
    run_mirror(slots, "stop")
    for q, v in enumerate(queues):
        v.oracle_drain(gen=gens[q])
    assert [v.ack for v in queues] == [0xFFFFFFFF, 1, 0, 7]
    check(slots, queues, "even generations", gens=gens)


def test_unusable_slots_copy_nothing():
    rng = np.random.default_rng(15)
    good = Queue(128, 0, rng)
    good.produce(100, rng)
    bad = [Queue(128, 0, rng) for _ in range(5)]
    for v in bad:
        v.produce(100, rng)
    slots = dd.cq_slots(6)
    attach(slots, 0, good)
    for q, v in enumerate(bad, start=1):
        attach(slots, q, v)
    w = slots.view(torch.int64)
    w[1, 2:3].fill_(1 | (1 << 32))                     # depth 1
    w[2, 2:3].fill_(65537 | (1 << 32))                 # depth above the maximum
    w[3, 3:4].fill_(128 << 32)                         # head == depth
    w[4, 0:1].fill_(bad[3].d_src.data_ptr() + 8)       # src not 16-byte aligned
    w[5, 1:2].fill_(0)                                 # no mirror
    gc.say("cq_mirror unusable slots")
    run_mirror(slots, "idle", idle=4)
    good.oracle_drain()
    st = dd.cq_slot_state(slots)
    check(slots[:1], [good], "usable slot beside unusable ones")
    assert (st["copied"][1:] == 0).all() and (st["ack"][1:] == 0).all()
    for v in bad:
        assert (gc.host(v.d_dst).view(np.uint32) == DST_FILL).all()


def _runs_concurrently(mirror, producer):
    """True when a mirror call on `mirror` sees a stop flag set on `producer`
    while it runs: its launch then lasts well under the ~0.2 s that 2^20 idle
    polls take. Two streams can share one hardware queue, and work on a shared
    queue runs one launch after the other."""
    slots = dd.cq_slots(1)                          # generation 0: nothing to copy
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mirror.wait_stream(torch.cuda.current_stream())
    producer.wait_stream(torch.cuda.current_stream())
    e0.record(mirror)
    dd.cq_mirror(slots, stop.view(torch.uint32), idle_polls=1 << 20, stream=mirror)
    e1.record(mirror)
    with torch.cuda.stream(producer):
        stop.fill_(1)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    gc.say(f"stream pair probe: mirror call {ms:.2f} ms")
    return ms < 20.0


@pytest.fixture(scope="module")
def stream_pair():
    """(mirror stream, producer stream, concurrent): a pair shown to run at
    the same time if one of 8 tries finds one. Where streams share hardware
    queues and none does, the tests still hold: the mirror call then ends idle
    before the producer runs, and the follow-up call after the stop flag (one
    more drain) does the copying. Either way every completion must be
    mirrored exactly once."""
    pair = None
    for _ in range(8):
        pair = torch.cuda.Stream(), torch.cuda.Stream()
        if _runs_concurrently(*pair):
            return (*pair, True)
    gc.say("no pair of streams ran concurrently: the calls run one after the other")
    return (*pair, False)


def _follow_up(slots, stop, concurrent):
    """One more mirror call after the stop flag: it drains once and leaves.
    After a concurrent run it must find nothing left to copy."""
    before = dd.cq_slot_state(slots)["copied"].copy()
    dd.cq_mirror(slots, stop.view(torch.uint32), idle_polls=1 << 10)
    torch.cuda.synchronize()
    after = dd.cq_slot_state(slots)["copied"]
    if concurrent:
        assert np.array_equal(before, after), (before, after)


def test_concurrent_producer_then_stop(stream_pair):
    """Completions arrive on another stream while the mirror runs (entry data
    in one launch, then dword 3 in the next, as a controller makes an entry
    valid only with its phase); the stop flag is set last. Every completion
    is mirrored exactly once, in order."""
    rng = np.random.default_rng(16)
    depths = [64, 65, 256, 1000, 4096, 4096, 65536, 3]
    queues = [Queue(d, int(rng.integers(0, 2 * d)), rng) for d in depths]
    slots = dd.cq_slots(len(queues))
    for q, v in enumerate(queues):
        attach(slots, q, v)
    # Every batch, prepared before the launch: (queue, positions, data, dword 3).
    batches = []
    for q, v in enumerate(queues):
        left = v.depth                     # a queue's worth, crossing the wrap
        while left:
            c = int(min(left, rng.integers(1, max(2, v.depth // 8) + 1)))
            pos, e = completions(v.depth, v.g, v.g + c, rng)
            v.src[pos] = e
            v.g += c
            left -= c
            batches.append((q, gc.dev(pos), gc.dev(e[:, :3].view(np.int32)),
                            gc.dev(e[:, 3].view(np.int32))))
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    mirror, producer, concurrent = stream_pair
    mirror.wait_stream(torch.cuda.current_stream())
    producer.wait_stream(torch.cuda.current_stream())
    gc.say(f"cq_mirror concurrent={concurrent}: {len(queues)} slots, {len(batches)} batches")
    dd.cq_mirror(slots, stop.view(torch.uint32), idle_polls=1 << 18, stream=mirror)
    with torch.cuda.stream(producer):
        # Each queue's batches in order, the queues taken round-robin.
        per_q = [[b for b in batches if b[0] == q] for q in range(len(queues))]
        while any(per_q):
            for q in range(len(queues)):
                if per_q[q]:
                    _, pos, data, dw3 = per_q[q].pop(0)
                    src = queues[q].d_src.view(-1, 4)
                    src[pos, 0:3] = data
                    src[pos, 3] = dw3
        stop.fill_(1)
    torch.cuda.synchronize()
    _follow_up(slots, stop, concurrent)
    for v in queues:
        v.oracle_drain()
        assert v.copied == v.depth
    check(slots, queues, "concurrent")


def test_detach_while_running(stream_pair):
    """The host detaches a queue (even generation) while completions keep
    arriving: the mirror acknowledges, stops copying it and keeps a valid
    prefix; a queue beside it is mirrored in full."""
    rng = np.random.default_rng(17)
    a, b = Queue(512, 100, rng), Queue(512, 0, rng)
    slots = dd.cq_slots(2)
    attach(slots, 0, a)
    attach(slots, 1, b)
    start_head, start_phase = a.head, a.phase
    plan = []
    for v in (a, b):
        pos, e = completions(v.depth, v.g, v.g + 400, rng)
        v.src[pos] = e
        v.g += 400
        plan.append((gc.dev(pos), gc.dev(e[:, :3].view(np.int32)),
                     gc.dev(e[:, 3].view(np.int32))))
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    mirror, producer, concurrent = stream_pair
    mirror.wait_stream(torch.cuda.current_stream())
    producer.wait_stream(torch.cuda.current_stream())
    gc.say(f"cq_mirror detach while running, concurrent={concurrent}")
    dd.cq_mirror(slots, stop.view(torch.uint32), idle_polls=1 << 18, stream=mirror)
    with torch.cuda.stream(producer):
        for i, (v, (pos, data, dw3)) in enumerate(zip((a, b), plan)):
            src = v.d_src.view(-1, 4)
            for lo in range(0, 400, 100):
                if i == 0 and lo == 200:
                    slots.view(torch.int64)[0, 2:3].fill_(512 | (2 << 32))
                src[pos[lo:lo + 100], 0:3] = data[lo:lo + 100]
                src[pos[lo:lo + 100], 3] = dw3[lo:lo + 100]
        stop.fill_(1)
    torch.cuda.synchronize()
    _follow_up(slots, stop, concurrent)
    st = dd.cq_slot_state(slots)
    assert st["ack"][0] == 1 and st["generation"][0] == 2, {k: list(v) for k, v in st.items()}
    c = int(st["copied"][0])
    assert 0 <= c <= 400
    # The oracle's drain of the whole queue, cut to the first c entries.
    full = a.dst.copy()
    oracle.cq_drain(a.src, full, 1, start_head, start_phase, 0)
    got = gc.host(a.d_dst).view(np.uint32)
    taken = (start_head + np.arange(c)) % a.depth
    assert np.array_equal(got[taken], full[taken])
    rest = np.setdiff1d(np.arange(a.depth), taken)
    assert (got[rest] == DST_FILL).all()
    h, p = state_at(a.depth, 100 + c)
    assert st["head"][0] == h and st["phase"][0] == p
    b.oracle_drain()
    check(slots[1:], [b], "queue beside the detached one")
