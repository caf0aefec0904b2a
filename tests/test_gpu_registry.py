"""GPU parity of the device registration cache (dmadesc_reg_register /
dmadesc_reg_deregister) with the oracle's O4b: every handle, kind and status,
the needed capacity, and the whole record table (start, end, handle,
references, in start order; storage in handle order) after every batch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import oracle
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

M = 1 << 20


def _compare_tables(dev_reg, ref, ctx):
    (s, e, h, r), storage = dev_reg.records()
    ws, we, wh, wr = ref.records()
    for name, got, want in (("start", s, ws), ("end", e, we), ("handle", h, wh), ("refs", r, wr)):
        if not np.array_equal(np.asarray(got, np.int64), np.asarray(want, np.int64)):
            raise AssertionError(f"{ctx}: table column {name} differs "
                                 f"({len(got)} vs {len(want)} records)")
    assert (np.diff(storage.astype(np.int64)) > 0).all(), f"{ctx}: storage not in handle order"
    assert dev_reg.next_id() == ref.next_id(), ctx


class Pair:
    """The device registry and the oracle registry, driven together."""

    def __init__(self, page_shift=12, capacity=0):
        self.dev = dd.DeviceRegistry(capacity, page_shift)
        self.ref = oracle.Registry(page_shift)
        self.cap = capacity

    def register(self, addr, size, ctx, grow=True):
        gc.say(f"registry register {ctx}: n={len(addr)} cap={self.dev.capacity}")
        out = self.dev.register(gc.dev(np.asarray(addr, np.uint64)),
                                gc.dev(np.asarray(size, np.uint64)), grow=grow)
        torch.cuda.synchronize()
        h, k, need = self.ref.register_batch(addr, size, self.dev.capacity if grow else self.cap)
        if grow:
            # The device call grew the table as often as the oracle's rule says;
            # replay the oracle against the final capacity.
            assert need <= self.dev.capacity
        np.testing.assert_array_equal(gc.host(out["kind"]), k, err_msg=f"{ctx} kind")
        np.testing.assert_array_equal(gc.host(out["handle"]), h, err_msg=f"{ctx} handle")
        assert out["needed"] == need or grow, (ctx, out["needed"], need)
        _compare_tables(self.dev, self.ref, ctx)
        return h, k

    def deregister(self, handles, ctx):
        gc.say(f"registry deregister {ctx}: n={len(handles)}")
        st = self.dev.deregister(gc.dev(np.asarray(handles, np.uint64)))
        torch.cuda.synchronize()
        want = self.ref.deregister_batch(handles)
        np.testing.assert_array_equal(gc.host(st), want, err_msg=f"{ctx} status")
        _compare_tables(self.dev, self.ref, ctx)


def test_register_experiment_as_batches():
    base = 0x7f00_0000_0000
    p = Pair()
    h, _ = p.register([base, base, base + 0x1000, base + 4 * M], [2 * M, 2 * M, M, 2 * M],
                      "experiment")
    assert p.dev.capacity == 32
    p.deregister([h[0]] * 4, "experiment deregister")
    p.deregister([h[0], 0, h[3], h[3]], "stale and repeated")
    assert p.dev.count() == 0


def test_capacity_grows_0_32_64_128_256():
    p = Pair()
    caps = []
    for i in range(0, 160, 20):
        p.register(np.arange(i, i + 20, dtype=np.uint64) * np.uint64(8 * M),
                   np.full(20, M, np.uint64), f"grow {i}")
        caps.append(p.dev.capacity)
    assert caps == [32, 64, 64, 128, 128, 128, 256, 256]


def test_refused_batch_changes_nothing():
    p = Pair(capacity=4)
    p.register([0, 16 * M], [M, M], "fill")
    p.cap = 4
    out = p.dev.register(gc.dev(np.array([32 * M, 48 * M, 64 * M], np.uint64)),
                         gc.dev(np.full(3, M, np.uint64)), grow=False)
    torch.cuda.synchronize()
    h, k, need = p.ref.register_batch([32 * M, 48 * M, 64 * M], [M, M, M], 4)
    assert out["needed"] == need == 8
    np.testing.assert_array_equal(gc.host(out["kind"]), k)
    assert (k == oracle.REG_NOSPACE).all() and (gc.host(out["handle"]) == 0).all()
    _compare_tables(p.dev, p.ref, "refused")


@pytest.mark.parametrize("page_shift", [12, 16])
def test_invalid_and_rounding(page_shift):
    p = Pair(page_shift)
    top = (1 << 64) - 1
    p.register([0, 5, 4095, top - 100, top - (1 << page_shift) + 1, 1 << 40, (1 << 40) + 1],
               [0, 1, 2, 50, 1, 1 << page_shift, 3], f"edges shift={page_shift}")


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(seed)
    p = Pair()
    live = []
    for rnd in range(30):
        n = int(rng.choice([1, 7, 255, 256, 257, 1000, 3000]))
        if rng.random() < 0.6 or not live:
            starts = rng.integers(0, 512, n).astype(np.uint64) * np.uint64(64 * 1024) + \
                rng.integers(0, 4096, n).astype(np.uint64)
            sizes = rng.choice([0, 1, 4096, 100_000, M, 3 * M, 9 * M], n).astype(np.uint64)
            if rnd % 5 == 0:                            # repeats of earlier items
                starts[n // 2:] = starts[:n - n // 2]
                sizes[n // 2:] = sizes[:n - n // 2]
            h, k = p.register(starts, sizes, f"seed {seed} round {rnd}")
        else:
            hs = rng.choice(live + [0, 10 ** 9], n).astype(np.uint64)
            p.deregister(hs, f"seed {seed} round {rnd}")
        (_, _, hh, _), _ = p.dev.records()
        live = [int(x) for x in hh]


def test_full_batch_on_a_large_table():
    rng = np.random.default_rng(42)
    p = Pair(capacity=2048)
    # 1024 disjoint regions, then one full batch: repeats, contained ranges,
    # nested new ranges and invalid ones.
    base = np.arange(1024, dtype=np.uint64) * np.uint64(64 * M)
    p.register(base, np.full(1024, 32 * M, np.uint64), "table")
    n = dd.REG_MAX_BATCH
    pick = rng.integers(0, 1024, n)
    kind = rng.integers(0, 4, n)
    starts = base[pick] + np.where(kind == 1, rng.integers(0, 16 * M, n), 0).astype(np.uint64)
    starts = np.where(kind >= 2, base[pick] + np.uint64(40 * M) +
                      rng.integers(0, 8, n).astype(np.uint64) * np.uint64(M), starts)
    sizes = np.where(kind == 0, 32 * M, np.where(kind == 1, M, (8 - (starts - base[pick] - np.uint64(40 * M)) // np.uint64(M)) * np.uint64(M)))
    sizes = np.where(kind >= 2, np.maximum(sizes.astype(np.int64), 1), sizes).astype(np.uint64)
    sizes[rng.random(n) < 0.01] = 0
    h, k = p.register(starts, sizes, "full batch")
    assert (k == oracle.REG_HIT_NEW).sum() > 1000 and (k == oracle.REG_NEW).sum() > 1000
    p.deregister(rng.choice(h[h > 0], n), "full deregister")


def _pages(x):
    return np.asarray(x, np.uint64) * np.uint64(4096)


def test_crowded_buckets_long_ranges_and_a_wide_span():
    # The batch relations go through a bucketed index of the batch's ranges:
    # a bucket holds a few ranges inline and sends the rest, and ranges longer
    # than a bucket, to a list every query walks. These batches crowd one
    # bucket far past its inline slots (identical and nested small ranges),
    # mix in ranges longer than a bucket, repeats and hits, and then spread
    # starts over the whole 64-bit space.
    rng = np.random.default_rng(7)
    p = Pair()
    table = _pages(np.arange(64, dtype=np.uint64) << np.uint64(22))      # 64 regions, 16 GiB apart
    p.register(table, np.full(64, 4 * M, np.uint64), "table")
    n = 20_000
    hot = np.uint64(0x50_0000_0000)
    k = rng.integers(0, 10, n)
    starts = np.zeros(n, np.uint64)
    sizes = np.zeros(n, np.uint64)
    crowd = k < 3                                   # the same few pages
    starts[crowd] = hot + _pages(rng.integers(0, 4, crowd.sum()))
    sizes[crowd] = 4096
    nest = (k >= 3) & (k < 5)                       # ranges around the crowd
    m = int(nest.sum())
    starts[nest] = hot - _pages(rng.integers(0, 8, m))
    sizes[nest] = _pages(rng.integers(1, 24, m))
    long_ = k == 5                                  # longer than a bucket
    m = int(long_.sum())
    starts[long_] = _pages(rng.integers(1 << 29, 1 << 30, m))
    sizes[long_] = _pages(rng.integers(1 << 17, 1 << 21, m))
    short = k == 6
    m = int(short.sum())
    starts[short] = _pages(rng.integers(1 << 28, 1 << 29, m)) + rng.integers(0, 4096, m).astype(np.uint64)
    sizes[short] = rng.integers(1, 1 << 20, m).astype(np.uint64)
    hits = k == 7                                   # inside the table's regions
    m = int(hits.sum())
    starts[hits] = table[rng.integers(0, 64, m)] + _pages(rng.integers(0, 512, m))
    sizes[hits] = _pages(rng.integers(1, 256, m))
    rep = k >= 8                                    # repeats of earlier items
    idx = np.nonzero(rep)[0]
    own = np.nonzero(~rep)[0]
    src = own[(rng.random(len(idx)) * np.searchsorted(own, idx)).astype(np.int64)]
    starts[idx] = starts[src]
    sizes[idx] = sizes[src]
    sizes[rng.random(n) < 0.005] = 0
    h, kd = p.register(starts, sizes, "crowded")
    assert (kd == oracle.REG_HIT_NEW).sum() > 1000 and (kd == oracle.REG_NEW).sum() > 1000
    live = h[h > 0]
    p.deregister(rng.choice(live, 4000), "crowded deregister")
    # Starts over the whole space, with ranges at both ends of it.
    n = 8192
    starts = rng.integers(0, 1 << 63, n, dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, n).astype(np.uint64)
    sizes = rng.integers(1, 1 << 30, n).astype(np.uint64)
    starts[:16] = np.arange(16, dtype=np.uint64) * np.uint64(4096)
    starts[16:32] = np.uint64((1 << 64) - (1 << 24)) + _pages(np.arange(16))
    sizes[16:32] = 4096
    starts[32:4096] = starts[rng.integers(0, 32, 4064)]
    sizes[32:4096] = sizes[rng.integers(0, 32, 4064)]
    p.register(starts, sizes, "wide span")


def test_whole_batches_on_one_record():
    # Every call of a full batch names one record: hits on one old record,
    # repeats of one new range, then deregistrations of one handle (its
    # references drop one by one, the rest are stale). The reference updates
    # of such a batch all land on one word.
    p = Pair(capacity=64)
    p.register(np.array([1 << 40], np.uint64), np.array([1 << 30], np.uint64), "one region")
    n = dd.REG_MAX_BATCH
    h, _ = p.register(np.full(n, (1 << 40) + 4096, np.uint64), np.full(n, M, np.uint64),
                      "hits on one record")
    h2, k2 = p.register(np.full(n - 1, 1 << 44, np.uint64), np.full(n - 1, M, np.uint64),
                        "repeats of one new range")
    assert (k2 == oracle.REG_NEW).sum() == 1
    p.deregister(np.full(n, h2[0], np.uint64), "one handle, every call")
    p.deregister(np.full(n, h[0], np.uint64), "the old record, every call")


def test_empty_batches_and_empty_table():
    p = Pair()
    p.register(np.zeros(0, np.uint64), np.zeros(0, np.uint64), "empty register")
    p.deregister(np.array([1, 2, 0], np.uint64), "deregister on an empty table")
    p.deregister(np.zeros(0, np.uint64), "empty deregister")


def test_workspace_of_exact_size_keeps_its_neighbour_intact():
    # A workspace of exactly dmadesc_workspace_bytes inside a larger buffer
    # whose tail holds a canary: a small batch on a large table must write
    # nothing past the workspace, for a register and a deregister batch.
    cap, n = 65536, 20
    reg = dd.DeviceRegistry(cap)
    need = dd.workspace_bytes(dd.OP_REGISTRY, n, cap)
    tail = 1 << 20
    buf = torch.full((need + tail,), 0xA5, dtype=torch.uint8, device="cuda")
    addr = gc.dev(np.arange(n, dtype=np.uint64) * np.uint64(8 * M))
    size = gc.dev(np.full(n, M, np.uint64))
    handle = torch.empty(n, dtype=torch.uint64, device="cuda")
    kind = torch.empty(n, dtype=torch.uint8, device="cuda")
    needed = torch.zeros(1, dtype=torch.uint64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    gc.say(f"registry exact workspace: n={n} cap={cap} ws={need}")
    rc = dd.lib().dmadesc_reg_register(*reg._table(), 12, addr.data_ptr(), size.data_ptr(), n,
                                       handle.data_ptr(), kind.data_ptr(), needed.data_ptr(),
                                       buf.data_ptr(), need, s)
    assert rc == 0
    torch.cuda.synchronize()
    assert (gc.host(kind) == oracle.REG_NEW).all() and reg.count() == n
    assert bool((buf[need:] == 0xA5).all()), "register wrote past its workspace"
    status = torch.empty(n, dtype=torch.uint8, device="cuda")
    rc = dd.lib().dmadesc_reg_deregister(*reg._table(), handle.data_ptr(), n,
                                         status.data_ptr(), buf.data_ptr(), need, s)
    assert rc == 0
    torch.cuda.synchronize()
    assert (gc.host(status) == oracle.DEREG_REMOVED).all() and reg.count() == 0
    assert bool((buf[need:] == 0xA5).all()), "deregister wrote past its workspace"
