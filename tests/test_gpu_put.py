"""GPU parity of dmadesc_build_put with the oracle's O6: first, count,
status, total and every descriptor slot (canary-filled on both sides, so
equal arrays also mean nothing else was written), bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import oracle
import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def check_put(src, dst, nbytes, pe, local_base, heap, shift, lkeys, peer_base, rkeys, cap,
              ctx=""):
    gc.say(f"build_put {ctx}: n={len(src)} cap={cap} shift={shift}")
    want = np.full(max(cap, 1), 0, oracle.PUT_DESC)
    want.view(np.uint64)[:] = np.uint64(gc.CANARY)
    o = oracle.build_put(src, dst, nbytes, pe, local_base, heap, shift, lkeys, peer_base,
                         rkeys, cap, desc=want)
    desc = torch.full((max(cap, 1), 4), gc.CANARY_I64, dtype=torch.int64,
                      device="cuda").view(torch.uint64)
    n = len(src)
    ws = torch.full((max(dd.workspace_bytes(dd.OP_BUILD_PUT, n), 8),), 0xAB,
                    dtype=torch.uint8, device="cuda")
    g = dd.build_put(gc.dev(np.asarray(src, np.uint64)), gc.dev(np.asarray(dst, np.uint64)),
                     gc.dev(np.asarray(nbytes, np.uint64)), gc.dev(np.asarray(pe, np.uint32)),
                     local_base, heap, shift, gc.dev(np.asarray(lkeys, np.uint32)),
                     gc.dev(np.asarray(peer_base, np.uint64)),
                     gc.dev(np.asarray(rkeys, np.uint32)), desc[:cap] if cap else desc[:0],
                     ws=ws)
    torch.cuda.synchronize()
    if n:
        # workspace header: blocks that ran, and bounded waits that expired
        blocks, timeouts = gc.host(ws[:8]).view(np.uint32)
        assert 1 <= blocks <= n and timeouts == 0, (ctx, blocks, timeouts)
    for k in ("first", "count", "status"):
        got = gc.host(g[k])
        if not np.array_equal(got, o[k]):
            bad = np.nonzero(got != o[k])[0]
            raise AssertionError(f"{ctx} {k}: {bad.size} differ, first at {bad[0]}: "
                                 f"oracle {o[k][bad[0]]} gpu {got[bad[0]]}")
    assert int(gc.host(g["total"])[0]) == o["total"], ctx
    gd = gc.host(desc).reshape(-1)
    wd = want.view(np.uint64)
    if not np.array_equal(gd, wd):
        bad = np.nonzero(gd != wd)[0]
        raise AssertionError(f"{ctx} descriptors: {bad.size} words differ, first in slot "
                             f"{bad[0] // 4}")
    return o


@pytest.mark.parametrize("n", [1, 1000, 100_001])
def test_vmm_workload_scaled(n):
    b = synth.put_batch(n)
    o = oracle.build_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                         b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], 0, write=False)
    check_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
              b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], o["total"], f"vmm n={n}")


def test_vmm_workload_full_size():
    b = synth.put_batch(1 << 24)
    o = oracle.build_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                         b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], 0, write=False)
    check_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
              b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], o["total"], "vmm full")


@pytest.mark.parametrize("shift", [12, 13, 16])
def test_small_chunks_many_pieces(shift):
    # Long puts over small chunks: hundreds of pieces each, both phase cases.
    rng = np.random.default_rng(shift)
    heap = 1 << 30
    n = 5000
    nbytes = rng.integers(1, 3 << 20, n).astype(np.uint64)
    src = rng.integers(0, heap - (3 << 20), n).astype(np.uint64)
    dst = rng.integers(0, heap - (3 << 20), n).astype(np.uint64)
    dst[::3] = src[::3] + np.uint64(4096 << 4)                # same phase
    dst[1::7] = (src[1::7] >> np.uint64(shift)) << np.uint64(shift)
    pe = rng.integers(0, 4, n).astype(np.uint32)
    nch = heap >> shift
    lk = rng.integers(1, 1 << 32, nch, dtype=np.uint64).astype(np.uint32)
    rk = rng.integers(1, 1 << 32, 4 * nch, dtype=np.uint64).astype(np.uint32)
    pb = np.arange(4, dtype=np.uint64) * np.uint64(1 << 44)
    o = oracle.build_put(src, dst, nbytes, pe, 1 << 45, heap, shift, lk, pb, rk, 0, write=False)
    check_put(src, dst, nbytes, pe, 1 << 45, heap, shift, lk, pb, rk, o["total"],
              f"small chunks {shift}")


def test_static_heap_message_limit():
    heap = 1 << 40
    src = np.array([0, 5, 1 << 35, 12], np.uint64)
    dst = np.array([8, 0, 4096, (1 << 39)], np.uint64)
    nbytes = np.array([1, 1 << 31, 5 * (1 << 31) + 3, (1 << 31) + 1], np.uint64)
    pe = np.array([1, 0, 2, 1], np.uint32)
    check_put(src, dst, nbytes, pe, 1 << 46, heap, 0, [9], [1 << 50, 2 << 50, 3 << 50],
              [7, 8, 9], 10, "static")


@pytest.mark.parametrize("frac", [0.0, 0.5, 0.999])
def test_status_and_enospc(frac):
    b = synth.put_batch(20_000, seed=3)
    b["len"][::97] = 0                                        # EINVAL
    b["pe"][5::101] = 8                                       # EINVAL
    b["src"][7::103] = np.uint64(b["heap"] - 100)             # ERANGE
    b["dst"][9::107] = np.uint64(b["heap"] - 100)             # ERANGE
    o = oracle.build_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                         b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], 0, write=False)
    cap = int(o["total"] * frac)
    r = check_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                  b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], cap,
                  f"status cap={cap}")
    assert ((r["status"] == 3).any()) == (cap < o["total"])


def test_empty_batch():
    b = synth.put_batch(1)
    z = np.zeros(0, np.uint64)
    check_put(z, z, z, np.zeros(0, np.uint32), b["local_base"], b["heap"], b["chunk_shift"],
              b["lkeys"], b["peer_base"], b["rkeys"], 4, "empty")


@pytest.mark.parametrize("seed", range(10))
def test_random_parameters(seed):
    """Seeded draws over the call's whole parameter space: chunk shift (0 =
    static heap, else 12..31), heap size, PE count, batch size (around the
    4,096-put block too), lengths from a byte to many chunks, invalid and
    out-of-heap puts, random key tables and bases, and a capacity below or
    at the total."""
    rng = np.random.default_rng(1000 + seed)
    shift = 0 if seed % 5 == 0 else int(rng.integers(12, 32))
    if shift:
        nch = int(rng.integers(1, min(1 << 12, (1 << 40) >> shift) + 1))
        heap = nch << shift
    else:
        nch, heap = 1, int(rng.integers(1 << 20, 1 << 41))
    npes = int(rng.integers(1, 17))
    n = [int(rng.integers(0, 300)), 4095, 4096, 4097, int(rng.integers(5000, 40_000))][seed % 5]
    unit = 1 << (shift if shift else 31)
    kind = rng.integers(0, 3, n)
    nbytes = np.where(kind == 0, rng.integers(1, 65, n),
                      np.where(kind == 1, rng.integers(1, unit + 1, n),
                               rng.integers(1, 4 * unit + 1, n))).astype(np.uint64)
    nbytes = np.minimum(nbytes, np.uint64(heap))
    src = (rng.random(n) * (heap - nbytes.astype(np.float64) + 1)).astype(np.uint64)
    dst = (rng.random(n) * (heap - nbytes.astype(np.float64) + 1)).astype(np.uint64)
    src = np.minimum(src, np.uint64(heap) - nbytes)
    dst = np.minimum(dst, np.uint64(heap) - nbytes)
    pe = rng.integers(0, npes, n).astype(np.uint32)
    if n:
        bad = rng.random(n)
        nbytes[bad < 0.01] = 0                                    # EINVAL
        pe[(bad >= 0.01) & (bad < 0.02)] = np.uint32(npes)        # EINVAL
        src[(bad >= 0.02) & (bad < 0.03)] = np.uint64(heap)       # ERANGE (a byte past)
    lk = rng.integers(0, 1 << 32, nch, dtype=np.uint64).astype(np.uint32)
    rk = rng.integers(0, 1 << 32, npes * nch, dtype=np.uint64).astype(np.uint32)
    pb = rng.integers(0, 1 << 56, npes, dtype=np.uint64)
    local_base = int(rng.integers(0, 1 << 56))
    o = oracle.build_put(src, dst, nbytes, pe, local_base, heap, shift, lk, pb, rk, 0, write=False)
    cap = int(o["total"]) if seed % 3 else int(o["total"] * rng.uniform(0.3, 1.0))
    check_put(src, dst, nbytes, pe, local_base, heap, shift, lk, pb, rk, cap,
              f"random seed={seed} shift={shift} heap={heap} npes={npes} n={n}")
