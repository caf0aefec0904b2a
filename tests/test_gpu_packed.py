"""GPU parity of dmadesc_build_prp_packed with the oracle's O2p: PRP1, PRP2,
status, the page total and every pool word (canary-filled on both sides, so
equal pools also mean nothing else was written), bit for bit."""
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


def _perm_lut(rng, p, base=synth.PHYS_BASE):
    return (np.uint64(base) + rng.permutation(p).astype(np.uint64) * np.uint64(65536))


def _need(lut, off, ln):
    return oracle.build_prp_packed(lut, off, ln, BUS, 1 << 50)["total"]


@pytest.mark.parametrize("name,n", [("tiny", None), ("small", 300_000), ("large", None),
                                    ("mixed", 1 << 20)])
def test_workload_scaled(name, n):
    d = synth.generate(name, n=n)
    pages = _need(d["lut"], d["off"], d["len"])
    gc.say(f"packed {name} n={d['n']} pages={pages}")
    gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, max(pages, 1), ctx=name, packed=True)


@pytest.mark.parametrize("name", ["small", "large", "mixed"])
def test_workload_full_size(name):
    d = synth.generate(name)
    pages = _need(d["lut"], d["off"], d["len"])
    gc.say(f"packed full {name} n={d['n']} pages={pages}")
    gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, max(pages, 1), ctx=name, packed=True)


def _chain_batch(rng, ms, p=1 << 14):
    lut = _perm_lut(rng, p)
    ms = np.asarray(ms, np.uint64)
    heap = p * 65536
    ln = (ms + np.uint64(1)) * np.uint64(4096) - rng.integers(0, 2, ms.size).astype(np.uint64) * np.uint64(8)
    off = rng.integers(0, (heap - int(ln.max())) // 4, ms.size).astype(np.uint64) * np.uint64(4)
    off -= off % np.uint64(4096)                     # page-aligned: pages = m + 1 exactly
    off += np.uint64(8) * (rng.random(ms.size) < 0.5).astype(np.uint64) * (ln % np.uint64(4096) != 0)
    return lut, off, ln


def test_list_starts_at_every_offset_near_page_ends():
    # Lists of 2..4 entries after a prefix that walks the start slot through
    # every residue around a page end, and long lists that end on each word
    # near 511.
    rng = np.random.default_rng(3)
    ms = []
    for lead in range(505, 515):
        ms += [lead] + [2, 3, 2, 4, 511, 512, 513, 2]
    lut, off, ln = _chain_batch(rng, ms)
    pages = _need(lut, off, ln)
    gc.check_prp_full(lut, off, ln, BUS, pages, ctx="page ends", packed=True)


@pytest.mark.parametrize("m", [2, 3, 509, 510, 511, 512, 513, 1021, 1022, 1023, 1024, 5000,
                               70_000])
def test_chain_sizes(m):
    rng = np.random.default_rng(m)
    lut, off, ln = _chain_batch(rng, [m, 7, m, 2, m], p=1 << 16)
    pages = _need(lut, off, ln)
    gc.check_prp_full(lut, off, ln, BUS, pages, ctx=f"m={m}", packed=True)


def test_random_mix_many_blocks():
    rng = np.random.default_rng(5)
    n = 50_000
    ms = rng.choice([0, 0, 1, 2, 3, 40, 510, 511, 512, 2000], n)
    lut, off, ln = _chain_batch(rng, np.maximum(ms, 1), p=1 << 16)
    ln[ms == 0] = rng.integers(1, 4096, int((ms == 0).sum())).astype(np.uint64) * np.uint64(4) % np.uint64(4096) + np.uint64(4)
    ln[rng.random(n) < 0.01] = 0                     # EINVAL
    off[rng.random(n) < 0.01] = np.uint64(1 << 40)  # ERANGE
    pages = _need(lut, off, ln)
    gc.check_prp_full(lut, off, ln, BUS, pages, ctx="mix", packed=True)


@pytest.mark.parametrize("frac", [0.0, 0.3, 0.97])
def test_enospc_suffix(frac):
    rng = np.random.default_rng(6)
    ms = rng.integers(2, 900, 20_000)
    lut, off, ln = _chain_batch(rng, ms, p=1 << 16)
    need = _need(lut, off, ln)
    pool_pages = int(need * frac)
    g = gc.check_prp_full(lut, off, ln, BUS, max(pool_pages, 1), ctx=f"enospc {frac}",
                          packed=True)[1]
    refused = g["status"] == 3                        # every request here has a list
    assert g["total"] == need and refused.any()
    assert refused[int(np.argmax(refused)):].all()    # the refused requests are a suffix


def test_empty_single_and_no_heap():
    lut = _perm_lut(np.random.default_rng(7), 64)
    e = np.zeros(0, np.uint64)
    gc.check_prp_full(lut, e, e, BUS, 1, ctx="empty", packed=True)
    gc.check_prp_full(lut, np.array([4096], np.uint64), np.array([4096 * 40], np.uint64), BUS, 1,
                      ctx="single", packed=True)
    gc.check_prp_full(np.zeros(0, np.uint64), np.array([0, 8], np.uint64),
                      np.array([4096, 4096 * 9], np.uint64), BUS, 1, ctx="no heap", packed=True)


def test_pool_probe_then_build():
    d = synth.generate("small", n=100_000)
    g, _ = gc.gpu_prp(d["lut"], d["off"], d["len"], BUS, 0, packed=True)
    o = oracle.build_prp_packed(d["lut"], d["off"], d["len"], BUS, 0)
    gc.assert_prp_columns_equal(o, g, "probe")
    gc.check_prp_full(d["lut"], d["off"], d["len"], BUS, max(g["total"], 1), ctx="after probe",
                      packed=True)
