"""Seeded random-parameter sweep of the PRP build, both list layouts, against
the oracle (O2 / O2p): every PRP1/PRP2/status, the page total and every pool
word (canary-filled on both sides). The draws cover batch sizes around both
block sizes (256 and 1,024 requests) and the switch between them at 2^19
requests, table sizes from one GPU page up, table entries with and without
low bits, request lengths from 4 bytes to chained lists, every status
(EINVAL, ERANGE, ENOSPC) and bus bases anywhere in 4 KiB-aligned space."""
from __future__ import annotations

import numpy as np
import pytest

from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

SIZES = [1, 255, 256, 257, 1023, 1024, 1025, 5000, 70_001, 1 << 19, (1 << 19) + 1, 600_000]


def draw(seed):
    rng = np.random.default_rng(2000 + seed)
    n = SIZES[seed % len(SIZES)]
    packed = bool(seed % 2)
    p = int(rng.choice([1, 2, 17, 4096, 65536]))                  # GPU pages in the heap
    heap = p << 16
    lut = np.uint64(int(rng.integers(0, 1 << 40)) << 16) + \
        rng.permutation(p).astype(np.uint64) * np.uint64(65536)
    if seed % 3 == 0:
        lut |= rng.integers(0, 1 << 16, p).astype(np.uint64)     # entries with low bits
    # Lengths: mostly one or two 4 KiB pages when the batch is large, so the
    # page layout's pool stays a few hundred MB; lists, some chained, otherwise.
    big = n > 100_000
    kind = rng.random(n)
    ln = np.where(kind < (0.9 if big else 0.3), rng.integers(1, 8193, n),
                  np.where(kind < (0.99 if big else 0.8), rng.integers(8193, 64 * 4096, n),
                           rng.integers(64 * 4096, 2100 * 4096, n))).astype(np.uint64)
    ln &= ~np.uint64(3)
    ln = np.maximum(ln, np.uint64(4))
    ln = np.minimum(ln, np.uint64(heap))
    off = (rng.random(n) * (heap - ln.astype(np.float64) + 1)).astype(np.uint64) & ~np.uint64(3)
    off = np.minimum(off, np.uint64(heap) - ln) & ~np.uint64(3)
    bad = rng.random(n)
    ln[bad < 0.005] = 0                                            # EINVAL: empty
    off[(bad >= 0.005) & (bad < 0.01)] += np.uint64(2)             # EINVAL: not 4-byte aligned
    off[(bad >= 0.01) & (bad < 0.015)] = np.uint64(heap)           # ERANGE: past the heap
    off[(bad >= 0.015) & (bad < 0.016)] = np.uint64(2 ** 64 - 4)   # EINVAL or ERANGE: wraps
    bus = int(rng.integers(0, 1 << 40)) << 12
    return rng, n, packed, lut, off, ln, bus


@pytest.mark.parametrize("seed", range(24))
def test_random_parameters(seed):
    import oracle
    rng, n, packed, lut, off, ln, bus = draw(seed)
    build = oracle.build_prp_packed if packed else oracle.build_prp
    need = build(lut, off, ln, bus, 1 << 50)["total"]
    pool_pages = need if seed % 4 else int(need * rng.uniform(0.2, 1.0))
    gc.say(f"prp random seed={seed} n={n} packed={packed} pages={need} pool={pool_pages}")
    gc.check_prp_full(lut, off, ln, bus, max(pool_pages, 1), ctx=f"random seed={seed}",
                      packed=packed)
