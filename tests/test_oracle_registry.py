"""Pins of the oracle's registry batches (O4b): the register experiment of
the NCCL course page as one batch, the capacity growth it prints, and a
record-list model replayed over random batches."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

M = 1 << 20


def test_register_experiment_as_batches():
    base = 0x7f00_0000_0000
    reg = oracle.Registry(12)
    h, k, need = reg.register_batch([base, base, base + 0x1000, base + 4 * M],
                                    [2 * M, 2 * M, M, 2 * M], 32)
    assert h[0] == h[1] == h[2] != h[3] and h[0] > 0
    assert k.tolist() == [oracle.REG_NEW, oracle.REG_HIT_NEW, oracle.REG_HIT_NEW,
                          oracle.REG_NEW]
    assert need == 32 and reg.refs(int(h[0])) == 3
    st = reg.deregister_batch([h[0]] * 4)
    assert st.tolist() == [oracle.DEREG_OK, oracle.DEREG_OK, oracle.DEREG_REMOVED,
                           oracle.DEREG_STALE]
    assert reg.count() == 1 and reg.refs(int(h[3])) == 1
    # The same ranges in a later batch hit the surviving record or make new ones.
    h2, k2, _ = reg.register_batch([base + 4 * M + 4096, base], [4096, 4096], 32)
    assert h2[0] == h[3] and k2[0] == oracle.REG_HIT
    assert k2[1] == oracle.REG_NEW and h2[1] > h[3]


def test_capacity_growth_0_32_64_128():
    reg = oracle.Registry(12)
    cap, seen = 0, []
    for i in range(130):
        h, k, need = reg.register_batch([i * 8 * M], [M], cap)
        if need > cap:
            assert k[0] == oracle.REG_NOSPACE and h[0] == 0 and reg.count() == i
            seen.append(need)
            cap = need
            h, k, need = reg.register_batch([i * 8 * M], [M], cap)
        assert k[0] == oracle.REG_NEW
    assert seen == [32, 64, 128, 256]
    assert reg.count() == 130


def test_refused_batch_changes_nothing():
    reg = oracle.Registry(12)
    reg.register_batch([0, 16 * M], [M, M], 2)
    before = reg.records()
    nid = reg.next_id()
    h, k, need = reg.register_batch([32 * M, 0], [M, 4096], 2)
    assert need == 4 and (k == oracle.REG_NOSPACE).all() and (h == 0).all()
    for a, b in zip(before, reg.records()):
        assert np.array_equal(a, b)
    assert reg.next_id() == nid


@pytest.mark.parametrize("seed", range(5))
def test_batches_match_record_list_model(seed):
    rng = np.random.default_rng(seed)
    reg, model = oracle.Registry(12), bf.RecordList(12)
    live = []
    for rnd in range(40):
        n = int(rng.integers(1, 60))
        if rng.random() < 0.6 or not live:
            starts = rng.integers(0, 64, n) * (256 * 1024) + rng.integers(0, 4096, n)
            sizes = rng.choice([0, 1, 4096, 100_000, M, 3 * M], n)
            if rnd % 7 == 0:                          # sometimes add exact repeats
                starts[n // 2:] = starts[:n - n // 2]
                sizes[n // 2:] = sizes[:n - n // 2]
            first_new = model.next
            want = [model.register(int(a), int(b)) for a, b in zip(starts, sizes)]
            h, k, need = reg.register_batch(starts, sizes, 1 << 20)
            names = {"invalid": oracle.REG_INVALID, "hit": oracle.REG_HIT}
            seen = set()
            for i, (wh, wk) in enumerate(want):
                assert int(h[i]) == wh
                if wk == "new":
                    assert k[i] == oracle.REG_NEW
                    seen.add(wh)
                elif wk == "hit" and wh >= first_new:
                    assert wh in seen and k[i] == oracle.REG_HIT_NEW
                else:
                    assert k[i] == names[wk]
            live = [r[2] for r in model.recs]
        else:
            hs = rng.choice(live + [10**6], n)            # one handle that never existed
            want = [model.deregister(int(x)) for x in hs]
            st = reg.deregister_batch(hs)
            codes = {"ok": oracle.DEREG_OK, "removed": oracle.DEREG_REMOVED,
                     "stale": oracle.DEREG_STALE}
            assert st.tolist() == [codes[w] for w in want]
            live = [r[2] for r in model.recs]
        s, e, hh, refs = reg.records()
        assert [list(map(int, t)) for t in zip(s, e, hh, refs)] == model.recs
