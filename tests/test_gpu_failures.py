"""Failure paths that must be loud: a slot-scan wait that expires refuses the
requests that need its prefix (PRP_EBUSY) and everything else stays exact;
the checked binding raises; the region-table check names the first faulty
region. The expired waits are forced from the host with the library's own
bound on a wait (dmadesc_debug_wait_limit), so every kernel still runs to its
normal end."""
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


class tight_waits:
    """Every look-back wait gives up at the first poll that finds a
    predecessor not yet published (restored on exit)."""

    def __enter__(self):
        self.old = dd.debug_wait_limit(0)

    def __exit__(self, *exc):
        dd.debug_wait_limit(self.old)


def _list_words_packed(o, off, ln):
    """[first word, end word) of every packed list, from the oracle's PRP2: the
    words of its data slots and chain pointers, plus word 511 of the page
    when its last slot is word 510 (that word is then the list's too)."""
    pages = ((off & np.uint64(4095)) + ln + np.uint64(4095)) >> np.uint64(12)
    spans = {}
    for i in np.nonzero((o["status"] == 0) & (pages >= 3))[0]:
        m = int(pages[i]) - 1
        w0 = (int(o["prp2"][i]) - BUS) // 8
        last = w0 - w0 // 512 + m - 1                  # its last data slot
        wl = last + last // 511                        # that slot's word
        spans[int(i)] = (w0, wl + 1 + (wl % 512 == 510))
    return spans


def _run_expired(packed, d, pool_pages, tries=4):
    """Runs the build with tight waits until some block's wait expires;
    returns (outputs, pool, expired blocks)."""
    n = d["n"]
    for t in range(tries):
        pool = torch.empty((pool_pages, 512), dtype=torch.uint64, device="cuda")
        pool.view(torch.int64).fill_(gc.CANARY_I64)
        ws = torch.zeros(dd.workspace_bytes(dd.OP_BUILD_PRP, n), dtype=torch.uint8, device="cuda")
        gc.say(f"expired-wait build packed={packed} n={n} try={t}")
        with tight_waits():
            out = dd.build_prp(gc.dev(d["lut"]), gc.dev(d["off"]), gc.dev(d["len"]), BUS, pool,
                               ws=ws, packed=packed, check=False)
        torch.cuda.synchronize()
        blocks, expired = gc.host(ws[:8]).view(np.uint32)
        assert blocks == -(-n // gc.prp_tile(n))
        if expired:
            return {k: gc.host(v) for k, v in out.items()}, pool, int(expired), ws
    pytest.fail(f"no look-back wait expired in {tries} runs at the tightest bound")


@pytest.mark.parametrize("packed", [True, False])
def test_expired_wait_refuses_only_list_requests_of_its_block(packed):
    d = synth.generate("mixed", n=(1 << 21) if packed else (1 << 18))
    off, ln = d["off"], d["len"]
    build = oracle.build_prp_packed if packed else oracle.build_prp
    need = build(d["lut"], off, ln, BUS, 1 << 50)["total"]
    o_pool = np.full((need, 512), gc.CANARY, dtype=np.uint64)
    o = build(d["lut"], off, ln, BUS, need, pool=o_pool)
    g, pool, expired, _ = _run_expired(packed, d, need)
    busy = g["status"] == dd.PRP_EBUSY
    assert busy.any(), "an expired block with list requests refuses them"
    # Refused requests: list requests the oracle builds, nothing written.
    pages = ((off & np.uint64(4095)) + ln + np.uint64(4095)) >> np.uint64(12)
    assert (o["status"][busy] == 0).all() and (pages[busy] >= 3).all()
    assert (g["prp1"][busy] == 0).all() and (g["prp2"][busy] == 0).all()
    # They come in whole blocks: every list request of a refused block is refused.
    tile = gc.prp_tile(d["n"])
    blk = np.unique(np.nonzero(busy)[0] // tile)
    assert len(blk) <= expired
    for b in blk:
        sl = slice(b * tile, (b + 1) * tile)
        assert (busy[sl] == ((o["status"][sl] == 0) & (pages[sl] >= 3))).all()
    # Everything else is exact.
    for k in ("prp1", "prp2", "status"):
        assert np.array_equal(g[k][~busy], o[k][~busy]), k
    # The batch total comes from the last block: exact, or UINT64_MAX when
    # that block's wait expired (certainly so when it refused requests).
    total = int(g["total_pages"][0])
    assert total in (o["total"], 2 ** 64 - 1)
    if busy[(d["n"] - 1) // tile * tile:].any():
        assert total == 2 ** 64 - 1
    gp = gc.host(pool)
    if not packed:
        gc.mask_padding(o_pool, gp, gc.padding_spans(o["prp2"], o["status"], off, ln, BUS))
    diff = np.flatnonzero((o_pool != gp).reshape(-1))
    # Every differing word is an untouched word of a refused request's list.
    assert (gp.reshape(-1)[diff] == np.uint64(gc.CANARY)).all()
    if packed:
        spans = _list_words_packed(o, off, ln)
        owned = np.zeros(o_pool.size, bool)
        for i in np.nonzero(busy)[0]:
            a, b = spans[int(i)]
            owned[a:b] = True
        assert owned[diff].all()
    else:
        refused_pages = set()
        for i in np.nonzero(busy)[0]:
            s0 = (int(o["prp2"][i]) - BUS) // 4096
            lp = (int(pages[i]) - 2 + 510) // 511
            refused_pages.update(range(s0, s0 + lp))
        assert set(np.unique(diff // 512).tolist()) <= refused_pages


def test_checked_build_raises_on_expired_wait():
    d = synth.generate("mixed", n=1 << 21)
    need = oracle.build_prp_packed(d["lut"], d["off"], d["len"], BUS, 1 << 50)["total"]
    pool = torch.empty((need, 512), dtype=torch.uint64, device="cuda")
    args = (gc.dev(d["lut"]), gc.dev(d["off"]), gc.dev(d["len"]), BUS, pool)
    for t in range(4):
        gc.say(f"checked build with tight waits, try {t}")
        try:
            with tight_waits():
                dd.build_prp_packed(*args)
        except dd.DmadescRefused as e:
            st = gc.host(e.out["status"])
            assert (st == dd.PRP_EBUSY).any()
            break
    else:
        pytest.fail("no look-back wait expired at the tightest bound")
    # At the default bound the same call is exact and raises nothing.
    out = dd.build_prp_packed(*args)
    assert not (gc.host(out["status"]) == dd.PRP_EBUSY).any()


def test_expired_wait_in_put_build():
    b = synth.put_batch(1 << 20)
    n = len(b["src"])
    o = oracle.build_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                         b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], 0)
    cap = o["total"]
    want = np.full(cap, 0, oracle.PUT_DESC)
    want.view(np.uint64)[:] = np.uint64(gc.CANARY)
    o = oracle.build_put(b["src"], b["dst"], b["len"], b["pe"], b["local_base"], b["heap"],
                         b["chunk_shift"], b["lkeys"], b["peer_base"], b["rkeys"], cap, desc=want)
    args = [gc.dev(b["src"]), gc.dev(b["dst"]), gc.dev(b["len"]), gc.dev(b["pe"]),
            b["local_base"], b["heap"], b["chunk_shift"], gc.dev(b["lkeys"]),
            gc.dev(b["peer_base"]), gc.dev(b["rkeys"])]
    for t in range(4):
        desc = torch.full((cap, 4), gc.CANARY_I64, dtype=torch.int64,
                          device="cuda").view(torch.uint64)
        ws = torch.zeros(dd.workspace_bytes(dd.OP_BUILD_PUT, n), dtype=torch.uint8, device="cuda")
        gc.say(f"expired-wait put build n={n} try={t}")
        with tight_waits():
            g = dd.build_put(*args, desc, ws=ws, check=False)
        torch.cuda.synchronize()
        if gc.host(ws[4:8]).view(np.uint32)[0]:
            break
    else:
        pytest.fail("no look-back wait expired at the tightest bound")
    st, first = gc.host(g["status"]), gc.host(g["first"])
    busy = st == dd.PRP_EBUSY
    assert busy.any()
    assert (o["status"][busy] == 0).all() and (first[busy] == np.uint64(2 ** 64 - 1)).all()
    assert np.array_equal(gc.host(g["count"]), o["count"])
    for k, got in (("first", first), ("status", st)):
        assert np.array_equal(got[~busy], o[k][~busy]), k
    gd = gc.host(desc).reshape(-1, 4)
    wd = want.view(np.uint64).reshape(-1, 4)
    diff = np.nonzero((gd != wd).any(axis=1))[0]
    assert (gd[diff] == np.uint64(gc.CANARY)).all()
    refused = np.zeros(cap, bool)
    for i in np.nonzero(busy)[0]:
        refused[int(o["first"][i]):int(o["first"][i]) + int(o["count"][i])] = True
    assert refused[diff].all()


@pytest.mark.parametrize("name", ["tiny", "small", "mixed"])
def test_table_check_accepts_the_workload_tables(name):
    d = synth.generate(name, n=16)
    dd.mr_table_check(gc.dev(d["rstart"]), gc.dev(d["rend"]))


def test_table_check_names_the_first_faulty_region():
    d = synth.generate("mixed", n=16)
    rs, re_ = d["rstart"].copy(), d["rend"].copy()
    cases = []
    a, b = rs.copy(), re_.copy()
    a[100], a[101] = a[101], a[100]                      # unsorted
    cases.append((a, b, 100))
    a, b = rs.copy(), re_.copy()
    b[2000] = a[2001] + np.uint64(4096)                  # overlaps the next
    cases.append((a, b, 2000))
    a, b = rs.copy(), re_.copy()
    a[3000] += np.uint64(8)                              # unaligned start
    cases.append((a, b, 3000))
    a, b = rs.copy(), re_.copy()
    b[7] = a[7]                                          # empty
    cases.append((a, b, 7))
    for a, b, want in cases:
        with pytest.raises(dd.DmadescError) as e:
            dd.mr_table_check(gc.dev(a), gc.dev(b))
        assert e.value.rc == -22 and f"region {want} " in str(e.value)
    dd.mr_table_check(gc.dev(rs[:0]), gc.dev(re_[:0]))   # empty table: valid
    with pytest.raises(dd.DmadescError):                 # 64 KiB pages: Mixed starts are
        dd.mr_table_check(gc.dev(rs), gc.dev(re_), page_shift=20)  # not 1 MiB aligned
