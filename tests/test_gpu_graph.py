"""The path's three calls captured once in a HIP graph (torch.cuda.graph) and
replayed: every replay must reproduce the eager outputs bit for bit (lookup
columns, PRP columns, the whole list pool, perm/qoff/n_invalid), with other
eager work and synchronizations between the replays and the outputs poisoned
before each replay. No call on the path records a memset or a host
synchronization (workspace headers are cleared by kernels), which is what
makes it capturable."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_dma_descriptor_amd as dd
import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

BUS = synth.LIST_BUS_BASE


class Path:
    """Lookup (if the workload has regions), PRP build, split on fixed
    device buffers, so that a captured graph and eager calls share them."""

    def __init__(self, d, packed):
        self.d, self.packed = d, packed
        self.n = d["n"]
        self.rs, self.re, self.rk = gc.dev(d["rstart"]), gc.dev(d["rend"]), gc.dev(d["rlkey"])
        self.off, self.ln = gc.dev(d["off"]), gc.dev(d["len"])
        self.qid, self.lut = gc.dev(d["qid"]), gc.dev(d["lut"])
        empty = torch.empty((0, 512), dtype=torch.uint64, device="cuda")
        probe = dd.build_prp(self.lut, self.off, self.ln, BUS, empty, packed=packed)
        pages = max(int(probe["total_pages"].cpu()[0]), 1)
        self.pool = torch.empty((pages, 512), dtype=torch.uint64, device="cuda")
        self.ws_prp = torch.empty(max(dd.workspace_bytes(dd.OP_BUILD_PRP, self.n), 1),
                                  dtype=torch.uint8, device="cuda")
        self.ws_sp = torch.empty(dd.workspace_bytes(dd.OP_PARTITION, self.n, d["nqueues"]),
                                 dtype=torch.uint8, device="cuda")
        need = dd.workspace_bytes(dd.OP_MR_LOOKUP, self.n, len(d["rstart"]))
        self.ws_lk = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        self.lk = self.pr = self.sp = None

    def run(self):
        d = self.d
        if len(d["rstart"]):
            self.lk = dd.mr_lookup(self.rs, self.re, self.rk, self.off, self.ln,
                                   va_base=d["va_base"], out=self.lk, ws=self.ws_lk)
        self.pr = dd.build_prp(self.lut, self.off, self.ln, BUS, self.pool, out=self.pr,
                               ws=self.ws_prp, packed=self.packed, check=False)
        self.sp = dd.partition_by_queue(self.qid, d["nqueues"], out=self.sp, ws=self.ws_sp,
                                        check=False)

    def outputs(self):
        out = {}
        for grp in (self.lk or {}, self.pr, self.sp):
            for k, v in grp.items():
                out[k] = v.clone()
        out["pool"] = self.pool.clone()
        return out

    def poison(self):
        for grp in (self.lk or {}, self.pr, self.sp):
            for v in grp.values():
                v.view(torch.uint8).fill_(0xC3)
        self.pool.view(torch.int64).fill_(gc.CANARY_I64)


def _equal(ref, got, ctx):
    for k, v in ref.items():
        if not torch.equal(v, got[k]):
            bad = (v != got[k]).nonzero()
            raise AssertionError(f"{ctx} {k}: {bad.shape[0]} elements differ, first {bad[0].tolist()}")


@pytest.mark.parametrize("name,n,packed", [("small", 100_003, True), ("mixed", 300_001, True),
                                           ("mixed", 300_001, False), ("mrheavy", 200_003, True),
                                           ("tiny", None, True)])
def test_graph_replays_match_eager(name, n, packed):
    d = synth.generate(name, n=n)
    if not d["lut_entries"]:
        # MR-heavy has no heap: give it the Mixed workload's table, so that
        # the graph holds the record-path lookup next to a PRP build.
        m = synth.generate("mixed", n=16)
        d.update(lut=m["lut"], lut_entries=m["lut_entries"], qid=np.zeros(d["n"], np.uint32),
                 nqueues=1)
    if not d["nqueues"]:
        d.update(qid=np.zeros(d["n"], np.uint32), nqueues=1)
    gc.say(f"graph {name} n={d['n']} packed={packed}")
    p = Path(d, packed)
    p.pool.view(torch.int64).fill_(gc.CANARY_I64)
    p.run()                                   # eager: allocates the outputs
    torch.cuda.synchronize()
    ref = p.outputs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        p.run()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        p.run()
    other = synth.generate("small", n=50_001)
    oq = gc.dev(other["qid"])
    for r in range(4):
        p.poison()
        # Eager work between the replays, on the same workspaces' neighbours.
        dd.partition_by_queue(oq, 64, check=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _equal(ref, p.outputs(), f"{name} replay {r}")
        blocks, expired = gc.host(p.ws_prp[:8]).view(np.uint32)
        assert expired == 0, (name, r)
    # And an eager call after the replays still gives the same outputs.
    p.poison()
    p.run()
    torch.cuda.synchronize()
    _equal(ref, p.outputs(), f"{name} eager after replays")
