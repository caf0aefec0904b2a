"""Pins of the oracle's completion-queue drain (O7) against a controller
model: every completion written comes out once, in order, across drains and
wraps; an even generation is acknowledged with the odd value before it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf


@pytest.mark.parametrize("depth", [2, 3, 64, 1000])
def test_drains_follow_the_controller(depth):
    ctl = bf.CqController(depth, seed=depth)
    dst = np.zeros((depth, 4), np.uint32)
    head, phase, ack = 0, 1, 0
    out = []
    rng = np.random.default_rng(depth)
    for _ in range(50):
        # A controller never has more than depth - 1 completions outstanding.
        k = int(rng.integers(0, depth))
        ctl.complete(k)
        h0 = head
        c, head, phase, ack = oracle.cq_drain(ctl.cq, dst, 7, head, phase, ack)
        assert c == k and ack == 0
        out += [dst[(h0 + j) % depth].copy() for j in range(c)]
        assert head == ctl.tail and phase == ctl.phase
    assert len(out) == len(ctl.log)
    assert all((a == b).all() for a, b in zip(out, ctl.log))


def test_nothing_new_copies_nothing():
    ctl = bf.CqController(8)
    ctl.complete(5)
    dst = np.zeros((8, 4), np.uint32)
    c, h, p, a = oracle.cq_drain(ctl.cq, dst, 1, 0, 1, 0)
    assert (c, h, p) == (5, 5, 1)
    before = dst.copy()
    assert oracle.cq_drain(ctl.cq, dst, 1, h, p, a)[0] == 0
    assert (dst == before).all()


def test_even_generation_is_acknowledged():
    ctl = bf.CqController(8)
    ctl.complete(3)
    dst = np.zeros((8, 4), np.uint32)
    c, h, p, a = oracle.cq_drain(ctl.cq, dst, 6, 0, 1, 0)
    assert (c, h, p, a) == (0, 0, 1, 5) and (dst == 0).all()
