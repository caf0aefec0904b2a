"""Seeded synthetic workloads for the batched DMA-descriptor path.

Thin ctypes wrapper over ``synth.c``. It only draws inputs (GPU-page
physical-address table, registered-region table, SoA request batch); it holds
none of the method's arithmetic, so both the CPU oracle and the GPU library
can consume what it returns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")

WORKLOADS = {"tiny": 1, "small": 2, "large": 3, "mrheavy": 4, "mixed": 5}

HEAP_VA_BASE = 0x0000700000000000
PHYS_BASE = 0x0000200000000000
LIST_BUS_BASE = 0x0000100000000000
NS_BLOCKS = 1 << 40
SLBA_STREAM = 0x51BA51BA51BA51BA


class _Shape(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_uint64),
        ("lut_entries", ctypes.c_uint64),
        ("regions", ctypes.c_uint64),
        ("nqueues", ctypes.c_uint32),
        ("page_shift", ctypes.c_uint32),
        ("va_base", ctypes.c_uint64),
        ("list_bus_base", ctypes.c_uint64),
        ("default_seed", ctypes.c_uint64),
    ]


def build() -> str:
    """Compile libsynth.so with the host C compiler."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _SO, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        p64 = ctypes.POINTER(ctypes.c_uint64)
        p32 = ctypes.POINTER(ctypes.c_uint32)
        lib.synth_shape_of.argtypes = [ctypes.c_int, ctypes.POINTER(_Shape)]
        lib.synth_shape_of.restype = ctypes.c_int
        lib.synth_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, p64]
        lib.synth_splitmix64.restype = None
        lib.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   p64, p64, p64, p32, p64, p64, p32]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill_slba.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, p64]
        lib.synth_fill_slba.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def _ptr(a, ctype):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def shape(name: str) -> dict:
    s = _Shape()
    if _lib().synth_shape_of(WORKLOADS[name], ctypes.byref(s)) != 0:
        raise ValueError(name)
    return {f: getattr(s, f) for f, _ in _Shape._fields_}


def splitmix64(seed: int, k: int) -> np.ndarray:
    out = np.empty(k, dtype=np.uint64)
    _lib().synth_splitmix64(seed, k, _ptr(out, ctypes.c_uint64))
    return out


def generate(name: str, n: int | None = None, seed: int = 0) -> dict:
    """Draws workload `name` with `n` requests (default: the workload's own
    count). Returns a dict with the shape fields and the arrays ``lut``,
    ``rstart``, ``rend``, ``rlkey``, ``off``, ``len``, ``qid`` (empty arrays
    where the workload has none)."""
    sh = shape(name)
    if n is None:
        n = sh["n"]
    P, R = sh["lut_entries"], sh["regions"]
    lut = np.empty(P, dtype=np.uint64)
    rstart = np.empty(R, dtype=np.uint64)
    rend = np.empty(R, dtype=np.uint64)
    rlkey = np.empty(R, dtype=np.uint32)
    off = np.empty(n, dtype=np.uint64)
    ln = np.empty(n, dtype=np.uint64)
    qid = np.empty(n, dtype=np.uint32)
    rc = _lib().synth_fill(WORKLOADS[name], seed, n,
                           _ptr(lut, ctypes.c_uint64), _ptr(rstart, ctypes.c_uint64),
                           _ptr(rend, ctypes.c_uint64), _ptr(rlkey, ctypes.c_uint32),
                           _ptr(off, ctypes.c_uint64), _ptr(ln, ctypes.c_uint64),
                           _ptr(qid, ctypes.c_uint32))
    if rc != 0:
        raise RuntimeError(f"synth_fill({name}) failed")
    out = dict(sh)
    out.update(name=name, n=n, lut=lut, rstart=rstart, rend=rend, rlkey=rlkey,
               off=off, len=ln, qid=qid)
    return out


def slba(name: str, n: int, seed: int = 0) -> np.ndarray:
    """Starting logical block of each of `n` requests of workload `name`
    (uniform over the namespace, room left for a 65536-block command)."""
    out = np.empty(n, dtype=np.uint64)
    if _lib().synth_fill_slba(WORKLOADS[name], seed, n, _ptr(out, ctypes.c_uint64)) != 0:
        raise ValueError(name)
    return out


QID_STREAM = 0x51D_51D_51D_51D


def queue_ids(n: int, nqueues: int, seed: int = 0, exponent: float = 1.1) -> np.ndarray:
    """Seeded destination queues for `n` requests: Zipf over `nqueues` queues
    with the given exponent (the Mixed workload's 1.1 over 64), drawn by
    inverting the cumulative weights with SplitMix64 uniforms."""
    w = np.arange(1, nqueues + 1, dtype=np.float64) ** -exponent
    cdf = np.cumsum(w) / w.sum()
    u = (splitmix64((seed or QID_STREAM) ^ QID_STREAM, n) >> np.uint64(11)).astype(np.float64) \
        / float(1 << 53)
    return np.minimum(np.searchsorted(cdf, u, side="right"), nqueues - 1).astype(np.uint32)


PUT_HEAP = 256 << 30          # symmetric heap of the put workload
PUT_CHUNK_SHIFT = 21          # 2 MiB chunks
PUT_NPES = 8
PUT_LOCAL_BASE = 0x0000600000000000
PUT_STREAM = 0x9075_9075_9075_9075


def put_batch(n: int, seed: int = 0, heap: int = PUT_HEAP, chunk_shift: int = PUT_CHUNK_SHIFT,
              npes: int = PUT_NPES) -> dict:
    """Seeded puts on a symmetric heap: lengths log-uniform 512 B .. 1 MiB in
    512 B steps (as the Mixed requests), source and destination offsets
    uniform and 4-byte aligned with room for the length, destination PE
    uniform; random nonzero 32-bit keys per chunk (local, and per PE remote)
    and one heap base per PE. Draws come from SplitMix64 streams."""
    r = splitmix64((seed or PUT_STREAM) ^ PUT_STREAM, 4 * n)
    u = (r[:n] >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    k = np.clip(np.floor(2049.0 ** u), 1, 2048).astype(np.uint64)
    length = k * np.uint64(512)
    room = np.uint64(heap) - length
    src = ((r[n:2 * n] % (room // np.uint64(4) + np.uint64(1))) * np.uint64(4))
    dst = ((r[2 * n:3 * n] % (room // np.uint64(4) + np.uint64(1))) * np.uint64(4))
    pe = (r[3 * n:] % np.uint64(npes)).astype(np.uint32)
    nchunks = heap >> chunk_shift if chunk_shift else 1
    kr = splitmix64(((seed or PUT_STREAM) ^ PUT_STREAM) + 1, nchunks * (npes + 1))
    keys = (kr >> np.uint64(32)).astype(np.uint32) | np.uint32(1)
    peer_base = np.uint64(0x0000400000000000) + np.arange(npes, dtype=np.uint64) * np.uint64(1 << 40)
    return dict(src=src, dst=dst, len=length, pe=pe, lkeys=keys[:nchunks],
                rkeys=keys[nchunks:], peer_base=peer_base, local_base=PUT_LOCAL_BASE,
                heap=heap, chunk_shift=chunk_shift, npes=npes)
