"""ctypes wrapper over the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library. Argument
marshalling only; every computation happens in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1 selects a build with AddressSanitizer and
# UndefinedBehaviorSanitizer (any report aborts); the process must then be
# started with the ASan runtime preloaded (LD_PRELOAD=$(gcc
# -print-file-name=libasan.so), ASAN_OPTIONS=detect_leaks=0), as
# tests/test_oracle_sanitized.py does.
SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_SO = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")

MISS, EXACT, CONTAINED, INVALID = 0, 1, 2, 3
OK, EINVAL, ERANGE, ENOSPC = 0, 1, 2, 3
REG_INVALID, REG_HIT, REG_NEW, REG_HIT_NEW, REG_NOSPACE = 0, 1, 2, 3, 4
DEREG_OK, DEREG_REMOVED, DEREG_STALE = 0, 1, 2


def build(sanitize: bool | None = None) -> str:
    """Compile the oracle with the host C compiler (single-threaded, -O2), or
    with ASan + UBSan (-O1, every report fatal) when sanitize is set (default:
    ORACLE_SANITIZE=1 in the environment)."""
    san = SANITIZE if sanitize is None else sanitize
    so = os.path.join(_HERE, "liboracle_san.so" if san else "liboracle.so")
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"] if san else ["-O2"])
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", so, _SRC]
    subprocess.run(cmd, check=True)
    return so


_lib_handle = None
_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        lib.orc_mr_lookup.argtypes = [_u64p, _u64p, _u32p, u64, ctypes.c_uint,
                                      _u64p, _u64p, u64, u64,
                                      _i32p, _u32p, _u8p, _u64p, _u64p]
        lib.orc_mr_lookup.restype = None
        lib.orc_build_prp.argtypes = [_u64p, u64, _u64p, _u64p, u64, u64, _u64p, u64,
                                      _u64p, _u64p, _u8p, _u64p]
        lib.orc_build_prp.restype = None
        lib.orc_build_prp_packed.argtypes = lib.orc_build_prp.argtypes
        lib.orc_build_prp_packed.restype = None
        lib.orc_partition.argtypes = [_u32p, u64, u32, _u32p, _u64p, _u64p]
        lib.orc_partition.restype = None
        lib.orc_emit_sqe.argtypes = [_u32p, _u64p, u32, _u8p, _u64p, _u64p, _u64p, _u64p, u64,
                                     ctypes.c_uint8, u32, ctypes.c_uint,
                                     ctypes.POINTER(_u8p), _u32p, _u32p, _u32p, _u64p, _u32p,
                                     _u32p]
        lib.orc_emit_sqe.restype = None
        lib.orc_build_put.argtypes = [_u64p, _u64p, _u64p, _u32p, u64, u64, u64, ctypes.c_uint,
                                      _u32p, _u64p, _u32p, u32, ctypes.c_void_p, u64,
                                      _u64p, _u32p, _u8p, _u64p]
        lib.orc_build_put.restype = None
        lib.orc_cq_drain.argtypes = [_u32p, _u32p, u32, u32, _u32p, _u32p, _u32p]
        lib.orc_cq_drain.restype = u64
        lib.orc_reg_create.argtypes = [ctypes.c_uint]
        lib.orc_reg_create.restype = ctypes.c_void_p
        lib.orc_reg_destroy.argtypes = [ctypes.c_void_p]
        lib.orc_reg_destroy.restype = None
        lib.orc_reg_register.argtypes = [ctypes.c_void_p, u64, u64]
        lib.orc_reg_register.restype = u64
        lib.orc_reg_deregister.argtypes = [ctypes.c_void_p, u64]
        lib.orc_reg_deregister.restype = ctypes.c_int
        lib.orc_reg_refs.argtypes = [ctypes.c_void_p, u64]
        lib.orc_reg_refs.restype = ctypes.c_int64
        lib.orc_reg_count.argtypes = [ctypes.c_void_p]
        lib.orc_reg_count.restype = u64
        lib.orc_reg_capacity.argtypes = [ctypes.c_void_p]
        lib.orc_reg_capacity.restype = u64
        lib.orc_reg_export.argtypes = [ctypes.c_void_p, _u64p, _u64p, _u64p, u64]
        lib.orc_reg_export.restype = u64
        lib.orc_reg_next_id.argtypes = [ctypes.c_void_p]
        lib.orc_reg_next_id.restype = u64
        lib.orc_reg_register_batch.argtypes = [ctypes.c_void_p, u64, _u64p, _u64p, u64,
                                               _u64p, _u8p]
        lib.orc_reg_register_batch.restype = u64
        lib.orc_reg_deregister_batch.argtypes = [ctypes.c_void_p, _u64p, u64, _u8p]
        lib.orc_reg_deregister_batch.restype = None
        _lib_handle = lib
    return _lib_handle


def _p(a, t):
    if a is None:
        return ctypes.cast(None, t)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _u64(a):
    return np.ascontiguousarray(a, dtype=np.uint64)


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.uint32)


def mr_lookup(start, end, lkey, off, length, va_base=0, page_shift=12):
    start, end, off, length = _u64(start), _u64(end), _u64(off), _u64(length)
    lkey = _u32(lkey)
    n = off.shape[0]
    out = dict(handle=np.empty(n, np.int32), lkey=np.empty(n, np.uint32),
               kind=np.empty(n, np.uint8), rbase=np.empty(n, np.uint64),
               rend=np.empty(n, np.uint64))
    _lib().orc_mr_lookup(_p(start, _u64p), _p(end, _u64p), _p(lkey, _u32p),
                         start.shape[0], page_shift, _p(off, _u64p), _p(length, _u64p),
                         n, va_base, _p(out["handle"], _i32p), _p(out["lkey"], _u32p),
                         _p(out["kind"], _u8p), _p(out["rbase"], _u64p),
                         _p(out["rend"], _u64p))
    return out


def build_prp(lut, off, length, list_bus_base, pool_pages, pool=None):
    """Runs O2. `pool` is None (lists not written), True (allocate a zeroed
    u64[pool_pages][512]) or a caller-owned u64 array of that shape."""
    lut, off, length = _u64(lut), _u64(off), _u64(length)
    n = off.shape[0]
    if pool is True:
        pool = np.zeros((pool_pages, 512), dtype=np.uint64)
    if pool is not None:
        assert pool.dtype == np.uint64 and pool.size >= pool_pages * 512
    out = dict(prp1=np.empty(n, np.uint64), prp2=np.empty(n, np.uint64),
               status=np.empty(n, np.uint8))
    total = np.zeros(1, np.uint64)
    _lib().orc_build_prp(_p(lut, _u64p), lut.shape[0], _p(off, _u64p), _p(length, _u64p),
                         n, list_bus_base, _p(pool, _u64p), pool_pages,
                         _p(out["prp1"], _u64p), _p(out["prp2"], _u64p),
                         _p(out["status"], _u8p), _p(total, _u64p))
    out["total"] = int(total[0])
    out["pool"] = pool
    return out


def build_prp_packed(lut, off, length, list_bus_base, pool_pages, pool=None):
    """Runs O2p (packed lists); arguments and result as build_prp."""
    lut, off, length = _u64(lut), _u64(off), _u64(length)
    n = off.shape[0]
    if pool is True:
        pool = np.zeros((pool_pages, 512), dtype=np.uint64)
    if pool is not None:
        assert pool.dtype == np.uint64 and pool.size >= pool_pages * 512
    out = dict(prp1=np.empty(n, np.uint64), prp2=np.empty(n, np.uint64),
               status=np.empty(n, np.uint8))
    total = np.zeros(1, np.uint64)
    _lib().orc_build_prp_packed(_p(lut, _u64p), lut.shape[0], _p(off, _u64p),
                                _p(length, _u64p), n, list_bus_base, _p(pool, _u64p),
                                pool_pages, _p(out["prp1"], _u64p), _p(out["prp2"], _u64p),
                                _p(out["status"], _u8p), _p(total, _u64p))
    out["total"] = int(total[0])
    out["pool"] = pool
    return out


def partition(qid, nqueues):
    qid = _u32(qid)
    n = qid.shape[0]
    perm = np.empty(n, np.uint32)
    qoff = np.empty(nqueues + 2, np.uint64)
    ninv = np.zeros(1, np.uint64)
    _lib().orc_partition(_p(qid, _u32p), n, nqueues, _p(perm, _u32p), _p(qoff, _u64p),
                         _p(ninv, _u64p))
    return dict(perm=perm, qoff=qoff, n_invalid=int(ninv[0]))


def emit_sqe(perm, qoff, status, length, slba, prp1, prp2, rings, depth, free_slots,
             tail, cursor, req_of_slot=None, opcode=0x02, nsid=1, lba_shift=9):
    """Runs O5 for one call. `rings` is a list of u8[depth[q], 64] arrays (or
    None for a refused queue) and `req_of_slot` a u32[nqueues, 65536] array
    (or None); both are updated in place. Returns dict(tail, cursor, placed)
    with new arrays."""
    perm, qoff = _u32(perm), _u64(qoff)
    status = np.ascontiguousarray(status, dtype=np.uint8)
    length, slba, prp1, prp2 = _u64(length), _u64(slba), _u64(prp1), _u64(prp2)
    nq = len(rings)
    depth, free_slots = _u32(depth), _u32(free_slots)
    tail, cursor = _u32(tail).copy(), _u64(cursor).copy()
    n = length.shape[0]
    placed = np.zeros(nq, np.uint32)
    if req_of_slot is not None:
        assert req_of_slot.dtype == np.uint32 and req_of_slot.size >= nq * 65536
    ring_ptrs = (_u8p * max(nq, 1))()
    for q, r in enumerate(rings):
        if r is not None:
            assert r.dtype == np.uint8 and r.flags["C_CONTIGUOUS"] and r.size >= int(depth[q]) * 64
            ring_ptrs[q] = r.ctypes.data_as(_u8p)
    _lib().orc_emit_sqe(_p(perm, _u32p), _p(qoff, _u64p), nq, _p(status, _u8p),
                        _p(length, _u64p), _p(slba, _u64p), _p(prp1, _u64p), _p(prp2, _u64p),
                        n, opcode, nsid, lba_shift, ring_ptrs, _p(depth, _u32p),
                        _p(free_slots, _u32p), _p(tail, _u32p), _p(cursor, _u64p),
                        _p(placed, _u32p), _p(req_of_slot, _u32p))
    return dict(tail=tail, cursor=cursor, placed=placed)


PUT_DESC = np.dtype([("laddr", "<u8"), ("raddr", "<u8"), ("len", "<u4"), ("lkey", "<u4"),
                     ("rkey", "<u4"), ("req", "<u4")])


def build_put(src, dst, nbytes, pe, local_base, heap_bytes, chunk_shift, lkeys, peer_base,
              rkeys, desc_cap, write=True, desc=None):
    """Runs O6; returns dict(desc (PUT_DESC[desc_cap] or None), first, count,
    status, total). `desc` may be a caller array of PUT_DESC[desc_cap]."""
    src, dst, nbytes, pe = _u64(src), _u64(dst), _u64(nbytes), _u32(pe)
    lkeys, peer_base, rkeys = _u32(lkeys), _u64(peer_base), _u32(rkeys)
    n = src.shape[0]
    if desc is None:
        desc = np.zeros(desc_cap, PUT_DESC) if write else None
    else:
        assert desc.dtype == PUT_DESC and desc.shape[0] >= desc_cap
    out = dict(first=np.empty(n, np.uint64), count=np.empty(n, np.uint32),
               status=np.empty(n, np.uint8))
    total = np.zeros(1, np.uint64)
    _lib().orc_build_put(_p(src, _u64p), _p(dst, _u64p), _p(nbytes, _u64p), _p(pe, _u32p), n,
                         local_base, heap_bytes, chunk_shift, _p(lkeys, _u32p),
                         _p(peer_base, _u64p), _p(rkeys, _u32p), peer_base.shape[0],
                         desc.ctypes.data if write else None, desc_cap,
                         _p(out["first"], _u64p), _p(out["count"], _u32p),
                         _p(out["status"], _u8p), _p(total, _u64p))
    out["desc"] = desc
    out["total"] = int(total[0])
    return out


def cq_drain(src, dst, gen, head, phase, ack):
    """Runs O7 on u32[depth, 4] arrays (dst updated in place); returns
    (copied, head, phase, ack)."""
    assert src.dtype == np.uint32 and dst.dtype == np.uint32 and src.flags["C_CONTIGUOUS"]
    h, p, a = (np.array([v], np.uint32) for v in (head, phase, ack))
    c = _lib().orc_cq_drain(_p(src, _u32p), _p(dst, _u32p), src.shape[0], gen, _p(h, _u32p),
                            _p(p, _u32p), _p(a, _u32p))
    return int(c), int(h[0]), int(p[0]), int(a[0])


class Registry:
    """Refcounted registration cache (O4)."""

    def __init__(self, page_shift=12):
        self._h = _lib().orc_reg_create(page_shift)

    def __del__(self):
        if getattr(self, "_h", None):
            _lib().orc_reg_destroy(self._h)
            self._h = None

    def register(self, addr, size):
        return int(_lib().orc_reg_register(self._h, addr, size))

    def deregister(self, handle):
        return int(_lib().orc_reg_deregister(self._h, handle))

    def refs(self, handle):
        return int(_lib().orc_reg_refs(self._h, handle))

    def count(self):
        return int(_lib().orc_reg_count(self._h))

    def capacity(self):
        return int(_lib().orc_reg_capacity(self._h))

    def table(self):
        k = self.count()
        s, e, h = (np.empty(k, np.uint64) for _ in range(3))
        _lib().orc_reg_export(self._h, _p(s, _u64p), _p(e, _u64p), _p(h, _u64p), k)
        return s, e, h

    def next_id(self):
        return int(_lib().orc_reg_next_id(self._h))

    def register_batch(self, addr, size, capacity):
        """O4b register batch; returns (handle u64[n], kind u8[n], needed capacity)."""
        addr, size = _u64(addr), _u64(size)
        n = addr.shape[0]
        h, k = np.empty(n, np.uint64), np.empty(n, np.uint8)
        need = _lib().orc_reg_register_batch(self._h, capacity, _p(addr, _u64p),
                                             _p(size, _u64p), n, _p(h, _u64p), _p(k, _u8p))
        return h, k, int(need)

    def deregister_batch(self, handles):
        """O4b deregister batch; returns status u8[n]."""
        handles = _u64(handles)
        st = np.empty(handles.shape[0], np.uint8)
        _lib().orc_reg_deregister_batch(self._h, _p(handles, _u64p), handles.shape[0],
                                        _p(st, _u8p))
        return st

    def records(self):
        """(start, end, handle, refs) of the live records in sorted order."""
        s, e, h = self.table()
        refs = np.array([self.refs(int(x)) for x in h], dtype=np.int64)
        return s, e, h, refs
