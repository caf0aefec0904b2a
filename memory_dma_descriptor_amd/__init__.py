"""dmadesc: batched DMA-descriptor building on AMD MI355X (gfx950).

Thin binding over the C ABI of libdmadesc.so (include/dmadesc.h): argument
marshalling only. Every step runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream. There is no CPU fallback: if
the library cannot be loaded, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

__all__ = ["mr_lookup", "build_prp", "build_prp_packed", "build_prp_packed_noalloc",
           "build_batch", "batch_workspace_bytes", "BATCH_PACKED",
           "partition_by_queue", "emit_sqe",
           "ring_addresses", "DeviceRegistry", "build_put", "cq_slots", "cq_attach",
           "cq_mirror", "cq_slot_state",
           "workspace_bytes", "DmadescError", "DmadescRefused", "lib", "LIB_PATH", "MAX_QUEUES",
           "SQ_MAX_DEPTH",
           "mr_table_check", "debug_wait_limit", "DEFAULT_WAIT_POLLS",
           "MISS", "EXACT", "CONTAINED", "INVALID",
           "PRP_OK", "PRP_EINVAL", "PRP_ERANGE", "PRP_ENOSPC", "PRP_EBUSY"]

LIB_PATH = _build.LIB
MAX_QUEUES = 256
SQ_MAX_DEPTH = 65536
OP_MR_LOOKUP, OP_BUILD_PRP, OP_PARTITION, OP_EMIT_SQE, OP_REGISTRY, OP_BUILD_PUT = 1, 2, 3, 4, 5, 6
REG_MAX_BATCH, REG_MAX_CAPACITY = 65536, 1 << 24
REG_INVALID, REG_HIT, REG_NEW, REG_HIT_NEW, REG_NOSPACE = 0, 1, 2, 3, 4
DEREG_OK, DEREG_REMOVED, DEREG_STALE = 0, 1, 2
MISS, EXACT, CONTAINED, INVALID = 0, 1, 2, 3
PRP_OK, PRP_EINVAL, PRP_ERANGE, PRP_ENOSPC, PRP_EBUSY = 0, 1, 2, 3, 4
DEFAULT_WAIT_POLLS = 1 << 22

_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32
_SIZE = ctypes.c_size_t

_EXPORTS = {
    "dmadesc_mr_lookup": ([_P, _P, _P, _U32, _U32, _P, _P, _U64, _U64,
                           _P, _P, _P, _P, _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_mr_table_check": ([_P, _P, _U32, _U32, _P, _P, _P], ctypes.c_int),
    "dmadesc_build_prp": ([_P, _U64, _P, _P, _U64, _U64, _P, _U64,
                           _P, _P, _P, _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_build_prp_packed": ([_P, _U64, _P, _P, _U64, _U64, _P, _U64,
                                  _P, _P, _P, _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_build_prp_packed_noalloc": ([_P, _U64, _P, _P, _U64, _U64, _P, _U64,
                                          _P, _P, _P, _P, _P], ctypes.c_int),
    "dmadesc_partition_by_queue": ([_P, _U64, _U32, _P, _P, _P, _P, _SIZE, _P],
                                   ctypes.c_int),
    "dmadesc_emit_sqe": ([_P, _P, _U32, _P, _P, _P, _P, _P, _U64, _U32, _U32, _U32,
                          _P, _P, _P, _P, _P, _P, _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_build_put": ([_P, _P, _P, _P, _U64, _U64, _U64, _U32, _P, _P, _P, _U32, _P, _U64,
                           _P, _P, _P, _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_cq_mirror": ([_P, _U32, _P, _U32, _P], ctypes.c_int),
    "dmadesc_reg_register": ([_P, _P, _P, _P, _P, _P, _U64, _U32, _P, _P, _U64, _P, _P, _P,
                              _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_reg_deregister": ([_P, _P, _P, _P, _P, _P, _U64, _P, _U64, _P, _P, _SIZE, _P],
                               ctypes.c_int),
    "dmadesc_build_batch": ([_P, _P, _P, _U32, _U32, _U64, _P, _U64, _P, _P, _P, _U64, _U32,
                             _U64, _P, _U64, _U32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _P, _P, _SIZE, _P], ctypes.c_int),
    "dmadesc_batch_workspace_bytes": ([_U64, _U32, _U32], _SIZE),
    "dmadesc_workspace_bytes": ([ctypes.c_int, _U64, _U32], _SIZE),
    "dmadesc_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "dmadesc_version": ([], ctypes.c_int),
    "dmadesc_debug_wait_limit": ([_U32], _U32),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Loads libdmadesc.so (building it in-tree first if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            _build.build()
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _EXPORTS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


class DmadescError(RuntimeError):
    def __init__(self, func: str, rc: int, detail: str = ""):
        msg = lib().dmadesc_strerror(rc).decode()
        super().__init__(f"{func} returned {rc}: {msg}" + (f" ({detail})" if detail else ""))
        self.rc = rc


class DmadescRefused(RuntimeError):
    """A call succeeded but refused part of its batch in a way the caller must
    act on: a slot-scan wait that expired (requests with PRP_EBUSY), or queue
    ids outside the queues (the split's overflow bucket). Raised after the
    stream is synchronized when the call was made with check=True; the
    outputs are complete and attached as `out`."""

    def __init__(self, msg: str, out: dict):
        super().__init__(msg)
        self.out = out


def _u32_at(t: torch.Tensor, byte: int) -> int:
    return int(t[byte:byte + 4].view(torch.int32).item()) & 0xFFFFFFFF


def _check_scan(func: str, ws: torch.Tensor, stream_dev, stream, out: dict) -> None:
    """After synchronizing, raises DmadescRefused when the slot scan's header
    (workspace bytes 4..7) counts blocks whose wait expired."""
    s = stream if stream is not None else torch.cuda.current_stream(stream_dev)
    s.synchronize()
    expired = _u32_at(ws, 4)
    if expired:
        raise DmadescRefused(f"{func}: the slot-scan wait of {expired} block(s) expired; "
                             "their requests carry PRP_EBUSY", out)


def _check(func: str, rc: int) -> None:
    if rc != 0:
        raise DmadescError(func, rc)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, n: int | None = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")
    return t.data_ptr() if t.numel() else 0


def _stream(device: torch.device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def workspace_bytes(op: int, n: int, param: int = 0) -> int:
    return int(lib().dmadesc_workspace_bytes(op, n, param))


def _workspace(op: int, n: int, param: int, device, ws):
    """(tensor, pointer, bytes) of a device workspace for `op`: the caller's
    `ws` (a contiguous uint8 device tensor, checked) or a new one."""
    need = workspace_bytes(op, n, param)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    ptr = _dev(ws, torch.uint8, "ws")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace needs {need} bytes, got {nbytes}")
    return ws, ptr, nbytes


def mr_lookup(reg_start: torch.Tensor, reg_end: torch.Tensor, reg_lkey: torch.Tensor,
              off: torch.Tensor, length: torch.Tensor, va_base: int = 0,
              page_shift: int = 12, out: dict | None = None, stream=None,
              ws: torch.Tensor | None = None, records: bool = True) -> dict:
    """Page-rounded containment lookup; returns dict(handle, lkey, kind, rbase, rend).
    Tables of more than 4,096 regions take the record path through a
    workspace (`ws`, or a new one); records=False passes none."""
    n, r = off.numel(), reg_start.numel()
    dev = off.device
    ws_ptr, ws_bytes = None, 0
    if records and workspace_bytes(OP_MR_LOOKUP, n, r) > 0:
        ws, ws_ptr, ws_bytes = _workspace(OP_MR_LOOKUP, n, r, dev, ws)
    if out is None:
        out = dict(handle=torch.empty(n, dtype=torch.int32, device=dev),
                   lkey=torch.empty(n, dtype=torch.uint32, device=dev),
                   kind=torch.empty(n, dtype=torch.uint8, device=dev),
                   rbase=torch.empty(n, dtype=torch.uint64, device=dev),
                   rend=torch.empty(n, dtype=torch.uint64, device=dev))
    rc = lib().dmadesc_mr_lookup(
        _dev(reg_start, torch.uint64, "reg_start", r), _dev(reg_end, torch.uint64, "reg_end", r),
        _dev(reg_lkey, torch.uint32, "reg_lkey", r), r, page_shift,
        _dev(off, torch.uint64, "off", n), _dev(length, torch.uint64, "len", n), n, va_base,
        _dev(out["handle"], torch.int32, "handle", n), _dev(out["lkey"], torch.uint32, "lkey", n),
        _dev(out["kind"], torch.uint8, "kind", n), _dev(out["rbase"], torch.uint64, "rbase", n),
        _dev(out["rend"], torch.uint64, "rend", n), ws_ptr, ws_bytes, _stream(dev, stream))
    _check("dmadesc_mr_lookup", rc)
    return out


def mr_table_check(reg_start: torch.Tensor, reg_end: torch.Tensor, page_shift: int = 12,
                   stream=None) -> None:
    """Raises DmadescError(-EINVAL) naming the first faulty region unless the
    table is sorted, non-overlapping and page-aligned (dmadesc_mr_table_check;
    synchronizes the stream)."""
    r = reg_start.numel()
    dev = reg_start.device
    scratch = torch.empty(1, dtype=torch.uint64, device=dev)
    bad = ctypes.c_uint64(0)
    rc = lib().dmadesc_mr_table_check(
        _dev(reg_start, torch.uint64, "reg_start", r), _dev(reg_end, torch.uint64, "reg_end", r),
        r, page_shift, scratch.data_ptr(), ctypes.addressof(bad), _stream(dev, stream))
    if rc != 0:
        detail = f"region {bad.value} is empty, unaligned or overlaps the next" \
            if bad.value != (1 << 64) - 1 else ""
        raise DmadescError("dmadesc_mr_table_check", rc, detail)


def debug_wait_limit(polls: int) -> int:
    """Sets the bound on slot-scan waits for later calls (tests of the
    PRP_EBUSY path); returns the previous bound."""
    return int(lib().dmadesc_debug_wait_limit(polls))


def build_prp(lut: torch.Tensor, off: torch.Tensor, length: torch.Tensor,
              list_bus_base: int, pool: torch.Tensor, out: dict | None = None,
              ws: torch.Tensor | None = None, stream=None, packed: bool = False,
              check: bool = True) -> dict:
    """GPU-page table -> PRP1/PRP2/status and chained lists in `pool`
    (u64[pool_pages, 512]); returns dict(prp1, prp2, status, total_pages).
    packed=True calls dmadesc_build_prp_packed (lists back to back).
    check=True synchronizes the stream and raises DmadescRefused if a
    slot-scan wait expired (check=False leaves the call asynchronous; the
    caller then reads workspace bytes 4..7 itself)."""
    n = off.numel()
    dev = off.device
    if pool.dim() != 2 or pool.shape[1] != 512:
        raise ValueError("pool must have shape [pool_pages, 512]")
    if out is None:
        out = dict(prp1=torch.empty(n, dtype=torch.uint64, device=dev),
                   prp2=torch.empty(n, dtype=torch.uint64, device=dev),
                   status=torch.empty(n, dtype=torch.uint8, device=dev),
                   total_pages=torch.empty(1, dtype=torch.uint64, device=dev))
    ws = _workspace(OP_BUILD_PRP, n, 0, dev, ws)
    fn = lib().dmadesc_build_prp_packed if packed else lib().dmadesc_build_prp
    rc = fn(
        _dev(lut, torch.uint64, "lut"), lut.numel(),
        _dev(off, torch.uint64, "off", n), _dev(length, torch.uint64, "len", n), n,
        list_bus_base, _dev(pool, torch.uint64, "pool"), pool.shape[0],
        _dev(out["prp1"], torch.uint64, "prp1", n), _dev(out["prp2"], torch.uint64, "prp2", n),
        _dev(out["status"], torch.uint8, "status", n),
        _dev(out["total_pages"], torch.uint64, "total_pages", 1),
        *ws[1:], _stream(dev, stream))
    name = "dmadesc_build_prp_packed" if packed else "dmadesc_build_prp"
    _check(name, rc)
    if check and n:
        _check_scan(name, ws[0], dev, stream, out)
    return out


def build_prp_packed(lut: torch.Tensor, off: torch.Tensor, length: torch.Tensor,
                     list_bus_base: int, pool: torch.Tensor, out: dict | None = None,
                     ws: torch.Tensor | None = None, stream=None, check: bool = True) -> dict:
    """dmadesc_build_prp_packed: the same PRP entries, lists back to back."""
    return build_prp(lut, off, length, list_bus_base, pool, out=out, ws=ws, stream=stream,
                     packed=True, check=check)


NOALLOC_MAX_N = 1 << 27


def build_prp_packed_noalloc(lut: torch.Tensor, off: torch.Tensor, length: torch.Tensor,
                             list_bus_base: int, pool: torch.Tensor, out: dict,
                             stream=None) -> dict:
    """dmadesc_build_prp_packed_noalloc: the packed build with the library's
    static scratch in place of a workspace. `out` (prp1, prp2, status,
    total_pages) is required, so that nothing is allocated here either."""
    n = off.numel()
    dev = off.device
    if pool.dim() != 2 or pool.shape[1] != 512:
        raise ValueError("pool must have shape [pool_pages, 512]")
    rc = lib().dmadesc_build_prp_packed_noalloc(
        _dev(lut, torch.uint64, "lut"), lut.numel(),
        _dev(off, torch.uint64, "off", n), _dev(length, torch.uint64, "len", n), n,
        list_bus_base, _dev(pool, torch.uint64, "pool"), pool.shape[0],
        _dev(out["prp1"], torch.uint64, "prp1", n), _dev(out["prp2"], torch.uint64, "prp2", n),
        _dev(out["status"], torch.uint8, "status", n),
        _dev(out["total_pages"], torch.uint64, "total_pages", 1), _stream(dev, stream))
    _check("dmadesc_build_prp_packed_noalloc", rc)
    return out


def partition_by_queue(qid: torch.Tensor, nqueues: int, out: dict | None = None,
                       ws: torch.Tensor | None = None, stream=None, check: bool = True) -> dict:
    """Stable split by queue id; returns dict(perm, qoff, n_invalid).
    check=True synchronizes the stream and raises DmadescRefused when some
    queue ids are >= nqueues (they sit, stably, in the overflow bucket);
    check=False leaves the call asynchronous."""
    n = qid.numel()
    dev = qid.device
    if out is None:
        out = dict(perm=torch.empty(n, dtype=torch.uint32, device=dev),
                   qoff=torch.empty(nqueues + 2, dtype=torch.uint64, device=dev),
                   n_invalid=torch.empty(1, dtype=torch.uint64, device=dev))
    ws = _workspace(OP_PARTITION, n, nqueues, dev, ws)
    rc = lib().dmadesc_partition_by_queue(
        _dev(qid, torch.uint32, "qid", n), n, nqueues,
        _dev(out["perm"], torch.uint32, "perm", n),
        _dev(out["qoff"], torch.uint64, "qoff", nqueues + 2),
        _dev(out["n_invalid"], torch.uint64, "n_invalid", 1),
        *ws[1:], _stream(dev, stream))
    _check("dmadesc_partition_by_queue", rc)
    if check:
        (stream if stream is not None else torch.cuda.current_stream(dev)).synchronize()
        bad = int(out["n_invalid"].view(torch.int64)[0].item())
        if bad:
            raise DmadescRefused(f"dmadesc_partition_by_queue: {bad} request(s) name a queue "
                                 f">= nqueues ({nqueues}); they are in the overflow bucket", out)
    return out


BATCH_PACKED = 1


def batch_workspace_bytes(n: int, nqueues: int, nregions: int) -> int:
    return int(lib().dmadesc_batch_workspace_bytes(n, nqueues, nregions))


def build_batch(lut: torch.Tensor, off: torch.Tensor, length: torch.Tensor,
                qid: torch.Tensor, nqueues: int, list_bus_base: int, pool: torch.Tensor,
                reg_start: torch.Tensor | None = None, reg_end: torch.Tensor | None = None,
                reg_lkey: torch.Tensor | None = None, va_base: int = 0, page_shift: int = 12,
                packed: bool = True, lookup: bool = True, out: dict | None = None,
                ws: torch.Tensor | None = None, stream=None, check: bool = True) -> dict:
    """dmadesc_build_batch: lookup (when lookup=True and a table is given),
    PRP build and split in one call. Returns one dict with the columns of
    mr_lookup, build_prp and partition_by_queue. check=True synchronizes and
    raises DmadescRefused on expired slot-scan waits or queue ids >= nqueues."""
    n = off.numel()
    dev = off.device
    if pool.dim() != 2 or pool.shape[1] != 512:
        raise ValueError("pool must have shape [pool_pages, 512]")
    lookup = lookup and reg_start is not None
    r = reg_start.numel() if lookup else 0
    if out is None:
        out = dict(prp1=torch.empty(n, dtype=torch.uint64, device=dev),
                   prp2=torch.empty(n, dtype=torch.uint64, device=dev),
                   status=torch.empty(n, dtype=torch.uint8, device=dev),
                   total_pages=torch.empty(1, dtype=torch.uint64, device=dev),
                   perm=torch.empty(n, dtype=torch.uint32, device=dev),
                   qoff=torch.empty(nqueues + 2, dtype=torch.uint64, device=dev),
                   n_invalid=torch.empty(1, dtype=torch.uint64, device=dev))
        if lookup:
            out.update(handle=torch.empty(n, dtype=torch.int32, device=dev),
                       lkey=torch.empty(n, dtype=torch.uint32, device=dev),
                       kind=torch.empty(n, dtype=torch.uint8, device=dev),
                       rbase=torch.empty(n, dtype=torch.uint64, device=dev),
                       rend=torch.empty(n, dtype=torch.uint64, device=dev))
    need = batch_workspace_bytes(n, nqueues, r)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    wptr = _dev(ws, torch.uint8, "ws")
    if ws.numel() < need:
        raise ValueError(f"workspace needs {need} bytes, got {ws.numel()}")
    if lookup:
        tbl = (_dev(reg_start, torch.uint64, "reg_start", r), _dev(reg_end, torch.uint64, "reg_end", r),
               _dev(reg_lkey, torch.uint32, "reg_lkey", r))
        lk = (_dev(out["handle"], torch.int32, "handle", n), _dev(out["lkey"], torch.uint32, "lkey", n),
              _dev(out["kind"], torch.uint8, "kind", n), _dev(out["rbase"], torch.uint64, "rbase", n),
              _dev(out["rend"], torch.uint64, "rend", n))
    else:
        tbl, lk = (None, None, None), (None,) * 5
    rc = lib().dmadesc_build_batch(
        *tbl, r, page_shift, va_base, _dev(lut, torch.uint64, "lut"), lut.numel(),
        _dev(off, torch.uint64, "off", n), _dev(length, torch.uint64, "len", n),
        _dev(qid, torch.uint32, "qid", n), n, nqueues, list_bus_base,
        _dev(pool, torch.uint64, "pool"), pool.shape[0], BATCH_PACKED if packed else 0, *lk,
        _dev(out["prp1"], torch.uint64, "prp1", n), _dev(out["prp2"], torch.uint64, "prp2", n),
        _dev(out["status"], torch.uint8, "status", n),
        _dev(out["total_pages"], torch.uint64, "total_pages", 1),
        _dev(out["perm"], torch.uint32, "perm", n),
        _dev(out["qoff"], torch.uint64, "qoff", nqueues + 2),
        _dev(out["n_invalid"], torch.uint64, "n_invalid", 1), wptr, ws.numel(),
        _stream(dev, stream))
    _check("dmadesc_build_batch", rc)
    if check:
        if n:
            _check_scan("dmadesc_build_batch", ws, dev, stream, out)
        else:
            (stream if stream is not None else torch.cuda.current_stream(dev)).synchronize()
        bad = int(out["n_invalid"].view(torch.int64)[0].item())
        if bad:
            raise DmadescRefused(f"dmadesc_build_batch: {bad} request(s) name a queue >= "
                                 f"nqueues ({nqueues})", out)
    return out


def ring_addresses(rings, device=None) -> torch.Tensor:
    """u64 device tensor of ring base addresses (None -> 0, a refused queue)
    from a list of device tensors holding depth x 64 bytes each."""
    addrs = [0 if r is None else r.data_ptr() for r in rings]
    if device is None:
        device = next(r.device for r in rings if r is not None)
    return torch.tensor(addrs, dtype=torch.int64).view(torch.uint64).to(device)


def emit_sqe(perm: torch.Tensor, qoff: torch.Tensor, status: torch.Tensor,
             length: torch.Tensor, slba: torch.Tensor, prp1: torch.Tensor,
             prp2: torch.Tensor, ring: torch.Tensor, depth: torch.Tensor,
             free_slots: torch.Tensor, tail: torch.Tensor, cursor: torch.Tensor,
             placed: torch.Tensor | None = None, req_of_slot: torch.Tensor | None = None,
             opcode: int = 0x02, nsid: int = 1, lba_shift: int = 9,
             ws: torch.Tensor | None = None, stream=None) -> dict:
    """NVMe submission entries for one window of each queue's bucket.
    `ring` holds each queue's ring address (see ring_addresses); `tail` and
    `cursor` are updated in place. Returns dict(placed, tail, cursor,
    req_of_slot)."""
    n = status.numel()
    nq = ring.numel()
    dev = status.device
    if placed is None:
        placed = torch.empty(nq, dtype=torch.uint32, device=dev)
    rid = 0
    if req_of_slot is not None:
        rid = _dev(req_of_slot, torch.uint32, "req_of_slot", nq * SQ_MAX_DEPTH)
    ws = _workspace(OP_EMIT_SQE, n, nq, dev, ws)
    rc = lib().dmadesc_emit_sqe(
        _dev(perm, torch.uint32, "perm", n), _dev(qoff, torch.uint64, "qoff", nq + 2), nq,
        _dev(status, torch.uint8, "status", n), _dev(length, torch.uint64, "len", n),
        _dev(slba, torch.uint64, "slba", n), _dev(prp1, torch.uint64, "prp1", n),
        _dev(prp2, torch.uint64, "prp2", n), n, opcode, nsid, lba_shift,
        _dev(ring, torch.uint64, "ring", nq), _dev(depth, torch.uint32, "depth", nq),
        _dev(free_slots, torch.uint32, "free_slots", nq), _dev(tail, torch.uint32, "tail", nq),
        _dev(cursor, torch.uint64, "cursor", nq), _dev(placed, torch.uint32, "placed", nq),
        rid, *ws[1:], _stream(dev, stream))
    _check("dmadesc_emit_sqe", rc)
    return dict(placed=placed, tail=tail, cursor=cursor, req_of_slot=req_of_slot)


def build_put(src: torch.Tensor, dst: torch.Tensor, nbytes: torch.Tensor, pe: torch.Tensor,
              local_base: int, heap_bytes: int, chunk_shift: int, lkeys: torch.Tensor,
              peer_base: torch.Tensor, rkeys: torch.Tensor, desc: torch.Tensor,
              out: dict | None = None, ws: torch.Tensor | None = None, stream=None,
              check: bool = True) -> dict:
    """RDMA put descriptors into `desc` (u64[desc_cap, 4], one 32-byte
    dmadesc_put_desc per row); returns dict(first, count, status, total).
    check=True synchronizes and raises DmadescRefused if a slot-scan wait
    expired."""
    n = src.numel()
    dev = src.device
    if desc.dim() != 2 or desc.shape[1] != 4:
        raise ValueError("desc must have shape [desc_cap, 4]")
    nchunks = heap_bytes >> chunk_shift if chunk_shift else 1
    if lkeys.numel() < nchunks or rkeys.numel() < peer_base.numel() * nchunks:
        raise ValueError("key tables smaller than the heap's chunks (lkeys[nchunks], "
                         "rkeys[npes * nchunks])")
    if out is None:
        out = dict(first=torch.empty(n, dtype=torch.uint64, device=dev),
                   count=torch.empty(n, dtype=torch.uint32, device=dev),
                   status=torch.empty(n, dtype=torch.uint8, device=dev),
                   total=torch.empty(1, dtype=torch.uint64, device=dev))
    ws = _workspace(OP_BUILD_PUT, n, 0, dev, ws)
    rc = lib().dmadesc_build_put(
        _dev(src, torch.uint64, "src", n), _dev(dst, torch.uint64, "dst", n),
        _dev(nbytes, torch.uint64, "bytes", n), _dev(pe, torch.uint32, "pe", n), n,
        local_base, heap_bytes, chunk_shift, _dev(lkeys, torch.uint32, "lkeys"),
        _dev(peer_base, torch.uint64, "peer_base"), _dev(rkeys, torch.uint32, "rkeys"),
        peer_base.numel(), _dev(desc, torch.uint64, "desc"), desc.shape[0],
        _dev(out["first"], torch.uint64, "first", n), _dev(out["count"], torch.uint32, "count", n),
        _dev(out["status"], torch.uint8, "status", n),
        _dev(out["total"], torch.uint64, "total", 1), *ws[1:], _stream(dev, stream))
    _check("dmadesc_build_put", rc)
    if check and n:
        _check_scan("dmadesc_build_put", ws[0], dev, stream, out)
    return out


# dmadesc_cq_slot as 6 little-endian u64 words: src, dst, depth | generation
# << 32, ack | head << 32, phase | reserved << 32, copied.
CQ_SLOT_WORDS = 6
CQ_MAX_SLOTS = 64


def cq_slots(n: int, device="cuda") -> torch.Tensor:
    """A zeroed table of n completion-queue mirror slots (u64[n, 6])."""
    if not 1 <= n <= CQ_MAX_SLOTS:
        raise ValueError(f"1..{CQ_MAX_SLOTS} slots")
    return torch.zeros((n, CQ_SLOT_WORDS), dtype=torch.int64, device=device).view(torch.uint64)


def cq_attach(slots: torch.Tensor, q: int, src: torch.Tensor, dst: torch.Tensor, depth: int,
              generation: int, head: int = 0, phase: int = 1) -> None:
    """Fills slot q (nothing copied; a fresh queue starts at head 0, phase 1)
    and then raises its generation (odd), on the current stream. src/dst:
    device tensors holding depth x 16 bytes."""
    if generation % 2 != 1:
        raise ValueError("an attached queue has an odd generation")
    if src.numel() * src.element_size() < 16 * depth or dst.numel() * dst.element_size() < 16 * depth:
        raise ValueError("src and dst must hold depth x 16 bytes")
    words = torch.tensor([src.data_ptr(), dst.data_ptr(), depth, head << 32, phase, 0],
                         dtype=torch.int64)
    row = slots[q].view(torch.int64)
    row.copy_(words.to(slots.device))
    row[2:3].copy_(torch.tensor([depth | (generation << 32)], dtype=torch.int64).to(slots.device))


def cq_mirror(slots: torch.Tensor, stop: torch.Tensor, idle_polls: int = 64, stream=None) -> None:
    """One resident call of the completion-queue mirror over all slots."""
    n = slots.shape[0]
    if slots.dim() != 2 or slots.shape[1] != CQ_SLOT_WORDS:
        raise ValueError("slots must be u64[n, 6]")
    rc = lib().dmadesc_cq_mirror(_dev(slots, torch.uint64, "slots"), n,
                                 _dev(stop, torch.uint32, "stop", 1), idle_polls,
                                 _stream(slots.device, stream))
    _check("dmadesc_cq_mirror", rc)


def cq_slot_state(slots: torch.Tensor) -> dict:
    """Host copy of every slot's generation, ack, head, phase and copied."""
    w = slots.view(torch.int64).cpu().numpy().view("<u8")
    return dict(depth=(w[:, 2] & 0xFFFFFFFF).astype("u4"), generation=(w[:, 2] >> 32).astype("u4"),
                ack=(w[:, 3] & 0xFFFFFFFF).astype("u4"), head=(w[:, 3] >> 32).astype("u4"),
                phase=(w[:, 4] & 0xFFFFFFFF).astype("u4"), copied=w[:, 5].copy())


class DeviceRegistry:
    """Registration cache kept in device memory (dmadesc_reg_register /
    dmadesc_reg_deregister). The record arrays are torch tensors owned here;
    when a register batch reports that it needs more room, the arrays are
    copied into larger ones (the C calls never allocate) and the batch is
    issued again."""

    def __init__(self, capacity: int = 0, page_shift: int = 12, device="cuda"):
        self.page_shift = page_shift
        self.device = torch.device(device)
        self.state = torch.tensor([0, 1], dtype=torch.int64).view(torch.uint64).to(self.device)
        self.capacity = 0
        self.start = self.end = self.id = self.refs = self.by_start = None
        self._needed = torch.zeros(1, dtype=torch.uint64, device=self.device)
        self.grow(capacity)

    def grow(self, capacity: int) -> None:
        if capacity > REG_MAX_CAPACITY:
            raise ValueError(f"capacity above {REG_MAX_CAPACITY}")
        if capacity <= self.capacity:
            return
        dev, c = self.device, capacity
        new = dict(start=torch.empty(c, dtype=torch.uint64, device=dev),
                   end=torch.empty(c, dtype=torch.uint64, device=dev),
                   id=torch.empty(c, dtype=torch.uint64, device=dev),
                   refs=torch.empty(c, dtype=torch.uint32, device=dev),
                   by_start=torch.empty(c, dtype=torch.uint32, device=dev))
        if self.capacity:
            k = self.count()
            for name, t in new.items():
                t[:k] = getattr(self, name)[:k]
        for name, t in new.items():
            setattr(self, name, t)
        self.capacity = capacity

    def count(self) -> int:
        return int(self.state.view(torch.int64)[0].item())

    def next_id(self) -> int:
        return int(self.state.view(torch.int64)[1].item())

    def _table(self):
        def ptr(t):
            return t.data_ptr() if t is not None else 0
        return (ptr(self.start), ptr(self.end), ptr(self.id), ptr(self.refs),
                ptr(self.by_start), self.state.data_ptr(), self.capacity)

    def register(self, addr: torch.Tensor, size: torch.Tensor, grow: bool = True,
                 stream=None) -> dict:
        """Returns dict(handle u64[n], kind u8[n], needed)."""
        n = addr.numel()
        dev = self.device
        handle = torch.empty(n, dtype=torch.uint64, device=dev)
        kind = torch.empty(n, dtype=torch.uint8, device=dev)
        while True:
            ws = _workspace(OP_REGISTRY, n, self.capacity, dev, None)
            rc = lib().dmadesc_reg_register(
                *self._table(), self.page_shift, _dev(addr, torch.uint64, "addr", n),
                _dev(size, torch.uint64, "size", n), n, _dev(handle, torch.uint64, "handle", n),
                _dev(kind, torch.uint8, "kind", n), self._needed.data_ptr(), *ws[1:], _stream(dev, stream))
            _check("dmadesc_reg_register", rc)
            needed = int(self._needed.view(torch.int64)[0].item())
            if needed <= self.capacity or not grow:
                return dict(handle=handle, kind=kind, needed=needed)
            self.grow(needed)

    def deregister(self, handles: torch.Tensor, stream=None) -> torch.Tensor:
        """Returns status u8[n]."""
        n = handles.numel()
        status = torch.empty(n, dtype=torch.uint8, device=self.device)
        ws = _workspace(OP_REGISTRY, n, self.capacity, self.device, None)
        rc = lib().dmadesc_reg_deregister(
            *self._table(), _dev(handles, torch.uint64, "handle", n), n,
            _dev(status, torch.uint8, "status", n), *ws[1:], _stream(self.device, stream))
        _check("dmadesc_reg_deregister", rc)
        return status

    def records(self):
        """(start, end, handle, refs) of the live records in start order, and
        the handles in storage order, as host numpy arrays."""
        import numpy as np
        k = self.count()
        if k == 0:
            z = np.zeros(0, np.uint64)
            return (z, z, z, np.zeros(0, np.int64)), z
        host = {name: getattr(self, name)[:k].cpu().numpy()
                for name in ("start", "end", "id", "refs", "by_start")}
        order = host["by_start"].astype(np.int64)
        return ((host["start"][order], host["end"][order], host["id"][order],
                 host["refs"][order].astype(np.int64)), host["id"])
