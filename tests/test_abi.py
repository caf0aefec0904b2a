"""The C-ABI library: loads, exports what include/dmadesc.h declares, and
rejects bad arguments on the host (these calls return before any GPU work,
so they run without a GPU)."""
import ctypes
import errno
import os
import re

import pytest

import memory_dma_descriptor_amd as dd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn), encoding="utf-8").read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dmadesc_\w+)\s*\(", src))
    return names


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"dmadesc_mr_lookup", "dmadesc_build_prp", "dmadesc_partition_by_queue",
            "dmadesc_emit_sqe", "dmadesc_reg_register", "dmadesc_reg_deregister",
            "dmadesc_build_put"} <= names
    lib = ctypes.CDLL(dd.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_version_and_strerror():
    lib = dd.lib()
    assert lib.dmadesc_version() == 1
    assert b"invalid" in lib.dmadesc_strerror(-errno.EINVAL)
    assert lib.dmadesc_strerror(0) == b"success"


def test_workspace_sizes():
    ws = dd.workspace_bytes
    # Lookup: no workspace up to 4,096 regions (the LDS kernel), then one
    # 64-byte record per run of 4 regions.
    assert ws(dd.OP_MR_LOOKUP, 1 << 20) == 0 and ws(dd.OP_MR_LOOKUP, 1 << 20, 4096) == 0
    assert ws(dd.OP_MR_LOOKUP, 1 << 20, 4097) == 1025 * 64
    assert ws(dd.OP_MR_LOOKUP, 0, 65536) == 16384 * 64
    assert ws(dd.OP_MR_LOOKUP, 5, (1 << 31) - 1) == (1 << 29) * 64
    assert ws(dd.OP_BUILD_PRP, 0) == 0
    assert ws(dd.OP_PARTITION, 100, 0) == 0            # nqueues 0 is invalid
    assert ws(dd.OP_PARTITION, 100, 257) == 0          # above the maximum
    assert ws(99, 10, 0) == 0
    for op, q in ((dd.OP_BUILD_PRP, 0), (dd.OP_PARTITION, 64)):
        sizes = [ws(op, n, q) for n in (1, 1000, 1 << 16, 1 << 20, 16 << 20, (1 << 32) - 1)]
        assert all(x % 256 == 0 and x > 0 for x in sizes), sizes
        assert sizes == sorted(sizes), sizes
        assert sizes[-1] < 1 << 32, sizes                 # small next to the batch itself
    assert ws(dd.OP_PARTITION, 1 << 20, 256) > ws(dd.OP_PARTITION, 1 << 20, 1)
    # Submission entries: per (queue, tile) a count, the placeable-lane masks
    # (128 bytes), a record and the block counts of its 1,024 positions (2
    # bytes each), per queue a record; independent of the batch, and under
    # 1/16 of the rings a call can fill (64 bytes per entry).
    assert ws(dd.OP_EMIT_SQE, 100, 0) == 0 and ws(dd.OP_EMIT_SQE, 100, 257) == 0
    e = [ws(dd.OP_EMIT_SQE, n, q) for q in (1, 64, 256) for n in (0, 1 << 24)]
    assert all(x % 256 == 0 and x > 0 for x in e) and e[0] == e[1] and e[2] < e[4]
    for q, x in zip((1, 64, 256), e[::2]):
        assert x <= q * 65536 * 64 // 16, (q, x)


EINVAL = -errno.EINVAL
NULL = None

# The probes below pass dummy pointers that host validation must reject. They
# run only where no GPU is visible, so a validation bug can never turn one of
# them into a launch on a real device.
import torch  # noqa: E402

no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                 reason="dummy-pointer probes run only without a GPU")
P = 0x1000   # a non-null pointer value never dereferenced: every call below is
             # rejected by host validation before anything is launched


@no_gpu_only
def test_lookup_rejects_bad_arguments():
    f = dd.lib().dmadesc_mr_lookup
    ok = [P, P, P, 4, 12, P, P, 8, 0, P, P, P, P, P, NULL, 0, NULL]
    for k, bad in [(4, 11), (4, 31), (7, 1 << 32), (3, 1 << 31), (0, NULL), (5, NULL),
                   (9, NULL), (13, NULL)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)
    # A record workspace given for a large table must be big enough and
    # 256-byte aligned (even for an empty batch); none at all is allowed.
    need = dd.workspace_bytes(dd.OP_MR_LOOKUP, 0, 5000)
    big = [P, P, P, 5000, 12, P, P, 0, 0, P, P, P, P, P]
    assert f(*big, P, need - 1, NULL) == EINVAL
    assert f(*big, P + 8, need, NULL) == EINVAL
    assert f(*big, P, need, NULL) == 0 and f(*big, NULL, 0, NULL) == 0


@no_gpu_only
def test_build_prp_rejects_bad_arguments():
    f = dd.lib().dmadesc_build_prp
    ok = [P, 16, P, P, 8, 0x10000, P, 4, P, P, P, P, P, 1 << 20, NULL]
    for k, bad in [(5, 0x10008), (1, 1 << 48), (4, 1 << 32), (11, NULL), (0, NULL),
                   (6, NULL), (6, P + 8), (2, NULL), (8, NULL), (12, NULL), (13, 8),
                   (12, P + 8), (12, P + 128)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_build_prp_packed_rejects_bad_arguments():
    f = dd.lib().dmadesc_build_prp_packed
    ok = [P, 16, P, P, 8, 0x10000, P, 4, P, P, P, P, P, 1 << 20, NULL]
    for k, bad in [(5, 0x10008), (1, 1 << 48), (4, 1 << 32), (11, NULL), (0, NULL),
                   (6, NULL), (6, P + 8), (2, NULL), (8, NULL), (12, NULL), (13, 8),
                   (12, P + 8), (12, P + 128)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)
    # Slot counts must stay below 2^62: (16 * lut_entries + 2) * n.
    args = list(ok)
    args[1], args[4] = (1 << 44), (1 << 20)
    assert f(*args) == EINVAL


@no_gpu_only
def test_partition_rejects_bad_arguments():
    f = dd.lib().dmadesc_partition_by_queue
    ok = [P, 100, 4, P, P, P, P, 1 << 20, NULL]
    for k, bad in [(2, 0), (2, 257), (1, 1 << 32), (4, NULL), (5, NULL), (0, NULL),
                   (3, NULL), (6, NULL), (7, 16), (6, P + 64)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_emit_sqe_rejects_bad_arguments():
    f = dd.lib().dmadesc_emit_sqe
    ok = [P, P, 4, P, P, P, P, P, 8, 2, 1, 9, P, P, P, P, P, P, NULL, P, 1 << 20, NULL]
    for k, bad in [(2, 0), (2, 257), (8, 1 << 32), (9, 256), (11, 8), (11, 17),
                   (1, NULL), (12, NULL), (13, NULL), (14, NULL), (15, NULL), (16, NULL),
                   (17, NULL), (0, NULL), (3, NULL), (4, NULL), (5, NULL), (6, NULL),
                   (7, NULL), (19, NULL), (20, 16), (19, P + 8)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_build_put_rejects_bad_arguments():
    f = dd.lib().dmadesc_build_put
    ok = [P, P, P, P, 8, 0, 1 << 30, 21, P, P, P, 4, P, 64, P, P, P, P, P, 1 << 20, NULL]
    for k, bad in [(4, 1 << 32), (11, 0), (11, 65537), (7, 11), (7, 32), (6, (1 << 30) + 5),
                   (6, 1 << 52), (8, NULL), (9, NULL), (10, NULL), (17, NULL), (12, NULL),
                   (12, P + 8), (0, NULL), (3, NULL), (14, NULL), (16, NULL), (18, NULL),
                   (19, 16), (18, P + 8)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_registry_rejects_bad_arguments():
    f = dd.lib().dmadesc_reg_register
    ok = [P, P, P, P, P, P, 64, 12, P, P, 8, P, P, P, P, 1 << 30, NULL]
    for k, bad in [(7, 11), (7, 31), (10, 65537), (6, (1 << 24) + 1), (5, NULL), (13, NULL),
                   (0, NULL), (4, NULL), (8, NULL), (11, NULL), (12, NULL), (14, NULL),
                   (15, 16), (14, P + 8)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)
    g = dd.lib().dmadesc_reg_deregister
    ok = [P, P, P, P, P, P, 64, P, 8, P, P, 1 << 30, NULL]
    for k, bad in [(8, 65537), (6, (1 << 24) + 1), (5, NULL), (0, NULL), (7, NULL), (9, NULL),
                   (10, NULL), (11, 16), (10, P + 8)]:
        args = list(ok)
        args[k] = bad
        assert g(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_cq_mirror_rejects_bad_arguments():
    f = dd.lib().dmadesc_cq_mirror
    ok = [P, 8, P, 64, NULL]
    for k, bad in [(0, NULL), (0, P + 4), (1, 0), (1, 65), (2, NULL), (3, 0), (3, (1 << 24) + 1)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


@no_gpu_only
def test_build_batch_rejects_bad_arguments():
    f = dd.lib().dmadesc_build_batch
    need = dd.batch_workspace_bytes(8, 4, 4)
    #     rs re rk nr ps  va lut lutn off len qid n  nq bus    pool pp flags
    ok = [P, P, P, 4, 12, 0, P, 16, P, P, P, 8, 4, 0x10000, P, 4, 1,
          P, P, P, P, P, P, P, P, P, P, P, P, P, need, NULL]
    for k, bad in [(16, 2), (16, 3), (12, 0), (12, 257), (11, 1 << 32), (13, 0x10008),
                   (1, NULL), (4, 11), (4, 31), (3, 1 << 31), (17, NULL), (21, NULL),
                   (6, NULL), (14, NULL), (14, P + 8), (8, NULL), (10, NULL), (22, NULL),
                   (25, NULL), (26, NULL), (27, NULL), (28, NULL), (29, NULL),
                   (30, need - 256), (29, P + 64), (7, 1 << 48)]:
        args = list(ok)
        args[k] = bad
        assert f(*args) == EINVAL, (k, bad)


def test_batch_workspace_sizes():
    ws = dd.batch_workspace_bytes
    assert ws(100, 0, 10) == 0 and ws(100, 257, 10) == 0 and ws(1 << 32, 64, 10) == 0
    assert ws(100, 64, 1 << 31) == 0
    a, b = ws(1 << 24, 64, 4096), ws(1 << 24, 64, 65536)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    # at least the PRP scan's and the split's own workspaces
    assert a >= dd.workspace_bytes(dd.OP_BUILD_PRP, 1 << 24) + \
        dd.workspace_bytes(dd.OP_PARTITION, 1 << 24, 64)
    assert ws(0, 64, 0) > 0


@no_gpu_only
def test_table_check_rejects_bad_arguments():
    f = dd.lib().dmadesc_mr_table_check
    bad = ctypes.c_uint64(0)
    ok = [P, P, 4, 12, P, ctypes.addressof(bad), NULL]
    for k, v in [(3, 11), (3, 31), (2, 1 << 31), (4, NULL), (4, P + 4), (0, NULL), (1, NULL)]:
        args = list(ok)
        args[k] = v
        bad.value = 5
        assert f(*args) == EINVAL, (k, v)
        assert bad.value == (1 << 64) - 1, (k, v)     # no faulty region named


def test_wait_limit_round_trip():
    # The bound is host state only: set, read back through the next call,
    # restore the default.
    assert dd.debug_wait_limit(7) == dd.DEFAULT_WAIT_POLLS
    assert dd.debug_wait_limit(0) == 7
    assert dd.debug_wait_limit(dd.DEFAULT_WAIT_POLLS) == 0


def test_status_codes_match_the_header():
    src = open(os.path.join(ROOT, "include", "dmadesc.h"), encoding="utf-8").read()
    for name in ("OK", "EINVAL", "ERANGE", "ENOSPC", "EBUSY"):
        v = int(re.search(rf"DMADESC_PRP_{name} = (\d+)", src).group(1))
        assert getattr(dd, f"PRP_{name}") == v, name
    polls = re.search(r"#define DMADESC_DEFAULT_WAIT_POLLS \(1u << (\d+)\)", src).group(1)
    assert dd.DEFAULT_WAIT_POLLS == 1 << int(polls)


def test_cq_slot_layout():
    # dmadesc_cq_slot is 48 bytes: two addresses, six u32 words, the count.
    src = open(os.path.join(ROOT, "include", "dmadesc.h"), encoding="utf-8").read()
    body = re.search(r"typedef struct dmadesc_cq_slot \{(.*?)\}", src, re.S).group(1)
    fields = re.findall(r"(uint\d+)_t\s+(\w+);", body)
    assert [n for _, n in fields] == ["src", "dst", "depth", "generation", "ack", "head",
                                      "phase", "reserved", "copied"]
    assert sum(int(t[4:]) // 8 for t, _ in fields) == 8 * dd.CQ_SLOT_WORDS


def test_registry_workspace_sizes():
    ws = dd.workspace_bytes
    assert ws(dd.OP_REGISTRY, 65537, 64) == 0 and ws(dd.OP_REGISTRY, 1, (1 << 24) + 1) == 0
    a, b, c = ws(dd.OP_REGISTRY, 1, 64), ws(dd.OP_REGISTRY, 65536, 64), ws(dd.OP_REGISTRY, 1, 1 << 20)
    assert 0 < a < b and a < c and all(x % 256 == 0 for x in (a, b, c))


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("n", [1, 20, 64, 1000, 65536])
@pytest.mark.parametrize("cap", [1, 32, 256, 4096, 65536, 1 << 20, 1 << 24])
def test_registry_workspace_holds_every_piece(n, cap):
    # The registry kernels keep, each in a 256-byte-aligned piece: per batch
    # item six u64 columns (rounded base and top, hit start, new base, insert
    # base and top), two more (miss base and top), one u8 class and six u32
    # columns (hit slot, rank, start rank, owner, new references, miss rank);
    # per record five u64 columns (starts, running maximum, three scratch)
    # and two u32 (new slot, scratch), the merged index over records and
    # items (u32), 16,384 chunk totals and four scalars; and two range
    # indexes over the batch (misses, inserts), each with nbk buckets (a power
    # of two near n / 4, 64..16,384) of a u32 count and 8 inline ranges
    # (16 bytes) with their u32 ranks, a u8 long flag per item and a u32
    # long count per 256-item tile of the largest batch, plus the inserts'
    # bucket prefixes (u32 per bucket), the bounds (two u64), each
    # classification block's smallest and largest start (u64, 256 blocks at
    # most) and the two long counts. A workspace of dmadesc_workspace_bytes
    # must hold all of them.
    nbk = 64
    while nbk < n // 4 and nbk < 16384:
        nbk *= 2
    index = 2 * (_a256(4 * nbk) + _a256(16 * 8 * nbk) + _a256(4 * 8 * nbk) + _a256(n)
                 + _a256(4 * 256))
    need = (8 * _a256(8 * n) + _a256(n) + 6 * _a256(4 * n) + 5 * _a256(8 * cap)
            + 2 * _a256(4 * cap) + _a256(4 * (cap + n)) + _a256(8 * 16384) + _a256(32)
            + index + _a256(4 * nbk) + _a256(16) + 2 * _a256(8 * 256) + _a256(8))
    assert dd.workspace_bytes(dd.OP_REGISTRY, n, cap) >= need, (n, cap)


def test_empty_lookup_is_a_no_op():
    # n == 0 with valid parameters launches nothing and succeeds.
    f = dd.lib().dmadesc_mr_lookup
    assert f(NULL, NULL, NULL, 0, 12, NULL, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL,
             NULL, 0, NULL) == 0


@pytest.mark.parametrize("name", ["mr_lookup", "build_prp", "build_prp_packed",
                                  "build_prp_packed_noalloc", "build_batch",
                                  "partition_by_queue", "emit_sqe", "build_put",
                                  "cq_mirror", "mr_table_check"])
def test_binding_names_match_abi(name):
    assert callable(getattr(dd, name))
    assert f"dmadesc_{name}" in _declared()
