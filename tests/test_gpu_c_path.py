"""The whole path from a plain C program, no PyTorch: it allocates device
memory with hipMalloc, copies a seeded batch in, calls dmadesc_mr_lookup,
dmadesc_build_prp_packed and dmadesc_partition_by_queue with workspaces
sized by dmadesc_workspace_bytes on one stream, and writes every output
back; each column and the whole list pool must equal the oracle's."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import memory_dma_descriptor_amd as dd
import oracle
import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "dmadesc.h"

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); exit(10); } } while (0)
#define CALL(x) do { int r_ = (x); if (r_ != 0) { \
    fprintf(stderr, "%s: %s\n", #x, dmadesc_strerror(r_)); exit(11); } } while (0)

static void *load(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { perror(path); exit(12); }
    void *p = malloc(bytes ? bytes : 1);
    if (bytes && fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short %s\n", path); exit(13); }
    fclose(f);
    return p;
}

static void save(const char *dir, const char *name, const void *p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/out_%s.bin", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { perror(path); exit(14); }
    fclose(f);
}

static void *up(const void *h, size_t bytes)
{
    void *d = NULL;
    CHECK(hipMalloc(&d, bytes ? bytes : 256));
    if (bytes) CHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void *down(const void *d, size_t bytes)
{
    void *h = malloc(bytes ? bytes : 1);
    if (bytes) CHECK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    return h;
}

int main(int argc, char **argv)
{
    if (argc != 9) return 2;
    const char *dir = argv[1];
    const uint64_t n = strtoull(argv[2], NULL, 10), lut_entries = strtoull(argv[3], NULL, 10);
    const uint32_t nreg = (uint32_t)strtoul(argv[4], NULL, 10);
    const uint32_t nq = (uint32_t)strtoul(argv[5], NULL, 10);
    const uint64_t bus = strtoull(argv[6], NULL, 10), pool_pages = strtoull(argv[7], NULL, 10);
    const uint64_t va_base = strtoull(argv[8], NULL, 10);

    uint64_t *d_lut = up(load(dir, "lut", lut_entries * 8), lut_entries * 8);
    uint64_t *d_off = up(load(dir, "off", n * 8), n * 8);
    uint64_t *d_len = up(load(dir, "len", n * 8), n * 8);
    uint32_t *d_qid = up(load(dir, "qid", n * 4), n * 4);
    uint64_t *d_rs = up(load(dir, "rstart", (size_t)nreg * 8), (size_t)nreg * 8);
    uint64_t *d_re = up(load(dir, "rend", (size_t)nreg * 8), (size_t)nreg * 8);
    uint32_t *d_rk = up(load(dir, "rlkey", (size_t)nreg * 4), (size_t)nreg * 4);

    int32_t *handle; uint32_t *lkey; uint8_t *kind; uint64_t *rbase, *rend;
    uint64_t *prp1, *prp2, *pool, *total, *qoff, *n_invalid; uint8_t *status; uint32_t *perm;
    CHECK(hipMalloc((void **)&handle, n * 4 + 4)); CHECK(hipMalloc((void **)&lkey, n * 4 + 4));
    CHECK(hipMalloc((void **)&kind, n + 16));      CHECK(hipMalloc((void **)&rbase, n * 8 + 8));
    CHECK(hipMalloc((void **)&rend, n * 8 + 8));   CHECK(hipMalloc((void **)&prp1, n * 8 + 8));
    CHECK(hipMalloc((void **)&prp2, n * 8 + 8));   CHECK(hipMalloc((void **)&status, n + 16));
    CHECK(hipMalloc((void **)&pool, pool_pages * 4096 + 16)); CHECK(hipMalloc((void **)&total, 8));
    CHECK(hipMalloc((void **)&perm, n * 4 + 4));   CHECK(hipMalloc((void **)&qoff, (nq + 2) * 8));
    CHECK(hipMalloc((void **)&n_invalid, 8));
    CHECK(hipMemset(pool, 0xC3, pool_pages * 4096));

    const size_t w_lk = dmadesc_workspace_bytes(DMADESC_OP_MR_LOOKUP, n, nreg);
    const size_t w_prp = dmadesc_workspace_bytes(DMADESC_OP_BUILD_PRP, n, 0);
    const size_t w_sp = dmadesc_workspace_bytes(DMADESC_OP_PARTITION, n, nq);
    void *ws_lk = NULL, *ws_prp = NULL, *ws_sp = NULL;
    if (w_lk) CHECK(hipMalloc(&ws_lk, w_lk));        /* hipMalloc is 256-byte aligned */
    CHECK(hipMalloc(&ws_prp, w_prp ? w_prp : 256));
    CHECK(hipMalloc(&ws_sp, w_sp ? w_sp : 256));

    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    CALL(dmadesc_mr_lookup(d_rs, d_re, d_rk, nreg, 12, d_off, d_len, n, va_base, handle, lkey,
                           kind, rbase, rend, ws_lk, w_lk, s));
    CALL(dmadesc_build_prp_packed(d_lut, lut_entries, d_off, d_len, n, bus, pool, pool_pages,
                                  prp1, prp2, status, total, ws_prp, w_prp, s));
    CALL(dmadesc_partition_by_queue(d_qid, n, nq, perm, qoff, n_invalid, ws_sp, w_sp, s));
    CHECK(hipStreamSynchronize(s));

    save(dir, "handle", down(handle, n * 4), n * 4);
    save(dir, "lkey", down(lkey, n * 4), n * 4);
    save(dir, "kind", down(kind, n), n);
    save(dir, "rbase", down(rbase, n * 8), n * 8);
    save(dir, "rend", down(rend, n * 8), n * 8);
    save(dir, "prp1", down(prp1, n * 8), n * 8);
    save(dir, "prp2", down(prp2, n * 8), n * 8);
    save(dir, "status", down(status, n), n);
    save(dir, "total", down(total, 8), 8);
    save(dir, "pool", down(pool, pool_pages * 4096), pool_pages * 4096);
    save(dir, "perm", down(perm, n * 4), n * 4);
    save(dir, "qoff", down(qoff, (nq + 2) * 8), (nq + 2) * 8);
    save(dir, "n_invalid", down(n_invalid, 8), 8);
    CHECK(hipStreamDestroy(s));
    printf("done %llu\n", (unsigned long long)n);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
@pytest.mark.parametrize("name,n", [("mixed", 300_001), ("mrheavy", 100_003), ("tiny", None)])
def test_path_from_a_c_program(tmp_path, name, n):
    d = synth.generate(name, n=n)
    if not d["lut_entries"]:                      # MR-heavy has no heap: borrow Mixed's table
        m = synth.generate("mixed", n=16)
        d.update(lut=m["lut"], lut_entries=m["lut_entries"])
    if not d["nqueues"]:
        d.update(qid=np.zeros(d["n"], np.uint32), nqueues=1)
    n, bus, va = d["n"], d["list_bus_base"], d["va_base"]
    pages = oracle.build_prp_packed(d["lut"], d["off"], d["len"], bus, 1 << 50)["total"]
    pool_pages = max(pages, 1)
    for k, dt in (("lut", np.uint64), ("off", np.uint64), ("len", np.uint64), ("qid", np.uint32),
                  ("rstart", np.uint64), ("rend", np.uint64), ("rlkey", np.uint32)):
        np.ascontiguousarray(d[k], dt).tofile(tmp_path / f"{k}.bin")
    dd.lib()                                      # the library is built in-tree beforehand
    libdir = os.path.dirname(dd.LIB_PATH)
    src, exe = tmp_path / "path.c", tmp_path / "path"
    src.write_text(PROGRAM)
    p = subprocess.run(["gcc", "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                        str(src), "-o", str(exe), f"-L{libdir}", "-ldmadesc",
                        f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
                        f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    gc.say(f"C program: {name} n={n} regions={len(d['rstart'])} pool={pool_pages}")
    r = subprocess.run([str(exe), str(tmp_path), str(n), str(d["lut_entries"]),
                        str(len(d["rstart"])), str(d["nqueues"]), str(bus), str(pool_pages),
                        str(va)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    out = lambda k, dt: np.fromfile(tmp_path / f"out_{k}.bin", dtype=dt)  # noqa: E731

    o = oracle.mr_lookup(d["rstart"], d["rend"], d["rlkey"], d["off"], d["len"], va_base=va)
    for k, dt in (("handle", np.int32), ("lkey", np.uint32), ("kind", np.uint8),
                  ("rbase", np.uint64), ("rend", np.uint64)):
        assert np.array_equal(out(k, dt), o[k]), f"{name} lookup {k}"
    want = np.full((pool_pages, 512), 0xC3C3C3C3C3C3C3C3, np.uint64)
    o = oracle.build_prp_packed(d["lut"], d["off"], d["len"], bus, pool_pages, pool=want)
    for k, dt in (("prp1", np.uint64), ("prp2", np.uint64), ("status", np.uint8)):
        assert np.array_equal(out(k, dt), o[k]), f"{name} prp {k}"
    assert int(out("total", np.uint64)[0]) == o["total"]
    assert np.array_equal(out("pool", np.uint64).reshape(pool_pages, 512), want), f"{name} pool"
    o = oracle.partition(d["qid"], d["nqueues"])
    assert np.array_equal(out("perm", np.uint32), o["perm"]), f"{name} perm"
    assert np.array_equal(out("qoff", np.uint64), o["qoff"]), f"{name} qoff"
    assert int(out("n_invalid", np.uint64)[0]) == o["n_invalid"]
