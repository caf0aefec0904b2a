"""The boundary from plain C: include/dmadesc.h compiles as C99 and C++11
with -pedantic, and a C program linked against libdmadesc.so calls the
host-only entry points (version, workspace sizes, error strings) and a call
the host refuses before anything is launched. No GPU is needed."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import memory_dma_descriptor_amd as dd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADER = os.path.join(INCLUDE, "dmadesc.h")

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                               reason="no host C/C++ compiler")

PROGRAM = r"""
#include <errno.h>
#include <stdio.h>
#include "dmadesc.h"

int main(void)
{
    if (dmadesc_version() != 1) return 1;
    size_t w = dmadesc_workspace_bytes(DMADESC_OP_BUILD_PRP, (uint64_t)1 << 20, 0);
    if (w == 0 || w % 256 != 0) return 2;
    if (dmadesc_workspace_bytes(DMADESC_OP_PARTITION, 1000, 0) != 0) return 3;
    if (dmadesc_batch_workspace_bytes(1000, 64, 4096) == 0) return 4;
    /* A table with entries but no pointer: refused on the host, nothing launched. */
    uint64_t total = 0;
    int rc = dmadesc_build_prp(NULL, 16, NULL, NULL, 1, 0, NULL, 0, NULL, NULL, NULL, &total,
                               NULL, 0, NULL);
    if (rc != -EINVAL) return 5;
    /* A list bus base that is not 4 KiB aligned. */
    rc = dmadesc_build_prp_packed(NULL, 0, NULL, NULL, 0, 4095, NULL, 0, NULL, NULL, NULL,
                                  &total, NULL, 0, NULL);
    if (rc != -EINVAL) return 6;
    rc = dmadesc_partition_by_queue(NULL, 0, 0, NULL, NULL, NULL, NULL, 0, NULL);
    if (rc != -EINVAL) return 7;
    printf("%s|%s\n", dmadesc_strerror(0), dmadesc_strerror(-EINVAL));
    return 0;
}
"""


@needs_gcc
@pytest.mark.parametrize("cmd", [["gcc", "-std=c99", "-x", "c"], ["g++", "-std=c++11", "-x", "c++"]])
def test_header_compiles_pedantic(cmd):
    p = subprocess.run(cmd + ["-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", HEADER],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr


@needs_gcc
def test_c_program_links_and_calls(tmp_path):
    dd.lib()                                   # builds the library in-tree if it is missing
    libdir = os.path.dirname(dd.LIB_PATH)
    src = tmp_path / "consumer.c"
    exe = tmp_path / "consumer"
    src.write_text(PROGRAM)
    p = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
                        str(src), "-o", str(exe), f"-L{libdir}", "-ldmadesc",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    ok, einval = r.stdout.strip().splitlines()[-1].split("|")
    assert ok == "success" and "invalid argument" in einval
