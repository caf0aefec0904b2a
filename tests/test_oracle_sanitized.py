"""The oracle's pin tests under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle is rebuilt with both (every report fatal) and the pin tests run in
a child process with the ASan runtime preloaded. A planted out-of-bounds
call (a split asked to read 1,000 queue ids from a 10-element array, on the
CPU) must be caught, which shows that the sanitizers are live in that
process."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_packed.py", "tests/test_oracle_put.py",
        "tests/test_oracle_registry.py", "tests/test_oracle_sqe.py", "tests/test_oracle_cq.py"]


def _asan_runtime():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


ASAN = _asan_runtime()
needs_asan = pytest.mark.skipif(ASAN is None, reason="gcc's ASan runtime is not installed")


def _env():
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=ASAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


@pytest.fixture(scope="module")
def sanitized_oracle():
    sys.path.insert(0, ROOT)
    import oracle
    return oracle.build(sanitize=True)


@needs_asan
def test_pins_pass_under_asan_and_ubsan(sanitized_oracle):
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=_env(), capture_output=True, text=True,
                       timeout=600)
    tail = (p.stdout + p.stderr)[-3000:]
    assert p.returncode == 0, tail
    assert "Sanitizer" not in p.stderr, tail


@needs_asan
def test_a_planted_overrun_is_caught(sanitized_oracle):
    snippet = (
        "import ctypes, numpy as np, oracle\n"
        "assert oracle.SANITIZE\n"
        "lib = oracle._lib()\n"
        "q = np.zeros(10, np.uint32); perm = np.zeros(1000, np.uint32)\n"
        "qoff = np.zeros(4, np.uint64); ninv = np.zeros(1, np.uint64)\n"
        "p = lambda a, t: a.ctypes.data_as(t)\n"
        "lib.orc_partition(p(q, oracle._u32p), 1000, 2, p(perm, oracle._u32p),\n"
        "                  p(qoff, oracle._u64p), p(ninv, oracle._u64p))\n"
        "print('not caught')\n")
    p = subprocess.run([sys.executable, "-c", snippet], cwd=ROOT, env=_env(),
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0 and "AddressSanitizer" in p.stderr, (p.stdout + p.stderr)[-2000:]
