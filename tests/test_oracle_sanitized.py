"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle is built a second time with -fsanitize=address,undefined (host
code only, gcc) and every quick pin of tests/test_oracle_pins.py runs
against that build in a child Python process that preloads the ASan
runtime: an out-of-bounds read or write (a wrong leading dimension or batch
stride in the C loops) or undefined behaviour (signed overflow in an index)
aborts the child, and the test fails.  The child also checks that the
sanitizer runtime is really mapped into it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r'''
import sys
sys.path[:0] = [{root!r}, {here!r}]
import numpy as np
import oracle
import test_oracle_pins as pins
from trsm_inputs import make_problem
orc = oracle.OracleLib({lib!r})
maps = open("/proc/self/maps").read()
assert "libasan" in maps and "libubsan" in maps, "sanitizer runtimes not loaded"
for check in pins.QUICK_CHECKS:
    for dtype in pins.DTYPES:
        check(orc, dtype)
        print("ok", check.__name__, dtype, flush=True)
# padded leading dimensions and the row-wise dot form
for dtype in pins.DTYPES:
    L, B = make_problem(dtype, 97, 13, seed=5, lda=101, ldb=99)
    orc.solve(L, B, 0.5)
L, B = make_problem("f64", 120, 7, seed=6)
assert np.array_equal(orc.solve(L, B, 1.0), orc.solve(L, B, 1.0, rowdot=True))
print("SANITIZED_OK", flush=True)
'''


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc has no ASan runtime here")
    tmp = tempfile.mkdtemp(prefix="oracle_san_")
    try:
        lib = os.path.join(tmp, "liboracle_san.so")
        flags = [f for f in oracle.CFLAGS if f != "-O2"] + [
            "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"]
        src = os.path.join(os.path.dirname(oracle.__file__), "oracle_lln.c")
        subprocess.run(["gcc", *flags, src, "-o", lib], check=True)
        env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
        code = CHILD.format(root=ROOT, here=HERE, lib=lib)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=900)
        assert r.returncode == 0 and "SANITIZED_OK" in r.stdout, (r.returncode, r.stdout[-2000:],
                                                                  r.stderr[-4000:])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
