"""The CPU code under AddressSanitizer + UndefinedBehaviorSanitizer: the
oracle against its pins, and libttt's host half (argument checks, launch
splitting) against the ABI and host-logic tests, each in a child process with
the sanitizer runtime preloaded.  A last test shows that the runtime does
report: an out-of-bounds read through the sanitized oracle is caught."""
import subprocess
import sys

import pytest

import sanitized as S


def _report(r):
    return f"rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-5000:]}"


def test_oracle_pins_under_asan_ubsan():
    lib = S.build_oracle()
    r = S.run_pytest("oracle", lib, S.gcc_runtime(), ["tests/test_oracle_pins.py"])
    assert r.returncode == 0, _report(r)


def test_host_checks_under_asan_ubsan():
    lib = S.build_libttt()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    r = S.run_pytest("libttt", lib, S.clang_runtime(), ["tests/test_abi.py", "tests/test_host_logic.py"])
    assert r.returncode == 0, _report(r)


_OVERFLOW = r"""
import sys, ctypes
import numpy as np
import oracle.oracle as m
m._LIB = sys.argv[1]
m.build = lambda force=False: sys.argv[1]
lib = m.load()
x, w, b, out = (np.ones(64) for _ in range(4))
p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
lib.oracle_ln_fwd(p(x), p(w), p(b), 80, 1e-6, p(out))  # 80 > 64: reads past the arrays
print("not caught", flush=True)
"""


def test_sanitizer_reports_an_overflow():
    lib = S.build_oracle()
    r = subprocess.run([sys.executable, "-c", _OVERFLOW, lib], cwd=S.ROOT, env=S.sanitizer_env(S.gcc_runtime()),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, _report(r)
