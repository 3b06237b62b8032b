"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code, for
the CPU test suite:

- the oracle (``oracle/ttt_oracle.c``), built with gcc;
- the host half of libttt (``ttt_host.cpp``: argument checks, splitting of a
  call into launches), built with clang for the host pass only and linked
  with the ordinary (unsanitized) kernel objects.

Both land under ``_build/san/``; neither replaces the product library.  The
sanitizer runtimes are preloaded into a child Python process
(``run_pytest``), which points the oracle or the binding at the sanitized
library before the tests import it.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
ORACLE_SRC = os.path.join(ROOT, "oracle", "ttt_oracle.c")
ORACLE_SAN = os.path.join(SAN, "libttt_oracle_san.so")
LIBTTT_SAN = os.path.join(SAN, "libttt_san.so")

SAN_FLAGS = ["address", "undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_oracle() -> str:
    os.makedirs(SAN, exist_ok=True)
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-D_DEFAULT_SOURCE",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    cmd += [f"-fsanitize={s}" for s in SAN_FLAGS]
    _run(cmd + [ORACLE_SRC, "-o", ORACLE_SAN, "-lm"])
    return ORACLE_SAN


def build_libttt() -> str:
    """ttt_host.cpp with the sanitizers on its host code, linked with the kernel
    objects of the ordinary build (built first if they are missing)."""
    from test_rnn_layers_amd import build_lib as bl

    os.makedirs(SAN, exist_ok=True)
    objs = []
    for src in bl.HIP_SOURCES:
        obj = os.path.join(bl.BUILD, src + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(bl.CSRC, src)):
            bl._compile(src, asm=False)
        objs.append(obj)
    host = []
    for s in SAN_FLAGS:
        host += ["-Xarch_host", f"-fsanitize={s}"]
    host += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan"]
    src = os.path.join(bl.CSRC, "ttt_host.cpp")
    obj = os.path.join(SAN, "ttt_host.san.o")
    hipcc = bl._hipcc()
    flags = [f for f in bl.COMMON if f != "-O3"] + ["-O1", "-g"]
    _run([hipcc] + flags + host + ["-c", src, "-o", obj])
    _run([hipcc, f"--offload-arch={bl.ARCH}", "-shared", "-fPIC"] + host + ["-o", LIBTTT_SAN, obj] + objs)
    return LIBTTT_SAN


def gcc_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_runtime() -> str:
    from test_rnn_layers_amd import build_lib as bl

    clang = os.path.join(os.path.dirname(os.path.realpath(bl._hipcc())), "..", "llvm", "bin", "clang++")
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


# The child process: point the oracle or the binding at the sanitized
# library, then run pytest on the given files.
_CHILD = r"""
import sys
which, lib = sys.argv[1], sys.argv[2]
if which == "oracle":
    import oracle.oracle as m
    m._LIB = lib
    m.build = lambda force=False: lib
else:
    import test_rnn_layers_amd.libttt as m
    m.LIB_PATH = lib
import pytest
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + sys.argv[3:])
if lib not in open("/proc/self/maps").read():
    print("the sanitized library was not loaded", flush=True)
    rc = rc or 3
sys.exit(rc)
"""


def sanitizer_env(runtime: str) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    # Python and the libraries it loads are not instrumented; leaks at exit
    # are theirs, so only memory errors and undefined behaviour are reported.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def run_pytest(which: str, lib: str, runtime: str, files: list[str], timeout: float = 600):
    env = sanitizer_env(runtime)
    return subprocess.run([sys.executable, "-c", _CHILD, which, lib] + files, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)
