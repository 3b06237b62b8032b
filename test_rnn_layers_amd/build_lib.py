"""Builds libttt.so in-tree with hipcc for gfx950.

    python -m test_rnn_layers_amd.build_lib          # build
    python -m test_rnn_layers_amd.build_lib --asm    # also keep the gfx950 assembly under _build/
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "lib", "libttt.so")
ARCH = "gfx950"

HIP_SOURCES = ["linear_token.hip", "linear_dual.hip", "mlp_dual.hip", "mlp_token.hip", "post_proj.hip"]
CXX_SOURCES = ["ttt_host.cpp"]

COMMON = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          # packed fp32 VALU ops are kept out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, asm: bool) -> str:
    hipcc = _hipcc()
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc] + COMMON + ["-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if asm and src.endswith(".hip"):
        s_out = os.path.join(BUILD, src + f"-{ARCH}.s")
        subprocess.run([hipcc, "-x", "hip"] + COMMON + ["--cuda-device-only", "-S", path, "-o", s_out],
                       check=True, capture_output=True)
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    srcs = [s for s in HIP_SOURCES + CXX_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    _build_c_example()
    if verbose:
        print(f"built {LIB} from {', '.join(srcs)}; {C_EXAMPLE}")
    return LIB


C_EXAMPLE = os.path.join(os.path.dirname(LIB), "ttt_c_example")


def _build_c_example() -> None:
    """A plain-C program that uses the library through include/ttt.h only."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), os.path.join(CSRC, "c_example.c"), "-o", C_EXAMPLE,
           "-L", os.path.dirname(LIB), "-lttt", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C example build failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    args = ap.parse_args()
    try:
        build(asm=args.asm)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
