"""Per-phase cycle breakdown of linear_dual_kernel from an instrumented build.

    python -m test_rnn_layers_amd.phase_stamps build        # on the CPU: lib/libttt_stamps.so
    python -m test_rnn_layers_amd.phase_stamps run --workload linear_1b --out profiles/...md   # on the GPU

The instrumented build compiles linear_dual.hip with TTT_PHASE_STAMPS: lane 0
of each wave records the shader clock (s_memtime, low 32 bits) in LDS at the
phase boundaries of mini-batches 256..319, and workgroup 0 (chain 0) copies
them out at the end.  The stamps add an s_memtime and an LDS write per
boundary, so the instrumented kernel is a little slower than the product
build; the run reports both launch times.

Column waves (0..3), per mini-batch m:
  k0 top of the step, k1 Z_m written (sequential product), k2 after the
  barrier, k3 products of mini-batch m done (before the second barrier).
Row waves (4..7):
  k0 top, k1 forward LayerNorm of m-2 done, k2 staging of m+2 done, k3 fetch
  of m+6 issued, k4 after the barrier, k5 backward LayerNorm of m done.
"""
from __future__ import annotations

import argparse
import os
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT_DIR = os.path.join(ROOT, "_build", "stamps")
LIB = os.path.join(PKG, "lib", "libttt_stamps.so")
ROW_NAMES = ["forward LayerNorm (m-2) + output store", "staging (m+2)", "fetch (m+6) issue", "wait at barrier 1",
             "backward LayerNorm (m)", "wait at barrier 2"]
COL_NAMES = ["Z = Y + C ng (sequential product)", "wait at barrier 1",
             "Zbar, state step, W to fp16, P, Y, causal, look-ahead, K^T", "wait at barrier 2"]


def build() -> str:
    from test_rnn_layers_amd import build_lib as bl

    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in bl.HIP_SOURCES + bl.CXX_SOURCES:
        if src == "linear_dual.hip":
            obj = os.path.join(OUT_DIR, "linear_dual.stamps.o")
            cmd = [bl._hipcc(), "-x", "hip"] + bl.COMMON + ["-DTTT_PHASE_STAMPS", "-c",
                                                             os.path.join(bl.CSRC, src), "-o", obj]
            subprocess.run(cmd, check=True, capture_output=True)
        else:
            obj = os.path.join(bl.BUILD, src + ".o")
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(bl.CSRC, src)):
                bl._compile(src, asm=False)
        objs.append(obj)
    subprocess.run([bl._hipcc(), f"--offload-arch={bl.ARCH}", "-shared", "-fPIC", "-o", LIB] + objs, check=True)
    return LIB


def _med(xs):
    return statistics.median(xs) if xs else float("nan")


def run(workload: str, reps: int) -> str:
    import ctypes

    import torch

    sys.path.insert(0, ROOT)
    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import WORKLOADS, workload_inputs

    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: run `python -m test_rnn_layers_amd.phase_stamps build` first")
    product = libttt.LIB_PATH
    w = next(x for x in WORKLOADS if x.name.startswith(workload))
    B, H, L = w.B, w.H, w.L
    N = L // 16
    inp = workload_inputs(w)
    dev = "cuda"
    x = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    W0, b0 = inp["W0"].to(dev).contiguous(), inp["b0"].to(dev).contiguous()
    cfg = libttt.linear_cfg(B, H, in_dtype=w.dtype, out_dtype="f32", rope=w.rope)
    out = torch.empty((B, H, L, 64), dtype=torch.float32, device=dev)
    st = libttt.LinearState.empty(B, H, 64, device=dev)
    stream = torch.cuda.current_stream()

    def timed(lib_path):
        libttt._lib = None
        libttt.LIB_PATH = lib_path
        lib = libttt.load()
        ms = []
        for _ in range(reps):
            libttt.ttt_linear_state_init(cfg, W0, b0, st, stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            libttt.ttt_linear_prefill(cfg, L, x["XQ"], x["XK"], x["XV"], eta, lw, lb, st, out, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return lib, ms

    _, ms_product = timed(product)
    first, count = 256, 64  # the stamped window of mini-batches (kStampFirst, kStampSteps)
    if N < first + count + 1:
        raise SystemExit(f"{w.name} has {N} mini-batches per chain; the stamped window needs {first + count + 1}")
    stamps = torch.zeros(count * 8 * 8, dtype=torch.int32, device=dev)
    libttt._lib = None
    libttt.LIB_PATH = LIB
    lib = libttt.load()
    lib.ttt_phase_stamps_set.argtypes = [ctypes.c_void_p]
    if lib.ttt_phase_stamps_set(ctypes.c_void_p(stamps.data_ptr())) != 0:
        raise SystemExit("ttt_phase_stamps_set failed")
    _, ms_stamped = timed(LIB)
    # 32-bit clock values: times relative to the first stamp, modulo 2^32
    raw = stamps.view(count, 8, 8).cpu().long().tolist()
    t0 = raw[0][0][0]
    s = [[[((t - t0 + (1 << 31)) % (1 << 32)) - (1 << 31) for t in wv] for wv in st] for st in raw]

    lo, hi = 0, count - 1  # window-relative steps that have a successor
    row = {k: [] for k in range(6)}
    col = {k: [] for k in range(4)}
    step = []
    for m in range(lo, hi):
        for wv in range(4, 8):
            a, b = s[m][wv], s[m + 1][wv]
            for k in range(5):
                row[k].append(a[k + 1] - a[k])
            row[5].append(b[0] - a[5])
        for wv in range(4):
            a, b = s[m][wv], s[m + 1][wv]
            for k in range(3):
                col[k].append(a[k + 1] - a[k])
            col[3].append(b[0] - a[3])
            step.append(b[0] - a[0])
    total = s[hi][0][0] - s[lo][0][0]
    mean_ms = statistics.mean(ms_stamped[1:] or ms_stamped)
    # the stamped launch covers N steps; the window covers hi - lo
    clock_ghz = total / (hi - lo) * N / (mean_ms * 1e-3) / 1e9
    lines = [f"# Phase breakdown of linear_dual_kernel ({w.name}), cycles per mini-batch", "",
             "Commands:", "", "```",
             "python -m test_rnn_layers_amd.phase_stamps build",
             f"python -m test_rnn_layers_amd.phase_stamps run --workload {workload} --reps {reps} --out <this file>",
             "```", "",
             f"- launch time, product build: median {_med(ms_product) * 1e3:.1f} us; instrumented build: median "
             f"{_med(ms_stamped) * 1e3:.1f} us ({reps} launches each); the stamps stretch every phase, so "
             f"the figures below are shares of an instrumented step, not of the product kernel's",
             f"- steady state (mini-batches {first}..{first + hi - 1} of chain 0): median step {_med(step):.0f} cycles; "
             f"s_memtime ticks at ~{clock_ghz:.2f} GHz against the launch time (an estimate: the slice is "
             f"scaled to the whole launch)", "",
             "Column waves (4 waves x steps; median and mean cycles):", "",
             "| part | median | mean |", "|---|---|---|"]
    for k, name in enumerate(COL_NAMES):
        lines.append(f"| {name} | {_med(col[k]):.0f} | {statistics.mean(col[k]):.0f} |")
    lines += ["", "Row waves:", "", "| part | median | mean |", "|---|---|---|"]
    for k, name in enumerate(ROW_NAMES):
        lines.append(f"| {name} | {_med(row[k]):.0f} | {statistics.mean(row[k]):.0f} |")
    seq = _med(col[0]) + _med(row[4])
    lines += ["", f"- sequential path inside the step (Z product + backward LayerNorm, medians): {seq:.0f} cycles; "
                  f"the rest of the step is the two barriers and the roles waiting for each other"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--workload", default="linear_1b", choices=["linear_1b", "linear_125m"])
    r.add_argument("--reps", type=int, default=5)
    r.add_argument("--out", default=None)
    a = ap.parse_args()
    if a.cmd == "build":
        print(build())
        return
    text = run(a.workload, a.reps)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
