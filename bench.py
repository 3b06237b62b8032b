"""Benchmark of the TTT hot path on one MI355X.

Default workload: TTT-Linear prefill, 1B-style layer (32 heads x 64,
mini-batch 16), B = 4, L = 8192, bf16 inputs, fp32 state and output, seeded
synthetic inputs resident in HBM.  One step = initialise the state from W0, b0
and run the whole prefill over the batch (one pass of every step of the path).

Prints one JSON line: throughput (tokens/s, a token = one position of one
sequence over all heads), the roofline of the dominant kernel measured with
HIP events on the launch stream, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload linear_1b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# algorithmic bytes per token-head of TTT-Linear prefill: q, k, v (bf16) +
# eta (fp32) + out (fp32)
LINEAR_BYTES_PER_TOKEN_HEAD = {("bf16", "f32"): 3 * 64 * 2 + 4 + 64 * 4, ("bf16", "bf16"): 3 * 64 * 2 + 4 + 64 * 2,
                               ("f32", "f32"): 3 * 64 * 4 + 4 + 64 * 4}
# state read + written once per chain: W, b (fp32)
LINEAR_STATE_BYTES_PER_CHAIN = 2 * (64 * 64 + 64) * 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="linear_1b",
                    choices=["linear_1b", "linear_125m", "mlp_350m", "decode_1b"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline_linear(inp, w, rope):
    """The oracle as it stands, on batch 0 (all heads, full L) of the workload,
    OpenMP over the heads."""
    import numpy as np

    import oracle

    H, L, D = w.H, w.L, 64
    f64 = lambda t: t.double().numpy()  # noqa: E731
    XQ, XK, XV = (np.ascontiguousarray(f64(inp[n][:1])) for n in ("XQ", "XK", "XV"))
    eta, lw, lb = f64(inp["eta"]), f64(inp["ln_w"]), f64(inp["ln_b"])
    W = np.ascontiguousarray(np.broadcast_to(f64(inp["W0"]), (1, H, D, D)))
    b = np.ascontiguousarray(np.broadcast_to(f64(inp["b0"]), (1, H, D)))
    G, gb = np.zeros_like(W), np.zeros_like(b)
    t0 = time.perf_counter()
    oracle.linear_batch(XQ, XK, XV, eta, 0, lw, lb, W, b, G, gb, K=16, rope=rope)
    dt = time.perf_counter() - t0
    return {"value": L / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"batch row 0 of the workload: {H} heads x {L} tokens (fp64 primal form), {dt:.2f} s"}


def bench_linear(args, w):
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import workload_inputs

    dev = "cuda"
    B, H, L, D = w.B, w.H, w.L, 64
    rope = w.rope
    inp = workload_inputs(w)
    cfg = libttt.linear_cfg(B, H, in_dtype=w.dtype, out_dtype=args.out_dtype, rope=rope)
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    # two resident input sets, alternated, so the 256 MB MALL does not serve
    # the inputs of the step from the previous one
    sets = []
    for s in range(2):
        xs = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
        if s == 1:
            xs = {n: t.flip(0).contiguous() for n, t in xs.items()}
        sets.append(xs)
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    W0, b0 = inp["W0"].to(dev).contiguous(), inp["b0"].to(dev).contiguous()
    out = torch.empty((B, H, L, D), dtype=odt, device=dev)
    st = libttt.LinearState.empty(B, H, D, device=dev)
    stream = torch.cuda.current_stream()

    ev = []

    def step(i, timed):
        x = sets[i % 2]
        libttt.ttt_linear_state_init(cfg, W0, b0, st, stream)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        libttt.ttt_linear_prefill(cfg, L, x["XQ"], x["XK"], x["XV"], eta, lw, lb, st, out, stream)
        if timed:
            e1.record(stream)
            ev.append((e0, e1))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)

    tokens = B * L
    per = LINEAR_BYTES_PER_TOKEN_HEAD[(w.dtype, args.out_dtype)]
    alg_bytes = per * B * H * L + LINEAR_STATE_BYTES_PER_CHAIN * B * H
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "TTT-Linear prefill tokens/sec (1B shape, L=8192) + % of HBM/MFMA roofline"
        if w.name.startswith("linear_1b") else f"TTT-Linear prefill tokens/sec ({w.name})",
        "value": tokens * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, W0 ~ N(0, 0.02^2), eta = sigmoid(N(0,1))/64)",
        "config": {"workload": w.name, "B": B, "H": H, "head_dim": D, "L": L, "mini_batch": 16,
                   "in_dtype": w.dtype, "out_dtype": args.out_dtype, "state_dtype": "f32", "rope": rope,
                   "parallelism": "single GPU, one workgroup per (batch, head) chain"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "linear_dual_kernel", "kernel_ms": kern_ms,
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_linear(inp, w, rope)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the (batch, head) "
              "chains are independent, so more GPUs would each take a share of the batch", file=sys.stderr)
        sys.exit(2)
    from test_rnn_layers_amd.synth import WORKLOADS

    w = {"linear_125m": WORKLOADS[1], "linear_1b": WORKLOADS[2], "mlp_350m": WORKLOADS[3],
         "decode_1b": WORKLOADS[4]}[args.workload]
    if w.kind == "linear":
        res = bench_linear(args, w)
    else:
        raise SystemExit(f"workload {args.workload} not wired yet")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
