"""Benchmark of the TTT hot path on one MI355X.

Default workload: TTT-Linear prefill, 1B-style layer (32 heads x 64,
mini-batch 16), B = 4, L = 8192, bf16 inputs, fp32 state and output, seeded
synthetic inputs resident in HBM.  One step = initialise the state from W0, b0
and run the whole prefill over the batch (one pass of every step of the path).

Other workloads (``--workload``):
  linear_125m  TTT-Linear prefill, B = 8, H = 12, L = 2048, rotary on
  mlp_350m     TTT-MLP prefill, B = 4, H = 16, L = 4096, hidden 256
  decode_1b    B = 64, H = 32: prefill 512 tokens, then 256 single-token
               decode calls; the value is decode tokens/s
  mlp_decode_350m  TTT-MLP, B = 16, H = 16: prefill 512 tokens, then 64
               single-token decode calls; the value is decode tokens/s
  post_proj_1b the steps after the layer: post-norm LayerNorm and output
               projection of the 1B-style layer output (M = B L = 32768
               rows, width 2048 -> 2048), bf16 in and out; tokens/s

Prints one JSON line: whole-step throughput, the roofline of the dominant
kernel (its launches timed with HIP events on the stream they run on), and
the CPU oracle timed on a bounded sample of the same workload.

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
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA, TFLOP/s
D, K, F = 64, 16, 256


# algorithmic HBM bytes of one TTT-Linear token of one head: q, k, v in + eta
# + out (prefill and decode alike)
def linear_token_bytes(in_dtype, out_dtype):
    e = {"bf16": 2, "f32": 4}
    return 3 * D * e[in_dtype] + 4 + D * e[out_dtype]


def decode_state_bytes(layout, positions):
    """Mean state bytes one chain reads and writes per decode call, over the
    calls at `positions`.  Every call reads W_s, b_s; a call that closes the
    mini-batch writes them.  Dense layout: read W_grad, b_grad unless the
    mini-batch is empty, write them.  Rows layout: read the p open rows
    [k_j | eta_j g_j] and b_grad, write the row added (none when the call
    closes the mini-batch) and b_grad."""
    wb = (D * D + D) * 4
    total = 0
    for pos in positions:
        p = pos % K
        n = wb
        if layout == "dense":
            n += (wb if p else 0) + wb
        else:
            n += p * 2 * D * 4 + (D * 4 if p else 0) + (2 * D * 4 if p != K - 1 else 0) + D * 4
        if p == K - 1:
            n += wb
        total += n
    return total / len(positions)


def mlp_decode_state_bytes(layout, positions):
    """Mean state bytes one TTT-MLP chain reads and writes per decode call:
    W1, b1, W2, b2 read, and written by a call that closes the mini-batch.
    Dense layout: W1_grad .. b2_grad read unless the mini-batch is empty, and
    written.  Rows layout: the p open rows [k | eta g1], [x2 | eta g2] and
    b1_grad, b2_grad read, the row added (none when the call closes the
    mini-batch) and b1_grad, b2_grad written."""
    par = (2 * D * F + F + D) * 4
    row = 2 * (D + F) * 4
    bias = (F + D) * 4
    total = 0
    for pos in positions:
        p = pos % K
        n = par
        if layout == "dense":
            n += (par if p else 0) + par
        else:
            n += p * row + (bias if p else 0) + (row if p != K - 1 else 0) + bias
        if p == K - 1:
            n += par
        total += n
    return total / len(positions)


# the state a prefill chain reads once and writes once: W, b (fp32)
LINEAR_STATE_BYTES = 2 * (D * D + D) * 4
# the state of one TTT-MLP chain, read once and written once: W1, b1, W2, b2
MLP_STATE_BYTES = 2 * (D * F + F + F * D + D) * 4
# MFMA flops of one TTT-MLP mini-batch of one chain (dual form):
#   X W1, Q W1, X2 W2, ng2 W2^T, Xb2 W2, X^T ng1, X2^T ng2   7 x 2*16*64*256
#   Q X^T, M2 ng2                                              2 x 2*16*16*64
#   M1 ng1, Xb2 X2^T                                           2 x 2*16*16*256
MLP_FLOPS_PER_BLOCK = 7 * 2 * K * D * F + 2 * 2 * K * K * D + 2 * 2 * K * K * F


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="linear_1b",
                    choices=["linear_1b", "linear_125m", "mlp_350m", "decode_1b", "mlp_decode_350m",
                             "post_proj_1b"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--rope", action="store_true", help="rotary on for a linear workload that has it off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget")
    ap.add_argument("--decode-eager", action="store_true",
                    help="decode workload: launch the decode calls one by one instead of replaying a HIP graph")
    ap.add_argument("--grad-layout", default="rows", choices=["rows", "dense"],
                    help="decode workloads: how the state holds the open mini-batch's gradients (the rows "
                         "[k_j | eta_j g_j], or their dense sums)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB twice (calibrates HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
class Timer:
    """HIP events around launches on one stream."""

    def __init__(self, stream):
        import torch

        self.torch, self.stream, self.pairs = torch, stream, {}

    def start(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.setdefault(name, []).append([e, None])

    def stop(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[name][-1][1] = e

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def stats(xs):
    xs = sorted(xs)
    q = lambda p: xs[min(len(xs) - 1, int(round(p * (len(xs) - 1))))]  # noqa: E731
    return {"mean": sum(xs) / len(xs), "p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "n": len(xs)}


def run_steps(args, step):
    import torch

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _profile_record(name, kernel, workload):
    """A committed rocprofv3 record of this kernel and workload, if it was
    taken on the kernel source as it is now."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(f"{kernel}@{workload}")
    from test_rnn_layers_amd.profile_summary import source_digest

    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE runs."""
    rec = _profile_record("traffic.json", kernel, workload)
    return None if rec is None else rec["hbm_bytes_per_launch"]


def measured_mfma(kernel, workload):
    """Matrix-core busy fraction from SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE."""
    rec = _profile_record("mfma.json", kernel, workload)
    if rec is None:
        return None
    return {"busy_frac_chip": rec["mfma_busy_frac_chip"],
            "busy_frac_occupied_cus": rec["mfma_busy_frac_occupied_cus"],
            "occupied_cus": rec["occupied_cus"], "counter_flops": rec["counter_flops"],
            "source": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs"}


def roofline(kernel, workload, *, bound, amount, kernel_ms, per_unit, units):
    peak, unit = (HBM_PEAK_GBS, "GB/s") if bound == "hbm" else (F16_MFMA_PEAK_TFLOPS, "TFLOP/s")
    scale = 1e9 if bound == "hbm" else 1e12
    achieved = amount / (kernel_ms["mean"] * 1e-3) / scale
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": measured_traffic(kernel, workload), "mfma_util_counter": measured_mfma(kernel, workload),
            "kernel": kernel, "kernel_ms": kernel_ms,
            "algorithmic_per_launch": amount, "algorithmic_per_unit": per_unit, "units_per_launch": units}


def copy_probe(mb):
    """A plain device copy of known size (for scaling the byte counters)."""
    import torch

    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy probe: {n * 4} bytes read, {n * 4} bytes written per copy", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# CPU oracle baselines (bounded samples)
# ---------------------------------------------------------------------------
def _f64(t):
    return t.double().numpy()


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def with_thread_sweep(fn, budget, *a):
    """fn(*a, budget) at the oracle's full thread count (the reported value),
    then at 1, 2, 4, ... threads below it with a quarter of the budget each
    (at least one unit of work per point)."""
    import oracle

    tmax = oracle.max_threads()
    res = fn(*a, budget)
    sweep = []
    t = 1
    try:
        while t < tmax:
            oracle.set_threads(t)
            sweep.append({"threads": t, "value": fn(*a, budget / 4)["value"]})
            t *= 2
    finally:
        oracle.set_threads(tmax)
    sweep.append({"threads": tmax, "value": res["value"]})
    model, nproc = host_cpu()
    res.update({"cpu_model": model, "nproc": nproc, "thread_sweep": sweep})
    return res


def cpu_linear(inp, w, rope, budget):
    """The oracle over whole batch rows of the workload (all heads, full L,
    OpenMP over the chains), cycling through the rows until the time budget
    is spent."""
    import numpy as np

    import oracle

    H, L = w.H, w.L
    eta, lw, lb = _f64(inp["eta"]), _f64(inp["ln_w"]), _f64(inp["ln_b"])
    x = {n: _f64(inp[n]) for n in ("XQ", "XK", "XV")}
    done, dt = 0, 0.0
    while done == 0 or dt < budget:
        r = done % w.B
        XQ, XK, XV = (np.ascontiguousarray(x[n][r:r + 1]) for n in ("XQ", "XK", "XV"))
        W = np.ascontiguousarray(np.broadcast_to(_f64(inp["W0"]), (1, H, D, D)))
        b = np.ascontiguousarray(np.broadcast_to(_f64(inp["b0"]), (1, H, D)))
        t0 = time.perf_counter()
        oracle.linear_batch(XQ, XK, XV, eta, 0, lw, lb, W, b, np.zeros_like(W), np.zeros_like(b), K=K, rope=rope)
        dt += time.perf_counter() - t0
        done += 1
    return {"value": done * L / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{done} batch rows of the workload's {w.B}, cycled ({H} heads x {L} tokens each), "
                      f"fp64 primal form, {dt:.1f} s"}


def cpu_mlp(inp, w, budget):
    import numpy as np

    import oracle

    H, L = w.H, w.L
    eta, lw, lb = _f64(inp["eta"]), _f64(inp["ln_w"]), _f64(inp["ln_b"])
    st0 = [_f64(inp[n]) for n in ("W1", "b1", "W2", "b2")]
    x = {n: _f64(inp[n]) for n in ("XQ", "XK", "XV")}
    done, dt = 0, 0.0
    while done == 0 or dt < budget:
        r = done % w.B
        XQ, XK, XV = (np.ascontiguousarray(x[n][r:r + 1]) for n in ("XQ", "XK", "XV"))
        st = [np.ascontiguousarray(a[None]) for a in st0]
        grads = [np.zeros_like(a) for a in st]
        t0 = time.perf_counter()
        oracle.mlp_batch(XQ, XK, XV, eta, 0, lw, lb, *st, *grads, K=K)
        dt += time.perf_counter() - t0
        done += 1
    return {"value": done * L / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{done} batch rows of the workload's {w.B}, cycled ({H} heads x {L} tokens each), "
                      f"fp64 primal form, {dt:.1f} s"}


def cpu_decode(inp, w, budget):
    """The oracle's decode rate: every sequence prefilled over 512 tokens
    (untimed), then its 256 decode tokens timed from a copy of that state,
    repeated until the budget is spent."""
    import numpy as np

    import oracle

    B, H, P, T = w.B, w.H, w.prefill, w.decode
    eta, lw, lb = _f64(inp["eta"]), _f64(inp["ln_w"]), _f64(inp["ln_b"])
    x = {n: _f64(inp[n]) for n in ("XQ", "XK", "XV")}
    W = np.ascontiguousarray(np.broadcast_to(_f64(inp["W0"]), (B, H, D, D)))
    b = np.ascontiguousarray(np.broadcast_to(_f64(inp["b0"]), (B, H, D)))
    G, gb = np.zeros_like(W), np.zeros_like(b)
    sl = lambda n, a, z: np.ascontiguousarray(x[n][:, :, a:z])  # noqa: E731
    oracle.linear_batch(sl("XQ", 0, P), sl("XK", 0, P), sl("XV", 0, P), np.ascontiguousarray(eta[:, :P]), 0, lw,
                        lb, W, b, G, gb, K=K)
    dq, dk, dv = sl("XQ", P, P + T), sl("XK", P, P + T), sl("XV", P, P + T)
    de = np.ascontiguousarray(eta[:, P:P + T])
    reps, dt = 0, 0.0
    while reps == 0 or dt < budget:
        s = [a.copy() for a in (W, b, G, gb)]
        t0 = time.perf_counter()
        oracle.linear_batch(dq, dk, dv, de, 0, lw, lb, *s, K=K, offset=P)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * B * T / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"all {B} sequences x {H} heads, {T} decode tokens after a {P}-token prefill (prefill "
                      f"untimed), {reps} repetitions, fp64 primal form, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def arithmetic(kind, in_dtype):
    """The arithmetic the timed kernel computes in (not the input format)."""
    if kind == "dual":
        if in_dtype == "bf16":
            return "bf16 in, fp16 MFMA operands (power-of-two range scaling), fp32 accumulate and state"
        return "fp32 in, fp32 MFMA (16x16x4), fp32 state"
    return f"{in_dtype} in, fp32 VALU arithmetic, fp32 state"


def common(args, w, value, elapsed, dtype, extra_cfg):
    return {"metric": None, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic: seeded N(0,1) q/k/v rounded to bf16, W ~ N(0, 0.02^2), zero biases, "
                    "eta = sigmoid(N(0,1))/64",
            "config": dict({"workload": w.name, "B": w.B, "H": w.H, "head_dim": D, "mini_batch": K,
                            "in_dtype": w.dtype, "out_dtype": args.out_dtype, "state_dtype": "f32",
                            "parallelism": "single GPU, one workgroup per (batch, head) chain"}, **extra_cfg)}


def input_sets(inp, dev):
    """Two resident input sets, alternated between steps, so that the 256 MB
    MALL does not serve one step's inputs from the previous step."""
    sets = []
    for s in range(2):
        xs = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
        if s == 1:
            xs = {n: t.flip(0).contiguous() for n, t in xs.items()}
        sets.append(xs)
    return sets


def bench_linear(args, w):
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import workload_inputs

    dev = "cuda"
    B, H, L = w.B, w.H, w.L
    rope = w.rope or args.rope
    inp = workload_inputs(w)
    cfg = libttt.linear_cfg(B, H, in_dtype=w.dtype, out_dtype=args.out_dtype, rope=rope)
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    sets = input_sets(inp, dev)
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    W0, b0 = inp["W0"].to(dev).contiguous(), inp["b0"].to(dev).contiguous()
    out = torch.empty((B, H, L, D), dtype=odt, device=dev)
    st = libttt.LinearState.empty(B, H, D, device=dev)
    stream = torch.cuda.current_stream()
    tm = Timer(stream)

    def step(i, timed):
        x = sets[i % 2]
        libttt.ttt_linear_state_init(cfg, W0, b0, st, stream)
        if timed:
            tm.start("prefill")
        libttt.ttt_linear_prefill(cfg, L, x["XQ"], x["XK"], x["XV"], eta, lw, lb, st, out, stream)
        if timed:
            tm.stop("prefill")

    elapsed = run_steps(args, step)
    per = linear_token_bytes(w.dtype, args.out_dtype)
    amount = per * B * H * L + LINEAR_STATE_BYTES * B * H
    res = common(args, w, B * L * args.steps / elapsed, elapsed, arithmetic("dual", w.dtype),
                 {"L": L, "rope": rope})
    res["metric"] = ("TTT-Linear prefill tokens/sec (1B shape, L=8192) + % of HBM/MFMA roofline"
                     if w.name.startswith("linear_1b") else f"TTT-Linear prefill tokens/sec ({w.name})")
    res["roofline"] = roofline("linear_dual_kernel", w.name + ("_rope" if rope and not w.rope else ""),
                               bound="hbm", amount=amount, kernel_ms=stats(tm.ms("prefill")),
                               per_unit=f"{per} B per token-head + {LINEAR_STATE_BYTES} B state per chain",
                               units=f"{B * H * L} token-heads, {B * H} chains")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_thread_sweep(cpu_linear, args.cpu_seconds, inp, w, rope)
    return res


def bench_mlp(args, w):
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import workload_inputs

    dev = "cuda"
    B, H, L = w.B, w.H, w.L
    inp = workload_inputs(w)
    cfg = libttt.mlp_cfg(B, H, in_dtype=w.dtype, out_dtype=args.out_dtype)
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    sets = input_sets(inp, dev)
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    init = [inp[n].to(dev).contiguous() for n in ("W1", "b1", "W2", "b2")]
    out = torch.empty((B, H, L, D), dtype=odt, device=dev)
    st = libttt.MlpState.empty(B, H, D, F, device=dev)
    stream = torch.cuda.current_stream()
    tm = Timer(stream)

    def step(i, timed):
        x = sets[i % 2]
        libttt.ttt_mlp_state_init(cfg, *init, st, stream)
        if timed:
            tm.start("prefill")
        libttt.ttt_mlp_prefill(cfg, L, x["XQ"], x["XK"], x["XV"], eta, lw, lb, st, out, stream)
        if timed:
            tm.stop("prefill")

    elapsed = run_steps(args, step)
    nblk = (L + K - 1) // K
    amount = MLP_FLOPS_PER_BLOCK * B * H * nblk
    res = common(args, w, B * L * args.steps / elapsed, elapsed, arithmetic("dual", w.dtype),
                 {"L": L, "mlp_hidden": F, "rope": False})
    res["metric"] = f"TTT-MLP prefill tokens/sec ({w.name})"
    res["roofline"] = roofline("mlp_dual_kernel", w.name, bound="mfma", amount=amount,
                               kernel_ms=stats(tm.ms("prefill")),
                               per_unit=f"{MLP_FLOPS_PER_BLOCK} MFMA flops per 16-token mini-batch per chain",
                               units=f"{B * H * nblk} chain mini-batches")
    hbm = linear_token_bytes(w.dtype, args.out_dtype) * B * H * L + MLP_STATE_BYTES * B * H
    res["roofline"]["hbm_gbs"] = hbm / (res["roofline"]["kernel_ms"]["mean"] * 1e-3) / 1e9
    res["roofline"]["note"] = ("64 chains on 256 CUs: one workgroup per chain, so at most a quarter of the "
                               "chip's matrix cores can be busy")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_thread_sweep(cpu_mlp, args.cpu_seconds, inp, w)
    return res


def bench_decode(args, w):
    """Prefill 512 tokens, then 256 single-token decode calls.  By default the
    256 calls are captured once in a HIP graph and replayed each step (the
    serving loop); --decode-eager launches them one by one from Python."""
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import workload_inputs

    dev = "cuda"
    B, H, P, T = w.B, w.H, w.prefill, w.decode
    inp = workload_inputs(w)
    cfg = libttt.linear_cfg(B, H, in_dtype=w.dtype, out_dtype=args.out_dtype, rope=w.rope,
                            grad_layout=args.grad_layout)
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    x = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    W0, b0 = inp["W0"].to(dev).contiguous(), inp["b0"].to(dev).contiguous()
    out = torch.empty((B, H, P + T, D), dtype=odt, device=dev)
    st = libttt.LinearState.empty(B, H, D, device=dev)
    # views of every decode token, made once
    views = [tuple(x[n][:, :, t:t + 1] for n in ("XQ", "XK", "XV")) + (eta[:, t:t + 1], out[:, :, t:t + 1])
             for t in range(P, P + T)]

    def prefill(stream):
        libttt.ttt_linear_state_init(cfg, W0, b0, st, stream)
        libttt.ttt_linear_prefill(cfg, P, x["XQ"][:, :, :P], x["XK"][:, :, :P], x["XV"][:, :, :P], eta[:, :P],
                                  lw, lb, st, out[:, :, :P], stream)

    def decode_all(stream, tm=None):
        for (q, k, v, e, o) in views:
            if tm:
                tm.start("token")
            libttt.ttt_linear_decode(cfg, 1, q, k, v, e, lw, lb, st, o, stream)
            if tm:
                tm.stop("token")

    graph = None
    if not args.decode_eager:
        # warm up eagerly, then capture the decode calls from the post-prefill
        # state (their positions are baked into the graph, so every replay
        # starts from a fresh prefill)
        prefill(torch.cuda.current_stream())
        decode_all(torch.cuda.current_stream())
        prefill(torch.cuda.current_stream())
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_all(torch.cuda.current_stream())
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    tm = Timer(stream)

    def step(i, timed):
        if timed:
            tm.start("prefill")
        prefill(stream)
        if timed:
            tm.stop("prefill")
            tm.start("decode")
        if graph is not None:
            graph.replay()
        else:
            decode_all(stream, tm if timed else None)
        if timed:
            tm.stop("decode")

    elapsed = run_steps(args, step)
    dec = stats(tm.ms("decode"))
    per_tok = linear_token_bytes(w.dtype, args.out_dtype)
    # per chain and decode call: the state read and written (mean over the
    # 256 positions), the token's inputs and output
    state_rw = decode_state_bytes(args.grad_layout, range(P, P + T))
    amount = (per_tok + state_rw) * B * H
    if graph is not None:
        # back-to-back replayed launches: the mean launch duration is the
        # replay time over the number of calls (gaps between launches included)
        kms = {k: (v / T if k != "n" else v * T) for k, v in dec.items()}
        how = "HIP graph of the 256 decode calls, replayed; per-call time = replay time / 256"
    else:
        kms = stats(tm.ms("token"))
        how = "256 decode calls launched one by one from Python; per-call HIP events"
    res = common(args, w, B * T / (dec["mean"] * 1e-3), elapsed, arithmetic("token", w.dtype),
                 {"prefill": P, "decode_steps": T, "rope": w.rope, "decode_launch": how,
                  "grad_layout": args.grad_layout,
                  "decode_phase_ms": dec, "prefill_ms": stats(tm.ms("prefill")),
                  "value_is": "decode tokens/s over the 256 decode calls (GPU time of the decode phase)",
                  "step_tokens_per_s": B * (P + T) * args.steps / elapsed})
    res["metric"] = f"TTT-Linear decode tokens/sec ({w.name})"
    res["roofline"] = roofline("linear_token_kernel", w.name, bound="hbm", amount=amount, kernel_ms=kms,
                               per_unit=f"{per_tok} B token in/out + {state_rw:g} B state read/write per chain "
                                        f"({args.grad_layout} W_grad, mean over the decode positions)",
                               units=f"{B * H} chains, one token each")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_thread_sweep(cpu_decode, args.cpu_seconds, inp, w)
    return res


def cpu_mlp_decode(inp, w, budget):
    """The oracle's TTT-MLP decode rate: every sequence prefilled over the
    prefill tokens (untimed), then its decode tokens timed from a copy of that
    state; only as many batch rows as the budget allows."""
    import numpy as np

    import oracle

    B, H, P, T = w.B, w.H, w.prefill, w.decode
    eta, lw, lb = _f64(inp["eta"]), _f64(inp["ln_w"]), _f64(inp["ln_b"])
    x = {n: _f64(inp[n]) for n in ("XQ", "XK", "XV")}
    st0 = [_f64(inp[n]) for n in ("W1", "b1", "W2", "b2")]
    sl = lambda n, r, a, z: np.ascontiguousarray(x[n][r:r + 1, :, a:z])  # noqa: E731
    rows, dt = 0, 0.0
    while rows == 0 or dt < budget:
        r = rows % B
        st = [np.ascontiguousarray(a[None]) for a in st0]
        grads = [np.zeros_like(a) for a in st]
        oracle.mlp_batch(sl("XQ", r, 0, P), sl("XK", r, 0, P), sl("XV", r, 0, P),
                         np.ascontiguousarray(eta[:, :P]), 0, lw, lb, *st, *grads, K=K)
        t0 = time.perf_counter()
        oracle.mlp_batch(sl("XQ", r, P, P + T), sl("XK", r, P, P + T), sl("XV", r, P, P + T),
                         np.ascontiguousarray(eta[:, P:P + T]), 0, lw, lb, *st, *grads, K=K, offset=P)
        dt += time.perf_counter() - t0
        rows += 1
    return {"value": rows * T / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{rows} batch rows of the workload's {B}, cycled ({H} heads, {T} decode tokens after a "
                      f"{P}-token prefill, prefill untimed), fp64 primal form, {dt:.1f} s"}


def bench_mlp_decode(args, w):
    """TTT-MLP: prefill, then single-token decode calls replayed from a HIP
    graph (as for TTT-Linear decode)."""
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import workload_inputs

    dev = "cuda"
    B, H, P, T = w.B, w.H, w.prefill, w.decode
    inp = workload_inputs(w)
    cfg = libttt.mlp_cfg(B, H, in_dtype=w.dtype, out_dtype=args.out_dtype, grad_layout=args.grad_layout)
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    x = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
    eta = inp["eta"].to(dev).contiguous()
    lw, lb = inp["ln_w"].to(dev).contiguous(), inp["ln_b"].to(dev).contiguous()
    init = [inp[n].to(dev).contiguous() for n in ("W1", "b1", "W2", "b2")]
    out = torch.empty((B, H, P + T, D), dtype=odt, device=dev)
    st = libttt.MlpState.empty(B, H, D, F, device=dev)
    views = [tuple(x[n][:, :, t:t + 1] for n in ("XQ", "XK", "XV")) + (eta[:, t:t + 1], out[:, :, t:t + 1])
             for t in range(P, P + T)]

    def prefill(stream):
        libttt.ttt_mlp_state_init(cfg, *init, st, stream)
        libttt.ttt_mlp_prefill(cfg, P, x["XQ"][:, :, :P], x["XK"][:, :, :P], x["XV"][:, :, :P], eta[:, :P],
                               lw, lb, st, out[:, :, :P], stream)

    def decode_all(stream):
        for (q, k, v, e, o) in views:
            libttt.ttt_mlp_decode(cfg, 1, q, k, v, e, lw, lb, st, o, stream)

    cur = torch.cuda.current_stream()
    prefill(cur)
    decode_all(cur)
    prefill(cur)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all(torch.cuda.current_stream())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    tm = Timer(stream)

    def step(i, timed):
        prefill(stream)
        if timed:
            tm.start("decode")
        graph.replay()
        if timed:
            tm.stop("decode")

    elapsed = run_steps(args, step)
    dec = stats(tm.ms("decode"))
    per_tok = linear_token_bytes(w.dtype, args.out_dtype)
    state_rw = mlp_decode_state_bytes(args.grad_layout, range(P, P + T))
    amount = (per_tok + state_rw) * B * H
    kms = {k: (v / T if k != "n" else v * T) for k, v in dec.items()}
    res = common(args, w, B * T / (dec["mean"] * 1e-3), elapsed, arithmetic("token", w.dtype),
                 {"prefill": P, "decode_steps": T, "mlp_hidden": F, "grad_layout": args.grad_layout,
                  "decode_launch": f"HIP graph of the {T} decode calls, replayed; per-call time = replay time / {T}",
                  "decode_phase_ms": dec,
                  "value_is": f"decode tokens/s over the {T} decode calls (GPU time of the decode phase)"})
    res["metric"] = f"TTT-MLP decode tokens/sec ({w.name})"
    res["roofline"] = roofline("mlp_token_kernel", w.name, bound="hbm", amount=amount, kernel_ms=kms,
                               per_unit=f"{per_tok} B token in/out + {state_rw:g} B state read/write per chain "
                                        f"({args.grad_layout} gradients, mean over the decode positions)",
                               units=f"{B * H} chains, one token each")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_thread_sweep(cpu_mlp_decode, args.cpu_seconds, inp, w)
    return res


# post-norm + output projection of the 1B-style layer: M = B L rows of the
# layer output, K = width = 32 heads x 64, N = the model width
POST_PROJ_1B = dict(name="post_proj_1b_M32768_K2048_N2048_bf16", M=4 * 8192, K=2048, N=2048, seed=1240)


def cpu_post_proj(inp, budget):
    """The oracle on blocks of 64 rows of the same inputs, cycled, until the
    budget is spent."""
    import oracle

    y = inp["y"].double().numpy()
    g, b, W = (inp[n].double().numpy() for n in ("gamma", "beta", "Wo"))
    M = y.shape[0]
    done, dt = 0, 0.0
    while done == 0 or dt < budget:
        r0 = (done * 64) % M
        t0 = time.perf_counter()
        oracle.post_proj(y[r0:r0 + 64], g, b, W, None, 1e-5)
        dt += time.perf_counter() - t0
        done += 1
    return {"value": done * 64 / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{done} blocks of 64 rows of the {M}-row workload, fp64, {dt:.1f} s"}


def bench_post_proj(args):
    import torch

    from test_rnn_layers_amd import libttt
    from test_rnn_layers_amd.synth import make_post_proj_inputs

    c = POST_PROJ_1B
    M, K, N = c["M"], c["K"], c["N"]
    dev = "cuda"
    inp = make_post_proj_inputs(M, K, N, seed=c["seed"])
    ys = [inp["y"].to(dev).contiguous(), inp["y"].flip(0).to(dev).contiguous()]  # two resident sets (MALL)
    g, b, W = (inp[n].to(dev).contiguous() for n in ("gamma", "beta", "Wo"))
    prepared = torch.empty(libttt.ttt_post_proj_prepared_bytes(K, N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    libttt.ttt_post_proj_prepare(K, N, g, b, W, None, prepared, stream)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    tm = Timer(stream)

    def step(i, timed):
        if timed:
            tm.start("proj")
        libttt.ttt_post_proj(M, K, N, ys[i % 2], K, 1e-5, prepared, out, N, "bf16", stream)
        if timed:
            tm.stop("proj")

    elapsed = run_steps(args, step)
    flops = 2 * M * K * N
    res = {"metric": f"post-norm + output projection tokens/sec ({c['name']})", "value": M * args.steps / elapsed,
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 MFMA operands (gamma folded into the weights), fp32 accumulate",
           "data": "synthetic: seeded bf16 rows N(m, s^2) with per-row m, s; gamma, beta near 1, 0; Wo ~ N(0, 0.02^2)",
           "config": {"workload": c["name"], "M": M, "K": K, "N": N, "in_dtype": "bf16", "out_dtype": "bf16",
                      "parallelism": "single GPU, 256x256 output tiles"}}
    res["roofline"] = roofline("post_proj_kernel", c["name"], bound="mfma", amount=flops,
                               kernel_ms=stats(tm.ms("proj")),
                               per_unit=f"2 K N = {2 * K * N} MFMA flops per row",
                               units=f"{M} rows")
    try:
        res["library_gemm"] = library_gemm(ys, prepared, M, K, N)
    except RuntimeError as e:  # a reference point only: never the reason the line is missing
        res["library_gemm"] = {"error": str(e)[:200]}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_thread_sweep(cpu_post_proj, args.cpu_seconds, inp)
    return res


def library_gemm(ys, prepared, M, K, N, reps=10):
    """Context for the projection's roofline: the vendor library's plain GEMM
    (torch.nn.functional.linear, bf16 in and out) on the same y and W' operands,
    without the LayerNorm fold.  Timed after, and apart from, the product path."""
    import torch

    Wt = prepared[:N * K * 2].view(torch.bfloat16).view(N, K)
    for i in range(3):
        torch.nn.functional.linear(ys[i % 2], Wt)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        torch.nn.functional.linear(ys[i % 2], Wt)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"what": "torch.nn.functional.linear (vendor BLAS) on the same bf16 y and W' operands, bf16 out, "
                    "no LayerNorm fold; not part of the measured path",
            "us_mean": round(ms * 1e3, 1), "tflops": round(2 * M * K * N / (ms * 1e-3) / 1e12, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the (batch, head) "
              "chains are independent, so more GPUs would each take a share of the batch", file=sys.stderr)
        sys.exit(2)
    if args.workload == "post_proj_1b":
        res = bench_post_proj(args)
        if args.copy_probe_mb:
            copy_probe(args.copy_probe_mb)
        print(json.dumps(res), flush=True)
        return
    from test_rnn_layers_amd.synth import WORKLOADS

    w = {"linear_125m": WORKLOADS[1], "linear_1b": WORKLOADS[2], "mlp_350m": WORKLOADS[3],
         "decode_1b": WORKLOADS[4], "mlp_decode_350m": WORKLOADS[5]}[args.workload]
    fn = {"linear": bench_linear, "mlp": bench_mlp, "decode": bench_decode, "mlp_decode": bench_mlp_decode}[w.kind]
    res = fn(args, w)
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
