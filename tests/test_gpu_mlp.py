"""GPU parity of TTT-MLP prefill (dual form, hidden width 4D, exact GELU)
against the CPU oracle, through the C ABI.  bf16 inputs, fp32 state:
max-abs tolerance 2e-2 on outputs and state."""
import numpy as np
import pytest
import torch

from harness import MlpGPU, TOL_BF16, bf16_half_ulp, make_inputs, max_abs, oracle_mlp, oracle_mlp_all
from test_rnn_layers_amd import libttt
from test_rnn_layers_amd.synth import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

STATE = ("W1", "b1", "W2", "b2", "W1_grad", "b1_grad", "W2_grad", "b2_grad")


def _report(name, **kv):
    print(f"[{name}] " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in kv.items()),
          flush=True)


def _compare(name, got, ref, chains, *, out_dtype="f32", tol=TOL_BF16):
    """got: GPU (out, 8 state arrays) over all chains; ref: oracle over `chains`."""
    B, H = got[0].shape[:2]
    idx = [b * H + h for (b, h) in chains]
    flat = [g.reshape((B * H,) + g.shape[2:])[idx] for g in got]
    out, ro = flat[0], ref[0]
    err = max_abs(out, ro)
    errs = {n: max_abs(flat[i + 1], ref[i + 1]) for i, n in enumerate(STATE)}
    _report(name, out=err, **errs)
    assert np.isfinite(out).all()
    if out_dtype == "bf16":
        assert np.max(np.abs(out - ro) - bf16_half_ulp(ro)) <= tol
    else:
        assert err <= tol, f"{name}: output max-abs {err}"
    for n, e in errs.items():
        assert e <= tol, f"{name}: {n} max-abs {e}"


def _run(name, inp, *, rope=False, pieces=(), out_dtype="f32", chains=None, token_eta=None, K=16, in_dtype="bf16",
         decode=(), tol=TOL_BF16, grad_layout="dense"):
    B, H, L, D = inp["XQ"].shape
    g = MlpGPU(inp, rope=rope, out_dtype=out_dtype, token_eta=token_eta, K=K, in_dtype=in_dtype,
               grad_layout=grad_layout)
    cuts = [0] + list(pieces) + [L]
    for i in range(len(cuts) - 1):
        g.run(cuts[i], cuts[i + 1], decode=cuts[i] in decode)
    got = g.result()
    if chains is None:  # every chain, through the oracle's OpenMP batch driver
        chains = [(b, h) for b in range(B) for h in range(H)]
        ref = [a.reshape((B * H,) + a.shape[2:]) for a in oracle_mlp_all(inp, rope=rope, token_eta=token_eta, K=K)]
    else:
        ref = oracle_mlp(inp, rope=rope, chains=chains, token_eta=token_eta, K=K)
    _compare(name, got, ref, chains, out_dtype=out_dtype, tol=tol)
    assert g.state.offset == L
    return got


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("L", [87, 96])
def test_small_rich_parity(rope, L):
    """Several chains, non-zero b1/b2/gamma/beta; L = 87 ends in an open
    mini-batch of 7 tokens, L = 96 on a boundary."""
    inp = make_inputs(2, 3, L, dtype="bf16", seed=21 + rope + L, rich=True, mlp_hidden=256)
    _run(f"mlp_small_L{L}_rope{int(rope)}", inp, rope=rope)


@pytest.mark.parametrize("L", [1, 9, 16, 17])
def test_short_sequences(L):
    """One token, a single open mini-batch, exactly one, one plus a token."""
    inp = make_inputs(1, 2, L, dtype="bf16", seed=40 + L, rich=True, mlp_hidden=256)
    _run(f"mlp_short_L{L}", inp)


def test_split_calls():
    """Prefill in pieces whose cuts are mini-batch boundaries; the last piece
    ends open."""
    inp = make_inputs(2, 2, 117, dtype="bf16", seed=51, rich=True, mlp_hidden=256)
    _run("mlp_split", inp, pieces=(32, 80), rope=True)


@pytest.mark.parametrize("L", [87, 96])
def test_token_eta(L):
    """A non-constant token_eta (per-position step scale); L = 87 ends in an
    open mini-batch, whose accumulated gradients carry no token_eta."""
    r = np.random.default_rng(L)
    te = (1.0 / np.arange(1, 17) + 0.05 * r.uniform(size=16)).astype(np.float32).astype(np.float64)
    inp = make_inputs(2, 3, L, dtype="bf16", seed=81 + L, rich=True, mlp_hidden=256)
    _run(f"mlp_token_eta_L{L}", inp, rope=True, pieces=(32,), token_eta=te)


# --- the primal (token) path: decoding, open mini-batches, fp32 inputs, K != 16
def test_decode_steps():
    """Prefill 20 tokens (ends inside a mini-batch), then single-token decode
    calls across two mini-batch boundaries, with rotary."""
    inp = make_inputs(2, 2, 52, dtype="bf16", seed=91, rich=True, mlp_hidden=256)
    cuts = [20] + list(range(21, 52))
    _run("mlp_decode", inp, rope=True, pieces=cuts, decode=set(cuts))


def test_prefill_from_open_minibatches():
    """Prefill calls that start inside a mini-batch: the head runs in the
    token kernel, the rest in the dual kernel."""
    inp = make_inputs(2, 3, 90, dtype="bf16", seed=92, rich=True, mlp_hidden=256)
    _run("mlp_open_pieces", inp, pieces=(5, 21, 40, 41, 75))


def test_fp32_inputs():
    """fp32 inputs run token by token in fp32 arithmetic: 1e-4 bar."""
    inp = make_inputs(1, 3, 37, dtype="f32", seed=93, rich=True, mlp_hidden=256)
    _run("mlp_f32", inp, in_dtype="f32", pieces=(10,), tol=1e-4)


@pytest.mark.parametrize("K", [1, 8])
def test_other_minibatch_sizes(K):
    inp = make_inputs(1, 2, 30, dtype="f32", seed=94 + K, rich=True, mlp_hidden=256)
    _run(f"mlp_K{K}", inp, in_dtype="f32", K=K, pieces=(7, 13), tol=1e-4)


def test_decode_token_eta():
    r = np.random.default_rng(5)
    te = (1.0 / np.arange(1, 17) + 0.05 * r.uniform(size=16)).astype(np.float32).astype(np.float64)
    inp = make_inputs(1, 3, 40, dtype="bf16", seed=95, rich=True, mlp_hidden=256)
    cuts = [9] + list(range(10, 40))
    _run("mlp_decode_token_eta", inp, pieces=cuts, decode=set(cuts), token_eta=te)


def test_decode_matches_prefill():
    """The same tokens prefilled in one call (dual kernel) and decoded one at
    a time (token kernel): outputs and state agree to the fp16-operand bar."""
    inp = make_inputs(2, 2, 48, dtype="bf16", seed=96, rich=True, mlp_hidden=256)
    a = MlpGPU(inp)
    a.run(0, 48)
    b = MlpGPU(inp)
    b.run(0, 16)
    for t in range(16, 48):
        b.run(t, t + 1, decode=True)
    ra, rb = a.result(), b.result()
    for x, y in zip(ra, rb):
        assert max_abs(x, y) <= TOL_BF16, max_abs(x, y)


def test_bf16_output():
    inp = make_inputs(1, 3, 70, dtype="bf16", seed=52, rich=True, mlp_hidden=256)
    _run("mlp_bf16_out", inp, out_dtype="bf16")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("te", [False, True])
def test_every_dual_instantiation(out_dtype, rope, te):
    """Each compiled variant of the dual-form MLP kernel (output dtype,
    rotary), with and without token_eta, on a ragged length."""
    token_eta = (0.5 + np.arange(16) / 16.0).tolist() if te else None
    inp = make_inputs(2, 2, 16 * 4 + 5, dtype="bf16", seed=71 + 2 * rope + te, rich=True, mlp_hidden=256)
    _run(f"mlp_dual_{out_dtype}_rope{int(rope)}_te{int(te)}", inp, rope=rope, out_dtype=out_dtype, token_eta=token_eta)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["dense", "rows"])
def test_every_token_instantiation(in_dtype, out_dtype, layout):
    """Each compiled variant of the MLP token kernel (input and output dtype,
    gradient layout): a prefill piece, then decode calls across a commit."""
    inp = make_inputs(1, 2, 40, dtype=in_dtype, seed=91, rich=True, mlp_hidden=256)
    cuts = (21, 29, 30, 33)
    _run(f"mlp_token_{in_dtype}_{out_dtype}_{layout}", inp, pieces=cuts, decode=set(cuts), out_dtype=out_dtype,
         in_dtype=in_dtype, tol=1e-4 if in_dtype == "f32" and out_dtype == "f32" else TOL_BF16, grad_layout=layout,
         rope=True)


def test_eta_zero_is_frozen_mlp():
    """With eta = 0 the fast weights never move: out = Q + LN(f(Q)) with the
    initial f, and the state keeps its initial values."""
    inp = make_inputs(1, 2, 50, dtype="bf16", seed=53, rich=True, mlp_hidden=256)
    inp["eta"] = torch.zeros_like(inp["eta"])
    got = _run("mlp_eta0", inp)
    for i, n in enumerate(("W1", "b1", "W2", "b2")):
        assert max_abs(got[1 + i][0], inp[n].double().numpy()) == 0.0
    for i in range(4, 8):
        assert np.all(got[1 + i] == 0.0)


def test_determinism():
    inp = make_inputs(1, 4, 100, dtype="bf16", seed=54, rich=True, mlp_hidden=256)
    a = MlpGPU(inp)
    a.run(0, 100)
    b = MlpGPU(inp)
    b.run(0, 100)
    ra, rb = a.result(), b.result()
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)


def test_open_offset_continues():
    """A call that starts inside a mini-batch continues it (it used to be
    refused): 20 tokens, then 20 more, equal to the oracle over all 40."""
    inp = make_inputs(1, 1, 40, dtype="bf16", seed=55, mlp_hidden=256)
    _run("mlp_open_continue", inp, pieces=(20,))


def test_full_350m_workload():
    """The 350M-shape TTT-MLP layer (B=4, H=16, L=4096) in one launch; every
    chain's outputs and final state against the oracle."""
    w = next(x for x in WORKLOADS if x.kind == "mlp")
    _run(w.name, workload_inputs(w))


def test_decode_workload():
    """The TTT-MLP decode workload (B16 H16: prefill 512 tokens in the dual
    kernel, then 64 single-token decode calls in the token kernel); every
    chain against the oracle."""
    w = next(x for x in WORKLOADS if x.kind == "mlp_decode")
    inp = workload_inputs(w)
    L = w.L
    cuts = [w.prefill] + list(range(w.prefill + 1, L))
    _run(w.name, inp, pieces=cuts, decode=set(cuts))


# --- the rows layout of the gradients (open rows [k | eta g1], [x2 | eta g2])
def test_rows_decode_steps():
    inp = make_inputs(2, 2, 52, dtype="bf16", seed=191, rich=True, mlp_hidden=256)
    cuts = [20] + list(range(21, 52))
    _run("mlp_rows_decode", inp, rope=True, pieces=cuts, decode=set(cuts), grad_layout="rows")


def test_rows_prefill_pieces():
    """Open heads and tails around dual-kernel bodies, in the rows layout."""
    inp = make_inputs(2, 3, 90, dtype="bf16", seed=192, rich=True, mlp_hidden=256)
    _run("mlp_rows_pieces", inp, pieces=(5, 21, 40, 41, 75), grad_layout="rows")


@pytest.mark.parametrize("K", [1, 8])
def test_rows_other_minibatch_sizes(K):
    inp = make_inputs(1, 2, 30, dtype="f32", seed=193 + K, rich=True, mlp_hidden=256)
    _run(f"mlp_rows_K{K}", inp, in_dtype="f32", K=K, pieces=(7, 13), tol=1e-4, grad_layout="rows")


def test_rows_decode_token_eta():
    r = np.random.default_rng(15)
    te = (1.0 / np.arange(1, 17) + 0.05 * r.uniform(size=16)).astype(np.float32).astype(np.float64)
    inp = make_inputs(1, 3, 40, dtype="bf16", seed=195, rich=True, mlp_hidden=256)
    cuts = [9] + list(range(10, 40))
    _run("mlp_rows_decode_token_eta", inp, pieces=cuts, decode=set(cuts), token_eta=te, grad_layout="rows")


def test_rows_K8_fp32_token_eta_rope():
    """Rows layout with fp32 inputs, K = 8, rotary and token_eta together."""
    r = np.random.default_rng(8)
    te = 1.0 / np.arange(1, 9) + 0.05 * r.uniform(size=8)
    inp = make_inputs(1, 2, 30, dtype="f32", seed=197, rich=True, mlp_hidden=256)
    cuts = [5, 11] + list(range(12, 30))
    _run("mlp_rows_K8_f32_te_rope", inp, in_dtype="f32", K=8, rope=True, pieces=cuts, decode=set(cuts[2:]),
         token_eta=te, tol=1e-4, grad_layout="rows")


def test_rows_matches_dense():
    """The same calls in both layouts agree to the bf16 bar.  (Not to fp32
    rounding: in the rows layout the prefill's trailing partial mini-batch runs
    in the fp32 token kernel, in the dense layout in the fp16-operand dual
    kernel.)"""
    inp = make_inputs(2, 2, 45, dtype="bf16", seed=196, rich=True, mlp_hidden=256)
    res = []
    for layout in ("dense", "rows"):
        g = MlpGPU(inp, grad_layout=layout)
        g.run(0, 23)
        for t in range(23, 45):
            g.run(t, t + 1, decode=True)
        res.append(g.result())
    for x, y in zip(res[0], res[1]):
        assert max_abs(x, y) <= TOL_BF16, max_abs(x, y)


def test_rows_decode_workload():
    w = next(x for x in WORKLOADS if x.kind == "mlp_decode")
    inp = workload_inputs(w)
    L = w.L
    cuts = [w.prefill] + list(range(w.prefill + 1, L))
    _run(w.name + "_rows", inp, pieces=cuts, decode=set(cuts), grad_layout="rows")


# per-batch learning rates, eta [B, H, L] ("代码连连看——TTT", compute_mini_batch
# takes eta per batch and head)
def test_per_batch_eta_prefill():
    """Open head (token kernel), whole mini-batches and an open tail (dual
    kernel), with rates that differ per batch row."""
    inp = make_inputs(3, 2, 16 * 4 + 7, dtype="bf16", seed=411, rich=True, mlp_hidden=256, eta_per_batch=True)
    assert inp["eta"].shape == (3, 2, 71)
    _run("mlp_per_batch_eta", inp, rope=True, pieces=(6,))


@pytest.mark.parametrize("grad_layout", ["dense", "rows"])
def test_per_batch_eta_decode(grad_layout):
    inp = make_inputs(3, 2, 44, dtype="bf16", seed=413, rich=True, mlp_hidden=256, eta_per_batch=True)
    cuts = [19] + list(range(20, 44))
    _run(f"mlp_per_batch_eta_decode_{grad_layout}", inp, pieces=cuts, decode=set(cuts), grad_layout=grad_layout)


def test_per_batch_eta_fp32_inputs():
    """fp32 inputs (every token in the token kernel) with per-batch rates."""
    inp = make_inputs(2, 2, 37, dtype="f32", seed=415, rich=True, mlp_hidden=256, eta_per_batch=True)
    _run("mlp_per_batch_eta_f32", inp, in_dtype="f32", pieces=(11,), tol=1e-4)


@pytest.mark.parametrize("grad_layout", ["dense", "rows"])
def test_decode_graph_replays_match_eager(grad_layout):
    """TTT-MLP decode calls captured in a HIP graph and replayed (as the
    benchmark runs them): every replay, with eager work and synchronisation
    in between, reproduces the eager outputs and final state bit for bit."""
    inp = make_inputs(2, 2, 40, dtype="bf16", seed=161, rich=True, mlp_hidden=256)
    P, T = 13, 20  # the prefill ends inside a mini-batch; decode crosses a boundary

    def fresh():
        g = MlpGPU(inp, grad_layout=grad_layout)
        g.run(0, P)
        return g

    def decode_calls(g):
        for t in range(P, P + T):
            g.run(t, t + 1, decode=True)

    ref = fresh()
    decode_calls(ref)
    want = ref.result()

    g = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_calls(g)
    torch.cuda.synchronize()
    saved = [t.clone() for t in g.state.tensors]  # post-prefill state
    for rep in range(3):
        # eager work between replays: restore the post-prefill state, clear the outputs
        for dst, src in zip(g.state.tensors, saved):
            dst.copy_(src)
        g.out[:, :, P:].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = g.result()
        assert np.array_equal(got[0][:, :, P:P + T], want[0][:, :, P:P + T]), rep
        for a, b in zip(got[1:], want[1:]):
            assert np.array_equal(a, b), rep

