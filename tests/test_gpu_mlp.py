"""GPU parity of TTT-MLP prefill (dual form, hidden width 4D, exact GELU)
against the CPU oracle, through the C ABI.  bf16 inputs, fp32 state:
max-abs tolerance 2e-2 on outputs and state."""
import numpy as np
import pytest
import torch

from harness import MlpGPU, TOL_BF16, bf16_half_ulp, make_inputs, max_abs, oracle_mlp
from test_rnn_layers_amd import libttt
from test_rnn_layers_amd.synth import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

STATE = ("W1", "b1", "W2", "b2", "W1_grad", "b1_grad", "W2_grad", "b2_grad")


def _report(name, **kv):
    print(f"[{name}] " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in kv.items()),
          flush=True)


def _compare(name, got, ref, chains, *, out_dtype="f32"):
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
        assert np.max(np.abs(out - ro) - bf16_half_ulp(ro)) <= TOL_BF16
    else:
        assert err <= TOL_BF16, f"{name}: output max-abs {err}"
    for n, e in errs.items():
        assert e <= TOL_BF16, f"{name}: {n} max-abs {e}"


def _run(name, inp, *, rope=False, pieces=(), out_dtype="f32", chains=None, token_eta=None):
    B, H, L, D = inp["XQ"].shape
    g = MlpGPU(inp, rope=rope, out_dtype=out_dtype, token_eta=token_eta)
    cuts = [0] + list(pieces) + [L]
    for i in range(len(cuts) - 1):
        g.run(cuts[i], cuts[i + 1])
    got = g.result()
    chains = [(b, h) for b in range(B) for h in range(H)] if chains is None else chains
    ref = oracle_mlp(inp, rope=rope, chains=chains, token_eta=token_eta)
    _compare(name, got, ref, chains, out_dtype=out_dtype)
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


def test_bf16_output():
    inp = make_inputs(1, 3, 70, dtype="bf16", seed=52, rich=True, mlp_hidden=256)
    _run("mlp_bf16_out", inp, out_dtype="bf16")


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


def test_open_offset_is_refused():
    """A call may only start on a mini-batch boundary."""
    inp = make_inputs(1, 1, 40, dtype="bf16", seed=55, mlp_hidden=256)
    g = MlpGPU(inp)
    g.run(0, 20)
    with pytest.raises(libttt.TTTError) as e:
        g.run(20, 40)
    assert e.value.name == "TTT_ERR_UNSUPPORTED"


def test_full_350m_workload_sampled():
    """The 350M-shape TTT-MLP layer (B=4, H=16, L=4096) in one launch; the
    oracle checks sampled chains, including the first and last."""
    w = next(x for x in WORKLOADS if x.kind == "mlp")
    inp = workload_inputs(w)
    B, H = w.B, w.H
    _run(w.name, inp, chains=[(0, 0), (1, 7), (2, 11), (B - 1, H - 1)])
