"""Input magnitudes at which fp16 operands would overflow.

For bf16 inputs the dual-form kernels run their products on fp16 MFMA
operands.  q.k dot products enter the 16x16 causal and look-ahead matrices;
at input rms 64 (or with XK a copy of XQ at rms 40) they reach 1e5..1e6,
beyond fp16's 65504.  The kernels carry ng times 2^8 and those matrices times
2^-8, so these inputs stay finite and within the bf16 bar of the oracle.
Each test first checks on the CPU that the case really holds dot products
above 65504."""
import numpy as np
import pytest
import torch

from harness import (LinearGPU, MlpGPU, TOL_BF16, make_inputs, max_abs, oracle_linear_all, oracle_mlp_all, to_f64)

pytestmark = pytest.mark.gpu

FP16_MAX = 65504.0


def _report(name, **kv):
    print(f"[{name}] " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in kv.items()),
          flush=True)


def _max_dot(inp):
    """Largest |q_i . k_j| and |k_i . k_j| within and between neighbouring
    mini-batches (the entries of the causal and look-ahead matrices)."""
    q, k = to_f64(inp["XQ"]), to_f64(inp["XK"])
    B, H, L, D = q.shape
    n = L // 16
    q = q[:, :, : 16 * n].reshape(B, H, n, 16, D)
    k = k[:, :, : 16 * n].reshape(B, H, n, 16, D)
    s = np.abs(np.einsum("bhnid,bhnjd->bhnij", q, k)).max()
    c = np.abs(np.einsum("bhnid,bhnjd->bhnij", k[:, :, 1:], k[:, :, :-1])).max() if n > 1 else 0.0
    return float(max(s, c))


def _large(seed, *, mlp=False, copy_q=False, L=16 * 6 + 5):
    """Inputs of rms 64 (or 40, with XK a copy of XQ).  For TTT-MLP the
    learning rate is scaled by 1/rms^2 (the step eta k^T g changes f(k) by
    ~eta |k|^2 g): with the default rate the inner MLP's weights grow by ~80
    per mini-batch at this scale and its hidden activations pass fp16's range
    within a few mini-batches, outside what fp16 operands can carry."""
    scale = 40.0 if copy_q else 64.0
    eta_scale = (1.0 / 64.0) / (scale * scale if mlp else 1.0)
    inp = make_inputs(2, 2, L, dtype="bf16", seed=seed, rich=True, scale=scale, mlp_hidden=256 if mlp else 0,
                      eta_scale=eta_scale)
    if copy_q:
        inp["XK"] = inp["XQ"].clone()
    return inp


@pytest.mark.parametrize("copy_q", [False, True])
def test_linear_large_inputs(copy_q):
    inp = _large(501 + copy_q, copy_q=copy_q)
    dots = _max_dot(inp)
    assert dots > FP16_MAX, dots
    g = LinearGPU(inp, in_dtype="bf16")
    g.run(0, inp["XQ"].shape[2])
    out, W, b, G, gb = g.result()
    ro, rW, rb, rG, rgb = oracle_linear_all(inp)
    err = max_abs(out, ro)
    _report(f"linear_large_copyq{int(copy_q)}", max_dot=dots, err=err, W=max_abs(W, rW) / max(1.0, np.abs(rW).max()))
    assert np.isfinite(out).all()
    assert err <= TOL_BF16
    sc = max(1.0, float(np.abs(rW).max()))
    assert max_abs(W, rW) <= TOL_BF16 * sc
    assert max_abs(G, rG) <= TOL_BF16 * max(1.0, float(np.abs(rG).max()))


def test_linear_large_inputs_prefill_matches_decode():
    """The same large inputs through whole-mini-batch prefill (fp16 operands)
    and through single-token decode calls (fp32 arithmetic) agree."""
    inp = _large(505)
    L = inp["XQ"].shape[2]
    a = LinearGPU(inp, in_dtype="bf16")
    a.run(0, L)
    b = LinearGPU(inp, in_dtype="bf16")
    for t in range(L):
        b.run(t, t + 1, decode=True)
    oa, ob = a.result()[0], b.result()[0]
    _report("linear_large_prefill_vs_decode", err=max_abs(oa, ob))
    assert max_abs(oa, ob) <= TOL_BF16


@pytest.mark.parametrize("copy_q", [False, True])
def test_mlp_large_inputs(copy_q):
    inp = _large(511 + copy_q, mlp=True, copy_q=copy_q)
    dots = _max_dot(inp)
    assert dots > FP16_MAX, dots
    g = MlpGPU(inp)
    L = inp["XQ"].shape[2]
    g.run(0, L)
    got = g.result()
    ref = oracle_mlp_all(inp)
    err = max_abs(got[0], ref[0])
    names = ("W1", "b1", "W2", "b2", "W1_grad", "b1_grad", "W2_grad", "b2_grad")
    rel = {n: max_abs(x, y) / max(1.0, float(np.abs(y).max())) for n, x, y in zip(names, got[1:], ref[1:])}
    _report(f"mlp_large_copyq{int(copy_q)}", max_dot=dots, err=err, **rel)
    assert np.isfinite(got[0]).all()
    assert err <= TOL_BF16
    for n, e in rel.items():
        assert e <= TOL_BF16, (n, e)
