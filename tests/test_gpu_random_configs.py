"""Seeded random configurations, TTT-Linear and TTT-MLP, against the CPU
oracle through the C ABI: batch and head counts, ragged lengths, mini-batch
sizes, rotary, input and output dtypes, gradient layouts, token_eta, and
calls cut at random points, some of them decode calls.  Every configuration
is drawn from a fixed seed, so a failure names a reproducible case; the bars
are those of the other parity tests (1e-4 fp32 inputs, 2e-2 bf16)."""
import numpy as np
import pytest

from harness import TOL_BF16, TOL_F32, make_inputs
from test_gpu_linear import _check_full
from test_gpu_mlp import _run

pytestmark = pytest.mark.gpu


def _draw(rng, mlp):
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 5 if mlp else 6))
    L = int(rng.integers(1, 81 if mlp else 101))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    K = 16 if rng.random() < 0.6 else int(rng.choice([1, 4, 8, 13]))
    rope = bool(rng.random() < 0.5)
    layout = "rows" if rng.random() < 0.5 else "dense"
    out_dtype = "bf16" if (dtype == "bf16" and rng.random() < 0.25) else "f32"
    te = (0.5 + rng.random(K)).tolist() if rng.random() < 0.3 else None
    ncut = int(rng.integers(0, 4)) if L > 1 else 0
    cuts = sorted(set(int(c) for c in rng.integers(1, L, size=ncut))) if ncut else []
    starts = [0] + cuts
    decode = {s for s in starts if rng.random() < 0.3}
    return dict(B=B, H=H, L=L, dtype=dtype, K=K, rope=rope, layout=layout, out_dtype=out_dtype, te=te, cuts=cuts,
                decode=decode)


def _cases(seed, n, mlp):
    rng = np.random.default_rng(seed)
    return [_draw(rng, mlp) for _ in range(n)]


@pytest.mark.parametrize("i,c", list(enumerate(_cases(2024, 24, mlp=False))))
def test_linear_random_configuration(i, c):
    inp = make_inputs(c["B"], c["H"], c["L"], dtype=c["dtype"], seed=1000 + i, rich=True)
    _check_full(f"random_linear_{i}_{c}", inp, dtype=c["dtype"], rope=c["rope"], K=c["K"], pieces=c["cuts"],
                out_dtype=c["out_dtype"], decode=c["decode"], grad_layout=c["layout"], token_eta=c["te"])


@pytest.mark.parametrize("i,c", list(enumerate(_cases(4048, 12, mlp=True))))
def test_mlp_random_configuration(i, c):
    inp = make_inputs(c["B"], c["H"], c["L"], dtype=c["dtype"], seed=2000 + i, rich=True, mlp_hidden=256)
    _run(f"random_mlp_{i}_{c}", inp, rope=c["rope"], pieces=tuple(c["cuts"]), out_dtype=c["out_dtype"],
         token_eta=c["te"], K=c["K"], in_dtype=c["dtype"], decode=c["decode"],
         tol=TOL_F32 if c["dtype"] == "f32" else TOL_BF16, grad_layout=c["layout"])


def test_linear_more_chains_than_cus():
    """288 chains: more workgroups than the chip has CUs, two per CU at a time."""
    inp = make_inputs(6, 48, 40, dtype="bf16", seed=3001, rich=True)
    _check_full("linear_288_chains", inp, dtype="bf16", pieces=[9], decode={9})


def test_mlp_more_chains_than_cus():
    """280 chains of TTT-MLP (one workgroup per CU, in several waves of dispatch)."""
    inp = make_inputs(5, 56, 36, dtype="bf16", seed=3002, rich=True, mlp_hidden=256)
    _run("mlp_280_chains", inp, pieces=(16,))
