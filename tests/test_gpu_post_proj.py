"""GPU parity of the post-norm LayerNorm and output projection (the steps
after the layer in "代码连连看——TTT", TTTBase.forward) against the CPU
oracle, through the C ABI.

Tolerances.  The kernel multiplies bf16 y by W' = bf16(diag(gamma) Wo) with
fp32 accumulation, which is the LayerNorm followed by the product with W'.
* When gamma * Wo is exactly representable in bf16 (``exact_weights``) the
  only differences are fp32 rounding: max-abs 2e-4 + 1e-4 |out|.
* Otherwise each weight carries a relative rounding error of at most 2^-9;
  these are independent, so the error of an output is about
  2^-9 sqrt(sum_k (xhat_k gamma_k Wo_kn)^2) / sqrt(3) (xhat the normalised
  row): the bound used is 6 2^-9 sqrt(sum_k (xhat gamma Wo)^2) + 1e-4 |out|.
bf16 outputs add half a bf16 ulp of the reference."""
import numpy as np
import pytest
import torch

import oracle
from harness import bf16_half_ulp
from test_rnn_layers_amd import libttt as T
from test_rnn_layers_amd.synth import make_post_proj_inputs

pytestmark = pytest.mark.gpu
EPS = 1e-5


def _gpu(inp, *, out_dtype="f32", ldy=None, ldo=None):
    dev = "cuda"
    y = inp["y"]
    M, K = y.shape
    N = inp["Wo"].shape[1]
    ldy = ldy or K
    ldo = ldo or N
    ybuf = torch.zeros((M, ldy), dtype=torch.bfloat16, device=dev)
    ybuf[:, :K] = y.to(dev)
    prepared = torch.empty(T.ttt_post_proj_prepared_bytes(K, N), dtype=torch.uint8, device=dev)
    g, b, W = (inp[n].to(dev).contiguous() for n in ("gamma", "beta", "Wo"))
    bias = inp["bias"].to(dev).contiguous() if inp["bias"] is not None else None
    T.ttt_post_proj_prepare(K, N, g, b, W, bias, prepared)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.full((M, ldo), float("nan"), dtype=odt, device=dev)
    T.ttt_post_proj(M, K, N, ybuf, ldy, EPS, prepared, out, ldo, out_dtype)
    torch.cuda.synchronize()
    res = out.double().cpu().numpy()
    if ldo > N:  # the columns past N are not written
        assert np.isnan(res[:, N:]).all()
    return res[:, :N]


def _ref(inp, rows):
    f = lambda n: inp[n].double().numpy()  # noqa: E731
    bias = f("bias") if inp["bias"] is not None else None
    return oracle.post_proj(f("y")[rows], f("gamma"), f("beta"), f("Wo"), bias, EPS)


def _spread(inp, rows):
    """sqrt(sum_k (xhat_k gamma_k Wo_kn)^2) per output (the rounding scale)."""
    y = inp["y"].double().numpy()[rows]
    xh = (y - y.mean(axis=1, keepdims=True)) / np.sqrt(y.var(axis=1, keepdims=True) + EPS)
    gw = inp["gamma"].double().numpy()[:, None] * inp["Wo"].double().numpy()
    return np.sqrt((xh ** 2) @ (gw ** 2))


def _check(name, inp, got, rows, *, exact, out_dtype="f32"):
    ref = _ref(inp, rows)
    g = got[rows]
    err = np.abs(g - ref)
    tol = (2e-4 if exact else 6 * 2.0 ** -9 * _spread(inp, rows)) + 1e-4 * np.abs(ref)
    if out_dtype == "bf16":
        tol = tol + bf16_half_ulp(ref)
    print(f"[{name}] max-abs {err.max():.3e}, max err/tol {np.max(err / tol):.3f}", flush=True)
    assert np.isfinite(g).all()
    assert (err <= tol).all(), f"{name}: {np.argwhere(err > tol)[:5]}"


@pytest.mark.parametrize("exact", [True, False])
@pytest.mark.parametrize("bias", [False, True])
def test_small_parity(exact, bias):
    """M = 300 (one full 256-row panel and a ragged one), K = 192, N = 512."""
    inp = make_post_proj_inputs(300, 192, 512, seed=11 + 2 * exact + bias, bias=bias, exact_weights=exact)
    got = _gpu(inp)
    _check(f"post_proj_small_exact{int(exact)}_bias{int(bias)}", inp, got, np.arange(300), exact=exact)


def test_bf16_output_and_strides():
    """bf16 output; y and out as row windows of wider buffers (ldy > K, ldo > N)."""
    inp = make_post_proj_inputs(257, 128, 256, seed=21, exact_weights=True)
    got = _gpu(inp, out_dtype="bf16", ldy=136, ldo=264)
    _check("post_proj_bf16_strided", inp, got, np.arange(257), exact=True, out_dtype="bf16")


@pytest.mark.parametrize("M", [1, 17, 255, 256, 512])
def test_row_counts(M):
    """Edge row counts: one row, less than a panel, exactly one and two panels."""
    inp = make_post_proj_inputs(M, 64, 256, seed=30 + M, exact_weights=True, offset=4.0)
    got = _gpu(inp)
    _check(f"post_proj_M{M}", inp, got, np.arange(M), exact=True)


def test_constant_rows():
    """A row with zero variance: LayerNorm gives beta, so the output is
    beta^T Wo (+ bias) whatever the constant."""
    inp = make_post_proj_inputs(40, 128, 256, seed=41, bias=True, exact_weights=True)
    inp["y"][3] = 2.5
    inp["y"][17] = -7.0
    got = _gpu(inp)
    _check("post_proj_constant_rows", inp, got, np.arange(40), exact=True)


@pytest.mark.parametrize("shape", [(32768, 2048, 2048), (16384, 768, 768)])
def test_full_size_sampled_rows(shape):
    """The 1B-style shape (M = B L = 4 x 8192, width 2048) and the 125M-style
    one (8 x 2048, width 768): the whole launch on the GPU, 96 sampled rows
    (first, last, panel edges, random) against the oracle."""
    M, K, N = shape
    inp = make_post_proj_inputs(M, K, N, seed=51 + K)
    got = _gpu(inp, out_dtype="bf16")
    r = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 257, M - 256, M - 1], r.choice(M, 90, replace=False)]))
    _check(f"post_proj_{M}x{K}x{N}", inp, got, rows, exact=False, out_dtype="bf16")


def test_after_the_layer():
    """The prefill writes its output as [B, L, H, D] bf16 (strides L*H*D, D,
    H*D), which is the [B*L, width] input of the projection: the composition
    equals the oracle's layer followed by its post-norm and projection."""
    from harness import oracle_linear_all
    from test_rnn_layers_amd.synth import make_inputs

    B, H, L, D = 2, 4, 64, 64
    inp = make_inputs(B, H, L, dtype="bf16", seed=61, rich=True)
    dev = "cuda"
    cfg = T.linear_cfg(B, H, in_dtype="bf16", out_dtype="bf16")
    st = T.LinearState.empty(B, H, D, device=dev)
    T.ttt_linear_state_init(cfg, inp["W0"].to(dev), inp["b0"].to(dev), st)
    ybuf = torch.empty((B, L, H, D), dtype=torch.bfloat16, device=dev)
    out_desc = T.ttt_tensor(ybuf.data_ptr(), L * H * D, D, H * D)
    x = {n: inp[n].to(dev).contiguous() for n in ("XQ", "XK", "XV")}
    T.ttt_linear_prefill(cfg, L, x["XQ"], x["XK"], x["XV"], inp["eta"].to(dev), inp["ln_w"].to(dev),
                         inp["ln_b"].to(dev), st, out_desc)
    pp = make_post_proj_inputs(1, H * D, 256, seed=62, bias=True)
    pp["y"] = ybuf.reshape(B * L, H * D).cpu()
    got = _gpu(pp)
    # the layer output against the oracle's, at the layer's bf16-output bar
    layer = oracle_linear_all(inp)[0]  # [B, H, L, D]
    y_ref = np.ascontiguousarray(layer.transpose(0, 2, 1, 3)).reshape(B * L, H * D)
    dlayer = np.abs(pp["y"].double().numpy() - y_ref) - bf16_half_ulp(y_ref)
    print(f"[post_proj_after_layer] layer output max-abs beyond half a bf16 ulp {dlayer.max():.3e}", flush=True)
    assert dlayer.max() <= 2e-2
    _check("post_proj_after_layer", pp, got, np.arange(B * L), exact=False)


@pytest.mark.parametrize("shape", [(192, 512, True), (2048, 2048, False), (320, 256, True)])
def test_prepared_weights(shape):
    """The prepared buffer itself: W'^T [N][K] must be bf16(gamma_k Wo[k][n])
    bit for bit (one fp32 product, rounded to nearest even), c1 the sum of
    the rounded W' column (a sum of bf16 values, exact in fp64 here, so bit
    for bit after the fp32 rounding) and c2 = beta^T Wo + bias to 1 ulp of
    fp32 (fp64 sums of fp32 products in another order)."""
    K, N, bias = shape
    inp = make_post_proj_inputs(8, K, N, seed=71 + K, bias=bias)
    dev = "cuda"
    g, b, W = (inp[n].to(dev).contiguous() for n in ("gamma", "beta", "Wo"))
    bv = inp["bias"].to(dev).contiguous() if bias else None
    prepared = torch.empty(T.ttt_post_proj_prepared_bytes(K, N), dtype=torch.uint8, device=dev)
    T.ttt_post_proj_prepare(K, N, g, b, W, bv, prepared)
    torch.cuda.synchronize()
    pc = prepared.cpu()
    wt = pc[:N * K * 2].view(torch.bfloat16).view(N, K)
    c1 = pc[N * K * 2:N * K * 2 + 4 * N].view(torch.float32).numpy()
    c2 = pc[N * K * 2 + 4 * N:].view(torch.float32).numpy()
    want = (inp["gamma"].float()[:, None] * inp["Wo"].float()).to(torch.bfloat16).t().contiguous()
    assert torch.equal(wt.view(torch.int16), want.view(torch.int16))
    c1_ref = want.double().sum(dim=1).numpy().astype(np.float32)
    assert np.array_equal(c1, c1_ref)
    c2_ref = inp["beta"].double().numpy() @ inp["Wo"].double().numpy()
    if bias:
        c2_ref = c2_ref + inp["bias"].double().numpy()
    ulp = np.spacing(np.abs(c2_ref).astype(np.float32)).astype(np.float64)
    assert (np.abs(c2.astype(np.float64) - c2_ref) <= ulp).all()
