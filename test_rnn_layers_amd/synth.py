"""Seeded synthetic inputs for the TTT hot path.

This module only draws random numbers; it holds none of the layer's
arithmetic.  The tests, the benchmark and the smoke check use it to feed the
same values to the HIP path and to the CPU oracle.

Recipe (shapes follow the TTT standard configs on the pages: hidden 768 = 12
heads x 64 for the 125m style, 1024 = 16 x 64 for 350m, 2048 = 32 x 64 for the
1b style; mini-batch 16):
  * one ``torch.Generator`` on the CPU, seeded, drawing in the fixed order
    XQ, XK, XV, eta-noise, W0 (TTT-MLP: W1 then W2), then optional extras;
  * XQ, XK, XV ~ N(0, 1) drawn in fp32 as [B, H, L, D] and rounded to bf16
    (round to nearest even) when the workload is bf16 (``scale`` multiplies
    the draws before rounding: the large-magnitude range tests);
  * eta[h, t] = sigmoid(N(0, 1)) / 64, shared over the batch (or, with
    ``eta_per_batch=True``, eta[b, h, t] drawn the same way, after every other
    draw, so the other values stay those of the shared case);
  * W0 ~ N(0, 0.02^2) per head, b0 = 0 (the TTTLinear init on the pages),
    LayerNorm gamma = 1, beta = 0 — unless ``rich=True``, which draws
    non-trivial b0, gamma, beta so that parity checks exercise every term.

Post-norm and output projection (``make_post_proj_inputs``): y [M, K] the
layer output as bf16 rows, N(offset_m, spread_m^2) with a per-row offset and
spread (drawn once per row) so that the LayerNorm has work to do; gamma =
1 + 0.2 N(0, 1), beta = 0.2 N(0, 1); Wo ~ N(0, 0.02^2) [K, N]; bias 0.05 N(0, 1)
or none.  With ``exact_weights=True`` gamma is a random power of two in
{+-1/2, +-1, +-2} and Wo is rounded to bf16, so that gamma * Wo is exactly
representable in bf16.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

D_HEAD = 64
MINI_BATCH = 16
MLP_HIDDEN = 256


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "linear", "mlp", "decode" (TTT-Linear) or "mlp_decode"
    B: int
    H: int
    L: int
    dtype: str         # "f32" or "bf16" (input dtype; the state is fp32)
    rope: bool
    seed: int
    prefill: int = 0   # decode workload: tokens prefilled before decoding
    decode: int = 0    # decode workload: single-token steps after the prefill


WORKLOADS = [
    Workload("linear_single_head_B1_H1_L64_f32", "linear", 1, 1, 64, "f32", False, 1234),
    Workload("linear_125m_B8_H12_L2048_bf16_rope", "linear", 8, 12, 2048, "bf16", True, 1235),
    Workload("linear_1b_B4_H32_L8192_bf16", "linear", 4, 32, 8192, "bf16", False, 1236),
    Workload("mlp_350m_B4_H16_L4096_F256_bf16", "mlp", 4, 16, 4096, "bf16", False, 1237),
    Workload("decode_1b_B64_H32_prefill512_decode256_bf16", "decode", 64, 32, 768, "bf16", False, 1238,
             prefill=512, decode=256),
    Workload("mlp_decode_350m_B16_H16_prefill512_decode64_bf16", "mlp_decode", 16, 16, 576, "bf16", False, 1239,
             prefill=512, decode=64),
]


def _dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(B: int, H: int, L: int, *, D: int = D_HEAD, dtype: str = "f32", seed: int = 0,
                mlp_hidden: int = 0, rich: bool = False, eta_scale: float = 1.0 / 64.0,
                eta_per_batch: bool = False, scale: float = 1.0) -> dict:
    """Draw one problem.  Returns CPU tensors:
    XQ, XK, XV [B, H, L, D] in ``dtype`` (N(0, scale^2)); eta [H, L] fp32
    ([B, H, L] with ``eta_per_batch``); ln_w, ln_b [H, D];
    linear: W0 [H, D, D], b0 [H, D]; MLP: W1 [H, D, F], b1 [H, F], W2 [H, F, D], b2 [H, D]."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, L, D)
    XQ = torch.randn(shape, generator=g, dtype=torch.float32) * scale
    XK = torch.randn(shape, generator=g, dtype=torch.float32) * scale
    XV = torch.randn(shape, generator=g, dtype=torch.float32) * scale
    eta = torch.sigmoid(torch.randn((H, L), generator=g, dtype=torch.float32)) * eta_scale
    out = {"XQ": XQ.to(_dtype(dtype)), "XK": XK.to(_dtype(dtype)), "XV": XV.to(_dtype(dtype)), "eta": eta}
    if mlp_hidden:
        F = mlp_hidden
        out["W1"] = torch.randn((H, D, F), generator=g, dtype=torch.float32) * 0.02
        out["W2"] = torch.randn((H, F, D), generator=g, dtype=torch.float32) * 0.02
        out["b1"] = torch.zeros((H, F), dtype=torch.float32)
        out["b2"] = torch.zeros((H, D), dtype=torch.float32)
    else:
        out["W0"] = torch.randn((H, D, D), generator=g, dtype=torch.float32) * 0.02
        out["b0"] = torch.zeros((H, D), dtype=torch.float32)
    out["ln_w"] = torch.ones((H, D), dtype=torch.float32)
    out["ln_b"] = torch.zeros((H, D), dtype=torch.float32)
    if rich:
        out["ln_w"] = 1.0 + 0.2 * torch.randn((H, D), generator=g, dtype=torch.float32)
        out["ln_b"] = 0.2 * torch.randn((H, D), generator=g, dtype=torch.float32)
        if mlp_hidden:
            out["b1"] = 0.05 * torch.randn((H, mlp_hidden), generator=g, dtype=torch.float32)
            out["b2"] = 0.05 * torch.randn((H, D), generator=g, dtype=torch.float32)
        else:
            out["b0"] = 0.05 * torch.randn((H, D), generator=g, dtype=torch.float32)
    if eta_per_batch:
        out["eta"] = torch.sigmoid(torch.randn((B, H, L), generator=g, dtype=torch.float32)) * eta_scale
    return out


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.H, w.L, dtype=w.dtype, seed=w.seed,
                       mlp_hidden=MLP_HIDDEN if w.kind in ("mlp", "mlp_decode") else 0)


def make_post_proj_inputs(M: int, K: int, N: int, *, seed: int = 0, bias: bool = False, offset: float = 1.0,
                          exact_weights: bool = False) -> dict:
    """y [M, K] bf16; gamma, beta [K], Wo [K, N], bias [N] (or None) fp32; CPU tensors."""
    g = torch.Generator().manual_seed(seed)
    mean = offset * torch.randn((M, 1), generator=g, dtype=torch.float32)
    spread = 0.5 + torch.rand((M, 1), generator=g, dtype=torch.float32) * 1.5
    y = (mean + spread * torch.randn((M, K), generator=g, dtype=torch.float32)).to(torch.bfloat16)
    gamma = 1.0 + 0.2 * torch.randn(K, generator=g, dtype=torch.float32)
    beta = 0.2 * torch.randn(K, generator=g, dtype=torch.float32)
    Wo = 0.02 * torch.randn((K, N), generator=g, dtype=torch.float32)
    bv = 0.05 * torch.randn(N, generator=g, dtype=torch.float32) if bias else None
    if exact_weights:
        pick = torch.randint(0, 6, (K,), generator=g)
        gamma = torch.tensor([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0])[pick]
        Wo = Wo.to(torch.bfloat16).to(torch.float32)
    return {"y": y, "gamma": gamma, "beta": beta, "Wo": Wo, "bias": bv}
