"""Shared helpers of the parity tests: run the HIP path through the C ABI and
the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from test_rnn_layers_amd import libttt
from test_rnn_layers_amd.synth import make_inputs

TOL_F32 = 1e-4   # max-abs error, fp32 inputs
TOL_BF16 = 2e-2  # max-abs error, bf16 inputs, fp32 state


def tol_for(dtype: str) -> float:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


class LinearGPU:
    """One TTT-Linear problem on the GPU: device inputs, state, out."""

    def __init__(self, inp: dict, *, K=16, rope=False, in_dtype="bf16", out_dtype="f32", layout="bhld",
                 device="cuda", grad_layout="dense", token_eta=None):
        self.inp = inp
        self.te = None if token_eta is None else torch.tensor(np.asarray(token_eta), dtype=torch.float32,
                                                              device=device)
        B, H, L, D = inp["XQ"].shape
        self.B, self.H, self.L, self.D = B, H, L, D
        self.grad_layout = grad_layout
        self.cfg = libttt.linear_cfg(B, H, K=K, in_dtype=in_dtype, out_dtype=out_dtype, rope=rope,
                                     grad_layout=grad_layout)
        self.K, self.rope, self.out_dtype = K, rope, out_dtype
        self.layout = layout
        self.x = {n: self._place(inp[n].to(device)) for n in ("XQ", "XK", "XV")}
        self.eta = inp["eta"].to(device)
        self.ln_w, self.ln_b = inp["ln_w"].to(device).contiguous(), inp["ln_b"].to(device).contiguous()
        self.W0, self.b0 = inp["W0"].to(device).contiguous(), inp["b0"].to(device).contiguous()
        odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        self.out = self._place(torch.full((B, H, L, D), float("nan"), dtype=odt, device=device))
        self.state = libttt.LinearState.empty(B, H, D, device=device)
        libttt.ttt_linear_state_init(self.cfg, self.W0, self.b0, self.state)

    def _place(self, t):
        """[B, H, L, D] contiguous -> the requested memory layout (same values)."""
        if self.layout == "bhld":
            return t.contiguous()
        # the pages' [B, L, H*D] projection output viewed as [B, H, L, D]
        B, H, L, D = t.shape
        return t.permute(0, 2, 1, 3).contiguous().view(B, L, H, D).permute(0, 2, 1, 3)

    def run(self, t0, t1, decode=False):
        """Tokens [t0, t1) in one prefill (or decode) call."""
        sl = slice(t0, t1)
        fn = libttt.ttt_linear_decode if decode else libttt.ttt_linear_prefill
        fn(self.cfg, t1 - t0, self.x["XQ"][:, :, sl], self.x["XK"][:, :, sl], self.x["XV"][:, :, sl],
           self.eta[..., sl], self.ln_w, self.ln_b, self.state, self.out[:, :, sl], token_eta=self.te)

    def result(self):
        """out, W, b, and the dense W_grad (built from the open rows in the rows
        layout: sum_j k_j (x) eta_j g_j), b_grad."""
        torch.cuda.synchronize()
        s = self.state
        G = to_f64(s.W_grad)
        if self.grad_layout == "rows":
            B, H, D = self.B, self.H, self.D
            rows = G.reshape(B, H, D // 2, 2 * D)[:, :, : s.offset % self.cfg.K]
            G = np.einsum("bhji,bhjc->bhic", rows[..., :D], rows[..., D:])
        return (to_f64(self.out), to_f64(s.W), to_f64(s.b), G, to_f64(s.b_grad))


def oracle_linear(inp: dict, *, K=16, rope=False, chains=None, L=None, token_eta=None):
    """Oracle outputs and final state for the listed (b, h) chains (default all).
    Returns out [n, L, D], W, b, G, gb per chain."""
    B, H, Lf, D = inp["XQ"].shape
    L = Lf if L is None else L
    chains = [(b, h) for b in range(B) for h in range(H)] if chains is None else chains
    outs, Ws, bs, Gs, gbs = [], [], [], [], []
    eta, lw, lb = to_f64(inp["eta"]), to_f64(inp["ln_w"]), to_f64(inp["ln_b"])
    W0, b0 = to_f64(inp["W0"]), to_f64(inp["b0"])
    for (b, h) in chains:
        q, k, v = (to_f64(inp[n][b, h, :L]) for n in ("XQ", "XK", "XV"))
        W, bb, G, gb = W0[h].copy(), b0[h].copy(), np.zeros((D, D)), np.zeros(D)
        e = eta[b, h, :L] if eta.ndim == 3 else eta[h, :L]
        o = oracle.linear_chain(q, k, v, e, lw[h], lb[h], W, bb, G, gb, K=K, rope=rope, token_eta=token_eta)
        outs.append(o)
        Ws.append(W)
        bs.append(bb)
        Gs.append(G)
        gbs.append(gb)
    return np.stack(outs), np.stack(Ws), np.stack(bs), np.stack(Gs), np.stack(gbs)


class MlpGPU:
    """One TTT-MLP problem on the GPU: device inputs, state, out."""

    def __init__(self, inp: dict, *, K=16, rope=False, out_dtype="f32", device="cuda", token_eta=None,
                 in_dtype="bf16", grad_layout="dense"):
        B, H, L, D = inp["XQ"].shape
        F = inp["W1"].shape[-1]
        self.B, self.H, self.L, self.D, self.F = B, H, L, D, F
        self.grad_layout = grad_layout
        self.cfg = libttt.mlp_cfg(B, H, F=F, K=K, in_dtype=in_dtype, out_dtype=out_dtype, rope=rope,
                                  grad_layout=grad_layout)
        self.te = None if token_eta is None else torch.tensor(np.asarray(token_eta), dtype=torch.float32,
                                                              device=device)
        self.x = {n: inp[n].to(device).contiguous() for n in ("XQ", "XK", "XV")}
        self.eta = inp["eta"].to(device)
        self.ln_w, self.ln_b = inp["ln_w"].to(device).contiguous(), inp["ln_b"].to(device).contiguous()
        odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        self.out = torch.full((B, H, L, D), float("nan"), dtype=odt, device=device)
        self.state = libttt.MlpState.empty(B, H, D, F, device=device)
        w = [inp[n].to(device).contiguous() for n in ("W1", "b1", "W2", "b2")]
        libttt.ttt_mlp_state_init(self.cfg, *w, self.state)

    def run(self, t0, t1, decode=False):
        sl = slice(t0, t1)
        fn = libttt.ttt_mlp_decode if decode else libttt.ttt_mlp_prefill
        fn(self.cfg, t1 - t0, self.x["XQ"][:, :, sl], self.x["XK"][:, :, sl],
                               self.x["XV"][:, :, sl], self.eta[..., sl], self.ln_w, self.ln_b, self.state,
                               self.out[:, :, sl], token_eta=self.te)

    def result(self):
        """out and the 8 state arrays; in the rows layout the dense W1_grad,
        W2_grad are rebuilt from the open rows (sum of outer products)."""
        torch.cuda.synchronize()
        st = [to_f64(t) for t in self.state.tensors]
        if self.grad_layout == "rows":
            B, H, D, F = self.B, self.H, self.D, self.F
            n = self.state.offset % self.cfg.K
            r1 = st[4].reshape(B, H, -1)[:, :, : 16 * (D + F)].reshape(B, H, 16, D + F)[:, :, :n]
            r2 = st[6].reshape(B, H, -1)[:, :, : 16 * (F + D)].reshape(B, H, 16, F + D)[:, :, :n]
            st[4] = np.einsum("bhji,bhjf->bhif", r1[..., :D], r1[..., D:])
            st[6] = np.einsum("bhjf,bhjc->bhfc", r2[..., :F], r2[..., F:])
        return (to_f64(self.out),) + tuple(st)


def oracle_mlp(inp: dict, *, K=16, rope=False, chains=None, L=None, token_eta=None):
    """Oracle outputs and final state (W1, b1, W2, b2, G1, gb1, G2, gb2) for the
    listed (b, h) chains (default all), each stacked over the chains."""
    B, H, Lf, D = inp["XQ"].shape
    F = inp["W1"].shape[-1]
    L = Lf if L is None else L
    chains = [(b, h) for b in range(B) for h in range(H)] if chains is None else chains
    eta, lw, lb = to_f64(inp["eta"]), to_f64(inp["ln_w"]), to_f64(inp["ln_b"])
    init = [to_f64(inp[n]) for n in ("W1", "b1", "W2", "b2")]
    res = [[] for _ in range(9)]
    for (b, h) in chains:
        q, k, v = (to_f64(inp[n][b, h, :L]) for n in ("XQ", "XK", "XV"))
        st = [a[h].copy() for a in init] + [np.zeros((D, F)), np.zeros(F), np.zeros((F, D)), np.zeros(D)]
        e = eta[b, h, :L] if eta.ndim == 3 else eta[h, :L]
        o = oracle.mlp_chain(q, k, v, e, lw[h], lb[h], *st, K=K, rope=rope, token_eta=token_eta)
        for i, a in enumerate([o] + st):
            res[i].append(a)
    return tuple(np.stack(r) for r in res)


def _eta_batch(inp, L):
    """eta for the oracle's batch drivers: flat, head stride L, and its batch
    stride (0 when shared over the batch)."""
    eta = to_f64(inp["eta"])[..., :L]
    if eta.ndim == 3:
        return np.ascontiguousarray(eta), eta.shape[1] * L
    return np.ascontiguousarray(eta), 0


def oracle_linear_all(inp: dict, *, K=16, rope=False, L=None, token_eta=None):
    """Every chain through the oracle's OpenMP batch driver (from W0, b0 tiled
    over the batch).  Returns out [B, H, L, D], W, b, G, gb [B, H, ...]."""
    B, H, Lf, D = inp["XQ"].shape
    L = Lf if L is None else L
    x = [np.ascontiguousarray(to_f64(inp[n][:, :, :L])) for n in ("XQ", "XK", "XV")]
    eta, eta_sB = _eta_batch(inp, L)
    W = np.ascontiguousarray(np.broadcast_to(to_f64(inp["W0"]), (B, H, D, D)))
    b = np.ascontiguousarray(np.broadcast_to(to_f64(inp["b0"]), (B, H, D)))
    G, gb = np.zeros_like(W), np.zeros_like(b)
    out = oracle.linear_batch(*x, eta, eta_sB, to_f64(inp["ln_w"]), to_f64(inp["ln_b"]), W, b, G, gb, K=K,
                              rope=rope, token_eta=token_eta)
    return out, W, b, G, gb


def oracle_mlp_all(inp: dict, *, K=16, rope=False, L=None, token_eta=None):
    """Every chain of a TTT-MLP problem through the OpenMP batch driver.
    Returns out [B, H, L, D] and the 8 state arrays [B, H, ...]."""
    B, H, Lf, D = inp["XQ"].shape
    F = inp["W1"].shape[-1]
    L = Lf if L is None else L
    x = [np.ascontiguousarray(to_f64(inp[n][:, :, :L])) for n in ("XQ", "XK", "XV")]
    eta, eta_sB = _eta_batch(inp, L)
    shapes = {"W1": (D, F), "b1": (F,), "W2": (F, D), "b2": (D,)}
    st = [np.ascontiguousarray(np.broadcast_to(to_f64(inp[n]), (B, H) + shapes[n])) for n in ("W1", "b1", "W2", "b2")]
    st += [np.zeros_like(a) for a in st]
    out = oracle.mlp_batch(*x, eta, eta_sB, to_f64(inp["ln_w"]), to_f64(inp["ln_b"]), *st, K=K, rope=rope,
                           token_eta=token_eta)
    return (out,) + tuple(st)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp of |x| (the rounding bound of a bf16 store)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8)


__all__ = ["LinearGPU", "oracle_linear", "oracle_linear_all", "MlpGPU", "oracle_mlp", "oracle_mlp_all", "max_abs", "tol_for", "make_inputs", "to_f64", "bf16_half_ulp",
           "TOL_F32", "TOL_BF16"]
