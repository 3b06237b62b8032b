"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula.  Each compares the oracle with an
independent route:
  * library routines (torch.nn.functional.layer_norm, gelu) and autograd;
  * central finite differences;
  * the defining statement of the method: the prediction for token i uses the
    parameters after one gradient step, from the mini-batch-start parameters,
    on the losses of tokens j <= i of its mini-batch, each weighted by its
    learning rate ("代码连连看——TTT", compute_mini_batch, primal branch); the
    step over the whole mini-batch is then carried to the next one;
  * the pages' claim that the dual branch computes the same thing as the
    primal branch (same listing; TTTLinear.ttt NOTE on dual/primal);
  * special cases: mini_batch_size = 1 is online gradient descent; eta = 0
    leaves the state untouched; cutting a sequence anywhere and carrying the
    state (TTTBase.forward remainder handling, TTTCache) changes nothing;
  * rotary embedding: identity at position 0, norm preserving, relative
    position property, and equal to multiplication by e^{i p theta} on
    complex pairs.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn


EPS = 1e-6


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# LayerNorm forward and fused LN + L2 backward
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("D", [4, 8, 64])
def test_ln_fwd_matches_library(orc, D):
    r = _rng(D)
    for _ in range(5):
        z = r.normal(size=D) * r.uniform(0.01, 5) + r.normal() * 3
        gam, bet = r.normal(size=D), r.normal(size=D)
        ref = Fn.layer_norm(torch.tensor(z), (D,), torch.tensor(gam), torch.tensor(bet), EPS).numpy()
        np.testing.assert_allclose(orc.ln_fwd(z, gam, bet, EPS), ref, rtol=1e-12, atol=1e-12)


def _l2_loss(z, t, gam, bet):
    return 0.5 * ((Fn.layer_norm(z, (z.shape[-1],), gam, bet, EPS) - t) ** 2).sum()


@pytest.mark.parametrize("D", [4, 8, 64])
def test_ln_l2_grad_finite_differences(orc, D):
    r = _rng(100 + D)
    z = r.normal(size=D) * 0.7 + 0.3
    t, gam, bet = r.normal(size=D), 1 + 0.3 * r.normal(size=D), 0.3 * r.normal(size=D)
    g = orc.ln_l2_grad(z, t, gam, bet, EPS)
    h = 1e-6
    T = lambda a: torch.tensor(a)  # noqa: E731
    fd = np.empty(D)
    for c in range(D):
        zp, zm = z.copy(), z.copy()
        zp[c] += h
        zm[c] -= h
        fd[c] = (_l2_loss(T(zp), T(t), T(gam), T(bet)) - _l2_loss(T(zm), T(t), T(gam), T(bet))).item() / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("D", [8, 64])
def test_ln_l2_grad_autograd(orc, D):
    r = _rng(200 + D)
    for scale in (0.01, 1.0, 30.0):
        z = torch.tensor(r.normal(size=D) * scale, requires_grad=True)
        t, gam, bet = (torch.tensor(r.normal(size=D)) for _ in range(3))
        (gz,) = torch.autograd.grad(_l2_loss(z, t, gam, bet), z)
        g = orc.ln_l2_grad(z.detach().numpy(), t.numpy(), gam.numpy(), bet.numpy(), EPS)
        np.testing.assert_allclose(g, gz.numpy(), rtol=1e-10, atol=1e-12 / scale)


# ----------------------------------------------------------------------------
# Rotary embedding
# ----------------------------------------------------------------------------
def _rope_complex(x, p, base=10000.0):
    """Rotation of the pairs (x_i, x_{i+D/2}) written as complex multiplication."""
    D = x.shape[-1]
    h = D // 2
    zc = x[:h] + 1j * x[h:]
    ang = p * base ** (-2.0 * np.arange(h) / D)
    w = zc * np.exp(1j * ang)
    return np.concatenate([w.real, w.imag])


def test_rope_properties(orc):
    r = _rng(7)
    D = 64
    x, y = r.normal(size=D), r.normal(size=D)
    np.testing.assert_array_equal(orc.rope_row(x, 0), x)
    for p in (1, 5, 15, 300):
        xr = orc.rope_row(x, p)
        assert abs(np.linalg.norm(xr) - np.linalg.norm(x)) < 1e-12
        np.testing.assert_allclose(xr, _rope_complex(x, p), rtol=1e-12, atol=1e-12)
    # relative position: <R_m x, R_n y> = <R_{m-n} x, y>
    for m, n in ((7, 3), (15, 0), (9, 9)):
        lhs = orc.rope_row(x, m) @ orc.rope_row(y, n)
        rhs = orc.rope_row(x, m - n) @ y
        assert abs(lhs - rhs) < 1e-11


# ----------------------------------------------------------------------------
# TTT-Linear: the oracle against the gradient-step definition (autograd)
# ----------------------------------------------------------------------------
def _linear_by_autograd(q, k, v, eta, gam, bet, W0, b0, K, offset=0, rope=False, loss_scale=0.5, token_eta=None):
    """Definition of the layer written with autograd.  Block boundaries are at
    absolute positions that are multiples of K; ``offset`` must be aligned.
    token_eta[i] scales the step used by the prediction of block row i (the
    pages' W1_bar = W1_init - grad_W1 * token_eta); the step carried to the
    next block is that of row K - 1."""
    assert offset % K == 0
    L, D = q.shape
    T = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))  # noqa: E731
    if rope:
        q = np.stack([_rope_complex(q[t], (offset + t) % K) for t in range(L)])
        k = np.stack([_rope_complex(k[t], (offset + t) % K) for t in range(L)])
    q, k, v, eta, gam, bet = map(T, (q, k, v, eta, gam, bet))
    W, b = T(W0), T(b0)
    outs = []
    for t in range(L):
        j0 = t - t % K
        Wp, bp = W.clone().requires_grad_(True), b.clone().requires_grad_(True)
        loss = 0.0
        for j in range(j0, t + 1):
            zj = k[j] @ Wp + bp
            loss = loss + eta[j] * loss_scale * ((Fn.layer_norm(zj, (D,), gam, bet, EPS) - (v[j] - k[j])) ** 2).sum()
        gW, gb = torch.autograd.grad(loss, (Wp, bp))
        te = 1.0 if token_eta is None else float(token_eta[(offset + t) % K])
        Wbar, bbar = W - te * gW, b - te * gb
        outs.append(q[t] + Fn.layer_norm(q[t] @ Wbar + bbar, (D,), gam, bet, EPS))
        if (t + 1) % K == 0:
            W, b = Wbar.detach(), bbar.detach()
    return torch.stack(outs).numpy(), W.numpy(), b.numpy()


def _problem(seed, L, D, rich=True):
    r = _rng(seed)
    q, k, v = (r.normal(size=(L, D)) for _ in range(3))
    eta = 1 / (1 + np.exp(-r.normal(size=L))) / 8
    W0 = r.normal(size=(D, D)) * 0.02
    if rich:
        b0 = 0.05 * r.normal(size=D)
        gam, bet = 1 + 0.2 * r.normal(size=D), 0.2 * r.normal(size=D)
    else:
        b0, gam, bet = np.zeros(D), np.ones(D), np.zeros(D)
    return q, k, v, eta, gam, bet, W0, b0


def _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K, offset=0, rope=False, token_eta=None):
    D = q.shape[1]
    W, b, G, gb = W0.copy(), b0.copy(), np.zeros((D, D)), np.zeros(D)
    out = orc.linear_chain(q, k, v, eta, gam, bet, W, b, G, gb, K=K, offset=offset, rope=rope, token_eta=token_eta)
    return out, W, b, G, gb


def _token_eta(K, seed):
    """A non-constant token_eta: 1/(i+1) (the usual choice for this factor)
    perturbed, so no two rows share a value."""
    r = _rng(seed)
    return 1.0 / np.arange(1, K + 1) + 0.05 * r.uniform(size=K)


@pytest.mark.parametrize("D,K,L,rope", [(8, 4, 11, False), (16, 1, 7, False), (64, 16, 40, False),
                                         (8, 4, 13, True), (64, 16, 35, True)])
def test_linear_matches_gradient_step_definition(orc, D, K, L, rope):
    prob = _problem(1000 + D * K + L, L, D)
    out, W, b, G, gb = _run_oracle_linear(orc, *prob, K=K, rope=rope)
    ref, Wr, br = _linear_by_autograd(*prob, K=K, rope=rope)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)
    # state: block-start W, b plus the open block's accumulated gradient
    if L % K == 0:
        np.testing.assert_allclose(W, Wr, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(b, br, rtol=1e-10, atol=1e-12)
        assert not G.any() and not gb.any()
    else:
        np.testing.assert_allclose(W, Wr, rtol=1e-10, atol=1e-12)  # committed blocks only
        assert np.abs(G).max() > 0


def test_online_gd_is_minibatch_one(orc):
    """mini_batch_size = 1: every token is its own mini-batch; the output of
    token t uses the state after the step on token t itself, and that state is
    carried — plain online gradient descent."""
    D, L = 16, 9
    q, k, v, eta, gam, bet, W0, b0 = _problem(31, L, D)
    out, W, b, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=1)
    Wt, bt = torch.tensor(W0), torch.tensor(b0)
    T = torch.tensor
    for t in range(L):
        Wp, bp = Wt.clone().requires_grad_(True), bt.clone().requires_grad_(True)
        z = T(k[t]) @ Wp + bp
        loss = 0.5 * ((Fn.layer_norm(z, (D,), T(gam), T(bet), EPS) - T(v[t] - k[t])) ** 2).sum()
        gW, gb_ = torch.autograd.grad(loss, (Wp, bp))
        Wt, bt = Wt - eta[t] * gW, bt - eta[t] * gb_
        o = T(q[t]) + Fn.layer_norm(T(q[t]) @ Wt + bt, (D,), T(gam), T(bet), EPS)
        np.testing.assert_allclose(out[t], o.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(W, Wt.numpy(), rtol=1e-10, atol=1e-13)


def test_loss_constant_reading(orc):
    """Half-square loss with 2*eta equals full-square loss with eta."""
    D, K, L = 8, 4, 8
    q, k, v, eta, gam, bet, W0, b0 = _problem(77, L, D)
    out, W, b, _, _ = _run_oracle_linear(orc, q, k, v, 2 * eta, gam, bet, W0, b0, K=K)
    ref, Wr, br = _linear_by_autograd(q, k, v, eta, gam, bet, W0, b0, K=K, loss_scale=1.0)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(W, Wr, rtol=1e-10, atol=1e-12)


def test_eta_zero_closed_form(orc):
    D, K, L = 64, 16, 37
    q, k, v, eta, gam, bet, W0, b0 = _problem(5, L, D)
    out, W, b, G, gb = _run_oracle_linear(orc, q, k, v, 0 * eta, gam, bet, W0, b0, K=K)
    ref = q + Fn.layer_norm(torch.tensor(q @ W0 + b0), (D,), torch.tensor(gam), torch.tensor(bet), EPS).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(W, W0)
    np.testing.assert_array_equal(b, b0)


@pytest.mark.parametrize("D,K,L,rope", [(8, 4, 11, False), (64, 16, 40, True), (16, 1, 6, False)])
def test_token_eta_matches_gradient_step_definition(orc, D, K, L, rope):
    """token_eta scales each row's step (and the carried step is the last
    row's): the oracle against the autograd definition with that scale."""
    prob = _problem(500 + D * K + L, L, D)
    te = _token_eta(K, D + L)
    out, W, b, _, _ = _run_oracle_linear(orc, *prob, K=K, rope=rope, token_eta=te)
    ref, Wr, br = _linear_by_autograd(*prob, K=K, rope=rope, token_eta=te)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(W, Wr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b, br, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dual", [False, True])
def test_constant_token_eta_equals_scaled_learning_rate(orc, dual):
    """eta_ij = token_eta_i * lr_j: a constant token_eta c is the same layer
    as token_eta = 1 with every learning rate times c."""
    D, K, L, c = 16, 4, 16, 0.37
    q, k, v, eta, gam, bet, W0, b0 = _problem(61, L, D)
    res = []
    for te, e in ((np.full(K, c), eta), (None, c * eta)):
        W, b = W0.copy(), b0.copy()
        if dual:
            o = orc.linear_chain_dual(q, k, v, e, gam, bet, W, b, K=K, token_eta=te)
        else:
            o = orc.linear_chain(q, k, v, e, gam, bet, W, b, np.zeros((D, D)), np.zeros(D), K=K, token_eta=te)
        res.append((o, W, b))
    for a, b_ in zip(*res):
        np.testing.assert_allclose(a, b_, rtol=1e-12, atol=1e-14)


def test_token_eta_on_last_row_only(orc):
    """token_eta = (0, ..., 0, 1): rows before the last predict with the
    block-start state (q + LN(q W_s + b_s)); the last row and the carried state
    are those of token_eta = 1.  A scale applied per key token instead of per
    output row would change the last row and the step."""
    D, K, L = 16, 4, 12
    q, k, v, eta, gam, bet, W0, b0 = _problem(62, L, D)
    te = np.zeros(K)
    te[-1] = 1.0
    out, W, b, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K, token_eta=te)
    ref, Wr, br, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K)
    np.testing.assert_allclose(W, Wr, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b, br, rtol=1e-13, atol=1e-15)
    T = torch.tensor
    for n in range(L // K):
        Ws, bs = W0.copy(), b0.copy()
        if n:
            _, Ws, bs, _, _ = _run_oracle_linear(orc, q[:n * K], k[:n * K], v[:n * K], eta[:n * K], gam, bet, W0,
                                                 b0, K=K)
        rows = slice(n * K, n * K + K - 1)
        closed = q[rows] + Fn.layer_norm(T(q[rows] @ Ws + bs), (D,), T(gam), T(bet), EPS).numpy()
        np.testing.assert_allclose(out[rows], closed, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[n * K + K - 1], ref[n * K + K - 1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,K,L,rope", [(8, 4, 16, False), (64, 16, 64, False), (64, 16, 48, True),
                                         (16, 1, 5, False), (8, 3, 12, True)])
def test_dual_equals_primal(orc, D, K, L, rope):
    q, k, v, eta, gam, bet, W0, b0 = _problem(9 + L, L, D)
    out_p, Wp, bp, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K, rope=rope)
    Wd, bd = W0.copy(), b0.copy()
    out_d = orc.linear_chain_dual(q, k, v, eta, gam, bet, Wd, bd, K=K, rope=rope)
    np.testing.assert_allclose(out_d, out_p, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Wd, Wp, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(bd, bp, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("D,K,L,rope", [(8, 4, 16, False), (64, 16, 48, True)])
def test_dual_equals_primal_token_eta(orc, D, K, L, rope):
    """The dual branch with eta_ij = token_eta_i * lr_j (its [K, K] eta and
    the last row for the step) against the primal per-token form."""
    q, k, v, eta, gam, bet, W0, b0 = _problem(19 + L, L, D)
    te = _token_eta(K, L)
    out_p, Wp, bp, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K, rope=rope, token_eta=te)
    Wd, bd = W0.copy(), b0.copy()
    out_d = orc.linear_chain_dual(q, k, v, eta, gam, bet, Wd, bd, K=K, rope=rope, token_eta=te)
    np.testing.assert_allclose(out_d, out_p, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Wd, Wp, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(bd, bp, rtol=1e-11, atol=1e-13)


def test_split_invariance_every_cut_token_eta(orc):
    D, K, L = 16, 8, 40
    q, k, v, eta, gam, bet, W0, b0 = _problem(43, L, D)
    te = _token_eta(K, 5)
    whole, Ww, bw, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K, token_eta=te)
    for s in range(1, L):
        W, b, G, gb = W0.copy(), b0.copy(), np.zeros((D, D)), np.zeros(D)
        o1 = orc.linear_chain(q[:s], k[:s], v[:s], eta[:s], gam, bet, W, b, G, gb, K=K, token_eta=te)
        o2 = orc.linear_chain(q[s:], k[s:], v[s:], eta[s:], gam, bet, W, b, G, gb, K=K, offset=s, token_eta=te)
        np.testing.assert_allclose(np.concatenate([o1, o2]), whole, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(W, Ww, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("rope", [False, True])
def test_split_invariance_every_cut(orc, rope):
    """Processing [0, s) then [s, L) with the carried state equals [0, L),
    for every cut s (remainder handling and TTTCache continuation)."""
    D, K, L = 64, 16, 64
    q, k, v, eta, gam, bet, W0, b0 = _problem(42, L, D)
    whole, Ww, bw, _, _ = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K, rope=rope)
    for s in range(1, L):
        W, b, G, gb = W0.copy(), b0.copy(), np.zeros((D, D)), np.zeros(D)
        o1 = orc.linear_chain(q[:s], k[:s], v[:s], eta[:s], gam, bet, W, b, G, gb, K=K, offset=0, rope=rope)
        o2 = orc.linear_chain(q[s:], k[s:], v[s:], eta[s:], gam, bet, W, b, G, gb, K=K, offset=s, rope=rope)
        np.testing.assert_allclose(np.concatenate([o1, o2]), whole, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(W, Ww, rtol=1e-12, atol=1e-14)


def test_prefill_then_single_token_decode(orc):
    D, K, L, P = 64, 16, 80, 24
    q, k, v, eta, gam, bet, W0, b0 = _problem(8, L, D)
    whole, Ww, bw, Gw, gbw = _run_oracle_linear(orc, q, k, v, eta, gam, bet, W0, b0, K=K)
    W, b, G, gb = W0.copy(), b0.copy(), np.zeros((D, D)), np.zeros(D)
    outs = [orc.linear_chain(q[:P], k[:P], v[:P], eta[:P], gam, bet, W, b, G, gb, K=K)]
    for t in range(P, L):
        outs.append(orc.linear_chain(q[t:t + 1], k[t:t + 1], v[t:t + 1], eta[t:t + 1], gam, bet, W, b, G, gb,
                                     K=K, offset=t))
    np.testing.assert_allclose(np.concatenate(outs), whole, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Ww, rtol=1e-12, atol=1e-14)


def test_batch_driver_matches_chains(orc):
    B, H, L, D, K = 2, 3, 20, 8, 4
    r = _rng(3)
    XQ, XK, XV = (r.normal(size=(B, H, L, D)) for _ in range(3))
    eta = r.uniform(0, 0.1, size=(H, L))
    lw, lb = 1 + 0.1 * r.normal(size=(H, D)), 0.1 * r.normal(size=(H, D))
    W0 = r.normal(size=(H, D, D)) * 0.02
    W = np.ascontiguousarray(np.broadcast_to(W0, (B, H, D, D)))
    b = np.zeros((B, H, D))
    G, gb = np.zeros_like(W), np.zeros_like(b)
    out = orc.linear_batch(XQ, XK, XV, eta, 0, lw, lb, W, b, G, gb, K=K, rope=True)
    for bi in range(B):
        for h in range(H):
            Wc, bc, Gc, gbc = W0[h].copy(), np.zeros(D), np.zeros((D, D)), np.zeros(D)
            oc = orc.linear_chain(XQ[bi, h], XK[bi, h], XV[bi, h], eta[h], lw[h], lb[h], Wc, bc, Gc, gbc,
                                  K=K, rope=True)
            np.testing.assert_array_equal(out[bi, h], oc)
            np.testing.assert_array_equal(W[bi, h], Wc)
            np.testing.assert_array_equal(G[bi, h], Gc)


# ----------------------------------------------------------------------------
# TTT-MLP
# ----------------------------------------------------------------------------
def test_gelu_matches_library(orc):
    xs = np.linspace(-6, 6, 97)
    for x in xs:
        xt = torch.tensor(x, requires_grad=True)
        y = Fn.gelu(xt, approximate="none")
        (dy,) = torch.autograd.grad(y, xt)
        assert abs(orc.gelu(x) - y.item()) < 1e-14
        assert abs(orc.gelu_grad(x) - dy.item()) < 1e-13


def _mlp_problem(seed, L, D, F):
    r = _rng(seed)
    q, k, v = (r.normal(size=(L, D)) for _ in range(3))
    eta = 1 / (1 + np.exp(-r.normal(size=L))) / 8
    W1, W2 = r.normal(size=(D, F)) * 0.2, r.normal(size=(F, D)) * 0.2
    b1, b2 = 0.05 * r.normal(size=F), 0.05 * r.normal(size=D)
    gam, bet = 1 + 0.2 * r.normal(size=D), 0.2 * r.normal(size=D)
    return q, k, v, eta, gam, bet, W1, b1, W2, b2


def _run_oracle_mlp(orc, q, k, v, eta, gam, bet, W1, b1, W2, b2, K, offset=0, rope=False, token_eta=None):
    D, F = W1.shape
    st = [W1.copy(), b1.copy(), W2.copy(), b2.copy(), np.zeros((D, F)), np.zeros(F), np.zeros((F, D)), np.zeros(D)]
    out = orc.mlp_chain(q, k, v, eta, gam, bet, *st, K=K, offset=offset, rope=rope, token_eta=token_eta)
    return out, st


def _mlp_by_autograd(q, k, v, eta, gam, bet, W1, b1, W2, b2, K, token_eta=None):
    L, D = q.shape
    T = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))  # noqa: E731
    q, k, v, eta, gam, bet = map(T, (q, k, v, eta, gam, bet))
    P = [T(W1), T(b1), T(W2), T(b2)]

    def f(x, p):
        return Fn.gelu(x @ p[0] + p[1], approximate="none") @ p[2] + p[3]

    outs = []
    for t in range(L):
        j0 = t - t % K
        Pp = [p.clone().requires_grad_(True) for p in P]
        loss = 0.0
        for j in range(j0, t + 1):
            loss = loss + eta[j] * 0.5 * ((Fn.layer_norm(f(k[j], Pp), (D,), gam, bet, EPS) - (v[j] - k[j])) ** 2).sum()
        grads = torch.autograd.grad(loss, Pp)
        te = 1.0 if token_eta is None else float(token_eta[t % K])
        Pbar = [p - te * g for p, g in zip(P, grads)]
        outs.append(q[t] + Fn.layer_norm(f(q[t], Pbar), (D,), gam, bet, EPS))
        if (t + 1) % K == 0:
            P = [p.detach() for p in Pbar]
    return torch.stack(outs).numpy(), [p.numpy() for p in P]


@pytest.mark.parametrize("D,F,K,L", [(8, 16, 4, 10), (64, 256, 16, 32), (8, 32, 1, 5)])
def test_mlp_matches_gradient_step_definition(orc, D, F, K, L):
    prob = _mlp_problem(D + F + L, L, D, F)
    out, st = _run_oracle_mlp(orc, *prob, K=K)
    ref, Pr = _mlp_by_autograd(*prob, K=K)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-10)
    for a, b in zip(st[:4], Pr):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("D,F,K,L", [(8, 16, 4, 10), (64, 256, 16, 32)])
def test_mlp_token_eta_matches_gradient_step_definition(orc, D, F, K, L):
    prob = _mlp_problem(7 + D + F + L, L, D, F)
    te = _token_eta(K, F)
    out, st = _run_oracle_mlp(orc, *prob, K=K, token_eta=te)
    ref, Pr = _mlp_by_autograd(*prob, K=K, token_eta=te)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-10)
    for a, b in zip(st[:4], Pr):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("D,F,K,L", [(8, 16, 4, 12), (64, 256, 16, 32)])
def test_mlp_dual_equals_primal_token_eta(orc, D, F, K, L):
    q, k, v, eta, gam, bet, W1, b1, W2, b2 = _mlp_problem(15 + L, L, D, F)
    te = _token_eta(K, D)
    out_p, st = _run_oracle_mlp(orc, q, k, v, eta, gam, bet, W1, b1, W2, b2, K=K, token_eta=te)
    sd = [W1.copy(), b1.copy(), W2.copy(), b2.copy()]
    out_d = orc.mlp_chain_dual(q, k, v, eta, gam, bet, *sd, K=K, token_eta=te)
    np.testing.assert_allclose(out_d, out_p, rtol=1e-10, atol=1e-11)
    for a, b in zip(sd, st[:4]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("D,F,K,L,rope", [(8, 16, 4, 12, False), (64, 256, 16, 32, True)])
def test_mlp_dual_equals_primal(orc, D, F, K, L, rope):
    q, k, v, eta, gam, bet, W1, b1, W2, b2 = _mlp_problem(5 + L, L, D, F)
    out_p, st = _run_oracle_mlp(orc, q, k, v, eta, gam, bet, W1, b1, W2, b2, K=K, rope=rope)
    sd = [W1.copy(), b1.copy(), W2.copy(), b2.copy()]
    out_d = orc.mlp_chain_dual(q, k, v, eta, gam, bet, *sd, K=K, rope=rope)
    np.testing.assert_allclose(out_d, out_p, rtol=1e-10, atol=1e-11)
    for a, b in zip(sd, st[:4]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-13)


def test_mlp_split_invariance(orc):
    D, F, K, L = 8, 16, 4, 14
    q, k, v, eta, gam, bet, W1, b1, W2, b2 = _mlp_problem(99, L, D, F)
    whole, stw = _run_oracle_mlp(orc, q, k, v, eta, gam, bet, W1, b1, W2, b2, K=K)
    for s in range(1, L):
        st = [W1.copy(), b1.copy(), W2.copy(), b2.copy(), np.zeros((D, F)), np.zeros(F), np.zeros((F, D)),
              np.zeros(D)]
        o1 = orc.mlp_chain(q[:s], k[:s], v[:s], eta[:s], gam, bet, *st, K=K, offset=0)
        o2 = orc.mlp_chain(q[s:], k[s:], v[s:], eta[s:], gam, bet, *st, K=K, offset=s)
        np.testing.assert_allclose(np.concatenate([o1, o2]), whole, rtol=1e-12, atol=1e-12)
        for a, b in zip(st, stw):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_mlp_eta_zero_closed_form(orc):
    D, F, K, L = 8, 16, 4, 9
    q, k, v, eta, gam, bet, W1, b1, W2, b2 = _mlp_problem(4, L, D, F)
    out, st = _run_oracle_mlp(orc, q, k, v, 0 * eta, gam, bet, W1, b1, W2, b2, K=K)
    T = torch.tensor
    h = Fn.gelu(T(q @ W1 + b1), approximate="none").numpy() @ W2 + b2
    ref = q + Fn.layer_norm(T(h), (D,), T(gam), T(bet), EPS).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert math.isclose(np.abs(st[0] - W1).max(), 0.0)


# ----------------------------------------------------------------------------
# Batch drivers (the all-chain checkers of the full-size GPU tests): each
# chain against the autograd definition, with learning rates that differ per
# batch row ([B, H, L], as "代码连连看——TTT" compute_mini_batch takes eta per
# batch and head), distinct per-chain start states and F != D, so that a
# wrong batch, head or state stride shows in some chain.
# ----------------------------------------------------------------------------
def _per_batch_eta(r, B, H, L):
    return 1 / (1 + np.exp(-r.normal(size=(B, H, L)))) / 8


@pytest.mark.parametrize("eta_per_batch", [False, True])
def test_linear_batch_driver_matches_definition(orc, eta_per_batch):
    B, H, L, D, K = 2, 3, 12, 8, 4
    r = _rng(301 + eta_per_batch)
    XQ, XK, XV = (r.normal(size=(B, H, L, D)) for _ in range(3))
    eta = _per_batch_eta(r, B, H, L) if eta_per_batch else _per_batch_eta(r, 1, H, L)[0]
    lw, lb = 1 + 0.2 * r.normal(size=(H, D)), 0.2 * r.normal(size=(H, D))
    W = r.normal(size=(B, H, D, D)) * 0.1  # every chain its own start state
    b = 0.05 * r.normal(size=(B, H, D))
    W0, b0 = W.copy(), b.copy()
    G, gb = np.zeros_like(W), np.zeros_like(b)
    out = orc.linear_batch(XQ, XK, XV, eta, H * L if eta_per_batch else 0, lw, lb, W, b, G, gb, K=K, rope=True)
    for bi in range(B):
        for h in range(H):
            e = eta[bi, h] if eta_per_batch else eta[h]
            ref, Wr, br = _linear_by_autograd(XQ[bi, h], XK[bi, h], XV[bi, h], e, lw[h], lb[h], W0[bi, h],
                                              b0[bi, h], K=K, rope=True)
            np.testing.assert_allclose(out[bi, h], ref, rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(W[bi, h], Wr, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(b[bi, h], br, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("eta_per_batch", [False, True])
def test_mlp_batch_driver_matches_definition(orc, eta_per_batch):
    B, H, L, D, F, K = 2, 2, 8, 8, 16, 4
    r = _rng(311 + eta_per_batch)
    XQ, XK, XV = (r.normal(size=(B, H, L, D)) for _ in range(3))
    eta = _per_batch_eta(r, B, H, L) if eta_per_batch else _per_batch_eta(r, 1, H, L)[0]
    lw, lb = 1 + 0.2 * r.normal(size=(H, D)), 0.2 * r.normal(size=(H, D))
    W1, W2 = r.normal(size=(B, H, D, F)) * 0.2, r.normal(size=(B, H, F, D)) * 0.2
    b1, b2 = 0.05 * r.normal(size=(B, H, F)), 0.05 * r.normal(size=(B, H, D))
    init = [a.copy() for a in (W1, b1, W2, b2)]
    G = [np.zeros_like(W1), np.zeros_like(b1), np.zeros_like(W2), np.zeros_like(b2)]
    out = orc.mlp_batch(XQ, XK, XV, eta, H * L if eta_per_batch else 0, lw, lb, W1, b1, W2, b2, *G, K=K)
    for bi in range(B):
        for h in range(H):
            e = eta[bi, h] if eta_per_batch else eta[h]
            ref, Pr = _mlp_by_autograd(XQ[bi, h], XK[bi, h], XV[bi, h], e, lw[h], lb[h],
                                       *[a[bi, h] for a in init], K=K)
            np.testing.assert_allclose(out[bi, h], ref, rtol=1e-9, atol=1e-10)
            for got, want in zip((W1, b1, W2, b2), Pr):
                np.testing.assert_allclose(got[bi, h], want, rtol=1e-9, atol=1e-12)


def test_batch_drivers_open_state_and_offset(orc):
    """Batch drivers started mid-mini-batch from a carried open state equal
    the per-chain routine (itself pinned by split invariance above) chain by
    chain, for both layers, with per-batch learning rates and token_eta."""
    B, H, D, F, K, P, L = 2, 2, 8, 16, 4, 6, 9
    r = _rng(321)
    XQ, XK, XV = (r.normal(size=(B, H, P + L, D)) for _ in range(3))
    eta = _per_batch_eta(r, B, H, P + L)
    lw, lb = 1 + 0.2 * r.normal(size=(H, D)), 0.2 * r.normal(size=(H, D))
    te = _token_eta(K, 3)
    # TTT-Linear: carry P tokens per chain, then the batch driver from offset P
    W, b = r.normal(size=(B, H, D, D)) * 0.1, 0.05 * r.normal(size=(B, H, D))
    G, gb = np.zeros_like(W), np.zeros_like(b)
    ref_out = np.empty((B, H, L, D))
    ref_state = [np.empty_like(a) for a in (W, b, G, gb)]
    for bi in range(B):
        for h in range(H):
            s = [W[bi, h].copy(), b[bi, h].copy(), G[bi, h].copy(), gb[bi, h].copy()]
            orc.linear_chain(XQ[bi, h, :P], XK[bi, h, :P], XV[bi, h, :P], eta[bi, h, :P], lw[h], lb[h], *s, K=K,
                             token_eta=te)
            for a, x in zip((W, b, G, gb), s):
                a[bi, h] = x
            t = [x.copy() for x in s]
            ref_out[bi, h] = orc.linear_chain(XQ[bi, h, P:], XK[bi, h, P:], XV[bi, h, P:], eta[bi, h, P:], lw[h],
                                              lb[h], *t, K=K, offset=P, token_eta=te)
            for a, x in zip(ref_state, t):
                a[bi, h] = x
    assert np.abs(G).max() > 0  # the carried state is open
    out = orc.linear_batch(XQ[:, :, P:], XK[:, :, P:], XV[:, :, P:], np.ascontiguousarray(eta[:, :, P:]), H * L,
                           lw, lb, W, b, G, gb, K=K, offset=P, token_eta=te)
    np.testing.assert_array_equal(out, ref_out)
    for a, x in zip((W, b, G, gb), ref_state):
        np.testing.assert_array_equal(a, x)
    # TTT-MLP, the same
    st = [r.normal(size=(B, H, D, F)) * 0.2, 0.05 * r.normal(size=(B, H, F)), r.normal(size=(B, H, F, D)) * 0.2,
          0.05 * r.normal(size=(B, H, D)), np.zeros((B, H, D, F)), np.zeros((B, H, F)), np.zeros((B, H, F, D)),
          np.zeros((B, H, D))]
    ref_out = np.empty((B, H, L, D))
    ref_state = [np.empty_like(a) for a in st]
    for bi in range(B):
        for h in range(H):
            s = [a[bi, h].copy() for a in st]
            orc.mlp_chain(XQ[bi, h, :P], XK[bi, h, :P], XV[bi, h, :P], eta[bi, h, :P], lw[h], lb[h], *s, K=K,
                          token_eta=te)
            for a, x in zip(st, s):
                a[bi, h] = x
            t = [x.copy() for x in s]
            ref_out[bi, h] = orc.mlp_chain(XQ[bi, h, P:], XK[bi, h, P:], XV[bi, h, P:], eta[bi, h, P:], lw[h],
                                           lb[h], *t, K=K, offset=P, token_eta=te)
            for a, x in zip(ref_state, t):
                a[bi, h] = x
    assert np.abs(st[4]).max() > 0 and np.abs(st[6]).max() > 0
    out = orc.mlp_batch(XQ[:, :, P:], XK[:, :, P:], XV[:, :, P:], np.ascontiguousarray(eta[:, :, P:]), H * L, lw,
                        lb, *st, K=K, offset=P, token_eta=te)
    np.testing.assert_array_equal(out, ref_out)
    for a, x in zip(st, ref_state):
        np.testing.assert_array_equal(a, x)


# ----------------------------------------------------------------------------
# Post-norm and output projection ("代码连连看——TTT", TTTBase.forward: the
# concatenated output goes through post_norm, a LayerNorm, then o_proj)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("K,N,bias", [(8, 3, False), (64, 48, True), (192, 64, False)])
def test_post_proj_matches_library(orc, K, N, bias):
    """Against torch: layer_norm over the width, then a matrix product."""
    r = _rng(K + N)
    y = r.normal(size=(7, K)) * r.uniform(0.1, 4, size=(7, 1)) + r.normal(size=(7, 1)) * 3
    gam, bet = r.normal(size=K), r.normal(size=K)
    Wo = r.normal(size=(K, N)) * 0.05
    bv = r.normal(size=N) if bias else None
    ref = Fn.layer_norm(torch.tensor(y), (K,), torch.tensor(gam), torch.tensor(bet), EPS) @ torch.tensor(Wo)
    if bias:
        ref = ref + torch.tensor(bv)
    np.testing.assert_allclose(orc.post_proj(y, gam, bet, Wo, bv, EPS), ref.numpy(), rtol=1e-11, atol=1e-11)


def test_post_proj_hand_example(orc):
    """A 2 x 4 case worked by hand (eps = 0): the row (1, 3, 5, 7) has mean 4
    and population variance 5, so LN gives (-3, -1, 1, 3) / sqrt(5); with
    gamma = 1, beta = (1, 0, 0, 0) and Wo = e_1 + e_4 (column 0) and all ones
    (column 1), the outputs are 1 + 0 and 1.  A constant row has variance 0:
    not allowed with eps = 0, so eps = 1 there: LN = 0, outputs beta Wo = (1, 1)."""
    y = np.array([[1.0, 3.0, 5.0, 7.0]])
    Wo = np.array([[1.0, 1.0], [0.0, 1.0], [0.0, 1.0], [1.0, 1.0]])
    gam, bet = np.ones(4), np.array([1.0, 0.0, 0.0, 0.0])
    out = orc.post_proj(y, gam, bet, Wo, None, 0.0)
    np.testing.assert_allclose(out, [[1.0 + 0.0, 1.0]], rtol=0, atol=1e-15)
    out = orc.post_proj(np.full((1, 4), 2.5), gam, bet, Wo, None, 1.0)
    np.testing.assert_allclose(out, [[1.0, 1.0]], rtol=0, atol=1e-15)


def test_post_proj_invariances(orc):
    """LayerNorm removes a per-row offset, and with eps = 0 a per-row positive
    scale; gamma = 0 leaves beta Wo (+ bias) on every row; the map is linear
    in (Wo, bias)."""
    r = _rng(5)
    K, N = 32, 24
    y = r.normal(size=(6, K))
    gam, bet = r.normal(size=K), r.normal(size=K)
    Wo, bv = r.normal(size=(K, N)), r.normal(size=N)
    base = orc.post_proj(y, gam, bet, Wo, bv, 0.0)
    shifted = orc.post_proj(y + r.normal(size=(6, 1)) * 10, gam, bet, Wo, bv, 0.0)
    scaled = orc.post_proj(y * r.uniform(0.1, 10, size=(6, 1)), gam, bet, Wo, bv, 0.0)
    np.testing.assert_allclose(shifted, base, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(scaled, base, rtol=1e-9, atol=1e-9)
    flat = orc.post_proj(y, np.zeros(K), bet, Wo, bv, EPS)
    np.testing.assert_allclose(flat, np.broadcast_to(bet @ Wo + bv, (6, N)), rtol=1e-12, atol=1e-12)
    W2, b2 = r.normal(size=(K, N)), r.normal(size=N)
    lin = orc.post_proj(y, gam, bet, Wo + 2 * W2, bv + 2 * b2, EPS)
    parts = orc.post_proj(y, gam, bet, Wo, bv, EPS) + 2 * orc.post_proj(y, gam, bet, W2, b2, EPS)
    np.testing.assert_allclose(lin, parts, rtol=1e-10, atol=1e-10)


def test_post_proj_rows_independent(orc):
    """Any subset of rows gives the same rows (the sampled full-size checks
    rely on it)."""
    r = _rng(6)
    y = r.normal(size=(9, 16))
    gam, bet, Wo = r.normal(size=16), r.normal(size=16), r.normal(size=(16, 5))
    full = orc.post_proj(y, gam, bet, Wo)
    np.testing.assert_array_equal(orc.post_proj(y[[2, 7, 3]], gam, bet, Wo), full[[2, 7, 3]])
