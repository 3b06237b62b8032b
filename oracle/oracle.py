"""ctypes front end of ``ttt_oracle.c`` (plain fp64 CPU reference).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark; never by the product path.

All arrays are numpy float64, C-contiguous.  State arrays are updated in
place, exactly as the C routines do.  See the C file for the definitions and
for the passages of the pages each routine follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f64 = ctypes.c_double

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (portable x86-64 code, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-D_DEFAULT_SOURCE",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_ln_fwd.argtypes = [_dp, _dp, _dp, _i32, _f64, _dp]
    lib.oracle_ln_l2_grad.argtypes = [_dp, _dp, _dp, _dp, _i32, _f64, _dp]
    lib.oracle_rope_row.argtypes = [_dp, _i32, _i64, _f64, _dp]
    lib.oracle_gelu.argtypes = [_f64]
    lib.oracle_gelu.restype = _f64
    lib.oracle_gelu_grad.argtypes = [_f64]
    lib.oracle_gelu_grad.restype = _f64
    chain_common = [_dp, _dp, _dp, _i64, _dp, _i64, _dp, _dp, _dp, _i32, _f64, _f64]
    lib.oracle_linear_chain.argtypes = [_i32, _i32, _i32, _i64] + chain_common + [_dp, _dp, _dp, _dp, _dp, _i64]
    lib.oracle_linear_chain_dual.argtypes = [_i32, _i32, _i32, _i64] + chain_common + [_dp, _dp, _dp, _i64]
    lib.oracle_linear_chain_dual.restype = _i32
    lib.oracle_mlp_chain.argtypes = [_i32, _i32, _i32, _i32, _i64] + chain_common + [_dp] * 9 + [_i64]
    lib.oracle_mlp_chain_dual.argtypes = [_i32, _i32, _i32, _i32, _i64] + chain_common + [_dp] * 5 + [_i64]
    lib.oracle_mlp_chain_dual.restype = _i32
    lib.oracle_linear_batch.argtypes = ([_i32] * 5 + [_i64, _dp, _dp, _dp, _dp, _i64, _dp, _dp, _dp, _i32, _f64,
                                                       _f64] + [_dp] * 5)
    lib.oracle_mlp_batch.argtypes = ([_i32] * 6 + [_i64, _dp, _dp, _dp, _dp, _i64, _dp, _dp, _dp, _i32, _f64, _f64]
                                     + [_dp] * 9)
    lib.oracle_post_proj.argtypes = [_i64, _i32, _i32, _dp, _dp, _dp, _f64, _dp, _dp, _dp]
    lib.oracle_max_threads.restype = _i32
    lib.oracle_set_threads.argtypes = [_i32]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous float64"
    return a.ctypes.data_as(_dp)


def _f(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _te(token_eta, K):
    """token_eta: None (all ones) or K values, the scale of output row i of a
    mini-batch (and, for i = K - 1, of the committed step)."""
    if token_eta is None:
        return None, None
    te = _f(token_eta)
    assert te.shape == (K,), f"token_eta must hold K = {K} values"
    return te, _p(te)


def ln_fwd(z, gamma, beta, eps=1e-6):
    z, gamma, beta = _f(z), _f(gamma), _f(beta)
    y = np.empty_like(z)
    load().oracle_ln_fwd(_p(z), _p(gamma), _p(beta), z.shape[-1], eps, _p(y))
    return y


def ln_l2_grad(z, target, gamma, beta, eps=1e-6):
    z, target, gamma, beta = _f(z), _f(target), _f(gamma), _f(beta)
    g = np.empty_like(z)
    load().oracle_ln_l2_grad(_p(z), _p(target), _p(gamma), _p(beta), z.shape[-1], eps, _p(g))
    return g


def rope_row(x, p, base=10000.0):
    x = _f(x)
    y = np.empty_like(x)
    load().oracle_rope_row(_p(x), x.shape[-1], int(p), base, _p(y))
    return y


def gelu(x: float) -> float:
    return load().oracle_gelu(float(x))


def gelu_grad(x: float) -> float:
    return load().oracle_gelu_grad(float(x))


def linear_chain(q, k, v, eta, gamma, beta, W, b, G, gb, *, K, offset=0, rope=False,
                 rope_base=10000.0, eps=1e-6, token_eta=None):
    """One chain, primal form.  q, k, v: [L, D]; eta: [L]; token_eta: [K] or
    None.  W, b, G, gb are float64 arrays updated in place.  Returns out [L, D]."""
    q, k, v, eta, gamma, beta = map(_f, (q, k, v, eta, gamma, beta))
    te, tp = _te(token_eta, K)
    L, D = q.shape
    out = np.empty((L, D))
    load().oracle_linear_chain(D, K, L, offset, _p(q), _p(k), _p(v), D, _p(eta), 1, tp, _p(gamma), _p(beta),
                               int(rope), rope_base, eps, _p(W), _p(b), _p(G), _p(gb), _p(out), D)
    return out


def linear_chain_dual(q, k, v, eta, gamma, beta, W, b, *, K, offset=0, rope=False,
                      rope_base=10000.0, eps=1e-6, token_eta=None):
    q, k, v, eta, gamma, beta = map(_f, (q, k, v, eta, gamma, beta))
    te, tp = _te(token_eta, K)
    L, D = q.shape
    out = np.empty((L, D))
    rc = load().oracle_linear_chain_dual(D, K, L, offset, _p(q), _p(k), _p(v), D, _p(eta), 1, tp, _p(gamma),
                                         _p(beta), int(rope), rope_base, eps, _p(W), _p(b), _p(out), D)
    if rc != 0:
        raise ValueError("dual form needs whole aligned mini-batches")
    return out


def mlp_chain(q, k, v, eta, gamma, beta, W1, b1, W2, b2, G1, gb1, G2, gb2, *, K, offset=0,
              rope=False, rope_base=10000.0, eps=1e-6, token_eta=None):
    q, k, v, eta, gamma, beta = map(_f, (q, k, v, eta, gamma, beta))
    te, tp = _te(token_eta, K)
    L, D = q.shape
    F = W1.shape[1]
    out = np.empty((L, D))
    load().oracle_mlp_chain(D, F, K, L, offset, _p(q), _p(k), _p(v), D, _p(eta), 1, tp, _p(gamma), _p(beta),
                            int(rope), rope_base, eps, _p(W1), _p(b1), _p(W2), _p(b2), _p(G1), _p(gb1),
                            _p(G2), _p(gb2), _p(out), D)
    return out


def mlp_chain_dual(q, k, v, eta, gamma, beta, W1, b1, W2, b2, *, K, offset=0, rope=False,
                   rope_base=10000.0, eps=1e-6, token_eta=None):
    q, k, v, eta, gamma, beta = map(_f, (q, k, v, eta, gamma, beta))
    te, tp = _te(token_eta, K)
    L, D = q.shape
    F = W1.shape[1]
    out = np.empty((L, D))
    rc = load().oracle_mlp_chain_dual(D, F, K, L, offset, _p(q), _p(k), _p(v), D, _p(eta), 1, tp, _p(gamma),
                                      _p(beta), int(rope), rope_base, eps, _p(W1), _p(b1), _p(W2), _p(b2),
                                      _p(out), D)
    if rc != 0:
        raise ValueError("dual form needs whole aligned mini-batches")
    return out


def linear_batch(XQ, XK, XV, eta, eta_sB, ln_w, ln_b, W, b, G, gb, *, K, offset=0, rope=False,
                 rope_base=10000.0, eps=1e-6, token_eta=None):
    """[B, H, L, D] inputs; eta flat with batch stride eta_sB and head stride L.
    State arrays [B, H, ...] float64, updated in place.  Returns out."""
    XQ, XK, XV, eta, ln_w, ln_b = map(_f, (XQ, XK, XV, eta, ln_w, ln_b))
    te, tp = _te(token_eta, K)
    B, H, L, D = XQ.shape
    out = np.empty_like(XQ)
    load().oracle_linear_batch(B, H, D, K, L, offset, _p(XQ), _p(XK), _p(XV), _p(eta), eta_sB, tp, _p(ln_w),
                               _p(ln_b), int(rope), rope_base, eps, _p(W), _p(b), _p(G), _p(gb), _p(out))
    return out


def mlp_batch(XQ, XK, XV, eta, eta_sB, ln_w, ln_b, W1, b1, W2, b2, G1, gb1, G2, gb2, *, K, offset=0,
              rope=False, rope_base=10000.0, eps=1e-6, token_eta=None):
    XQ, XK, XV, eta, ln_w, ln_b = map(_f, (XQ, XK, XV, eta, ln_w, ln_b))
    te, tp = _te(token_eta, K)
    B, H, L, D = XQ.shape
    F = W1.shape[-1]
    out = np.empty_like(XQ)
    load().oracle_mlp_batch(B, H, D, F, K, L, offset, _p(XQ), _p(XK), _p(XV), _p(eta), eta_sB, tp, _p(ln_w),
                            _p(ln_b), int(rope), rope_base, eps, _p(W1), _p(b1), _p(W2), _p(b2), _p(G1),
                            _p(gb1), _p(G2), _p(gb2), _p(out))
    return out


def post_proj(y, gamma, beta, Wo, bias=None, eps=1e-6):
    """out = LayerNorm(y) Wo (+ bias) row by row: y [M, K], gamma/beta [K],
    Wo [K, N], bias [N] or None.  Returns [M, N] float64."""
    y, gamma, beta, Wo = map(_f, (y, gamma, beta, Wo))
    M, K = y.shape
    N = Wo.shape[1]
    assert Wo.shape[0] == K and gamma.shape == (K,) and beta.shape == (K,)
    out = np.empty((M, N))
    bp = _p(_f(bias)) if bias is not None else None
    load().oracle_post_proj(M, K, N, _p(y), _p(gamma), _p(beta), eps, _p(Wo), bp, _p(out))
    return out


def max_threads() -> int:
    return int(load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Thread count of the batch drivers from now on."""
    load().oracle_set_threads(int(n))
