"""Python binding of libttt (ctypes).  Argument marshalling only: every step of
the TTT hot path runs in the library's HIP kernels; torch supplies device
memory and streams.  The functions carry the C names of include/ttt.h.

There is no fallback: if libttt.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libttt.so")

TTT_OK = 0
STATUS_NAMES = {0: "TTT_OK", 1: "TTT_ERR_NULL", 2: "TTT_ERR_SHAPE", 3: "TTT_ERR_DTYPE", 4: "TTT_ERR_ALIGN",
                5: "TTT_ERR_ALIAS", 6: "TTT_ERR_STATE", 7: "TTT_ERR_UNSUPPORTED", 8: "TTT_ERR_HIP"}
TTT_F32, TTT_BF16 = 0, 1
TTT_GRAD_DENSE, TTT_GRAD_ROWS = 0, 1

EXPORTS = ["ttt_linear_state_init", "ttt_linear_prefill", "ttt_linear_decode", "ttt_mlp_state_init",
           "ttt_mlp_prefill", "ttt_mlp_decode", "ttt_post_proj_prepared_bytes", "ttt_post_proj_prepare",
           "ttt_post_proj", "ttt_status_string", "ttt_last_error"]


class ttt_tensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("sB", c_int64), ("sH", c_int64), ("sL", c_int64)]


class ttt_eta(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("sB", c_int64), ("sH", c_int64), ("token_eta", c_void_p)]


class ttt_linear_cfg(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("D", c_int32), ("K", c_int32), ("in_dtype", c_int32),
                ("out_dtype", c_int32), ("rope", c_int32), ("rope_base", c_float), ("ln_eps", c_float),
                ("grad_layout", c_int32)]


class ttt_linear_state(ctypes.Structure):
    _fields_ = [("W", c_void_p), ("b", c_void_p), ("W_grad", c_void_p), ("b_grad", c_void_p), ("offset", c_int64)]


class ttt_mlp_cfg(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("D", c_int32), ("F", c_int32), ("K", c_int32),
                ("in_dtype", c_int32), ("out_dtype", c_int32), ("rope", c_int32), ("rope_base", c_float),
                ("ln_eps", c_float), ("grad_layout", c_int32)]


class ttt_mlp_state(ctypes.Structure):
    _fields_ = [("W1", c_void_p), ("b1", c_void_p), ("W2", c_void_p), ("b2", c_void_p), ("W1_grad", c_void_p),
                ("b1_grad", c_void_p), ("W2_grad", c_void_p), ("b2_grad", c_void_p), ("offset", c_int64)]


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


_lib = None


def load():
    """Loads libttt.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m test_rnn_layers_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.ttt_status_string.argtypes = [c_int32]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_last_error.argtypes = []
    lib.ttt_last_error.restype = ctypes.c_char_p
    lib.ttt_linear_state_init.argtypes = [P(ttt_linear_cfg), c_void_p, c_void_p, P(ttt_linear_state), c_void_p]
    call = [P(ttt_linear_cfg), c_int32, ttt_tensor, ttt_tensor, ttt_tensor, ttt_eta, c_void_p, c_void_p,
            P(ttt_linear_state), ttt_tensor, c_void_p]
    lib.ttt_linear_prefill.argtypes = call
    lib.ttt_linear_decode.argtypes = call
    lib.ttt_mlp_state_init.argtypes = [P(ttt_mlp_cfg), c_void_p, c_void_p, c_void_p, c_void_p, P(ttt_mlp_state),
                                       c_void_p]
    lib.ttt_mlp_prefill.argtypes = [P(ttt_mlp_cfg), c_int32, ttt_tensor, ttt_tensor, ttt_tensor, ttt_eta, c_void_p,
                                    c_void_p, P(ttt_mlp_state), ttt_tensor, c_void_p]
    lib.ttt_mlp_decode.argtypes = lib.ttt_mlp_prefill.argtypes
    lib.ttt_post_proj_prepared_bytes.argtypes = [c_int32, c_int32]
    lib.ttt_post_proj_prepared_bytes.restype = ctypes.c_size_t
    lib.ttt_post_proj_prepare.argtypes = [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p]
    lib.ttt_post_proj.argtypes = [c_int32, c_int32, c_int32, c_void_p, c_int64, c_float, c_void_p, c_void_p,
                                  c_int64, c_int32, c_void_p]
    for f in ("ttt_linear_state_init", "ttt_linear_prefill", "ttt_linear_decode", "ttt_mlp_state_init",
              "ttt_mlp_prefill", "ttt_mlp_decode", "ttt_post_proj_prepare", "ttt_post_proj"):
        getattr(lib, f).restype = c_int32
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def tensor(t) -> ttt_tensor:
    """[B, H, L, D] torch tensor (D contiguous) -> ttt_tensor."""
    if isinstance(t, ttt_tensor):
        return t
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("activations must be [B, H, L, D] with D contiguous")
    return ttt_tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _check_te(cfg, token_eta):
    if token_eta is not None and token_eta.numel() != cfg.K:
        raise ValueError(f"token_eta holds {token_eta.numel()} values; the mini-batch size is {cfg.K}")


def eta_desc(t, token_eta=None) -> ttt_eta:
    """eta as [H, L] (shared over the batch) or [B, H, L], token stride 1;
    token_eta: None or a contiguous fp32 device tensor of K values."""
    if isinstance(t, ttt_eta):
        return t
    if t.stride(-1) != 1:
        raise ValueError("eta must have token stride 1")
    te = None
    if token_eta is not None:
        import torch

        if token_eta.dim() != 1 or not token_eta.is_contiguous() or token_eta.dtype != torch.float32:
            raise ValueError("token_eta must be a contiguous fp32 vector of K values")
        te = token_eta.data_ptr()
    if t.dim() == 2:
        return ttt_eta(t.data_ptr(), 0, t.stride(0), te)
    if t.dim() == 3:
        return ttt_eta(t.data_ptr(), t.stride(0), t.stride(1), te)
    raise ValueError("eta must be [H, L] or [B, H, L]")


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != TTT_OK:
        raise TTTError(status, load().ttt_last_error().decode())


def dtype_code(dt) -> int:
    import torch

    if dt in (torch.float32, "f32"):
        return TTT_F32
    if dt in (torch.bfloat16, "bf16"):
        return TTT_BF16
    raise ValueError(f"unsupported dtype {dt}")


class LinearState:
    """Device buffers of a ttt_linear_state plus the ctypes struct (keeps the
    tensors alive).  ``offset`` is maintained by the library."""

    def __init__(self, W, b, W_grad, b_grad):
        self.W, self.b, self.W_grad, self.b_grad = W, b, W_grad, b_grad
        self.struct = ttt_linear_state(W.data_ptr(), b.data_ptr(), W_grad.data_ptr(), b_grad.data_ptr(), 0)

    @classmethod
    def empty(cls, B, H, D=64, device="cuda"):
        import torch

        f = dict(device=device, dtype=torch.float32)
        return cls(torch.empty((B, H, D, D), **f), torch.empty((B, H, D), **f), torch.empty((B, H, D, D), **f),
                   torch.empty((B, H, D), **f))

    @property
    def offset(self) -> int:
        return self.struct.offset


class MlpState:
    def __init__(self, W1, b1, W2, b2, W1_grad, b1_grad, W2_grad, b2_grad):
        self.tensors = (W1, b1, W2, b2, W1_grad, b1_grad, W2_grad, b2_grad)
        self.W1, self.b1, self.W2, self.b2 = W1, b1, W2, b2
        self.W1_grad, self.b1_grad, self.W2_grad, self.b2_grad = W1_grad, b1_grad, W2_grad, b2_grad
        self.struct = ttt_mlp_state(*[t.data_ptr() for t in self.tensors], 0)

    @classmethod
    def empty(cls, B, H, D=64, F=256, device="cuda"):
        import torch

        shapes = [(B, H, D, F), (B, H, F), (B, H, F, D), (B, H, D)]
        return cls(*[torch.empty(s, device=device, dtype=torch.float32) for s in shapes * 2])

    @property
    def offset(self) -> int:
        return self.struct.offset


def linear_cfg(B, H, *, K=16, in_dtype="bf16", out_dtype="f32", rope=False, rope_base=10000.0, ln_eps=1e-6, D=64,
               grad_layout="dense"):
    layout = {"dense": TTT_GRAD_DENSE, "rows": TTT_GRAD_ROWS}.get(grad_layout, grad_layout)
    return ttt_linear_cfg(B, H, D, K, dtype_code(in_dtype), dtype_code(out_dtype), int(rope), rope_base, ln_eps,
                          int(layout))


def mlp_cfg(B, H, *, F=256, K=16, in_dtype="bf16", out_dtype="f32", rope=False, rope_base=10000.0, ln_eps=1e-6,
            D=64, grad_layout="dense"):
    layout = {"dense": TTT_GRAD_DENSE, "rows": TTT_GRAD_ROWS}.get(grad_layout, grad_layout)
    return ttt_mlp_cfg(B, H, D, F, K, dtype_code(in_dtype), dtype_code(out_dtype), int(rope), rope_base, ln_eps,
                       int(layout))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def ttt_linear_state_init(cfg, W0, b0, state, stream=None):
    _check(load().ttt_linear_state_init(ctypes.byref(cfg), _ptr(W0), _ptr(b0), ctypes.byref(_st(state)),
                                        _stream(stream)))


def _st(state):
    return state.struct if hasattr(state, "struct") else state


def ttt_linear_prefill(cfg, L, XQ, XK, XV, eta, ln_w, ln_b, state, out, stream=None, token_eta=None):
    _check_te(cfg, token_eta)
    _check(load().ttt_linear_prefill(ctypes.byref(cfg), int(L), tensor(XQ), tensor(XK), tensor(XV),
                                     eta_desc(eta, token_eta),
                                     _ptr(ln_w), _ptr(ln_b), ctypes.byref(_st(state)), tensor(out),
                                     _stream(stream)))


def ttt_linear_decode(cfg, T, XQ, XK, XV, eta, ln_w, ln_b, state, out, stream=None, token_eta=None):
    _check_te(cfg, token_eta)
    _check(load().ttt_linear_decode(ctypes.byref(cfg), int(T), tensor(XQ), tensor(XK), tensor(XV),
                                    eta_desc(eta, token_eta),
                                    _ptr(ln_w), _ptr(ln_b), ctypes.byref(_st(state)), tensor(out),
                                    _stream(stream)))


def ttt_mlp_state_init(cfg, W1, b1, W2, b2, state, stream=None):
    _check(load().ttt_mlp_state_init(ctypes.byref(cfg), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                     ctypes.byref(_st(state)), _stream(stream)))


def ttt_mlp_prefill(cfg, L, XQ, XK, XV, eta, ln_w, ln_b, state, out, stream=None, token_eta=None):
    _check_te(cfg, token_eta)
    _check(load().ttt_mlp_prefill(ctypes.byref(cfg), int(L), tensor(XQ), tensor(XK), tensor(XV),
                                  eta_desc(eta, token_eta),
                                  _ptr(ln_w), _ptr(ln_b), ctypes.byref(_st(state)), tensor(out), _stream(stream)))


def ttt_mlp_decode(cfg, T, XQ, XK, XV, eta, ln_w, ln_b, state, out, stream=None, token_eta=None):
    _check_te(cfg, token_eta)
    _check(load().ttt_mlp_decode(ctypes.byref(cfg), int(T), tensor(XQ), tensor(XK), tensor(XV),
                                 eta_desc(eta, token_eta),
                                 _ptr(ln_w), _ptr(ln_b), ctypes.byref(_st(state)), tensor(out), _stream(stream)))


def ttt_status_string(status: int) -> str:
    return load().ttt_status_string(int(status)).decode()


def ttt_last_error() -> str:
    return load().ttt_last_error().decode()


def ttt_post_proj_prepared_bytes(K, N) -> int:
    return int(load().ttt_post_proj_prepared_bytes(int(K), int(N)))


def ttt_post_proj_prepare(K, N, gamma, beta, Wo, bias, prepared, stream=None):
    """gamma, beta [K], Wo [K, N] (row-major), bias [N] or None: fp32 device
    tensors; prepared: a device buffer of ttt_post_proj_prepared_bytes(K, N)."""
    _check(load().ttt_post_proj_prepare(int(K), int(N), _ptr(gamma), _ptr(beta), _ptr(Wo), _ptr(bias),
                                        _ptr(prepared), _stream(stream)))


def ttt_post_proj(M, K, N, y, ldy, eps, prepared, out, ldo, out_dtype="f32", stream=None):
    """y [M, K] bf16 rows of stride ldy; out [M, N] rows of stride ldo."""
    _check(load().ttt_post_proj(int(M), int(K), int(N), _ptr(y), int(ldy), float(eps), _ptr(prepared), _ptr(out),
                                int(ldo), dtype_code(out_dtype), _stream(stream)))
