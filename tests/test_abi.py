"""libttt loads, exports every function include/ttt.h declares, and rejects bad
arguments with the documented status before touching the GPU.  The error
paths return before any HIP call, so these run without a GPU (the pointers
below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from test_rnn_layers_amd import libttt as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char \*|ttt_status |size_t )\s*(ttt_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert set(_declared()) == set(T.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = T.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in T.STATUS_NAMES.items():
        assert T.ttt_status_string(code) == name


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
B, H, L, D = 2, 3, 40, 64
MB = 1 << 20
BASE = 0x7F0000000000


def _addr(i):
    return BASE + i * 64 * MB


def _args(**over):
    es = 2
    a = dict(
        cfg=T.linear_cfg(B, H, in_dtype="bf16", out_dtype="f32"),
        L=L,
        XQ=T.ttt_tensor(_addr(0), H * L * D, L * D, D),
        XK=T.ttt_tensor(_addr(1), H * L * D, L * D, D),
        XV=T.ttt_tensor(_addr(2), H * L * D, L * D, D),
        eta=T.ttt_eta(_addr(3), 0, L),
        ln_w=_addr(4),
        ln_b=_addr(5),
        state=T.ttt_linear_state(_addr(6), _addr(7), _addr(8), _addr(9), 0),
        out=T.ttt_tensor(_addr(10), H * L * D, L * D, D),
    )
    del es
    a.update(over)
    return a


def _call(fn="ttt_linear_prefill", **over):
    a = _args(**over)
    lib = T.load()
    cfg = ctypes.byref(a["cfg"]) if a["cfg"] is not None else None
    st = ctypes.byref(a["state"]) if a["state"] is not None else None
    rc = getattr(lib, fn)(cfg, a["L"], a["XQ"], a["XK"], a["XV"], a["eta"], a["ln_w"], a["ln_b"], st, a["out"],
                          None)
    return rc, a


def _cfg(**kw):
    c = T.linear_cfg(B, H, in_dtype="bf16", out_dtype="f32")
    for k, v in kw.items():
        setattr(c, k, v)
    return c


CASES = [
    ("null cfg", dict(cfg=None), "TTT_ERR_NULL"),
    ("null XQ", dict(XQ=T.ttt_tensor(None, H * L * D, L * D, D)), "TTT_ERR_NULL"),
    ("null eta", dict(eta=T.ttt_eta(None, 0, L)), "TTT_ERR_NULL"),
    ("null ln", dict(ln_w=None), "TTT_ERR_NULL"),
    ("null state", dict(state=None), "TTT_ERR_NULL"),
    ("null W_grad", dict(state=T.ttt_linear_state(_addr(6), _addr(7), None, _addr(9), 0)), "TTT_ERR_NULL"),
    ("D=32", dict(cfg=_cfg(D=32)), "TTT_ERR_SHAPE"),
    ("K=0", dict(cfg=_cfg(K=0)), "TTT_ERR_SHAPE"),
    ("K=17", dict(cfg=_cfg(K=17)), "TTT_ERR_SHAPE"),
    ("B=0", dict(cfg=_cfg(B=0)), "TTT_ERR_SHAPE"),
    ("L=0", dict(L=0), "TTT_ERR_SHAPE"),
    ("eps=0", dict(cfg=_cfg(ln_eps=0.0)), "TTT_ERR_SHAPE"),
    ("dtype", dict(cfg=_cfg(in_dtype=7)), "TTT_ERR_DTYPE"),
    ("grad_layout", dict(cfg=_cfg(grad_layout=2)), "TTT_ERR_UNSUPPORTED"),
    ("misaligned token_eta", dict(eta=T.ttt_eta(_addr(3), 0, L, _addr(11) + 4)), "TTT_ERR_ALIGN"),
    ("out overlaps token_eta", dict(eta=T.ttt_eta(_addr(3), 0, L, _addr(10) + 256)), "TTT_ERR_ALIAS"),
    ("misaligned XK", dict(XK=T.ttt_tensor(_addr(1) + 8, H * L * D, L * D, D)), "TTT_ERR_ALIGN"),
    ("odd token stride", dict(XV=T.ttt_tensor(_addr(2), H * L * 68, L * 68, 68 + 2)), "TTT_ERR_ALIGN"),
    ("negative stride", dict(XQ=T.ttt_tensor(_addr(0), H * L * D, L * D, -D)), "TTT_ERR_ALIGN"),
    ("misaligned state", dict(state=T.ttt_linear_state(_addr(6) + 4, _addr(7), _addr(8), _addr(9), 0)),
     "TTT_ERR_ALIGN"),
    ("out overlaps XQ", dict(out=T.ttt_tensor(_addr(0) + 4096, H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("out overlaps state", dict(out=T.ttt_tensor(_addr(8), H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("out rows overlap", dict(out=T.ttt_tensor(_addr(10), H * L * D, L * D, 32)), "TTT_ERR_ALIAS"),
    ("XQ overlaps W", dict(XQ=T.ttt_tensor(_addr(6) + 1024, H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("eta overlaps b_grad", dict(eta=T.ttt_eta(_addr(9), 0, L)), "TTT_ERR_ALIAS"),
    ("ln_b overlaps W_grad", dict(ln_b=_addr(8) + 512), "TTT_ERR_ALIAS"),
    ("token_eta overlaps b", dict(eta=T.ttt_eta(_addr(3), 0, L, _addr(7))), "TTT_ERR_ALIAS"),
    ("state buffers overlap", dict(state=T.ttt_linear_state(_addr(6), _addr(6) + 64, _addr(8), _addr(9), 0)),
     "TTT_ERR_ALIAS"),
    ("negative offset", dict(state=T.ttt_linear_state(_addr(6), _addr(7), _addr(8), _addr(9), -3)),
     "TTT_ERR_STATE"),
]


@pytest.mark.parametrize("fn", ["ttt_linear_prefill", "ttt_linear_decode"])
@pytest.mark.parametrize("label,over,expect", CASES, ids=[c[0] for c in CASES])
def test_error_paths(fn, label, over, expect):
    rc, a = _call(fn, **over)
    assert T.STATUS_NAMES[rc] == expect, (label, T.ttt_last_error())
    assert T.ttt_last_error(), "a failed call leaves a message"
    if a["state"] is not None:
        assert a["state"].offset == over.get("state", a["state"]).offset  # unchanged on error


def test_state_init_errors():
    lib = T.load()
    st = T.ttt_linear_state(_addr(6), _addr(7), _addr(8), _addr(9), 5)
    assert T.STATUS_NAMES[lib.ttt_linear_state_init(ctypes.byref(_cfg()), None, _addr(4), ctypes.byref(st), None)] \
        == "TTT_ERR_NULL"
    assert T.STATUS_NAMES[lib.ttt_linear_state_init(ctypes.byref(_cfg(D=16)), _addr(1), _addr(4), ctypes.byref(st),
                                                    None)] == "TTT_ERR_SHAPE"
    assert st.offset == 5


# ---------------------------------------------------------------------------
# TTT-MLP entry points
# ---------------------------------------------------------------------------
F = 256


def _mlp_cfg(**kw):
    c = T.mlp_cfg(B, H, in_dtype="bf16", out_dtype="f32")
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _mlp_state(offset=0, **over):
    p = [_addr(20 + i) for i in range(8)]
    for i, v in over.items():
        p[int(i[1:])] = v
    return T.ttt_mlp_state(*p, offset)


def _mlp_call(fn="ttt_mlp_prefill", **over):
    a = dict(cfg=_mlp_cfg(), L=L, XQ=T.ttt_tensor(_addr(0), H * L * D, L * D, D),
             XK=T.ttt_tensor(_addr(1), H * L * D, L * D, D), XV=T.ttt_tensor(_addr(2), H * L * D, L * D, D),
             eta=T.ttt_eta(_addr(3), 0, L), ln_w=_addr(4), ln_b=_addr(5), state=_mlp_state(),
             out=T.ttt_tensor(_addr(10), H * L * D, L * D, D))
    a.update(over)
    cfg = ctypes.byref(a["cfg"]) if a["cfg"] is not None else None
    st = ctypes.byref(a["state"]) if a["state"] is not None else None
    rc = getattr(T.load(), fn)(cfg, a["L"], a["XQ"], a["XK"], a["XV"], a["eta"], a["ln_w"], a["ln_b"], st,
                               a["out"], None)
    return rc, a


MLP_CASES = [
    ("null cfg", dict(cfg=None), "TTT_ERR_NULL"),
    ("null state", dict(state=None), "TTT_ERR_NULL"),
    ("null W2_grad", dict(state=_mlp_state(s6=None)), "TTT_ERR_NULL"),
    ("null XV", dict(XV=T.ttt_tensor(None, H * L * D, L * D, D)), "TTT_ERR_NULL"),
    ("F=128", dict(cfg=_mlp_cfg(F=128)), "TTT_ERR_SHAPE"),
    ("K=0", dict(cfg=_mlp_cfg(K=0)), "TTT_ERR_SHAPE"),
    ("K=17", dict(cfg=_mlp_cfg(K=17)), "TTT_ERR_SHAPE"),
    ("D=32", dict(cfg=_mlp_cfg(D=32)), "TTT_ERR_SHAPE"),
    ("L=0", dict(L=0), "TTT_ERR_SHAPE"),
    ("dtype", dict(cfg=_mlp_cfg(in_dtype=7)), "TTT_ERR_DTYPE"),
    ("misaligned token_eta", dict(eta=T.ttt_eta(_addr(3), 0, L, _addr(11) + 8)), "TTT_ERR_ALIGN"),
    ("negative offset", dict(state=_mlp_state(offset=-16)), "TTT_ERR_STATE"),
    ("misaligned b1", dict(state=_mlp_state(s1=_addr(21) + 4)), "TTT_ERR_ALIGN"),
    ("state buffers overlap", dict(state=_mlp_state(s3=_addr(20) + 1024)), "TTT_ERR_ALIAS"),
    ("out overlaps XK", dict(out=T.ttt_tensor(_addr(1), H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("out overlaps state", dict(out=T.ttt_tensor(_addr(24), H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("XV overlaps W2", dict(XV=T.ttt_tensor(_addr(22), H * L * D, L * D, D)), "TTT_ERR_ALIAS"),
    ("ln_w overlaps b1_grad", dict(ln_w=_addr(25)), "TTT_ERR_ALIAS"),
]


@pytest.mark.parametrize("fn", ["ttt_mlp_prefill", "ttt_mlp_decode"])
@pytest.mark.parametrize("label,over,expect", MLP_CASES, ids=[c[0] for c in MLP_CASES])
def test_mlp_error_paths(fn, label, over, expect):
    rc, a = _mlp_call(fn, **over)
    assert T.STATUS_NAMES[rc] == expect, (label, T.ttt_last_error())
    assert T.ttt_last_error()
    if a["state"] is not None:
        assert a["state"].offset == over.get("state", _mlp_state()).offset  # unchanged on error


def test_mlp_state_init_errors():
    lib = T.load()
    st = _mlp_state(offset=7)
    assert T.STATUS_NAMES[lib.ttt_mlp_state_init(ctypes.byref(_mlp_cfg()), _addr(1), None, _addr(3), _addr(4),
                                                 ctypes.byref(st), None)] == "TTT_ERR_NULL"
    assert T.STATUS_NAMES[lib.ttt_mlp_state_init(ctypes.byref(_mlp_cfg(F=64)), _addr(1), _addr(2), _addr(3),
                                                 _addr(4), ctypes.byref(st), None)] == "TTT_ERR_SHAPE"
    assert st.offset == 7


def test_c_example_is_built_against_the_header():
    """The plain-C example links libttt and imports the entry points it uses
    from it (it is run, against the oracle, by a GPU test)."""
    import subprocess
    from test_rnn_layers_amd.build_lib import C_EXAMPLE

    assert os.path.exists(C_EXAMPLE)
    und = subprocess.run(["nm", "-D", "--undefined-only", C_EXAMPLE], capture_output=True, text=True).stdout
    for sym in ("ttt_linear_state_init", "ttt_linear_prefill", "ttt_linear_decode", "ttt_last_error"):
        assert sym in und, sym


# --- post-norm and output projection
def _pp_args(**over):
    a = dict(M=300, K=128, N=256, y=_addr(0), ldy=128, eps=1e-5, prepared=_addr(1), out=_addr(2), ldo=256,
             out_dtype=T.TTT_F32, stream=None)
    a.update(over)
    return a


def _pp_call(a):
    lib = T.load()
    return lib.ttt_post_proj(a["M"], a["K"], a["N"], a["y"], a["ldy"], a["eps"], a["prepared"], a["out"],
                             a["ldo"], a["out_dtype"], a["stream"])


@pytest.mark.parametrize("label,over,expect", [
    ("y NULL", dict(y=0), "TTT_ERR_NULL"),
    ("prepared NULL", dict(prepared=0), "TTT_ERR_NULL"),
    ("out NULL", dict(out=0), "TTT_ERR_NULL"),
    ("M = 0", dict(M=0), "TTT_ERR_SHAPE"),
    ("K not a multiple of 64", dict(K=96, ldy=96), "TTT_ERR_SHAPE"),
    ("N not a multiple of 256", dict(N=128, ldo=128), "TTT_ERR_SHAPE"),
    ("ldy < K", dict(ldy=64), "TTT_ERR_SHAPE"),
    ("ldo < N", dict(ldo=255), "TTT_ERR_SHAPE"),
    ("eps = 0", dict(eps=0.0), "TTT_ERR_SHAPE"),
    ("out dtype", dict(out_dtype=7), "TTT_ERR_DTYPE"),
    ("y misaligned", dict(y=_addr(0) + 2), "TTT_ERR_ALIGN"),
    ("ldy not a multiple of 8", dict(ldy=132), "TTT_ERR_ALIGN"),
    ("prepared misaligned", dict(prepared=_addr(1) + 8), "TTT_ERR_ALIGN"),
    ("out misaligned", dict(out=_addr(2) + 4), "TTT_ERR_ALIGN"),
    ("ldo not a multiple of 16 bytes", dict(ldo=258), "TTT_ERR_ALIGN"),
    ("out overlaps y", dict(out=_addr(0) + 4096), "TTT_ERR_ALIAS"),
    ("out overlaps prepared", dict(out=_addr(1) + 16), "TTT_ERR_ALIAS"),
])
def test_post_proj_error_paths(label, over, expect):
    s = _pp_call(_pp_args(**over))
    assert T.STATUS_NAMES[s] == expect, (label, T.ttt_last_error())
    assert T.ttt_last_error()


def test_post_proj_prepare_errors():
    lib = T.load()
    K, N = 128, 256
    assert T.ttt_post_proj_prepared_bytes(K, N) == K * N * 2 + N * 8
    assert T.ttt_post_proj_prepared_bytes(0, N) == 0
    args = dict(K=K, N=N, gamma=_addr(0), beta=_addr(1), Wo=_addr(2), bias=None, prepared=_addr(3))
    cases = [(dict(gamma=0), "TTT_ERR_NULL"), (dict(Wo=0), "TTT_ERR_NULL"), (dict(prepared=0), "TTT_ERR_NULL"),
             (dict(K=100), "TTT_ERR_SHAPE"), (dict(N=300), "TTT_ERR_SHAPE"), (dict(prepared=_addr(3) + 4),
                                                                             "TTT_ERR_ALIGN"),
             (dict(prepared=_addr(2) + 64), "TTT_ERR_ALIAS"), (dict(bias=_addr(3) + 32), "TTT_ERR_ALIAS")]
    for over, expect in cases:
        a = dict(args, **over)
        s = lib.ttt_post_proj_prepare(a["K"], a["N"], a["gamma"], a["beta"], a["Wo"], a["bias"], a["prepared"], None)
        assert T.STATUS_NAMES[s] == expect, (over, T.ttt_last_error())
