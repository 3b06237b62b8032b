"""The library used from plain C through include/ttt.h (csrc/c_example.c,
built with the library): TTT-Linear prefill of 27 tokens, then decode of 13
with the carried state, fp32.  Its outputs and final state are compared with
the oracle over the whole sequence at the fp32 bar."""
import os
import subprocess

import numpy as np
import pytest
import torch

from harness import TOL_F32, max_abs, oracle_linear
from test_rnn_layers_amd.build_lib import C_EXAMPLE

pytestmark = pytest.mark.gpu


def test_c_program_matches_oracle(tmp_path):
    path = str(tmp_path / "c_example.bin")
    r = subprocess.run([C_EXAMPLE, path], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(path, "rb").read()
    B, H, L, D, Lp = np.frombuffer(raw[:20], dtype=np.int32)
    a = np.frombuffer(raw[20:], dtype=np.float32)
    shapes = [(B, H, L, D)] * 3 + [(H, L), (H, D, D), (H, D), (H, D), (H, D), (B, H, L, D), (B, H, D, D), (B, H, D)]
    parts, off = [], 0
    for s in shapes:
        n = int(np.prod(s))
        parts.append(a[off:off + n].reshape(s))
        off += n
    assert off == a.size
    XQ, XK, XV, eta, W0, b0, lw, lb, out, W, b = parts
    inp = {k: torch.from_numpy(v.copy()) for k, v in
           dict(XQ=XQ, XK=XK, XV=XV, eta=eta, W0=W0, b0=b0, ln_w=lw, ln_b=lb).items()}
    ro, rW, rb, _, _ = oracle_linear(inp, K=16)
    assert 0 < Lp < L
    assert max_abs(out.reshape(B * H, L, D).astype(np.float64), ro) <= TOL_F32
    assert max_abs(W.reshape(rW.shape).astype(np.float64), rW) <= TOL_F32
    assert max_abs(b.reshape(rb.shape).astype(np.float64), rb) <= TOL_F32
