"""Host-side logic that needs no GPU: bench.py's traffic models and its
one-GPU contract, the seeded input recipe, and the binding's argument checks."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from test_rnn_layers_amd import libttt  # noqa: E402
from test_rnn_layers_amd.synth import WORKLOADS, make_inputs, workload_inputs  # noqa: E402

D, K, F = 64, 16, 256
WB = (D * D + D) * 4          # W, b of TTT-Linear, bytes
MLP_PAR = (2 * D * F + F + D) * 4


def test_linear_decode_bytes_dense():
    """Dense layout over one mini-batch: W_s, b_s read by every call, G, gb
    read by all but the first and written by all, W_s, b_s written once."""
    cycle = range(512, 512 + K)
    per_call = [bench.decode_state_bytes("dense", [p]) for p in cycle]
    assert per_call[0] == 2 * WB                  # read W_s, b_s; write G, gb (clear G not read)
    assert per_call[5] == 3 * WB                  # read W_s, b_s, G, gb; write G, gb
    assert per_call[K - 1] == 4 * WB              # ... and the commit writes W_s, b_s
    assert bench.decode_state_bytes("dense", cycle) == pytest.approx(sum(per_call) / K)


def test_linear_decode_bytes_rows():
    """Rows layout: p open rows of 2D floats read, one row written (none on
    the closing call), b_grad read unless empty and always written."""
    row = 2 * D * 4
    assert bench.decode_state_bytes("rows", [0]) == WB + row + D * 4
    assert bench.decode_state_bytes("rows", [7]) == WB + 7 * row + D * 4 + row + D * 4
    assert bench.decode_state_bytes("rows", [15]) == WB + 15 * row + D * 4 + D * 4 + WB
    cycle = range(0, K)
    assert bench.decode_state_bytes("rows", cycle) < bench.decode_state_bytes("dense", cycle) / 2


def test_mlp_decode_bytes():
    cycle = range(0, K)
    dense = [bench.mlp_decode_state_bytes("dense", [p]) for p in cycle]
    assert dense[0] == 2 * MLP_PAR and dense[3] == 3 * MLP_PAR and dense[K - 1] == 4 * MLP_PAR
    rows = bench.mlp_decode_state_bytes("rows", cycle)
    assert rows < bench.mlp_decode_state_bytes("dense", cycle) / 2
    # a rows-layout call never moves more than W1..b2 twice plus 16 rows of both layers
    assert max(bench.mlp_decode_state_bytes("rows", [p]) for p in cycle) <= 2 * MLP_PAR + 16 * 2 * (D + F) * 4 + 4 * (
        F + D) * 4


def test_linear_token_bytes():
    assert bench.linear_token_bytes("bf16", "f32") == 3 * D * 2 + 4 + D * 4 == 644
    assert bench.linear_token_bytes("f32", "bf16") == 3 * D * 4 + 4 + D * 2


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_inputs_are_seeded_and_bf16_rounded():
    a = make_inputs(2, 3, 40, dtype="bf16", seed=5, rich=True)
    b = make_inputs(2, 3, 40, dtype="bf16", seed=5, rich=True)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert a["XQ"].dtype == torch.bfloat16 and a["eta"].dtype == torch.float32
    f = make_inputs(2, 3, 40, dtype="f32", seed=5, rich=True)
    # the bf16 values are the fp32 draws rounded to nearest
    assert torch.equal(f["XQ"].to(torch.bfloat16), a["XQ"])
    assert float(a["eta"].min()) > 0 and float(a["eta"].max()) < 1 / 64


def test_workload_shapes():
    names = {w.name: w for w in WORKLOADS}
    w = names["linear_1b_B4_H32_L8192_bf16"]
    assert (w.B, w.H, w.L, w.dtype, w.rope) == (4, 32, 8192, "bf16", False)
    w = names["decode_1b_B64_H32_prefill512_decode256_bf16"]
    assert (w.B, w.H, w.prefill, w.decode, w.L) == (64, 32, 512, 256, 768)
    small = workload_inputs(WORKLOADS[0])
    assert small["XQ"].shape == (1, 1, 64, 64) and small["W0"].shape == (1, 64, 64)


def test_binding_checks_token_eta_length():
    cfg = libttt.linear_cfg(1, 1, K=16)
    with pytest.raises(ValueError):
        libttt._check_te(cfg, torch.ones(8))
    libttt._check_te(cfg, torch.ones(16))
    with pytest.raises(ValueError):
        libttt.eta_desc(torch.ones(1, 8), token_eta=torch.ones(16, dtype=torch.float64))


def test_binding_cfg_layouts():
    assert libttt.linear_cfg(2, 3, grad_layout="rows").grad_layout == libttt.TTT_GRAD_ROWS
    assert libttt.mlp_cfg(2, 3, grad_layout="rows").grad_layout == libttt.TTT_GRAD_ROWS
    assert libttt.mlp_cfg(2, 3).grad_layout == libttt.TTT_GRAD_DENSE
    d = libttt.eta_desc(torch.ones(3, 40))
    assert d.sB == 0 and d.sH == 40 and not d.token_eta
    d = libttt.eta_desc(torch.ones(2, 3, 40))
    assert (d.sB, d.sH) == (120, 40)
    np.testing.assert_equal(libttt.STATUS_NAMES[7], "TTT_ERR_UNSUPPORTED")


def _counter_csv(path, rows):
    import csv

    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_profile_traffic_scaling(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE of a kernel scaled by what they read for the copy probe."""
    from test_rnn_layers_amd import profile_summary as ps

    monkeypatch.setattr(ps, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    mb = 64
    _counter_csv(str(tmp_path / "f" / "p_counter_collection.csv"),
                 [(1, 512, "linear_dual_kernel", "FETCH_SIZE", 1000.0), (2, 512, "linear_dual_kernel", "FETCH_SIZE", 1000.0),
                  (3, 4096, "__amd_rocclr_copyBuffer", "FETCH_SIZE", mb * 512.0),
                  (4, 4096, "__amd_rocclr_copyBuffer", "FETCH_SIZE", mb * 512.0)])
    _counter_csv(str(tmp_path / "w" / "p_counter_collection.csv"),
                 [(1, 512, "linear_dual_kernel", "WRITE_SIZE", 300.0),
                  (3, 4096, "__amd_rocclr_copyBuffer", "WRITE_SIZE", mb * 1024.0),
                  (4, 4096, "__amd_rocclr_copyBuffer", "WRITE_SIZE", mb * 1024.0)])
    ps.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "linear_dual_kernel", "wl", mb, "cmd")
    import json

    rec = json.load(open(tmp_path / "traffic.json"))["linear_dual_kernel@wl"]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1000 * 1024 * 2 + 300 * 1024)


def test_profile_sq_per_wave(tmp_path):
    """Per-wave figures of the shader-sequencer summary (cycle counters in units of 4 cycles)."""
    from test_rnn_layers_amd import profile_summary as ps

    rows = [(1, 512, "mlp_dual_kernel", "SQ_WAVES", 8.0), (1, 512, "mlp_dual_kernel", "SQ_WAVE_CYCLES", 8000.0),
            (1, 512, "mlp_dual_kernel", "SQ_INSTS_VALU", 1600.0), (1, 512, "mlp_dual_kernel", "SQ_ACTIVE_INST_VALU", 2000.0),
            (1, 512, "other_kernel", "SQ_INSTS_VALU", 1e9)]
    _counter_csv(str(tmp_path / "p" / "p_counter_collection.csv"), rows)
    text = ps.sq_summary([str(tmp_path / "p")], "mlp_dual_kernel", "cmd", 2)
    assert "8 waves per dispatch, 4000 cycles each" in text
    assert "VALU instructions: 200 (100 per mini-batch)" in text
    assert "SQ_ACTIVE_INST_VALU: 25.0% of the wave's cycles" in text
