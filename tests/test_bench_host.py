"""bench.py's host-side logic on the CPU: the one-GPU guard, the algorithmic byte and flop
counts its roofline divides by (written out again here from the layer's definition: each
touched expert's weights read once, each grouped row read and its output written once,
6 H I flops per row and expert), and the traffic record that is used only while the
kernel sources it was measured on are unchanged."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.configs import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_r1_decode_accounting():
    """r1_decode with 141 touched experts: bf16 weights of the touched experts and the
    shared expert, 1024 routed and 128 shared rows."""
    cfg = CONFIGS["r1_decode"]
    T, H, I, k = 128, 7168, 2048, 8
    acct = bench.ffn_accounting(cfg, 141)
    rows_r, rows = T * k, T * k + T
    w13 = (141 + 1) * 2 * I * H * 2
    gu_bytes = w13 + rows * H * 2 + rows * I * 2
    assert acct["gate_up"]["bytes"] == pytest.approx(gu_bytes, rel=1e-12)
    assert acct["gate_up"]["flops"] == pytest.approx(2.0 * rows * H * 2 * I, rel=1e-12)
    # down: W2 of the same experts, h read, fp32 expert outputs written
    w2 = (141 + 1) * I * H * 2
    assert acct["down"]["bytes"] == pytest.approx(w2 + rows * I * 2 + rows * H * 4, rel=1e-12)
    assert acct["down"]["flops"] == pytest.approx(2.0 * rows * I * H, rel=1e-12)
    assert acct["gate_up"]["bound"] == "hbm" and acct["gate_up"]["kernel"] == "k_gateup_stream"
    # 6 H I flops per (row, expert) over both launches
    total = acct["gate_up"]["flops"] + acct["down"]["flops"]
    assert total == pytest.approx(6.0 * H * I * rows, rel=1e-12)
    assert rows_r == 1024


def test_prefill_and_fp8_bounds_and_kernels():
    pre = bench.ffn_accounting(CONFIGS["r1_prefill"], 207)
    assert pre["gate_up"]["bound"] == "mfma" and pre["gate_up"]["kernel"] == "k_tiled2<gate/up>"
    f8 = bench.ffn_accounting(CONFIGS["e384_fp8"], 384)
    assert f8["gate_up"]["bound"] == "hbm" and f8["gate_up"]["kernel"] == "k_fp8<gate/up>"
    # fp8 weights: one byte a weight plus its share of a 128 x 128 fp32 scale
    H, I = 7168, 2048
    w13 = (384 + 1) * 2 * I * H * (1.0 + 4.0 / (128 * 128))
    assert f8["gate_up"]["bytes"] > w13
    mx = bench.ffn_accounting(CONFIGS["ep32_mxfp4"], 32)
    assert mx["gate_up"]["bound"] == "mfma" and mx["gate_up"]["kernel"].startswith("k_tiled2")


def test_generic_shapes_name_their_kernels():
    cfg = CONFIGS["r1_decode"].with_(H=200, I=136, shared_I=72)
    assert bench.ffn_accounting(cfg, 8)["gate_up"]["kernel"] == "k_gateup_generic"


def test_traffic_record_is_used_only_on_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    import hashlib

    rec = {"workload": "w", "traffic_bytes": 123.0, "sources": [str(src)],
           "source_sha256_16": hashlib.sha256(b"// kernel v1\n").hexdigest()[:16]}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w") == 123.0
    src.write_text("// kernel v2\n")                 # the kernel changed since the counters
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("absent") is None


def test_percentile():
    v = [1.0, 2.0, 3.0, 4.0, 5.0]
    assert bench.percentile(v, 50) == 3.0
    assert bench.percentile(v, 10) == pytest.approx(1.4)
