"""The measurement probes on the GPU: they run, and the rates they give lie between sane
bounds for an MI355X (datasheet: 8 TB/s HBM; dense bf16 2.5, fp8 and INT8 5.0, FP4 10.1
PFLOP/s at 2.4 GHz), i.e. each is a measured ceiling below its datasheet figure."""
import pytest
import torch

import mixture_experts_layer_04_amd as moe

pytestmark = pytest.mark.gpu

DATASHEET_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "int8": 5000.0, "mxfp4a4": 10100.0}


def _time_s(fn):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3


def test_probe_hbm_read_rate():
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    gbs = buf.numel() / _time_s(lambda: moe.moe_probe_hbm_read(buf, sink)) / 1e9
    print("hbm read GB/s", gbs, flush=True)
    assert 1000.0 < gbs < 8000.0
    assert int(sink[0]) == 0            # all-zero data never hits the sink's mark


@pytest.mark.parametrize("dt", sorted(DATASHEET_TFLOPS))
def test_probe_mfma_rate(dt):
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    iters = 2000
    flops = moe.moe_probe_mfma(dt, iters, sink)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    per = {"bf16": 16384, "fp8": 65536, "int8": 32768, "mxfp4a4": 65536}[dt]
    assert flops == n_cu * 16 * iters * 8 * per
    tf = flops / _time_s(lambda: moe.moe_probe_mfma(dt, iters, sink)) / 1e12
    print(dt, "dense MFMA TFLOP/s", tf, flush=True)
    assert 0.1 * DATASHEET_TFLOPS[dt] < tf < 1.01 * DATASHEET_TFLOPS[dt]
