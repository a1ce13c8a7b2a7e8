"""moe_layer_forward_overlap (shared expert on a side stream, forked and joined by events)
against the oracle, and against moe_layer_forward: the same kernels on the same rows, so every
output is bit-identical; and the pair of streams captured into a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import TOL, describe, make_layer

pytestmark = pytest.mark.gpu

CASES = [
    # streaming kernels (few rows per expert), shared expert with its own I
    MoEConfig("ovl_bf16_stream", T=24, H=256, E=16, k=4, I=128, score="sigmoid", use_bias=True,
              scale=2.5, shared_I=256, seed=91, weight_seed=91),
    # LDS-tiled kernels, ragged tiles, f32 output
    MoEConfig("ovl_bf16_tiled", T=600, H=256, E=6, k=2, I=128, score="softmax", shared_I=128,
              out="f32", seed=92, weight_seed=92),
    MoEConfig("ovl_fp8", T=200, H=256, E=8, k=2, I=256, score="softmax", shared_I=128,
              wdt="fp8", seed=93, weight_seed=93),
    MoEConfig("ovl_mxfp4_stream", T=40, H=1024, E=16, k=3, I=512, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=512, wdt="mxfp4", seed=94, weight_seed=94),
    MoEConfig("ovl_no_shared", T=100, H=256, E=8, k=2, I=128, score="softmax", seed=95,
              weight_seed=95),
]


def _outputs(cfg, layer, dev, fj=None):
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    dt = torch.float32 if cfg.out == "f32" else torch.bfloat16
    out = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    if fj is None:
        layer.forward(dev.x, out, idx, w, counts)
    else:
        layer.forward_overlap(dev.x, out, fj, idx, w, counts)
    torch.cuda.synchronize()
    return [t.cpu() for t in (out, idx, w, counts)]


def _same(a, b):
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and x.shape == y.shape
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_overlap_equals_plain_forward(cfg):
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    layer = make_layer(cfg, dev)
    fj = moe.ForkJoin()
    plain = _outputs(cfg, layer, dev)
    for _ in range(2):  # twice: the second call reuses the workspace and the events
        ovl = _outputs(cfg, layer, dev, fj)
        _same(ovl, plain)
    # and against the oracle: routing bit-exact, output within the format's tolerance
    want = O.layer_forward(host)
    assert np.array_equal(ovl[1].numpy(), want["topk_idx"])
    assert np.array_equal(ovl[3].numpy(), want["counts"])
    err = O.rel_err(ovl[0].float().numpy().astype(np.float64), want["out"])
    print(cfg.name, "overlap rel err", err, flush=True)
    assert err <= TOL[cfg.wdt]


def test_overlap_equals_plain_forward_r1_decode():
    cfg = CONFIGS["r1_decode"]
    print("case", describe(cfg), flush=True)
    dev = device_problem(cfg, host=host_problem(cfg))
    layer = make_layer(cfg, dev)
    _same(_outputs(cfg, layer, dev, moe.ForkJoin()), _outputs(cfg, layer, dev))


def test_overlap_graph_replays():
    """Capture the overlapped forward (two streams) into a graph; replay it three times on
    new activations, with eager library calls in between, and check every replay against the
    eager result for the same activations."""
    cfg = CASES[0]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    layer = make_layer(cfg, dev)
    fj = moe.ForkJoin()
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    xs = [dev.x.clone()]
    g = torch.Generator(device="cuda").manual_seed(96)
    for _ in range(3):
        xs.append(torch.randn(dev.x.shape, device="cuda", generator=g).to(torch.bfloat16))
    x_static = xs[0].clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        layer.forward_overlap(x_static, out, fj)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        layer.forward_overlap(x_static, out, fj, stream=cap)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for i, x in enumerate(xs[1:]):
        want = torch.empty_like(out)
        layer.forward(x, want)                  # eager, between replays
        x_static.copy_(x)
        graph.replay()
        layer.forward(xs[0], other)             # more eager work on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), i
