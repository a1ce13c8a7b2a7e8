"""moe_route without the logits output on bf16 inputs: the selection is made from bf16
matrix-core dot products with a proven error bound and kept only where the bound separates
the chosen experts from the rest; every other token is routed by the exact fp64 kernels.
Either way the expert ids must equal the oracle's bit for bit, and the weights (from exact
logits of the chosen experts) to 1e-6 relative, as with the logits output."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import describe

pytestmark = pytest.mark.gpu


def _route_dev(cfg, dev, with_logits):
    T, E, k = cfg.T, cfg.E, cfg.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    moe.moe_route(dev.x, dev.wr, dev.bias, k, cfg.score, cfg.scale, idx, w, logits)
    torch.cuda.synchronize()
    if with_logits:
        return idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    return idx.cpu().numpy(), w.cpu().numpy()


def _oracle_route(cfg, host):
    return O.route(O.bf16_to_f64(host.x), O.bf16_to_f64(host.wr), host.bias, cfg.k, cfg.score,
                   cfg.scale)


def _check(cfg, host, dev):
    idx, w = _route_dev(cfg, dev, with_logits=False)
    want = _oracle_route(cfg, host)
    bad = np.nonzero((idx != want["topk_idx"]).any(axis=1))[0]
    assert bad.size == 0, (describe(cfg), bad[:10])
    np.testing.assert_allclose(w, want["topk_w"], rtol=1e-6, atol=0)
    return idx, w


@pytest.mark.parametrize("name", ["r1_decode", "r1_prefill", "e384_fp8"])
def test_fast_route_full_size(name):
    """All tokens of the three routed workloads at their real sizes, against the oracle; and
    the exact path (the logits output requested) on the same inputs, its logits within one
    fp32 ulp of the oracle's on a handful of entries (fp64 sums in another order)."""
    cfg = CONFIGS[name]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    idx, w = _check(cfg, host, dev)
    idx_x, w_x, lg = _route_dev(cfg, dev, with_logits=True)
    assert np.array_equal(idx, idx_x)
    np.testing.assert_allclose(w, w_x, rtol=1e-6, atol=0)
    want = O.router_logits(O.bf16_to_f64(host.x), O.bf16_to_f64(host.wr))
    ulps = np.abs(lg.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1 and (ulps > 0).sum() <= max(2, ulps.size // 100000)


SMALL = [
    MoEConfig("fast_sigmoid_bias", T=77, H=192, E=100, k=6, I=64, score="sigmoid",
              use_bias=True, scale=2.5, seed=141, weight_seed=141),
    MoEConfig("fast_softmax", T=300, H=512, E=64, k=8, I=64, score="softmax", seed=142,
              weight_seed=142),
    MoEConfig("fast_softmax_bias_e1000", T=40, H=64, E=1000, k=16, I=64, score="softmax",
              use_bias=True, seed=143, weight_seed=143),
    MoEConfig("fast_single_token", T=1, H=128, E=3, k=1, I=64, score="sigmoid", seed=144,
              weight_seed=144),
    # router weights of 1e-12: every sigmoid score rounds to 0.5 in fp32, all keys tie, every
    # token takes the exact path (and the lowest k ids)
    MoEConfig("fast_all_ties", T=257, H=256, E=48, k=4, I=64, score="sigmoid",
              use_bias=False, w_std=1e-12, seed=145, weight_seed=145),
    # router weights 1000x smaller than usual: keys a few fp32 ulps apart, a mix of tokens
    # on both paths
    MoEConfig("fast_near_ties_softmax", T=200, H=320, E=70, k=3, I=64, score="softmax",
              use_bias=True, w_std=2e-5, seed=146, weight_seed=146),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_fast_route_small(cfg):
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    _check(cfg, host, dev)


def test_fast_route_repeated_calls_share_workspace():
    """Two calls on one workspace (the token list's count is reset by the first kernel), the
    second with fewer tokens."""
    cfg = SMALL[0]
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    ws = moe.workspace(moe.lib().moe_route_workspace_size(cfg.T, cfg.H, cfg.E))
    want = _oracle_route(cfg, host)
    for T in (cfg.T, 13):
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        moe.moe_route(dev.x[:T], dev.wr, dev.bias, cfg.k, cfg.score, cfg.scale, idx, w, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), want["topk_idx"][:T])
        np.testing.assert_allclose(w.cpu().numpy(), want["topk_w"][:T], rtol=1e-6, atol=0)
