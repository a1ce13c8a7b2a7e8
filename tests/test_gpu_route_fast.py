"""moe_route without the logits output on bf16 inputs from 512 tokens on: the selection is
made from bf16 matrix-core dot products with a proven error bound and kept only where the
bound separates the chosen experts from the rest; every other token is routed by the exact
fp64 kernels. (Below 512 tokens the exact kernels route every token.)
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
    # ragged token and expert counts (T not a multiple of the 32-token tiles, E not of 64)
    MoEConfig("fast_sigmoid_bias", T=777, H=192, E=100, k=6, I=64, score="sigmoid",
              use_bias=True, scale=2.5, seed=141, weight_seed=141),
    MoEConfig("fast_softmax", T=600, H=512, E=64, k=8, I=64, score="softmax", seed=142,
              weight_seed=142),
    MoEConfig("fast_softmax_bias_e1000", T=520, H=64, E=1000, k=16, I=64, score="softmax",
              use_bias=True, seed=143, weight_seed=143),
    # below 512 tokens: the exact kernels alone
    MoEConfig("exact_single_token", T=1, H=128, E=3, k=1, I=64, score="sigmoid", seed=144,
              weight_seed=144),
    # router weights of 1e-12: every sigmoid score rounds to 0.5 in fp32, all keys tie, every
    # token is listed for the exact kernels (and takes the lowest k ids)
    MoEConfig("fast_all_ties", T=700, H=256, E=48, k=4, I=64, score="sigmoid",
              use_bias=False, w_std=1e-12, seed=145, weight_seed=145),
    # router weights 1000x smaller than usual: keys a few fp32 ulps apart, a mix of tokens
    # on both paths
    MoEConfig("fast_near_ties_softmax", T=640, H=320, E=70, k=3, I=64, score="softmax",
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
    second with fewer tokens, both on the certified router."""
    cfg = SMALL[0]
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    ws = moe.workspace(moe.lib().moe_route_workspace_size(cfg.T, cfg.H, cfg.E))
    want = _oracle_route(cfg, host)
    for T in (cfg.T, 530):
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        moe.moe_route(dev.x[:T], dev.wr, dev.bias, cfg.k, cfg.score, cfg.scale, idx, w, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), want["topk_idx"][:T])
        np.testing.assert_allclose(w.cpu().numpy(), want["topk_w"][:T], rtol=1e-6, atol=0)


def test_layer_with_fast_route_graph_replays():
    """The layer at 600 tokens (the certified router, its token list and count in the
    workspace) captured into a HIP graph and replayed on new activations, with eager calls
    on the same workspace in between: every replay equals the eager result bit for bit."""
    from moe_cases import make_layer
    cfg = MoEConfig("fast_graph", T=600, H=256, E=32, k=4, I=128, score="sigmoid",
                    use_bias=True, scale=2.5, shared_I=128, seed=147, weight_seed=147)
    print("case", describe(cfg), flush=True)
    dev = device_problem(cfg, host=host_problem(cfg))
    layer = make_layer(cfg, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(148)
    xs = [torch.randn(dev.x.shape, device="cuda", generator=g).to(torch.bfloat16)
          for _ in range(3)]
    x_static = dev.x.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        layer.forward(x_static, out, stream=cap)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        layer.forward(x_static, out, stream=cap)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for i, x in enumerate(xs):
        want = torch.empty_like(out)
        layer.forward(x, want)                  # eager, between replays
        x_static.copy_(x)
        graph.replay()
        layer.forward(dev.x, other)             # more eager work on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), i


BF16_NAN = np.uint16(0x7FC0)


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_fast_route_exact_ties_and_nan_token(score):
    """On the certified router: router rows 3, 7 and 12 identical (with equal bias) so their
    keys tie exactly, and token 5 all NaN. Tied tokens and the NaN token are listed for the
    exact kernels: ties go to the lower id, the NaN token takes ids 0..k-1 with NaN
    weights; every other token matches the oracle."""
    cfg = MoEConfig("fast_ties_nan", T=600, H=256, E=16, k=2, I=64, score=score,
                    use_bias=True, scale=1.0, seed=149, weight_seed=149)
    host = host_problem(cfg)
    x, wr, bias = host.x.copy(), host.wr.copy(), host.bias.copy()
    wr[7] = wr[3]
    wr[12] = wr[3]
    bias[7] = bias[3] = bias[12] = bias[3] + 1.0
    x[5, :] = BF16_NAN
    T, k = cfg.T, cfg.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(_bf16_dev(x), _bf16_dev(wr), torch.from_numpy(bias).cuda(), k, score, cfg.scale,
                  idx, w)
    torch.cuda.synchronize()
    want = O.route(O.bf16_to_f64(x), O.bf16_to_f64(wr), bias, k, score, cfg.scale)
    got_idx, got_w = idx.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(got_idx, want["topk_idx"])
    assert got_idx[5].tolist() == [0, 1] and np.isnan(got_w[5]).all()
    ok = np.arange(T) != 5
    np.testing.assert_allclose(got_w[ok], want["topk_w"][ok], rtol=1e-6, atol=0)
    chosen = set(got_idx[ok].ravel().tolist())
    assert 3 in chosen and 12 not in chosen


def _route_listed(x, wr, bias, k, score, scale):
    """moe_route on a workspace of its own; returns ids, weights and the number of tokens
    handed to the exact kernels (the int32 count that closes the route workspace)."""
    T, H = x.shape
    E = wr.shape[0]
    ws = moe.workspace(moe.lib().moe_route_workspace_size(T, H, E))
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(x, wr, bias, k, score, scale, idx, w, ws=ws)
    torch.cuda.synchronize()
    listed = ws[ws.numel() - 256: ws.numel() - 252].view(torch.int32).item()
    return idx.cpu().numpy(), w.cpu().numpy(), listed


@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_fast_route_refines_grouped_ties(score):
    """Router rows in groups of four identical rows (with equal bias inside a group): the
    k-th key of most tokens falls inside a group of exactly tied keys, which no bound can
    separate. The wavefront refines them from exact logits of the few candidates: with
    sigmoid the exact keys settle every token (ties to the lower id), so none reaches the
    exact kernels; with softmax the exact ties are left to the exact kernels. Ids equal the
    oracle's either way."""
    cfg = MoEConfig("fast_grouped_ties", T=640, H=256, E=64, k=6, I=64, score=score,
                    use_bias=score == "sigmoid", scale=1.0, seed=150, weight_seed=150)
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    x, wr = host.x, host.wr.copy()
    for g in range(0, cfg.E, 4):
        wr[g + 1: g + 4] = wr[g]
    bias = None
    if cfg.use_bias:
        bias = host.bias.copy()
        for g in range(0, cfg.E, 4):
            bias[g + 1: g + 4] = bias[g]
    got_idx, got_w, listed = _route_listed(
        _bf16_dev(x), _bf16_dev(wr), None if bias is None else torch.from_numpy(bias).cuda(),
        cfg.k, score, cfg.scale)
    want = O.route(O.bf16_to_f64(x), O.bf16_to_f64(wr), bias, cfg.k, score, cfg.scale)
    assert np.array_equal(got_idx, want["topk_idx"])
    np.testing.assert_allclose(got_w, want["topk_w"], rtol=1e-6, atol=0)
    if score == "sigmoid":
        assert listed == 0, listed
    else:
        assert 0 < listed <= cfg.T, listed


@pytest.mark.parametrize("name", ["r1_prefill", "e384_fp8"])
def test_fast_route_refinement_at_size(name):
    """At full size the bounds leave a few hundred tokens undecided (362 of e384_fp8's 4096,
    302 of r1_prefill's 8192 before refinement); the refinement settles all of them on
    these inputs, with ids equal to the oracle's (checked by the full-size test above)."""
    cfg = CONFIGS[name]
    dev = device_problem(cfg, host=host_problem(cfg))
    _, _, listed = _route_listed(dev.x, dev.wr, dev.bias, cfg.k, cfg.score, cfg.scale)
    assert listed <= 4, listed
