"""moe_bias_update (auxiliary-loss-free balancing of the selection bias) on the GPU against
the oracle: bit-exact on its own, and bit-exact over a closed loop in which each batch's
routed counts update the bias the next batch is routed with."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
from synth.configs import MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import TOL, describe, run_layer

pytestmark = pytest.mark.gpu


def _counts_around_mean(rng, E, m):
    """Loads paired around an integer mean m (so some sit exactly on it), shuffled."""
    d = rng.integers(0, m + 1, E // 2)
    d[: max(1, E // 8)] = 0
    c = np.concatenate([m + d, m - d, [m] * (E % 2)]).astype(np.int32)
    return rng.permutation(c)


@pytest.mark.parametrize("E", [1, 7, 64, 100, 257, 1000, 1024])
def test_bias_update_bit_exact(E):
    rng = np.random.default_rng(80 + E)
    print("case bias_update E", E, flush=True)
    cases = [
        (_counts_around_mean(rng, E, 37), 0.001),
        (rng.integers(0, 5000, E).astype(np.int32), 2.0 ** -10),
        (np.where(rng.random(E) < 0.5, 0, rng.integers(0, 9, E)).astype(np.int32), -0.25),
        (np.zeros(E, np.int32), 0.5),
        (rng.integers(0, 200, E).astype(np.int32), 0.0),
    ]
    bias0 = rng.standard_normal(E).astype(np.float32)
    special = np.array([0.0, -0.0, 1e30, -1e-30, 3.0, 2.0 ** -24], np.float32)
    bias0[: min(E, special.size)] = special[: min(E, special.size)]
    for counts, u in cases:
        dcounts = torch.from_numpy(counts).cuda()
        dbias = torch.from_numpy(bias0.copy()).cuda()
        moe.moe_bias_update(dcounts, u, dbias)
        torch.cuda.synchronize()
        want = O.bias_update(bias0, counts, u)
        got = dbias.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (E, u)


def test_bias_update_large_counts_exact_sign():
    """Loads near 2^21 each over 1000 experts, one of them a single token above the rest:
    the mean is not an integer and only that expert is above it."""
    E = 1000
    counts = np.full(E, 2_000_000, np.int32)
    counts[417] += 1
    dbias = torch.zeros(E, dtype=torch.float32, device="cuda")
    moe.moe_bias_update(torch.from_numpy(counts).cuda(), 1.0, dbias)
    torch.cuda.synchronize()
    want = O.bias_update(np.zeros(E, np.float32), counts, 1.0)
    assert np.array_equal(dbias.cpu().numpy(), want)
    assert want[417] == -1.0 and (np.delete(want, 417) == 1.0).all()


def test_balancing_loop_through_the_layer():
    """Eight batches: moe_layer_forward routes with the current bias and returns the counts,
    moe_bias_update moves the bias from them. At every step the routing, the counts and the
    updated bias are bit-identical to the oracle's, the (fp32) output is within the bf16
    tolerance, and the load skew that a tilted starting bias causes shrinks."""
    cfg = MoEConfig("bf16_balance_loop", T=512, H=128, E=32, k=4, I=64, score="sigmoid",
                    use_bias=True, scale=2.5, shared_I=64, out="f32", seed=72, weight_seed=72)
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    host.bias = np.linspace(0.0, 0.12, cfg.E).astype(np.float32)     # favours high ids
    dev = device_problem(cfg, host=host)
    dev.bias.copy_(torch.from_numpy(host.bias))
    u = 0.01
    ratios = []
    for step in range(8):
        got = run_layer(cfg, dev, with_logits=False)
        want = O.layer_forward(host)
        assert np.array_equal(got["topk_idx"], want["topk_idx"]), step
        counts = O.permutation(want["topk_idx"], cfg.E)[0]
        assert np.array_equal(got["counts"], counts), step
        assert O.rel_err(got["out"], want["out"]) <= TOL["bf16"], step
        ratios.append(counts.max() / counts.mean())
        moe.moe_bias_update(torch.from_numpy(got["counts"]).cuda(), u, dev.bias)
        host.bias = O.bias_update(host.bias, counts, u)
        torch.cuda.synchronize()
        assert np.array_equal(dev.bias.cpu().numpy().view(np.uint32),
                              host.bias.view(np.uint32)), step
    print("max/mean load per step", [round(r, 3) for r in ratios], flush=True)
    assert ratios[-1] < ratios[0]
