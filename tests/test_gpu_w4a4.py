"""W4A4 (MOE_MXFP4_A4): the MXFP4 activation quantiser bit-exact against the oracle's, and
layers and pre-routed rows whose expert GEMMs run on the FP4 scaled matrix instruction,
against the oracle with the same quantisation of activations and of h."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import TOL, describe, problems, run_layer, run_rows

pytestmark = pytest.mark.gpu


def _bf16_bits(a32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quantize_mxfp4_bit_exact():
    rng = np.random.default_rng(101)
    n, H = 64, 512
    v = rng.standard_normal((n, H)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (n, 1)))
    v[0, :32] = 0.0                                        # an all-zero block
    v[1, :32] = [3.0, -1.5, 0.75, 0.25, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0] + [0.0] * 22  # ties
    v[2, :32] = 7.9                                        # saturation above 6
    v[3, :32] = np.float32(2.0 ** -130)                    # amax below 2^-125
    v[4, 32:64] = -0.0
    bits = _bf16_bits(v)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q = torch.empty((n, H // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((n, H // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp4(x, q, qs)
    torch.cuda.synchronize()
    codes, scales, _ = O.quantise_rows_mxfp4(O.bf16_to_f64(bits).astype(np.float32))
    want = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(q.cpu().numpy(), want)
    assert np.array_equal(qs.cpu().numpy(), scales)


A4_LAYERS = [
    MoEConfig("w4a4_routed_shared", T=300, H=256, E=8, k=2, I=128, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, wdt="mxfp4a4", seed=102, weight_seed=102),
    MoEConfig("w4a4_softmax_f32out_k4", T=160, H=384, E=12, k=4, I=256, score="softmax",
              out="f32", wdt="mxfp4a4", seed=103, weight_seed=103),
    MoEConfig("w4a4_single_token", T=1, H=128, E=4, k=2, I=128, score="softmax", shared_I=256,
              wdt="mxfp4a4", seed=104, weight_seed=104),
]


@pytest.mark.parametrize("cfg", A4_LAYERS, ids=lambda c: c.name)
def test_w4a4_layer_matches_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_layer(cfg, dev)
    want = O.layer_forward(host)
    assert np.array_equal(got["topk_idx"], want["topk_idx"])
    assert np.array_equal(got["counts"], want["counts"])
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err", err, flush=True)
    assert err <= TOL["mxfp4"]


A4_ROWS = [
    MoEConfig("w4a4_rows_ragged", T=1500, H=512, E=5, k=1, I=256, score="none", act="bf16",
              wdt="mxfp4a4", out="bf16", seed=105, weight_seed=105, dirichlet_alpha=0.5),
    MoEConfig("w4a4_rows_f32out", T=257, H=384, E=9, k=1, I=384, score="none", act="bf16",
              wdt="mxfp4a4", out="f32", seed=106, weight_seed=106, dirichlet_alpha=0.5),
]


@pytest.mark.parametrize("cfg", A4_ROWS, ids=lambda c: c.name)
def test_w4a4_rows_match_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_rows(cfg, dev)
    want = O.layer_forward(host)
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err", err, flush=True)
    assert err <= TOL["mxfp4"]


def test_ep32_w4a4_full_size():
    """ep32_w4a4 at its real size: the rows covering every expert and the first and last
    rows of every expert's last tile against the oracle, all rows finite."""
    from moe_cases import TILE_ROWS, cover_tokens, oracle_layer, with_device_banks

    cfg = CONFIGS["ep32_w4a4"]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    rows = cover_tokens(host.topk_idx, cfg.E, TILE_ROWS[cfg.name], False)
    want = oracle_layer(with_device_banks(host, dev), tokens=rows)   # before the library runs
    got = run_rows(cfg, dev)
    err = O.rel_err(got["out"][rows], want["out"])
    print("ep32_w4a4 sampled rel err", len(rows), "rows", err, flush=True)
    assert err <= TOL["mxfp4"]
    assert np.isfinite(got["out"]).all()
