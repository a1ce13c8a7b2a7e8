"""W8A8 (MOE_INT8) on the INT8 matrix units against the oracle, through the C ABI: the INT8
activation quantiser bit-exact, the seeded INT8 weight banks byte-identical on host and
device, small layers (routing bit-exact, outputs within the low-precision tolerance) and
the R1-shaped decode and prefill layers at their real sizes."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
import synth
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import (TILE_ROWS, TOL, cover_tokens, describe, oracle_layer, problems,
                       run_layer, with_device_banks)

pytestmark = pytest.mark.gpu


def test_quantize_int8_matches_oracle_bit_exact():
    """moe_quantize_int8: INT8 codes and fp32 scales equal the oracle's, decided in fp32 on
    both sides from the same bf16 input (zero, tie-laden, tiny and wide-range blocks)."""
    rng = np.random.default_rng(141)
    n, H = 37, 640
    v = rng.normal(0, 1, (n, H)) * 10.0 ** rng.uniform(-6, 3, (n, 1))
    v[3, :128] = 0.0
    v[4, 128:256] *= 1e-30
    v[5, :128] = np.round(rng.uniform(-100, 100, 128)) + 0.5
    v[5, 0] = 127.0          # scale 1: every other element of the block is a tie
    xb = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    q = torch.empty((n, H), dtype=torch.int8, device="cuda")
    qs = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
    moe.moe_quantize_int8(xb.cuda(), q, qs)
    torch.cuda.synchronize()
    codes, scales, _ = O.quantise_rows_int8(O.bf16_to_f64(bits).astype(np.float32))
    assert np.array_equal(qs.cpu().numpy(), scales)
    assert np.array_equal(q.cpu().numpy(), codes)


def test_int8_bank_device_matches_host():
    c_dev, s_dev = synth.dev_int8_bank(3, 4, 3, 256, 384, 0.02)
    c, s = synth.int8_bank(3, 4, 0, 3, 256, 384, 0.02)
    assert np.array_equal(c_dev.cpu().numpy(), c) and np.array_equal(s_dev.cpu().numpy(), s)


W8A8_SMALL = [
    MoEConfig("int8_sigmoid_bias_shared", T=100, H=256, E=8, k=2, I=256, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, wdt="int8", seed=151, weight_seed=151),
    MoEConfig("int8_softmax_ragged_f32out", T=333, H=384, E=5, k=3, I=128, score="softmax",
              shared_I=256, wdt="int8", out="f32", seed=152, weight_seed=152),
    MoEConfig("int8_decode_like", T=24, H=512, E=32, k=4, I=256, score="sigmoid", use_bias=True,
              scale=2.5, shared_I=256, wdt="int8", seed=153, weight_seed=153),
    MoEConfig("int8_single_token", T=1, H=128, E=4, k=2, I=128, score="softmax", wdt="int8",
              seed=154, weight_seed=154),
]


@pytest.mark.parametrize("cfg", W8A8_SMALL, ids=lambda c: c.name)
def test_w8a8_layer_matches_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_layer(cfg, dev)
    want = O.layer_forward(host)
    assert np.array_equal(got["topk_idx"], want["topk_idx"])
    assert np.array_equal(got["counts"], want["counts"])
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err", err, flush=True)
    assert err <= TOL["int8"], (describe(cfg), err)


def test_r1_decode_int8_full_size():
    """The R1-shaped decode layer with W8A8 experts at its real size: routing of all 128 tokens
    bit-exact (the bf16 layer's), the outputs of all tokens against the oracle."""
    cfg = CONFIGS["r1_decode_int8"]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    want = oracle_layer(with_device_banks(host, dev))   # before the library runs
    got = run_layer(cfg, dev, with_logits=False)
    assert np.array_equal(got["topk_idx"], want["topk_idx"])
    assert np.array_equal(got["counts"], want["counts"])
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err (all tokens)", err, flush=True)
    assert err <= TOL["int8"]


def test_r1_prefill_int8_full_size():
    """The skewed R1-shaped prefill layer with W8A8 experts at its real size: routing of all
    8192 tokens bit-exact; the tokens that cover every touched expert and the first and last
    rows of every expert's (and the shared group's) last tile against the oracle."""
    cfg = CONFIGS["r1_prefill_int8"]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    route = O.route(O.decode_act(cfg.act, host.x), O.decode_act(cfg.act, host.wr), host.bias,
                    cfg.k, cfg.score, cfg.scale)
    tokens = cover_tokens(route["topk_idx"], cfg.E, TILE_ROWS[cfg.name], True)
    want = oracle_layer(with_device_banks(host, dev), tokens=tokens)
    got = run_layer(cfg, dev, with_logits=False)
    assert np.array_equal(got["topk_idx"], want["topk_idx"])
    err = O.rel_err(got["out"][tokens], want["out"])
    print(cfg.name, "sampled rel err", len(tokens), "tokens", err, flush=True)
    assert err <= TOL["int8"]
    assert np.isfinite(got["out"]).all()
