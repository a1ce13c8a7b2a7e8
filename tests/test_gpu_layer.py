"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Bit-exact: expert ids, counts, offsets and the permutation maps. Floating point: router
logits (fp64 sums rounded once on both sides; at most 1 ulp on a handful of entries; the
full-size layers run without the logits output, as a caller would, which routes through
the certified bf16 router),
routing weights (1e-6 relative), layer outputs (max |err| / RMS of the oracle output:
1e-4 fp32, 2e-2 bf16).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
import synth
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import (TILE_ROWS, TOL, cover_tokens, describe, experts, make_layer, oracle_layer,
                       problems, run_layer, run_rows, with_device_banks)

pytestmark = pytest.mark.gpu

SMALL = [
    CONFIGS["tiny_fp32"],
    MoEConfig("bf16_sigmoid_bias_shared", T=77, H=256, E=24, k=4, I=192, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, seed=11, weight_seed=11),
    MoEConfig("bf16_softmax_ragged", T=300, H=512, E=16, k=8, I=256, score="softmax", seed=12,
              weight_seed=12),
    MoEConfig("f32_k_equals_e_shared", T=33, H=192, E=5, k=5, I=64, score="sigmoid", use_bias=True,
              shared_I=64, act="f32", wdt="f32", out="f32", seed=13, weight_seed=13),
    MoEConfig("bf16_single_token", T=1, H=128, E=8, k=3, I=64, score="softmax", shared_I=64,
              seed=14, weight_seed=14),
    MoEConfig("bf16_one_expert", T=40, H=128, E=1, k=1, I=128, score="softmax", seed=15,
              weight_seed=15),
    MoEConfig("bf16_f32_out_k16", T=70, H=256, E=40, k=16, I=128, score="sigmoid", use_bias=True,
              scale=2.5, out="f32", seed=16, weight_seed=16),
    # more than 32 rows per expert: the LDS-tiled grouped GEMMs with ragged 128-row tiles
    MoEConfig("bf16_t3_sigmoid_shared", T=900, H=512, E=10, k=3, I=256, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, seed=19, weight_seed=19),
    MoEConfig("bf16_t3_softmax_f32out", T=1200, H=768, E=5, k=2, I=384, score="softmax",
              out="f32", seed=20, weight_seed=20),
    MoEConfig("bf16_tiled_sigmoid_shared", T=600, H=256, E=12, k=3, I=192, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, seed=17, weight_seed=17),
    MoEConfig("bf16_tiled_softmax_f32out", T=1000, H=384, E=6, k=2, I=128, score="softmax",
              out="f32", seed=18, weight_seed=18),
    # decode-sized groups with I a multiple of 512: the down projection stages h in LDS
    # (ragged 16-row tiles: the shared expert's 37 rows)
    MoEConfig("bf16_stream_lds_shared", T=37, H=320, E=12, k=3, I=1024, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=512, seed=22, weight_seed=22),
    MoEConfig("bf16_stream_lds_f32out", T=6, H=192, E=5, k=2, I=512, score="softmax",
              out="f32", seed=23, weight_seed=23),
    # H or I a multiple of 8 but not of 64: the plain dot-product kernels (h kept in fp32)
    MoEConfig("bf16_h200_i136_shared72", T=90, H=200, E=12, k=4, I=136, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=72, seed=24, weight_seed=24),
    MoEConfig("f32_h136_i200", T=50, H=136, E=6, k=2, I=200, score="softmax", act="f32",
              wdt="f32", out="f32", seed=25, weight_seed=25),
    # a group of more tiles than one tile block (the shared expert's 2100 rows: nine tiles)
    MoEConfig("bf16_tile_blocks", T=2100, H=512, E=3, k=1, I=128, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, out="f32", seed=21, weight_seed=21),
]


def check_routing(got, want, cfg):
    assert np.array_equal(got["topk_idx"], want["topk_idx"]), describe(cfg)
    assert np.array_equal(got["counts"], want["counts"]), describe(cfg)
    if "logits" in got:
        a = got["logits"].view(np.int32).astype(np.int64)
        b = want["logits"].view(np.int32).astype(np.int64)
        ulps = np.abs(a - b)
        assert ulps.max() <= 1 and (ulps > 0).sum() <= max(2, ulps.size // 100000), describe(cfg)
    np.testing.assert_allclose(got["topk_w"], want["topk_w"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_matches_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_layer(cfg, dev)
    want = O.layer_forward(host)
    check_routing(got, want, cfg)
    err = O.rel_err(got["out"], want["out"])
    assert err <= TOL[cfg.wdt], (describe(cfg), err)


def test_layer_deterministic():
    cfg = SMALL[1]
    _, dev = problems(cfg)
    layer = make_layer(cfg, dev)
    a = run_layer(cfg, dev, layer)
    b = run_layer(cfg, dev, layer)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_empty_batch():
    cfg = SMALL[1].with_(T=0)
    dev = device_problem(cfg)
    layer = make_layer(cfg, dev)
    out = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    counts = torch.full((cfg.E,), -1, dtype=torch.int32, device="cuda")
    layer.forward(dev.x, out, counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().tolist() == [0] * cfg.E


def test_standalone_entry_points():
    """moe_route, moe_permute, moe_grouped_ffn and moe_combine one by one, composed as
    moe_layer_forward composes them: the expert rows stay fp32 until the combine rounds once
    (rows rounded to bf16 and then combined into a bf16 output are rounded twice; that is
    covered row by row in test_gpu_parity_more)."""
    cfg = SMALL[1]
    host, dev = problems(cfg)
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    want = O.layer_forward(host)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_route(dev.x, dev.wr, dev.bias, k, cfg.score, cfg.scale, idx, w, logits)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm_src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv_perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    x_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_permute(idx, E, counts, offsets, perm_src, inv_perm, dev.x, x_perm)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(experts(dev.routed), x_perm, offsets, y_perm)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(y_perm, inv_perm, w, out)
    torch.cuda.synchronize()
    check_routing({"topk_idx": idx.cpu().numpy(), "counts": counts.cpu().numpy(),
                   "logits": logits.cpu().numpy(), "topk_w": w.cpu().numpy()}, want, cfg)
    assert np.array_equal(offsets.cpu().numpy(), want["offsets"])
    assert np.array_equal(perm_src.cpu().numpy(), want["perm_src"])
    assert np.array_equal(inv_perm.cpu().numpy(), want["inv_perm"])
    xp = x_perm.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xp, host.x[want["perm_src"] // k])
    # grouped FFN rows against the oracle's expert FFN, row by row
    x64 = O.bf16_to_f64(host.x)
    y64 = np.zeros((T * k, H))
    for e in range(E):
        r0, r1 = want["offsets"][e], want["offsets"][e + 1]
        if r1 > r0:
            w13, w2 = O.expert_weights(host.routed, e)
            y64[r0:r1] = O.expert_ffn(x64[want["perm_src"][r0:r1] // k], w13, w2)
    yg = y_perm.float().cpu().numpy().astype(np.float64)
    assert O.rel_err(yg, y64) <= TOL["bf16"]
    # combine of the routed part only
    routed = O.combine(y64, want["inv_perm"], want["topk_w"])
    assert O.rel_err(out.float().cpu().numpy(), routed) <= TOL["bf16"]


def test_device_generator_matches_host():
    w_dev = synth.dev_words(99, 5, 0, 4097).cpu().numpy().view(np.uint32)
    assert np.array_equal(w_dev, synth.words(99, 5, 0, 4097))
    b_dev = synth.dev_normal(7, 4, (3, 2, 1000), 0.02, "bf16").view(torch.int16).cpu().numpy()
    assert np.array_equal(b_dev.view(np.uint16), synth.normal_bf16(7, 4, (3, 2, 1000), 0.02))
    f_dev = synth.dev_normal(7, 1, (5, 999), 1.0, "f32").cpu().numpy()
    assert np.array_equal(f_dev.view(np.uint32), synth.normal_f32(7, 1, (5, 999), 1.0).view(np.uint32))
    c_dev, s_dev = synth.dev_fp8_bank(3, 4, 2, 256, 384, 0.02)
    c, s = synth.fp8_bank(3, 4, 0, 2, 256, 384, 0.02)
    assert np.array_equal(c_dev.cpu().numpy(), c) and np.array_equal(s_dev.cpu().numpy(), s)
    p_dev, q_dev = synth.dev_mxfp4_bank(3, 4, 2, 64, 256, 0.02)
    p, q = synth.mxfp4_bank(3, 4, 0, 2, 64, 256, 0.02)
    assert np.array_equal(p_dev.cpu().numpy(), p) and np.array_equal(q_dev.cpu().numpy(), q)


def test_r1_decode_full_size():
    """DeepSeek-R1-shaped decode layer at its real size: routing of all 128 tokens bit-exact,
    and the outputs of all 128 tokens (every touched expert, every ragged 16-row tile)
    against the oracle."""
    cfg = CONFIGS["r1_decode"]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    want = oracle_layer(with_device_banks(host, dev))   # before the library runs
    got = run_layer(cfg, dev, with_logits=False)
    check_routing(got, want, cfg)
    err = O.rel_err(got["out"], want["out"])
    print("r1_decode rel err (all tokens)", err, flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["r1_decode_fp8", "r1_decode_mxfp4"])
def test_r1_decode_low_precision_full_size(name):
    """r1_decode with fp8 or MXFP4 expert weights at its real size: the routing is the bf16
    layer's, bit-exact; the outputs of all tokens against the oracle's decode of the same
    weights."""
    cfg = CONFIGS[name]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    want = oracle_layer(with_device_banks(host, dev))   # before the library runs
    got = run_layer(cfg, dev, with_logits=False)
    check_routing(got, want, cfg)
    err = O.rel_err(got["out"], want["out"])
    print(name, "rel err (all tokens)", err, flush=True)
    assert err <= TOL[cfg.wdt]


def _full_size_sampled(name):
    """A routed workload at its real size: routing of every token bit-exact; the outputs of
    the tokens that cover every touched expert and the first and last rows of every
    expert's (and the shared group's) last tile against the oracle; all outputs finite."""
    cfg = CONFIGS[name]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    want_route = O.route(O.decode_act(cfg.act, host.x), O.decode_act(cfg.act, host.wr), host.bias,
                         cfg.k, cfg.score, cfg.scale)
    tokens = cover_tokens(want_route["topk_idx"], cfg.E, TILE_ROWS[name], cfg.shared_I > 0)
    print(name, "sampled tokens", len(tokens), flush=True)
    want = oracle_layer(with_device_banks(host, dev), tokens=tokens)   # before the library runs
    got = run_layer(cfg, dev, with_logits=False)
    check_routing(got, want, cfg)
    assert set(np.unique(want["topk_idx"][tokens])) == set(np.nonzero(want["counts"])[0])
    err = O.rel_err(got["out"][tokens], want["out"])
    print(name, "sampled rel err", err, flush=True)
    assert err <= TOL[cfg.wdt]
    assert np.isfinite(got["out"]).all()


def test_r1_prefill_full_size():
    """DeepSeek-R1-shaped prefill layer with Zipf-skewed routing at its real size."""
    _full_size_sampled("r1_prefill")


FP8_SMALL = [
    MoEConfig("fp8_softmax_shared", T=100, H=256, E=8, k=2, I=256, score="softmax", shared_I=128,
              act="bf16", wdt="fp8", out="bf16", seed=31, weight_seed=31),
    MoEConfig("fp8_sigmoid_bias_ragged", T=333, H=384, E=5, k=3, I=128, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=256, act="bf16", wdt="fp8", out="f32", seed=32,
              weight_seed=32),
    MoEConfig("fp8_single_token", T=1, H=128, E=4, k=2, I=128, score="softmax", act="bf16",
              wdt="fp8", out="bf16", seed=33, weight_seed=33),
]


def test_quantize_fp8_matches_oracle_bit_exact():
    """moe_quantize_fp8: E4M3 codes and fp32 scales equal the oracle's, decided in fp32 on both
    sides from the same bf16 input (zeros, subnormal-range and wide-range blocks included)."""
    rng = np.random.default_rng(40)
    n, H = 37, 640
    v = rng.normal(0, 1, (n, H)) * 10.0 ** rng.uniform(-6, 3, (n, 1))
    v[3, :128] = 0.0                       # all-zero block
    v[4, 128:256] *= 1e-30                 # far below the E4M3 range
    v[5, :] = rng.choice([-1.0, 1.0], H) * 2.0 ** rng.integers(-12, 12, H)
    xb = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    x = xb.cuda()
    q = torch.empty((n, H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
    moe.moe_quantize_fp8(x, q, qs)
    torch.cuda.synchronize()
    codes, scales, _ = O.quantise_rows_e4m3(O.bf16_to_f64(bits).astype(np.float32))
    assert np.array_equal(qs.cpu().numpy(), scales)
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("cfg", FP8_SMALL, ids=lambda c: c.name)
def test_fp8_layer_matches_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_layer(cfg, dev)
    want = O.layer_forward(host)
    check_routing(got, want, cfg)
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err", err, flush=True)
    assert err <= TOL["fp8"], (describe(cfg), err)


def test_e384_fp8_full_size():
    """384 routed experts, top-8 + shared, fp8 block-scaled weights and activations, T=4096,
    at its real size."""
    _full_size_sampled("e384_fp8")


MX_ROWS = [
    MoEConfig("mxfp4_rows_small", T=700, H=256, E=6, k=1, I=128, score="none", act="bf16",
              wdt="mxfp4", out="bf16", seed=51, weight_seed=51, dirichlet_alpha=0.5),
    MoEConfig("mxfp4_rows_f32out_ragged", T=257, H=384, E=9, k=1, I=384, score="none", act="bf16",
              wdt="mxfp4", out="f32", seed=52, weight_seed=52, dirichlet_alpha=0.5),
    MoEConfig("mxfp4_rows_dma_ragged", T=1500, H=512, E=5, k=1, I=256, score="none", act="bf16",
              wdt="mxfp4", out="f32", seed=54, weight_seed=54, dirichlet_alpha=0.5),
]


@pytest.mark.parametrize("cfg", MX_ROWS, ids=lambda c: c.name)
def test_mxfp4_rows_match_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_rows(cfg, dev)
    want = O.layer_forward(host)
    err = O.rel_err(got["out"], want["out"])
    print(cfg.name, "rel err", err, flush=True)
    assert err <= TOL["mxfp4"], (describe(cfg), err)


def test_rows_forward_timed_matches_untimed():
    """The timed pre-routed entry point runs the same kernels: identical output, and stage
    times that add up (no route stage)."""
    cfg = MX_ROWS[0]
    _, dev = problems(cfg)
    want = run_rows(cfg, dev)["out"]
    e = experts(dev.routed)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(moe.moe_rows_workspace_size(e, moe.DTYPES[cfg.act], cfg.T))
    ev = moe.StageEvents()
    moe.moe_rows_forward_timed(e, dev.x, dev.topk_idx.view(-1), dev.topk_w.view(-1), out, ws, ev)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)
    st = ev.elapsed_ms()
    # events [0] and [1] are recorded back to back: only the recording gap separates them
    assert st["route"] < 0.05 and all(v >= 0 for v in st.values()) and st["gate_up"] > 0


MX_ROUTED = [
    # many rows per expert: the tiled kernel
    MoEConfig("mxfp4_routed_shared", T=300, H=256, E=8, k=2, I=128, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=128, act="bf16", wdt="mxfp4", out="bf16",
              seed=53, weight_seed=53),
    # decode-like (at most 32 rows per expert, H and I multiples of 512): the streaming
    # kernels, with ragged 16-row tiles, an f32 output, and a shared expert
    MoEConfig("mxfp4_stream_shared", T=40, H=1024, E=16, k=3, I=512, score="sigmoid",
              use_bias=True, scale=2.5, shared_I=512, act="bf16", wdt="mxfp4", out="bf16",
              seed=54, weight_seed=54),
    MoEConfig("mxfp4_stream_f32out", T=9, H=512, E=6, k=2, I=1024, score="softmax",
              act="bf16", wdt="mxfp4", out="f32", seed=55, weight_seed=55),
]


@pytest.mark.parametrize("cfg", MX_ROUTED, ids=lambda c: c.name)
def test_mxfp4_routed_layer_matches_oracle(cfg):
    print("case", describe(cfg), flush=True)
    host, dev = problems(cfg)
    got = run_layer(cfg, dev)
    want = O.layer_forward(host)
    check_routing(got, want, cfg)
    assert O.rel_err(got["out"], want["out"]) <= TOL["mxfp4"]


@pytest.mark.parametrize("name", ["ep32_mxfp4"])
def test_ep32_full_size(name):
    """One GPU's expert-parallel share: 32 local MXFP4 experts, 16384 received rows with
    Dirichlet(0.5)-multinomial loads; the rows covering every expert and the first and last
    rows of every expert's last tile against the oracle, all rows finite."""
    cfg = CONFIGS[name]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    rows = cover_tokens(host.topk_idx, cfg.E, TILE_ROWS[name], False)
    print(name, "sampled rows", len(rows), flush=True)
    want = oracle_layer(with_device_banks(host, dev), tokens=rows)   # before the library runs
    got = run_rows(cfg, dev)
    err = O.rel_err(got["out"][rows], want["out"])
    print(name, "sampled rel err", err, flush=True)
    assert err <= TOL[cfg.wdt]
    assert np.isfinite(got["out"]).all()
