"""More parity of the HIP library against the oracle, through the C ABI:

  * moe_permute at the full sizes of the routed and pre-routed workloads (r1_prefill,
    e384_fp8, ep32_mxfp4), where T * E exceeds one scan chunk: counts, offsets, perm_src
    and inv_perm bit-exact against oracle.permutation, and every gathered row bit-exact;
  * moe_grouped_ffn on its own for every expert format and kernel family (streaming,
    LDS-staged streaming down, 128- and 256-row tiles, fp8, MXFP4 streaming and tiled, W4A4,
    fp32), each with fp32 and bf16 output rows, row by row against oracle.expert_ffn on the
    same (quantised) activations;
  * moe_grouped_ffn_prequant (fp8, INT8, W4A4) on the oracle's own codes and scales against
    oracle.expert_ffn, and on the library quantisers' codes bit-identical to
    moe_grouped_ffn on the bf16 rows.
The expert ids fed to moe_permute come from the oracle's routing (or the workload's
pre-routed ids), never from the library.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_04_amd as moe
import oracle as O
import synth
from synth import TID_X
from synth.configs import CONFIGS, MoEConfig
from synth.problem import device_problem, host_problem

from moe_cases import TOL, describe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["r1_prefill", "e384_fp8", "ep32_mxfp4"])
def test_permute_full_size(name):
    cfg = CONFIGS[name]
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    if cfg.routed:
        idx = O.route(O.decode_act(cfg.act, host.x), O.decode_act(cfg.act, host.wr), host.bias,
                      cfg.k, cfg.score, cfg.scale)["topk_idx"]
    else:
        idx = host.topk_idx
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    assert T * E > 65536  # more than one chunk of the permutation scan
    counts, offsets, perm_src, inv_perm = O.permutation(idx, E)
    x = synth.dev_normal(cfg.seed, TID_X, (T, H), cfg.x_std, cfg.act)
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    g_counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    g_offsets = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    g_src = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    g_inv = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    x_perm = torch.empty((T * k, H), dtype=x.dtype, device="cuda")
    moe.moe_permute(d_idx, E, g_counts, g_offsets, g_src, g_inv, x, x_perm)
    torch.cuda.synchronize()
    assert np.array_equal(g_counts.cpu().numpy(), counts)
    assert np.array_equal(g_offsets.cpu().numpy(), offsets)
    assert np.array_equal(g_src.cpu().numpy(), perm_src)
    assert np.array_equal(g_inv.cpu().numpy(), inv_perm)
    want_rows = torch.from_numpy(perm_src.astype(np.int64) // k).cuda()
    assert torch.equal(x_perm.view(torch.int16), x.view(torch.int16)[want_rows])


# (name, weight format, H, I, E, rows): shapes chosen to reach each kernel family
FFN_CASES = [
    ("bf16_stream", "bf16", 256, 192, 8, 60),            # <= 32 rows per expert
    ("bf16_stream_lds_down", "bf16", 320, 512, 5, 37),   # I % 512 == 0: h staged in LDS
    ("bf16_tiled128", "bf16", 384, 128, 4, 700),         # H % 256 != 0: 128-row tiles
    ("bf16_tiled256", "bf16", 512, 256, 3, 900),         # 256-row tiles
    ("f32_stream", "f32", 128, 64, 6, 50),
    ("fp8", "fp8", 256, 256, 5, 400),
    ("int8", "int8", 384, 256, 5, 400),
    ("mxfp4_stream", "mxfp4", 512, 512, 6, 40),          # H, I multiples of 512, few rows
    ("mxfp4_tiled", "mxfp4", 256, 128, 4, 600),
    ("w4a4", "mxfp4a4", 256, 128, 4, 500),
    ("bf16_generic", "bf16", 200, 136, 5, 300),          # H, I multiples of 8, not of 64
    ("f32_generic", "f32", 136, 200, 4, 120),
]


@pytest.mark.parametrize("y_dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", FFN_CASES, ids=lambda c: c[0])
def test_grouped_ffn_alone(case, y_dt):
    name, wdt, H, I, E, rows = case
    act = "f32" if wdt == "f32" else "bf16"
    cfg = MoEConfig(f"ffn_{name}", T=rows, H=H, E=E, k=1, I=I, score="none", act=act, wdt=wdt,
                    out=y_dt, seed=140 + len(name), weight_seed=140 + len(name),
                    dirichlet_alpha=0.7)
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    counts = np.bincount(host.topk_idx[:, 0], minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    # rows r0..r1 of x_perm belong to expert e: here, x's rows in order
    x64 = O.decode_act(act, host.x)
    if wdt == "fp8":
        a = O.quantise_rows_e4m3(x64.astype(np.float32))[2]
    elif wdt == "int8":
        a = O.quantise_rows_int8(x64.astype(np.float32))[2]
    elif wdt == "mxfp4a4":
        a = O.quantise_rows_mxfp4(x64.astype(np.float32))[2]
    else:
        a = x64
    requant = {"fp8": True, "int8": "int8", "mxfp4a4": "mxfp4"}.get(wdt, False)
    want = np.zeros((rows, H))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            w13, w2 = O.expert_weights(host.routed, e)
            want[r0:r1] = O.expert_ffn(a[r0:r1], w13, w2, requant_h=requant)
    ydt = torch.float32 if y_dt == "f32" else torch.bfloat16
    y = torch.full((rows + 8, H), float("nan"), dtype=ydt, device="cuda")  # 8 guard rows
    moe.moe_grouped_ffn(moe.Experts.from_bank(dev.routed), dev.x,
                        torch.from_numpy(offsets).cuda(), y[:rows])
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isnan(got[rows:]).all()                # nothing written past the last row
    err = O.rel_err(got[:rows], want)
    tol = TOL[wdt] if not (wdt == "f32" and y_dt == "bf16") else TOL["bf16"]
    print(name, y_dt, "rel err", err, flush=True)
    assert err <= tol, (name, y_dt, err)


PREQUANT = {"fp8": (O.quantise_rows_e4m3, moe.moe_quantize_fp8, 1, 128, torch.uint8, torch.float32),
            "int8": (O.quantise_rows_int8, moe.moe_quantize_int8, 1, 128, torch.int8, torch.float32),
            "mxfp4a4": (O.quantise_rows_mxfp4, moe.moe_quantize_mxfp4, 2, 32, torch.uint8,
                        torch.uint8)}


@pytest.mark.parametrize("y_dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", [c for c in FFN_CASES if c[1] in PREQUANT], ids=lambda c: c[0])
def test_grouped_ffn_prequant(case, y_dt):
    """Rows handed over already quantised. The oracle's codes and scales, uploaded as they
    are, give oracle.expert_ffn's rows within the format's tolerance; the codes and scales of
    the library's moe_quantize_* on the bf16 rows give exactly moe_grouped_ffn's bits."""
    name, wdt, H, I, E, rows = case
    quantise, lib_quantise, per_byte, blk, code_dt, scale_dt = PREQUANT[wdt]
    cfg = MoEConfig(f"ffn_{name}", T=rows, H=H, E=E, k=1, I=I, score="none", act="bf16", wdt=wdt,
                    out=y_dt, seed=150 + len(name), weight_seed=150 + len(name),
                    dirichlet_alpha=0.7)
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    counts = np.bincount(host.topk_idx[:, 0], minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    codes, scales, a = quantise(O.decode_act("bf16", host.x).astype(np.float32))
    if per_byte == 2:  # E2M1 nibbles, element 2i in the low nibble of byte i
        codes = codes[:, 0::2] | (codes[:, 1::2] << 4)
    requant = {"fp8": True, "int8": "int8", "mxfp4a4": "mxfp4"}[wdt]
    want = np.zeros((rows, H))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            w13, w2 = O.expert_weights(host.routed, e)
            want[r0:r1] = O.expert_ffn(a[r0:r1], w13, w2, requant_h=requant)
    experts = moe.Experts.from_bank(dev.routed)
    d_off = torch.from_numpy(offsets).cuda()
    ydt = torch.float32 if y_dt == "f32" else torch.bfloat16
    y = torch.full((rows + 8, H), float("nan"), dtype=ydt, device="cuda")  # 8 guard rows
    d_codes = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8)).cuda().view(code_dt)
    d_scales = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    moe.moe_grouped_ffn_prequant(experts, d_codes, d_scales, d_off, y[:rows])
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isnan(got[rows:]).all()                # nothing written past the last row
    err = O.rel_err(got[:rows], want)
    print(name, y_dt, "rel err", err, flush=True)
    assert err <= TOL[wdt], (name, y_dt, err)
    # the library's quantiser, then the pre-quantised call: the bits of moe_grouped_ffn
    q = torch.empty((rows, H // per_byte), dtype=code_dt, device="cuda")
    qs = torch.empty((rows, H // blk), dtype=scale_dt, device="cuda")
    lib_quantise(dev.x, q, qs)
    y_pre = torch.empty((rows, H), dtype=ydt, device="cuda")
    y_ref = torch.empty((rows, H), dtype=ydt, device="cuda")
    moe.moe_grouped_ffn_prequant(experts, q, qs, d_off, y_pre)
    moe.moe_grouped_ffn(experts, dev.x, d_off, y_ref)
    torch.cuda.synchronize()
    assert torch.equal(y_pre.view(torch.int16 if y_dt == "bf16" else torch.int32),
                       y_ref.view(torch.int16 if y_dt == "bf16" else torch.int32))


def _split_h(h64):
    """h as the bf16 kernels carry it into the down GEMM: fp32 h rounded to bf16 (hi) plus
    the residual fp32(h) - hi coded as MXFP4 per 32 features (OCP MX rule)."""
    h32 = h64.astype(np.float32).astype(np.float64)
    hi = torch.from_numpy(h32.astype(np.float32)).to(torch.bfloat16).double().numpy()
    return hi + O.quantise_rows_mxfp4((h32 - hi).astype(np.float32))[2]


@pytest.mark.parametrize("case", [c for c in FFN_CASES if c[1] == "bf16" and c[2] % 64 == 0 and
                                  c[3] % 64 == 0], ids=lambda c: c[0])
def test_bf16_down_carries_h_residual(case):
    """The bf16 kernels' arithmetic, pinned tighter than the tolerance: with fp32 output
    rows, every kernel family's result equals a float64 simulation of h as bf16 plus its
    MXFP4-coded residual to 1e-4 of the RMS (without the residual the two differ by about
    1e-3)."""
    name, wdt, H, I, E, rows = case
    cfg = MoEConfig(f"ffn_{name}", T=rows, H=H, E=E, k=1, I=I, score="none", act="bf16", wdt=wdt,
                    out="f32", seed=140 + len(name), weight_seed=140 + len(name),
                    dirichlet_alpha=0.7)
    print("case", describe(cfg), flush=True)
    host = host_problem(cfg)
    dev = device_problem(cfg, host=host)
    counts = np.bincount(host.topk_idx[:, 0], minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    x64 = O.bf16_to_f64(host.x)
    sim = np.zeros((rows, H))
    plain = np.zeros((rows, H))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            w13, w2 = O.expert_weights(host.routed, e)
            h = O.silu(x64[r0:r1] @ w13[:I].T) * (x64[r0:r1] @ w13[I:].T)
            sim[r0:r1] = _split_h(h) @ w2.T
            hb = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).double().numpy()
            plain[r0:r1] = hb @ w2.T
    y = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(moe.Experts.from_bank(dev.routed), dev.x, torch.from_numpy(offsets).cuda(), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(sim ** 2))
    d = np.sqrt(np.mean((got - sim) ** 2)) / rms
    print(name, "rms diff vs simulation", d, "plain bf16 h would be",
          np.sqrt(np.mean((plain - sim) ** 2)) / rms, flush=True)
    assert np.sqrt(np.mean((plain - sim) ** 2)) / rms > 3e-4   # the check has teeth here
    assert d <= 1e-4
