"""Pins of the CPU oracle to things other than itself (CPU only).

Each check ties one step of the oracle to a definition it can be checked against
by eye or by an independent route: brute-force enumeration, closed forms,
library routines (torch's float8 codecs and float64 ops), the OCP MX tables,
invariants and hand-worked fixtures under tests/golden/.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth.configs import MoEConfig
from synth.problem import HostProblem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- codecs

def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert O.e4m3_to_f64(np.array([0x7E], np.uint8))[0] == 448.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000), rng.normal(0, 0.01, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),
        # exact midpoints between neighbouring codes (ties) and the grid itself
        (O.e4m3_to_f64(np.arange(126, dtype=np.uint8)) + O.e4m3_to_f64(np.arange(1, 127, dtype=np.uint8))) / 2,
        O.e4m3_to_f64(np.arange(127, dtype=np.uint8)),
    ]).astype(np.float32)
    v = np.concatenate([v, -v])
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.encode_e4m3_rne_sat(v)
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 463.9, 464.0, 1e6, -1e6, -470.0], np.float32)
    got = O.encode_e4m3_rne_sat(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e2m1_decode_is_the_ocp_table():
    # OCP Microscaling Formats (MX) v1.0, FP4 E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = O.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == table
    assert list(got[8:]) == [-t for t in table]


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = O.e8m0_to_f64(codes)
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255], want[:255])


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(2).integers(0, 2 ** 16, 5000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_to_f64(bits), want)


def test_mxfp4_matrix_decode_nibble_order_and_scale():
    # byte 0x31 holds element 0 = 1 (low nibble, 0.5) and element 1 = 3 (high nibble, 1.5)
    packed = np.array([[0x31] + [0] * 15], np.uint8)         # one row of 32 elements
    scale = np.array([[128]], np.uint8)                       # 2^1
    got = O.decode_matrix("mxfp4", {"w": packed, "scale": scale})
    assert got.shape == (1, 32)
    assert got[0, 0] == 1.0 and got[0, 1] == 3.0 and not got[0, 2:].any()


def test_fp8_matrix_decode_block_scales():
    codes = np.full((256, 128), 0x38, np.uint8)              # 1.0
    scale = np.array([[2.0], [0.5]], np.float32)
    got = O.decode_matrix("fp8", {"w": codes, "scale": scale})
    assert np.all(got[:128] == 2.0) and np.all(got[128:] == 0.5)


def test_activation_quantiser_steps():
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, (8, 256)).astype(np.float32)
    v[2, :128] = 0.0
    codes, s, deq = O.quantise_rows_e4m3(v)
    amax = np.abs(v.reshape(8, 2, 128)).max(axis=2)
    # scale: fp32 amax/448, or 1 for an all-zero block
    want_s = np.where(amax == 0, 1.0, amax / np.float32(448)).astype(np.float32)
    assert np.array_equal(s, want_s)
    # codes: torch's RNE conversion of the fp32 quotient
    q = (v.reshape(8, 2, 128) / s[:, :, None]).astype(np.float32).reshape(8, 256)
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)
    # the block maximum maps to 448 exactly
    assert np.max(np.abs(O.e4m3_to_f64(codes[0, :128]))) == 448.0
    rel = np.abs(deq - v) / np.maximum(np.abs(v), 1e-30)
    assert np.all((rel <= 2.0 ** -4 + 1e-12) | (np.abs(v) < np.repeat(s, 128, axis=1) * 2.0 ** -6))


# ----------------------------------------------------------------------------- selection

def _brute_force_topk(keys: np.ndarray, k: int):
    """All C(E,k) subsets; the chosen one is the unique S where every member beats every
    non-member under (key larger, or equal key and lower index), NaN below everything."""
    E = len(keys)

    def beats(a, b):  # expert a ranks above expert b
        ka, kb = keys[a], keys[b]
        if math.isnan(ka) and math.isnan(kb):
            return a < b
        if math.isnan(ka):
            return False
        if math.isnan(kb):
            return True
        return ka > kb or (ka == kb and a < b)

    winners = [S for S in itertools.combinations(range(E), k)
               if all(beats(a, b) for a in S for b in range(E) if b not in S)]
    assert len(winners) == 1
    return list(winners[0])


def test_topk_matches_brute_force_with_ties_and_nan():
    rng = np.random.default_rng(4)
    for trial in range(400):
        E = int(rng.integers(2, 11))
        k = int(rng.integers(1, min(E, 4) + 1))
        keys = rng.integers(-3, 4, E).astype(np.float32)        # many ties
        if trial % 3 == 0:
            keys[rng.integers(0, E)] = np.nan
        if trial % 5 == 0:
            keys[rng.integers(0, E)] = -0.0
        got = O.select_topk(keys[None, :], k)[0]
        assert list(got) == _brute_force_topk(keys.tolist(), k), (keys, k)


def test_topk_ascending_distinct():
    rng = np.random.default_rng(5)
    keys = rng.normal(size=(50, 32)).astype(np.float32)
    idx = O.select_topk(keys, 6)
    assert np.all(np.diff(idx, axis=1) > 0)


def _tiny_problem(T=24, H=64, E=6, k=2, I=32, fn="softmax", bias=None, scale=1.0, shared_I=0,
                  seed=0, wr_zero=False):
    rng = np.random.default_rng(seed)
    cfg = MoEConfig("t", T=T, H=H, E=E, k=k, I=I, score=fn, use_bias=bias is not None,
                    scale=scale, shared_I=shared_I, act="f32", wdt="f32", out="f32")

    class Bank:
        fmt = "f32"

        def __init__(self, n, I):
            self.w13s = rng.normal(0, 0.2, (n, 2 * I, H)).astype(np.float32)
            self.w2s = rng.normal(0, 0.2, (n, H, I)).astype(np.float32)

        def w13(self, e):
            return {"w": self.w13s[e]}

        def w2(self, e):
            return {"w": self.w2s[e]}

    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    wr = np.zeros((E, H), np.float32) if wr_zero else rng.normal(0, 0.3, (E, H)).astype(np.float32)
    return HostProblem(cfg, x, wr, bias, Bank(E, I), Bank(1, shared_I) if shared_I else None)


def test_zero_router_picks_lowest_indices_equal_weights():
    for fn, scale in (("softmax", 1.0), ("sigmoid", 2.5)):
        p = _tiny_problem(E=7, k=3, fn=fn, scale=scale, wr_zero=True)
        r = O.route(O.f32_to_f64(p.x), O.f32_to_f64(p.wr), None, 3, fn, scale)
        assert np.all(r["topk_idx"] == np.array([0, 1, 2]))
        assert np.allclose(r["topk_w"], scale / 3, rtol=0, atol=1e-15)


def test_bias_is_selection_only():
    E, k = 8, 3
    S0 = [1, 4, 6]
    bias = np.zeros(E, np.float32)
    bias[S0] = 10.0
    p = _tiny_problem(E=E, k=k, fn="sigmoid", bias=bias, scale=2.5, seed=7)
    x64, wr64 = O.f32_to_f64(p.x), O.f32_to_f64(p.wr)
    r = O.route(x64, wr64, bias, k, "sigmoid", 2.5)
    assert np.all(r["topk_idx"] == np.array(S0))
    # weights come from the unbiased sigmoid scores of S0
    l = (x64 @ wr64.T).astype(np.float32).astype(np.float64)[:, S0]
    s = 1 / (1 + np.exp(-l))
    assert np.allclose(r["topk_w"], 2.5 * s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_k_equals_e_softmax_is_full_softmax():
    p = _tiny_problem(E=5, k=5, fn="softmax", seed=8)
    x64, wr64 = O.f32_to_f64(p.x), O.f32_to_f64(p.wr)
    r = O.route(x64, wr64, None, 5, "softmax", 1.0)
    l = torch.from_numpy((x64 @ wr64.T).astype(np.float32).astype(np.float64))
    assert np.allclose(r["topk_w"], torch.softmax(l, dim=1).numpy(), rtol=1e-13, atol=0)


def test_softmax_renormalised_equals_softmax_over_selected_logits():
    p = _tiny_problem(E=16, k=4, fn="softmax", seed=9)
    x64, wr64 = O.f32_to_f64(p.x), O.f32_to_f64(p.wr)
    r = O.route(x64, wr64, None, 4, "softmax", 1.0)
    l = np.take_along_axis(r["logits"].astype(np.float64), r["topk_idx"].astype(np.int64), 1)
    want = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    assert np.allclose(r["topk_w"], want, rtol=1e-13, atol=0)


def test_router_logits_brute_force_dot_products():
    rng = np.random.default_rng(10)
    x = rng.normal(0, 1, (5, 33)).astype(np.float32)
    w = rng.normal(0, 0.1, (7, 33)).astype(np.float32)
    got = O.router_logits(O.f32_to_f64(x), O.f32_to_f64(w))
    for t in range(5):
        for e in range(7):
            exact = math.fsum(float(a) * float(b) for a, b in zip(x[t], w[e]))
            assert got[t, e] == np.float32(exact)


def test_sigmoid_scores_closed_form():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4 (ln 3 rounded to fp32)
    l = np.array([[0.0, math.log(3.0), -math.log(3.0)]], np.float32)
    s = O.scores(l, "sigmoid")[0]
    assert s[0] == 0.5
    assert abs(s[1] - 0.75) < 1e-7 and abs(s[2] - 0.25) < 1e-7
    assert abs(s[1] + s[2] - 1.0) < 1e-15


def test_softmax_scores_closed_form():
    # logits ln 1 .. ln 4 -> softmax 0.1, 0.2, 0.3, 0.4
    l = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    s = O.scores(l, "softmax")[0]
    assert np.allclose(s, [0.1, 0.2, 0.3, 0.4], rtol=0, atol=1e-7)


# ----------------------------------------------------------------------------- permutation

def test_permutation_matches_loop_construction():
    rng = np.random.default_rng(11)
    for _ in range(20):
        T, E, k = int(rng.integers(1, 40)), int(rng.integers(1, 12)), 0
        k = int(rng.integers(1, E + 1))
        idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm_src, inv_perm = O.permutation(idx, E)
        # loop construction: walk experts ascending, tokens ascending
        rows = []
        for e in range(E):
            for t in range(T):
                for j in range(k):
                    if idx[t, j] == e:
                        rows.append(t * k + j)
        assert list(perm_src) == rows
        assert list(counts) == [int((idx == e).sum()) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
        assert np.array_equal(inv_perm[perm_src], np.arange(T * k))


# ----------------------------------------------------------------------------- experts and layer

def test_expert_ffn_matches_torch_swiglu():
    rng = np.random.default_rng(12)
    a = rng.normal(0, 1, (9, 48))
    w13 = rng.normal(0, 0.2, (2 * 40, 48))
    w2 = rng.normal(0, 0.2, (48, 40))
    ta, t13, t2 = (torch.from_numpy(v) for v in (a, w13, w2))
    want = (torch.nn.functional.silu(ta @ t13[:40].T) * (ta @ t13[40:].T)) @ t2.T
    assert np.allclose(O.expert_ffn(a, w13, w2), want.numpy(), rtol=1e-12, atol=1e-14)


def test_single_expert_layer_is_plain_swiglu():
    p = _tiny_problem(E=1, k=1, fn="softmax", seed=13)
    res = O.layer_forward(p)
    b = p.routed
    ta = torch.from_numpy(p.x.astype(np.float64))
    t13 = torch.from_numpy(b.w13s[0].astype(np.float64))
    t2 = torch.from_numpy(b.w2s[0].astype(np.float64))
    I = p.cfg.I
    want = (torch.nn.functional.silu(ta @ t13[:I].T) * (ta @ t13[I:].T)) @ t2.T
    assert np.allclose(res["topk_w"], 1.0)
    assert np.allclose(res["out"], want.numpy(), rtol=1e-12, atol=1e-13)


def test_zero_gate_leaves_only_shared_expert():
    p = _tiny_problem(E=4, k=2, shared_I=24, seed=14)
    p.routed.w13s[:, : p.cfg.I] = 0.0
    res = O.layer_forward(p)
    sh = O.expert_ffn(O.f32_to_f64(p.x), O.f32_to_f64(p.shared.w13s[0]), O.f32_to_f64(p.shared.w2s[0]))
    assert np.array_equal(res["out"], sh)


def _dense_reference(p, res):
    """Every expert on every token, weight 0 off the chosen set, plus the shared expert."""
    x64 = O.f32_to_f64(p.x)
    T, E = p.cfg.T, p.cfg.E
    W = np.zeros((T, E))
    for t in range(T):
        for j in range(p.cfg.k):
            W[t, res["topk_idx"][t, j]] = res["topk_w"][t, j]
    out = np.zeros((T, p.cfg.H))
    for e in range(E):
        y = O.expert_ffn(x64, O.f32_to_f64(p.routed.w13s[e]), O.f32_to_f64(p.routed.w2s[e]))
        out += W[:, e:e + 1] * y
    if p.shared is not None:
        out += O.expert_ffn(x64, O.f32_to_f64(p.shared.w13s[0]), O.f32_to_f64(p.shared.w2s[0]))
    return out


@pytest.mark.parametrize("fn,bias,scale,shared_I", [("softmax", False, 1.0, 0),
                                                    ("sigmoid", True, 2.5, 40)])
def test_sparse_equals_dense(fn, bias, scale, shared_I):
    rng = np.random.default_rng(15)
    b = rng.uniform(-0.1, 0.1, 9).astype(np.float32) if bias else None
    p = _tiny_problem(T=30, E=9, k=3, fn=fn, bias=b, scale=scale, shared_I=shared_I, seed=16)
    res = O.layer_forward(p)
    dense = _dense_reference(p, res)
    assert np.max(np.abs(res["out"] - dense)) <= 1e-12 * np.max(np.abs(dense))
    # routed weights sum to the scale
    assert np.allclose(res["topk_w"].sum(1), scale, rtol=1e-14)


def test_sample_of_tokens_equals_full_layer():
    p = _tiny_problem(T=20, E=6, k=2, shared_I=16, seed=17)
    full = O.layer_forward(p)
    sub = O.layer_forward(p, tokens=[3, 11, 19])
    assert np.allclose(sub["out"], full["out"][[3, 11, 19]], rtol=1e-14, atol=1e-15)


def test_token_permutation_equivariance():
    p = _tiny_problem(T=16, E=6, k=2, shared_I=16, seed=18)
    res = O.layer_forward(p)
    perm = np.random.default_rng(19).permutation(16)
    p2 = HostProblem(p.cfg, p.x[perm], p.wr, None, p.routed, p.shared)
    res2 = O.layer_forward(p2)
    assert np.array_equal(res2["topk_idx"], res["topk_idx"][perm])
    assert np.allclose(res2["out"], res["out"][perm], rtol=1e-13, atol=1e-14)


def test_expert_relabelling_invariance():
    p = _tiny_problem(T=16, E=6, k=2, fn="sigmoid", bias=np.linspace(-0.05, 0.05, 6).astype(np.float32),
                      scale=2.5, seed=20)
    res = O.layer_forward(p)
    pi = np.array([3, 0, 5, 1, 4, 2])           # new expert i is old expert pi[i]
    q = _tiny_problem(T=16, E=6, k=2, fn="sigmoid", bias=p.bias[pi], scale=2.5, seed=20)
    q.x, q.wr = p.x, p.wr[pi]
    q.routed.w13s, q.routed.w2s = p.routed.w13s[pi], p.routed.w2s[pi]
    res2 = O.layer_forward(q)
    old_of_new = pi[res2["topk_idx"]]
    assert np.array_equal(np.sort(old_of_new, axis=1), res["topk_idx"])
    assert np.allclose(res2["out"], res["out"], rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- golden fixtures

def test_golden_hand_worked_layer():
    """Hand-worked one-token layers in tests/golden/hand_worked.json (see its notes)."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        T, H = len(c["x"]), len(c["x"][0])
        E, k, I = len(c["router"]), c["k"], len(c["w2"][0][0])
        cfg = MoEConfig("g", T=T, H=H, E=E, k=k, I=I, score=c["score"], use_bias=c["bias"] is not None,
                        scale=c["scale"], shared_I=0, act="f32", wdt="f32", out="f32")

        class Bank:
            fmt = "f32"

            def w13(self, e):
                return {"w": np.array(c["w13"][e], np.float32)}

            def w2(self, e):
                return {"w": np.array(c["w2"][e], np.float32)}

        bias = None if c["bias"] is None else np.array(c["bias"], np.float32)
        p = HostProblem(cfg, np.array(c["x"], np.float32), np.array(c["router"], np.float32), bias,
                        Bank(), None)
        res = O.layer_forward(p)
        assert res["topk_idx"].tolist() == c["expect_topk_idx"], c["name"]
        assert np.allclose(res["topk_w"], c["expect_topk_w"], rtol=0, atol=c["atol"]), c["name"]
        assert np.allclose(res["out"], c["expect_out"], rtol=0, atol=c["atol"]), c["name"]
