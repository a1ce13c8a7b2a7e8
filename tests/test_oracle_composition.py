"""Pins of the oracle's composed steps (CPU only): the weighted combine and the
re-quantisation of the low-precision expert paths.

Each codec of the oracle is pinned on its own in test_oracle.py and
test_oracle_mxfp4_act.py. Here the steps that put them together are pinned:
  * combine: the weighted sum of moe_ffn ("Decoding Trillion-Parameter MoE LLMs",
    section "Routing: Top-K Experts Plus a Shared Expert") through the inverse
    permutation, against the un-permutation identity, closed forms and the layer's own
    per-expert accumulation (a second route through the same sum);
  * the fused SwiGLU + re-quantisation of the FP8/FP4 grouped GEMM (GC-MoE record,
    key_changes, fourth item): h quantised from its fp32 value per 1 x 128 (fp8) or
    1 x 32 (MXFP4) block before the down projection, composed here independently with
    torch's float8_e4m3fn codec and a literal OCP E2M1 value table. The inputs are built
    so that h sits on a rounding tie in fp32 but not in float64: a quantiser fed the
    float64 h picks the other code, and these tests fail;
  * the fp8 / W4A4 layer: the router sees the unquantised activations, and the routed
    and shared experts both take the quantised ones.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from synth.configs import MoEConfig
from synth.problem import host_problem

# ----------------------------------------------------------------------------- combine


def _routing(T, k, E, rng):
    """k distinct experts per token, ascending, with uneven loads."""
    p = rng.dirichlet(np.full(E, 0.5))
    idx = np.stack([np.sort(rng.choice(E, size=k, replace=False, p=p)) for _ in range(T)])
    return idx.astype(np.int32)


def test_combine_unpermutes_with_unit_weights():
    """k = 1, weight 1, no shared term: combine is the inverse of the dispatch gather, so
    rows gathered into expert order come back in token order exactly."""
    rng = np.random.default_rng(3)
    T, E, H = 57, 6, 5
    idx = _routing(T, 1, E, rng)
    _, _, perm_src, inv_perm = O.permutation(idx, E)
    z = rng.normal(size=(T, H))
    y_perm = z[perm_src]                       # row r holds token perm_src[r] (k = 1)
    out = O.combine(y_perm, inv_perm, np.ones((T, 1)))
    assert np.array_equal(out, z)


def test_combine_equal_rows_give_scaled_row():
    """When every expert returns the same vector v for a token, the weighted sum is
    (sum of its weights) * v: scale * v for renormalised weights."""
    rng = np.random.default_rng(4)
    T, E, H, k, scale = 20, 9, 7, 3, 2.5
    idx = _routing(T, k, E, rng)
    _, _, perm_src, inv_perm = O.permutation(idx, E)
    v = rng.normal(size=(T, H))
    s = rng.uniform(0.1, 1.0, (T, k))
    w = scale * s / s.sum(axis=1, keepdims=True)
    y_perm = v[perm_src // k]
    out = O.combine(y_perm, inv_perm, w)
    np.testing.assert_allclose(out, scale * v, rtol=1e-14, atol=1e-14)


def test_combine_hand_worked():
    """Two tokens, k = 2, E = 3, H = 1, worked by hand.
    Token 0 chose experts {0, 2} with weights 0.25, 0.75; token 1 chose {1, 2} with 0.5,
    0.5. Rows in expert order: r0 = (t0, e0), r1 = (t1, e1), r2 = (t0, e2), r3 = (t1, e2).
    With expert outputs y = [10, 20, 30, 40] and a shared output [1, 2]:
    out0 = 0.25*10 + 0.75*30 + 1 = 26, out1 = 0.5*20 + 0.5*40 + 2 = 32."""
    idx = np.array([[0, 2], [1, 2]], np.int32)
    counts, offsets, perm_src, inv_perm = O.permutation(idx, 3)
    assert list(perm_src) == [0, 2, 1, 3] and list(inv_perm) == [0, 2, 1, 3]
    y = np.array([[10.0], [20.0], [30.0], [40.0]])
    w = np.array([[0.25, 0.75], [0.5, 0.5]])
    out = O.combine(y, inv_perm, w, shared64=np.array([[1.0], [2.0]]))
    assert out.tolist() == [[26.0], [32.0]]
    # without the shared term
    assert O.combine(y, inv_perm, w).tolist() == [[25.0], [30.0]]


@pytest.mark.parametrize("with_shared", [False, True])
def test_combine_matches_layer_accumulation(with_shared):
    """The layer accumulates per expert (rows of each expert found by comparing ids);
    combine sums through inv_perm. Both routes must give the same output, with expert
    outputs computed once per permuted row and placed in expert order."""
    rng = np.random.default_rng(5 + with_shared)
    T, H, E, k, I = 33, 16, 7, 3, 8
    cfg = MoEConfig("combine_pin", T=T, H=H, E=E, k=k, I=I, score="sigmoid", use_bias=True,
                    scale=2.5, shared_I=8 if with_shared else 0, act="f32", wdt="f32", out="f32",
                    seed=91, weight_seed=91)
    prob = host_problem(cfg)
    # the layer's own route and accumulation
    want = O.layer_forward(prob)
    x64 = O.f32_to_f64(prob.x)
    rows = T * k
    y_perm = np.zeros((rows, H))
    for e in range(E):
        r0, r1 = want["offsets"][e], want["offsets"][e + 1]
        if r1 > r0:
            w13, w2 = O.expert_weights(prob.routed, e)
            y_perm[r0:r1] = O.expert_ffn(x64[want["perm_src"][r0:r1] // k], w13, w2)
    shared = None
    if with_shared:
        w13, w2 = O.expert_weights(prob.shared, 0)
        shared = O.expert_ffn(x64, w13, w2)
    got = O.combine(y_perm, want["inv_perm"], want["topk_w"], shared)
    np.testing.assert_allclose(got, want["out"], rtol=1e-12, atol=1e-12)
    # a dropped shared term, or the permutation used the wrong way round, would differ
    scale = np.abs(want["out"]).max()
    if with_shared:
        dropped = O.combine(y_perm, want["inv_perm"], want["topk_w"])
        assert np.abs(dropped - want["out"]).max() > 0.05 * scale
    wrong = O.combine(y_perm, want["perm_src"], want["topk_w"], shared)
    assert np.abs(wrong - want["out"]).max() > 0.05 * scale


# ------------------------------------------------------- re-quantisation of h, fp8


def _silu_at(target: float, lo: float, hi: float) -> float:
    """A float64 z in [lo, hi] whose float64 SiLU lies about 2^-33 relative above `target`
    (torch's SiLU and the oracle's both: far above float64's last bit, far below half an
    fp32 step), so h is above the tie in float64 and on it after rounding to fp32."""
    f = lambda z: F.silu(torch.tensor([z], dtype=torch.float64)).item()
    goal = target * (1 + 2.0 ** -33)
    a, b = lo, hi
    for _ in range(200):
        m = 0.5 * (a + b)
        if f(m) > goal:
            b = m
        else:
            a = m
    z = b
    for v in (f(z), float(O.silu(np.array([z]))[0])):
        assert target < v < target * (1 + 2.0 ** -27) and np.float32(v) == np.float32(target), (v, target)
    return z


def _tie_expert(H, I, zs):
    """One SwiGLU expert whose h is chosen element by element: the up rows all pick input
    column 0 (set to 1) and gate row i picks input column 1 + i, so h_i = SiLU(a_{1+i})."""
    w13 = np.zeros((2 * I, H))
    for i in range(I):
        w13[i, 1 + i] = 1.0
        w13[I + i, 0] = 1.0
    a = np.zeros((1, H))
    a[0, 0] = 1.0
    a[0, 1:1 + len(zs)] = zs
    return a, w13


def _h_fp64(a, w13):
    I = w13.shape[0] // 2
    ta, tw = torch.from_numpy(a), torch.from_numpy(w13)
    return (F.silu(ta @ tw[:I].T) * (ta @ tw[I:].T)).numpy()


def _fp8_deq_torch(v32: np.ndarray, block=128) -> np.ndarray:
    """Per 1 x block: s = fp32(amax / 448) (1 for a zero block), q = e4m3(fp32(v / s)) with
    torch's float8_e4m3fn conversion, value q * s."""
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32))
    R, C = t.shape
    tb = t.reshape(R, C // block, block)
    amax = tb.abs().amax(dim=2, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (tb / s).to(torch.float8_e4m3fn)
    return (q.double() * s.double()).reshape(R, C).numpy()


def test_expert_ffn_fp8_requant_from_fp32_h():
    """expert_ffn(requant_h=True) = (fp8 per 1x128 of fp32(h)) @ W2^T, composed with torch.
    h_0 = SiLU(448) = 448 sets the block scale to 1; h_1 is SiLU at just above 1.0625, the
    midpoint of E4M3's 1 and 1.125: fp32(h_1) = 1.0625 rounds to even (1), the float64
    h_1 would round up to 1.125."""
    H, I = 256, 128
    z1 = _silu_at(1.0625, 1.0, 2.0)
    a, w13 = _tie_expert(H, I, [448.0, z1, -0.3, 2.7])
    h64 = _h_fp64(a, w13)
    assert h64[0, 0] == 448.0 and np.float32(h64[0, 1]) == np.float32(1.0625) and h64[0, 1] > 1.0625
    rng = np.random.default_rng(6)
    w2 = rng.normal(0, 0.1, (H, I))
    want = _fp8_deq_torch(h64.astype(np.float32)) @ w2.T
    got = O.expert_ffn(a, w13, w2, requant_h=True)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    # the composition has teeth: h_1 goes to 1 from its fp32 value; quantised from the
    # float64 value (above the tie) it would go to 1.125, and y would differ
    hq = _fp8_deq_torch(h64.astype(np.float32))
    assert hq[0, 1] == 1.0
    h_wrong = hq.copy()
    h_wrong[0, 1] = 1.125
    assert np.abs(h_wrong @ w2.T - got).max() > 1e-3


def test_expert_ffn_fp8_requant_blocks_are_per_row_and_128_wide():
    """Two rows, two 128-blocks each, with very different magnitudes: each (row, block)
    takes its own scale. A scale per row, per column block over all rows, or per 64 would
    change the quantised values."""
    rng = np.random.default_rng(7)
    H, I, R = 64, 256, 2
    a = rng.normal(size=(R, H))
    w13 = rng.normal(0, 0.3, (2 * I, H))
    w13[:I // 2] *= 100.0        # first block of h: much larger values
    w2 = rng.normal(0, 0.1, (H, I))
    a[1] *= 1e-3                 # second row: much smaller values
    h64 = _h_fp64(a, w13)
    want = _fp8_deq_torch(h64.astype(np.float32)) @ w2.T
    got = O.expert_ffn(a, w13, w2, requant_h="fp8")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-300)
    # one scale per row (block = I) would lose the small block's precision
    coarse = _fp8_deq_torch(h64.astype(np.float32), block=I) @ w2.T
    assert np.abs(coarse - want).max() > 1e-6 * np.abs(want).max()


# ------------------------------------------------------ re-quantisation of h, MXFP4

# OCP Microscaling Formats (MX) v1.0, FP4 E2M1: code m (0..7) has magnitude E2M1[m].
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mxfp4_deq_table(v32: np.ndarray, block=32) -> np.ndarray:
    """Per 1 x block: X = 2^(floor(log2 amax) - 2) (1 for a zero block); each element the
    nearest E2M1 magnitude of |v| / X by brute force over the table (saturating at 6; on a
    tie the even code); value sign * magnitude * X."""
    v = np.asarray(v32, np.float32).astype(np.float64)
    R, C = v.shape
    out = np.empty_like(v)
    for r in range(R):
        for b in range(C // block):
            blk = v[r, b * block:(b + 1) * block]
            amax = np.abs(blk).max()
            X = 1.0 if amax == 0 else 2.0 ** (math.floor(math.log2(amax)) - 2)
            for j, x in enumerate(blk):
                a = min(abs(x) / X, 6.0)
                best = min(range(8), key=lambda m: (abs(E2M1[m] - a), m % 2))
                out[r, b * block + j] = math.copysign(E2M1[best] * X, x)
    return out


def test_expert_ffn_mxfp4_requant_from_fp32_h():
    """expert_ffn(requant_h='mxfp4') = (MXFP4 per 1x32 of fp32(h)) @ W2^T. h_0 = SiLU(5)
    (in [4, 8)) sets the block scale to 1; h_1 is just above 1.25, the midpoint of E2M1's 1
    and 1.5: fp32(h_1) = 1.25 rounds to the even code (1), the float64 value to 1.5."""
    H, I = 128, 64
    z1 = _silu_at(1.25, 1.0, 2.0)
    a, w13 = _tie_expert(H, I, [5.0, z1, -0.7, 3.1, 0.05])
    h64 = _h_fp64(a, w13)
    assert np.float32(h64[0, 1]) == np.float32(1.25) and h64[0, 1] > 1.25
    rng = np.random.default_rng(8)
    w2 = rng.normal(0, 0.1, (H, I))
    hq = _mxfp4_deq_table(h64.astype(np.float32))
    assert hq[0, 1] == 1.0
    want = hq @ w2.T
    got = O.expert_ffn(a, w13, w2, requant_h="mxfp4")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    h_wrong = hq.copy()
    h_wrong[0, 1] = 1.5      # the float64 h_1's code
    assert np.abs(h_wrong @ w2.T - got).max() > 1e-3


def test_expert_ffn_mxfp4_requant_random_rows():
    rng = np.random.default_rng(9)
    H, I, R = 96, 128, 5
    a = rng.normal(size=(R, H))
    w13 = rng.normal(0, 0.2, (2 * I, H))
    w2 = rng.normal(0, 0.1, (H, I))
    h64 = _h_fp64(a, w13)
    want = _mxfp4_deq_table(h64.astype(np.float32)) @ w2.T
    got = O.expert_ffn(a, w13, w2, requant_h="mxfp4")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ the quantised layer


def _layer_by_hand(prob, deq_act, deq_h):
    """The quantised layer composed outside the oracle's layer_forward: routing from the
    unquantised activations (taken from the pinned route), expert and shared FFNs on the
    quantised activations, h re-quantised by deq_h, weighted sum plus shared output."""
    cfg = prob.cfg
    x64 = O.bf16_to_f64(prob.x)
    r = O.route(x64, O.bf16_to_f64(prob.wr), prob.bias, cfg.k, cfg.score, cfg.scale)
    xq = deq_act(x64.astype(np.float32))
    out = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = int(r["topk_idx"][t, j])
            w13, w2 = O.expert_weights(prob.routed, e)
            I = w13.shape[0] // 2
            g = xq[t:t + 1] @ w13[:I].T
            u = xq[t:t + 1] @ w13[I:].T
            h = F.silu(torch.from_numpy(g)).numpy() * u
            out[t] += r["topk_w"][t, j] * (deq_h(h.astype(np.float32)) @ w2.T)[0]
    w13, w2 = O.expert_weights(prob.shared, 0)
    I = w13.shape[0] // 2
    h = F.silu(torch.from_numpy(xq @ w13[:I].T)).numpy() * (xq @ w13[I:].T)
    out += deq_h(h.astype(np.float32)) @ w2.T
    return r, out


@pytest.mark.parametrize("wdt", ["fp8", "mxfp4a4"])
def test_quantised_layer_composition(wdt):
    """The fp8 and W4A4 layers equal their composition by hand (router on the bf16 x,
    routed and shared experts on the quantised x, h re-quantised), and their routing
    equals the bf16 layer's on the same x and router."""
    cfg = MoEConfig("q_layer", T=12, H=256, E=6, k=2, I=128, score="softmax", shared_I=128,
                    act="bf16", wdt=wdt, out="bf16", seed=92, weight_seed=92)
    prob = host_problem(cfg)
    want = O.layer_forward(prob)
    ref = O.layer_forward(host_problem(cfg.with_(wdt="bf16")))
    assert np.array_equal(want["logits"], ref["logits"])
    assert np.array_equal(want["topk_idx"], ref["topk_idx"])
    if wdt == "fp8":
        deq = _fp8_deq_torch
    else:
        deq = _mxfp4_deq_table
    r, out = _layer_by_hand(prob, deq, deq)
    assert np.array_equal(r["topk_idx"], want["topk_idx"])
    np.testing.assert_allclose(want["out"], out, rtol=1e-11, atol=1e-11 * np.abs(out).max())
    # the shared expert fed the unquantised x would give another output
    x64 = O.bf16_to_f64(prob.x)
    w13, w2 = O.expert_weights(prob.shared, 0)
    I = w13.shape[0] // 2
    xq = deq(x64.astype(np.float32))

    def shared_out(a):
        h = F.silu(torch.from_numpy(a @ w13[:I].T)).numpy() * (a @ w13[I:].T)
        return deq(h.astype(np.float32)) @ w2.T

    assert np.abs(shared_out(x64) - shared_out(xq)).max() > 1e-3 * np.abs(out).max()
