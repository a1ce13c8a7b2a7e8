"""Pins of the oracle's INT8 (W8A8) parts (CPU only): the quantiser against torch's
round-half-to-even and against brute force, hand-worked blocks, the block decode of INT8
weights, exact integer products, the re-quantisation of h from its fp32 value, and the W8A8
layer composed independently.

The pages name W8A8 -- weights and activations as INT8 on INT8 matrix units ("Trillion-
Parameter LLM Architecture Explained and Cost-Efficient Inference in Practice", section 3.1)
-- without a recipe; the reading pinned here is symmetric INT8 with fp32 scales amax / 127
per 1 x 128 activation block and per 128 x 128 weight block.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle as O
import synth
from synth.configs import MoEConfig
from synth.problem import host_problem


def _torch_int8(v32, block=128):
    """Per 1 x block: s = fp32(amax / 127) (1 for a zero block); q = torch.round (half to
    even) of fp32(v / s), clamped to +-127."""
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32))
    R, C = t.shape
    tb = t.reshape(R, C // block, block)
    amax = tb.abs().amax(dim=2, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
    q = torch.round(tb / s).clamp(-127, 127)
    return q.to(torch.int8).reshape(R, C).numpy(), s[:, :, 0].numpy(), (q.double() * s.double()).reshape(R, C).numpy()


def test_int8_quantiser_matches_torch():
    rng = np.random.default_rng(21)
    v = (rng.normal(0, 1, (64, 512)) * 10.0 ** rng.uniform(-5, 4, (64, 1))).astype(np.float32)
    v[0, :128] = 0.0
    v[1, :128] = np.round(rng.uniform(-127, 127, 128)) + 0.5   # every element a tie
    v[1, 0] = 127.0                                            # (scale 1)
    codes, s, deq = O.quantise_rows_int8(v)
    tc, ts, td = _torch_int8(v)
    assert np.array_equal(s, ts) and np.array_equal(codes, tc)
    np.testing.assert_array_equal(deq, td)


def test_int8_quantiser_hand_worked():
    """A block with amax 127 has scale 1: codes are the values rounded half to even
    (63.5 -> 64, -63.5 -> -64, 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2); a zero block
    gets scale 1 and zero codes; a block with amax 254 has scale 2."""
    v = np.zeros((3, 128), np.float32)
    v[0, :8] = [127.0, 63.5, -63.5, 0.5, 1.5, 2.5, -2.5, 126.6]
    v[2, :3] = [254.0, 5.0, -3.0]      # 5 / 2 = 2.5 -> 2; -3 / 2 = -1.5 -> -2
    codes, s, deq = O.quantise_rows_int8(v)
    assert codes[0, :8].tolist() == [127, 64, -64, 0, 2, 2, -2, 127]
    assert s.tolist() == [[1.0], [1.0], [2.0]]
    assert (codes[1] == 0).all()
    assert codes[2, :3].tolist() == [127, 2, -2] and deq[2, :3].tolist() == [254.0, 4.0, -4.0]


def test_int8_quantiser_is_the_nearest_code():
    """Brute force: every code is the nearest of the 255 integers -127..127 to v / s (ties
    to the even one), and the error is at most half a scale step."""
    rng = np.random.default_rng(22)
    v = rng.normal(0, 3, (40, 128)).astype(np.float32)
    codes, s, deq = O.quantise_rows_int8(v)
    grid = np.arange(-127, 128, dtype=np.float64)
    for r in range(40):
        x = (v[r] / s[r, 0]).astype(np.float32).astype(np.float64)
        d = np.abs(x[:, None] - grid[None, :])
        best = d.min(axis=1)
        for j in range(128):
            cand = grid[d[j] == best[j]]
            want = cand[0] if len(cand) == 1 else cand[cand % 2 == 0][0]
            assert codes[r, j] == want
    assert (np.abs(deq - v) <= s.repeat(128, axis=1) / 2 * (1 + 1e-6)).all()


def test_int8_weight_decode_is_code_times_block_scale():
    """decode_matrix('int8'): element (r, c) is its code times the scale of its 128 x 128
    block, checked element by element on a 256 x 384 matrix with six different scales."""
    codes, scales = synth.int8_bank(5, 4, 0, 1, 256, 384, 0.02)
    w = O.decode_matrix("int8", {"w": codes[0], "scale": scales[0]})
    rng = np.random.default_rng(23)
    for r, c in zip(rng.integers(0, 256, 500), rng.integers(0, 384, 500)):
        assert w[r, c] == float(codes[0, r, c]) * float(scales[0, r // 128, c // 128])
    assert len(np.unique(scales[0])) == 6


def test_int8_products_match_integer_accumulation():
    """The fp64 product of two dequantised INT8 matrices (fp32 scales) is their exact integer
    matrix product times the product of the scales (exact in fp64: two 24-bit mantissas), up
    to fp64 rounding of the oracle's sums: what an INT8 matrix unit with int32 accumulation
    computes before its scales are applied."""
    rng = np.random.default_rng(24)
    a = rng.integers(-127, 128, (16, 256)).astype(np.int64)
    b = rng.integers(-127, 128, (24, 256)).astype(np.int64)
    sa, sb = float(np.float32(0.0125)), float(np.float32(0.003))
    got = (a * sa).astype(np.float64) @ (b * sb).astype(np.float64).T
    acc = a @ b.T                                   # exact: |acc| <= 256 * 127^2 < 2^23
    want = acc.astype(np.float64) * (sa * sb)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14 * np.abs(want).max())
    assert np.abs(acc).max() < 2 ** 24              # exact in fp32 too


def _silu_at(target, lo, hi):
    """A float64 z whose float64 SiLU (torch's and the oracle's) lies about 2^-33 relative
    above `target`: above the tie in float64, on it after rounding to fp32."""
    f = lambda z: F.silu(torch.tensor([z], dtype=torch.float64)).item()
    goal = target * (1 + 2.0 ** -33)
    a, b = lo, hi
    for _ in range(200):
        m = 0.5 * (a + b)
        if f(m) > goal:
            b = m
        else:
            a = m
    for v in (f(b), float(O.silu(np.array([b]))[0])):
        assert target < v < target * (1 + 2.0 ** -27) and np.float32(v) == np.float32(target)
    return b


def test_expert_ffn_int8_requant_from_fp32_h():
    """expert_ffn(requant_h='int8') = (INT8 per 1x128 of fp32(h)) @ W2^T, composed with
    torch. h_0 = SiLU(127) = 127 sets the block scale to 1; h_1 is SiLU just above 2.5: its
    fp32 value 2.5 rounds to the even code 2, its float64 value would round to 3."""
    H, I = 256, 128
    z1 = _silu_at(2.5, 2.0, 3.0)
    w13 = np.zeros((2 * I, H))
    for i in range(I):
        w13[i, 1 + i] = 1.0
        w13[I + i, 0] = 1.0
    a = np.zeros((1, H))
    a[0, 0] = 1.0
    a[0, 1:4] = [127.0, z1, -40.3]
    ta, tw = torch.from_numpy(a), torch.from_numpy(w13)
    h64 = (F.silu(ta @ tw[:I].T) * (ta @ tw[I:].T)).numpy()
    assert h64[0, 0] == 127.0 and np.float32(h64[0, 1]) == np.float32(2.5) and h64[0, 1] > 2.5
    w2 = np.random.default_rng(25).normal(0, 0.1, (H, I))
    _, _, hq = _torch_int8(h64.astype(np.float32))
    assert hq[0, 1] == 2.0
    got = O.expert_ffn(a, w13, w2, requant_h="int8")
    np.testing.assert_allclose(got, hq @ w2.T, rtol=1e-13, atol=1e-13)
    h_wrong = hq.copy()
    h_wrong[0, 1] = 3.0
    assert np.abs(h_wrong @ w2.T - got).max() > 1e-3


def test_w8a8_layer_composition():
    """The W8A8 layer equals its composition by hand: routing from the bf16 x (the bf16
    layer's routing, bit for bit), routed and shared experts on the INT8-quantised x with
    INT8 weights, h re-quantised to INT8 per 1x128."""
    cfg = MoEConfig("w8a8_layer", T=10, H=256, E=6, k=2, I=128, score="sigmoid", use_bias=True,
                    scale=2.5, shared_I=128, act="bf16", wdt="int8", out="bf16", seed=93,
                    weight_seed=93)
    prob = host_problem(cfg)
    want = O.layer_forward(prob)
    ref = O.layer_forward(host_problem(cfg.with_(wdt="bf16")))
    assert np.array_equal(want["logits"], ref["logits"])
    assert np.array_equal(want["topk_idx"], ref["topk_idx"])
    x64 = O.bf16_to_f64(prob.x)
    _, _, xq = _torch_int8(x64.astype(np.float32))

    def ffn(a, bank, e):
        w13, w2 = O.expert_weights(bank, e)
        I = w13.shape[0] // 2
        h = F.silu(torch.from_numpy(a @ w13[:I].T)).numpy() * (a @ w13[I:].T)
        return _torch_int8(h.astype(np.float32))[2] @ w2.T

    out = ffn(xq, prob.shared, 0)
    for t in range(cfg.T):
        for j in range(cfg.k):
            out[t] += want["topk_w"][t, j] * ffn(xq[t:t + 1], prob.routed, int(want["topk_idx"][t, j]))[0]
    np.testing.assert_allclose(want["out"], out, rtol=1e-11, atol=1e-11 * np.abs(out).max())
