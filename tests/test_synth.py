"""The seeded input generator (CPU side): known-answer vectors of Philox4x32-10,
determinism, value distributions and the calibrated routing skew."""
import numpy as np

import oracle as O
import synth
from synth.configs import CONFIGS
from synth.problem import host_problem, preroute


def test_philox_known_answer_vectors():
    # Random123 known-answer vectors for philox4x32 with 10 rounds
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert list(synth.philox_block(ctr, key)) == want


def test_generation_is_slice_consistent():
    a = synth.normal_bf16(7, 4, (1000,), 0.02)
    b = synth.normal_bf16(7, 4, (300,), 0.02, start=500)
    assert np.array_equal(a[500:800], b)


def test_normal_fill_equals_per_element_words():
    """The normal fills take all four words of a Philox block at once where they can; at any
    start and length they equal the per-element definition: word i of the stream, its top
    16 bits picking a quantile interval and its low 16 bits the point inside it (fp32)."""
    q = synth.quantile_table()
    std = np.float32(0.5)
    for start in range(9):
        for n in (1, 2, 3, 4, 5, 7, 8, 17, 64):
            got = synth.normal_f32(7, 3, (n,), 0.5, start=start)
            w = synth.words(7, 3, start, n)
            a, b = q[w >> 16], q[(w >> 16) + 1]
            f = (w & 0xFFFF).astype(np.float32) * np.float32(1.0 / 65536.0)
            z = a + f * (b - a)
            assert np.array_equal(got, (z * std).astype(np.float32)), (start, n)


def test_normal_statistics():
    v = synth.normal_f32(11, 1, (2_000_000,), 1.0)
    assert abs(v.mean()) < 3e-3 and abs(v.std() - 1.0) < 3e-3
    # quantile-table tails reach about 4.3 sigma
    assert 4.0 < np.abs(v).max() < 4.5
    u = synth.uniform_f32(11, 3, (100000,), -0.1, 0.1)
    assert u.min() >= -0.1 and u.max() < 0.1 and abs(u.mean()) < 2e-3


def test_fp8_bank_roundtrip_error():
    codes, s = synth.fp8_bank(3, 4, 0, 1, 256, 256, 0.02)
    w = synth.normal_f32(3, 4, (256, 256), 0.02)
    deq = O.decode_matrix("fp8", {"w": codes[0], "scale": s[0]})
    blk_amax = np.abs(w.reshape(2, 128, 2, 128)).max(axis=(1, 3))
    assert np.allclose(s[0], (blk_amax / np.float32(448)).astype(np.float32), rtol=0, atol=0)
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 above the subnormal range
    big = np.abs(w) > np.repeat(np.repeat(s[0], 128, 0), 128, 1) * 2.0 ** -6
    assert np.all(np.abs(deq - w)[big] <= np.abs(w)[big] * 2.0 ** -4 + 1e-12)


def test_mxfp4_bank_roundtrip_error():
    packed, sc = synth.mxfp4_bank(3, 4, 0, 1, 64, 256, 0.02)
    w = synth.normal_f32(3, 4, (64, 256), 0.02)
    deq = O.decode_matrix("mxfp4", {"w": packed[0], "scale": sc[0]})
    # every block's scale is 2^(floor(log2 amax) - 2): the largest element lands in [4, 8)
    amax = np.abs(w.reshape(64, 8, 32)).max(axis=2)
    ratio = amax / O.e8m0_to_f64(sc[0])
    assert np.all((ratio >= 4) & (ratio < 8))
    # E2M1 steps are at most 2 (between 4 and 6): error <= 1 scale unit up to 6 units,
    # and magnitudes in (6, 8) units saturate to 6 (error < 2 units)
    unit = O.e8m0_to_f64(sc[0])[:, :, None]
    err = np.abs(deq - w).reshape(64, 8, 32)
    inside = np.abs(w).reshape(64, 8, 32) <= 6 * unit
    assert np.all(err[inside] <= unit.repeat(32, 2)[inside])
    assert np.all(err <= 2 * unit)


def test_bf16_problem_bytes_deterministic():
    cfg = CONFIGS["tiny_fp32"].with_(act="bf16", wdt="bf16", out="bf16")
    p1, p2 = host_problem(cfg), host_problem(cfg)
    assert np.array_equal(p1.x, p2.x) and np.array_equal(p1.routed.w13(3)["w"], p2.routed.w13(3)["w"])


def test_preroute_counts_dirichlet():
    cfg = CONFIGS["ep32_mxfp4"]
    idx, w = preroute(cfg)
    counts = np.bincount(idx[:, 0], minlength=cfg.E)
    assert counts.sum() == cfg.T and idx.shape == (cfg.T, 1)
    assert counts.max() > 2 * cfg.T / cfg.E     # alpha = 0.5 gives uneven loads
    assert w.min() >= 0 and w.max() < 1


def test_prefill_skew_top10_share():
    """r1_prefill's routing (oracle, all 8192 tokens) gives the top 10% of experts 40% +- 1%."""
    cfg = CONFIGS["r1_prefill"]
    p = host_problem(cfg)
    r = O.route(O.bf16_to_f64(p.x), O.bf16_to_f64(p.wr), p.bias, cfg.k, cfg.score, cfg.scale)
    counts = np.bincount(r["topk_idx"].reshape(-1), minlength=cfg.E)
    share = np.sort(counts)[::-1][:26].sum() / counts.sum()
    assert abs(share - 0.40) <= 0.01, share
