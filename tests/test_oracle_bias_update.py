"""Pins of the oracle's selection-bias update (auxiliary-loss-free balancing).

The pages name the technique and its purpose, not its rule, so the pins are the rule's
hand-worked value, exact-arithmetic properties, and the purpose itself: iterated on a
router whose scores favour some experts, the update must even out the expert loads.
"""
import numpy as np

import oracle as O


def test_hand_worked_step_uses_the_mean_load():
    """E = 4, loads 8, 0, 0, 0: the mean is 2, so expert 0 is lowered by u and the three
    idle experts are raised by u (a median reading would leave the idle ones alone)."""
    got = O.bias_update(np.array([0.25, -1.0, 0.0, 3.0], np.float32), [8, 0, 0, 0], 0.5)
    assert got.dtype == np.float32
    assert got.tolist() == [-0.25, -0.5, 0.5, 3.5]


def test_balanced_loads_are_a_fixed_point():
    rng = np.random.default_rng(1)
    bias = rng.standard_normal(64).astype(np.float32)
    for c in (0, 1, 37):
        got = O.bias_update(bias, np.full(64, c, np.int32), 1e-3)
        assert np.array_equal(got.view(np.uint32), bias.view(np.uint32))


def test_steps_are_exactly_u_and_follow_integer_comparison():
    """With a zero bias and u a power of two every step is exact: each expert moves by
    +u, -u or 0, decided by comparing E * load with the total load in integers."""
    rng = np.random.default_rng(2)
    for E in (1, 7, 256, 1024):
        counts = rng.integers(0, 50, E).astype(np.int32)
        counts[: E // 3] = counts[0]             # several experts exactly tied
        total = int(counts.sum())
        u = 2.0 ** -7
        got = O.bias_update(np.zeros(E, np.float32), counts, u).astype(np.float64)
        below = E * counts.astype(np.int64) < total
        above = E * counts.astype(np.int64) > total
        want = np.where(below, u, np.where(above, -u, 0.0))
        assert np.array_equal(got, want)


def test_exact_mean_boundaries_at_large_counts():
    """Loads one apart around a mean that is not an integer, at counts near the int32
    range: the sign must still follow the exact rational comparison."""
    E = 1000
    base = 2_000_000
    counts = np.full(E, base, np.int64)
    counts[0] += 1                               # mean = base + 1/1000
    got = O.bias_update(np.zeros(E, np.float32), counts, 1.0)
    assert got[0] == -1.0 and (got[1:] == 1.0).all()


def test_relabelling_experts_permutes_the_update():
    rng = np.random.default_rng(3)
    E = 96
    bias = rng.standard_normal(E).astype(np.float32)
    counts = rng.integers(0, 40, E)
    p = rng.permutation(E)
    a = O.bias_update(bias, counts, 0.01)[p]
    b = O.bias_update(bias[p], counts[p], 0.01)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_scaling_every_load_changes_nothing():
    rng = np.random.default_rng(4)
    bias = rng.standard_normal(33).astype(np.float32)
    counts = rng.integers(0, 20, 33)
    a = O.bias_update(bias, counts, 0.03)
    b = O.bias_update(bias, counts * 7, 0.03)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _load_ratio(s64, bias, k, E):
    idx = O.select_topk(O.selection_keys(s64, bias), k)
    c = np.bincount(idx.ravel(), minlength=E)
    return c, c.max() / c.mean()


def test_iterated_update_balances_a_skewed_router():
    """The purpose of the bias: router logits with a per-expert offset rising from 0 to 3
    send about 3.6x the mean load to the favourite expert; 400 steps of the update at
    u = 0.004 bring the largest load within 1.3x of the mean, while the weights stay those
    of the unbiased scores. The opposite sign makes the skew worse, which this detects."""
    rng = np.random.default_rng(5)
    T, E, k, u = 1024, 16, 2, 0.004
    logits = rng.standard_normal((T, E)) + np.linspace(0.0, 3.0, E)[None, :]
    s64 = O.scores(logits.astype(np.float32), "sigmoid")
    bias = np.zeros(E, np.float32)
    c, first = _load_ratio(s64, bias, k, E)
    ratios = []
    for _ in range(400):
        bias = O.bias_update(bias, c, u)
        c, r = _load_ratio(s64, bias, k, E)
        ratios.append(r)
    assert first >= 3.0
    assert max(ratios[-20:]) <= 1.3
    # weights of the balanced selection are renormalised unbiased scores
    idx = O.select_topk(O.selection_keys(s64, bias), k)
    w = O.routing_weights(s64, idx, 1.0)
    sel = np.take_along_axis(s64, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-15)


def test_step_is_the_ieee_fp32_sum_of_bias_and_fp32_step():
    """The bias and the step u are fp32 numbers and the new bias is their fp32 sum: equal,
    bit for bit, to torch's float32 add of b and u * sign (including -0 + 0 = +0 at the
    mean, and u values such as 0.01 that fp32 cannot hold exactly)."""
    import torch

    rng = np.random.default_rng(6)
    E = 512
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32)
    bias[:4] = [-0.0, 0.0, 1e-40, -1e-40]
    counts = rng.integers(0, 3, E).astype(np.int32)
    counts[:4] = 1                                   # choose the mean for the first four
    counts[4:] = np.where(np.arange(4, E) % 2 == 0, 0, 2)
    assert counts.sum() == E
    for u in (0.01, 1e-3, 2.0 ** -10, -0.3):
        got = O.bias_update(bias, counts, u)
        sgn = np.sign(counts.sum() / E - counts.astype(np.float64)).astype(np.float32)
        want = (torch.from_numpy(bias) + torch.tensor(u, dtype=torch.float32) *
                torch.from_numpy(sgn)).numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), u
    assert O.bias_update(np.array([-0.0], np.float32), [5], 0.01).view(np.uint32)[0] == 0
