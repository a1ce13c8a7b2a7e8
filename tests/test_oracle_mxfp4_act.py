"""Pins of the oracle's MXFP4 activation quantiser (the W4A4 path): the E2M1 encoder against
the format's own value table, rounding and saturation worked by hand, and the OCP MX shared
scale against its definition on blocks whose answer is known."""
import numpy as np

import oracle as O

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_every_code_round_trips():
    codes = np.arange(16, dtype=np.uint8)
    vals = O.e2m1_to_f64(codes)
    back = O.encode_e2m1_rne_sat(vals)
    assert back.tolist() == codes.tolist()   # including -0 -> 0x8


def test_ties_go_to_the_even_code_and_large_values_saturate():
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             0.2499: 0.0, 0.2501: 0.5, 5.01: 6.0, 7.0: 6.0, 1e9: 6.0, 0.0: 0.0}
    for v, want in cases.items():
        for sgn in (1.0, -1.0):
            got = O.e2m1_to_f64(O.encode_e2m1_rne_sat(np.array([sgn * v])))[0]
            assert got == sgn * want or (want == 0.0 and got == 0.0), (sgn * v, got)


def test_nearest_value_by_brute_force():
    rng = np.random.default_rng(7)
    v = rng.uniform(-8, 8, 20000)
    got = O.e2m1_to_f64(O.encode_e2m1_rne_sat(v))
    g = np.array(GRID)
    best = g[np.abs(np.abs(v)[:, None] - g[None, :]).argmin(axis=1)] * np.sign(v)
    # away from the midpoints (ties are pinned above) the nearest grid value is unique
    mids = (g[1:] + g[:-1]) / 2
    clear = np.abs(np.abs(v)[:, None] - mids[None, :]).min(axis=1) > 1e-9
    assert np.array_equal(got[clear], best[clear])


def test_shared_scale_is_the_ocp_mx_rule():
    """amax 3.0 -> floor(log2 3) = 1 -> e = -1: the block maps onto [-6, 6] exactly; amax
    4 -> e = 0; amax 7.9 -> e = 0 and 7.9 saturates to 6; a zero block takes e = 0."""
    blocks = np.zeros((4, 32), np.float32)
    blocks[0, :3] = [3.0, -1.5, 0.75]
    blocks[1, :2] = [4.0, 1.0]
    blocks[2, :2] = [7.9, -2.0]
    codes, sc, deq = O.quantise_rows_mxfp4(blocks)
    assert sc.tolist() == [[126], [127], [127], [127]]
    assert deq[0, :3].tolist() == [3.0, -1.5, 0.75]
    assert deq[1, :2].tolist() == [4.0, 1.0]
    assert deq[2, :2].tolist() == [6.0, -2.0]
    assert (deq[3] == 0).all() and (codes[3] == 0).all()


def test_representable_blocks_are_fixed_points_and_error_is_bounded():
    rng = np.random.default_rng(8)
    R, C = 64, 256
    e = rng.integers(-20, 20, (R, C // 32))
    codes = rng.integers(0, 16, (R, C)).astype(np.uint8)
    codes[:, ::32] = 6 | (codes[:, ::32] & 8)   # each block's largest magnitude is 4 * 2^e
    v = (O.e2m1_to_f64(codes).reshape(R, C // 32, 32) * np.exp2(e)[:, :, None]).reshape(R, C)
    c2, s2, deq = O.quantise_rows_mxfp4(v.astype(np.float32))
    assert np.array_equal(deq, v)
    assert np.array_equal(s2.astype(np.int64) - 127, e)
    # arbitrary values: error at most one grid step (2 * 2^e at the top) plus saturation
    x = rng.standard_normal((R, C)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (R, 1)))
    _, s3, d3 = O.quantise_rows_mxfp4(x)
    scale = np.repeat(np.exp2(s3.astype(np.float64) - 127), 32, axis=1)
    assert (np.abs(d3 - x) <= 2.0 * scale + 1e-300).all()
