"""Pins of the oracle's E4M3 quantizer (the FP8 attention's inputs).

Independent checks: the format's landmarks (127 non-negative finite codes,
largest 448, smallest subnormal 2^-9, smallest normal 2^-6, 8 codes per
binade), rounding against a brute-force nearest search over the grid with
ties to the even code, and the per-problem scale mapping max|x| to 448.
"""
import numpy as np

import oracle


def test_e4m3_grid_landmarks():
    g = oracle.e4m3_grid()
    assert len(g) == 127 and g[0] == 0.0
    assert g[-1] == 448.0 and g[1] == 2.0 ** -9 and g[8] == 2.0 ** -6
    assert np.all(np.diff(g) > 0)
    # 8 codes per binade above the subnormals, each a power of two times 1 + m/8
    for e in range(-6, 9):
        b = g[(g >= 2.0 ** e) & (g < 2.0 ** (e + 1))]
        assert len(b) == (7 if e == 8 else 8)
        np.testing.assert_array_equal(b, 2.0 ** e * (1 + np.arange(len(b)) / 8))


def test_e4m3_round_is_nearest_with_ties_to_even():
    g = oracle.e4m3_grid()
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 5000), rng.uniform(-1, 1, 5000) * 2.0 ** rng.integers(-12, 2, 5000)])
    r = oracle.e4m3_round(x)
    for xi, ri in zip(x[:2000], r[:2000]):
        d = np.abs(g - abs(xi))
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert ri == np.copysign(g[code], xi)
    mids = (g[1:] + g[:-1]) / 2                                     # exact midpoints
    rm = oracle.e4m3_round(mids)
    lo_even = np.arange(len(g) - 1) % 2 == 0
    np.testing.assert_array_equal(rm, np.where(lo_even, g[:-1], g[1:]))


def test_scale_maps_the_largest_magnitude_to_448():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((100, 16)) * 3).astype(np.float32)
    s = oracle.fp8_scale(x)
    assert s == np.float32(np.max(np.abs(x)) / 448.0)
    assert oracle.fp8_ratio(x) == np.float32(448.0 / np.max(np.abs(x)))
    q = oracle.fp8_quantize(x)
    assert np.max(np.abs(q)) == 448.0
    assert oracle.fp8_scale(np.zeros((3, 4))) == 1.0 and oracle.fp8_ratio(np.zeros((3, 4))) == 1.0
    np.testing.assert_array_equal(oracle.fp8_quantize(np.zeros((3, 4))), 0.0)
    # dequantized values stay within half a code step (2^-4 relative above the subnormals)
    deq = q * s
    big = np.abs(x) >= 2.0 ** -6 * s
    assert np.all(np.abs(deq[big] - x[big]) <= 2.0 ** -4 * np.abs(x[big]) * (1 + 1e-6))
