"""Pins of the Lloyd-Max derivation (oracle/codebook.py) against the textbook
table, numerical integration and optimality - nothing here reuses the
derivation's own formulas."""

import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook


@pytest.fixture(scope="module")
def lm():
    return codebook.lloyd_max_gaussian()


def test_levels_match_published_table(lm, golden):
    g = golden("lloyd_max_n01_3bit.txt")
    levels, bounds, it = lm
    assert it < 1000
    pos = levels[4:]
    for c, ref in zip(pos, g["level"]):
        assert abs(c - ref) <= 1e-4, (c, ref)
    for b, ref in zip(bounds[3:], g["boundary"]):
        assert abs(b - ref) <= 1e-3, (b, ref)


def test_levels_symmetric_and_sorted(lm):
    levels, bounds, _ = lm
    assert all(a < b for a, b in zip(levels, levels[1:]))
    for k in range(8):
        assert levels[7 - k] == -levels[k]
    assert bounds[3] == 0.0


def test_centroid_condition_by_quadrature(lm):
    """Each level is the conditional mean of N(0,1) over its cell, checked by
    scipy quadrature (independent of the erfc closed form)."""
    levels, bounds, _ = lm
    edges = [-np.inf] + list(bounds) + [np.inf]
    for k, c in enumerate(levels):
        lo, hi = edges[k], edges[k + 1]
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), lo, hi, epsabs=1e-14, epsrel=1e-13)[0]
        m0 = stats.norm.cdf(hi) - stats.norm.cdf(lo)
        assert abs(m1 / m0 - c) < 1e-10, (k, m1 / m0, c)


def test_nearest_neighbour_condition(lm):
    levels, bounds, _ = lm
    for k, b in enumerate(bounds):
        assert abs(b - 0.5 * (levels[k] + levels[k + 1])) < 1e-15


def test_distortion_matches_table_and_quadrature(lm, golden):
    g = golden("lloyd_max_n01_3bit.txt")
    levels, bounds, _ = lm
    D = codebook.distortion(levels, bounds)
    assert abs(D - g["mse"]) < 2e-5
    edges = [-np.inf] + list(bounds) + [np.inf]
    Dq = sum(integrate.quad(lambda x, c=c: (x - c) ** 2 * stats.norm.pdf(x), edges[k], edges[k + 1],
                            epsabs=1e-14, epsrel=1e-12)[0] for k, c in enumerate(levels))
    assert abs(D - Dq) < 1e-10


def test_distortion_is_a_local_minimum(lm):
    """Moving any level (with boundaries re-optimised) or any boundary alone
    raises the mean squared error."""
    levels, bounds, _ = lm
    D0 = codebook.distortion(levels, bounds)
    for k in range(8):
        for eps in (1e-3, -1e-3):
            lv = list(levels)
            lv[k] += eps
            assert codebook.distortion(lv, codebook.boundaries_of(lv)) > D0
    for k in range(7):
        for eps in (1e-3, -1e-3):
            bd = list(bounds)
            bd[k] += eps
            assert codebook.distortion(levels, bd) > D0


def test_monte_carlo_distortion(lm):
    levels, bounds, _ = lm
    x = np.random.default_rng(7).standard_normal(2_000_000)
    idx = np.searchsorted(np.asarray(bounds), x, side="right")
    mse = np.mean((x - np.asarray(levels)[idx]) ** 2)
    # standard error of the mean of (x-Q(x))^2 is ~ 4e-5 here
    assert abs(mse - codebook.distortion(levels, bounds)) < 3e-4


def test_codec_table_grid_and_exactness(lm):
    levels, _, _ = lm
    q, thr = codebook.codec_table()
    ints = codebook.codec_table_integers()
    for c, qc, n in zip(levels, q, ints):
        assert qc * 2 ** 15 == n
        assert abs(qc - c) <= 2 ** -16
        assert np.float32(qc) == qc            # exact in float32
    for k, t in enumerate(thr):
        assert t == 0.5 * (q[k] + q[k + 1])
        assert np.float32(t) == t
        assert (t * 2 ** 16) == int(t * 2 ** 16)
    assert thr[3] == 0.0
    # any sum of 128 levels with signs is an integer multiple of 2^-15 below 2^24 units
    assert 128 * max(ints) < 2 ** 24
    # the grid costs almost nothing in distortion
    D_opt = codebook.distortion(*lm[:2])
    D_q = codebook.distortion(q, thr)
    assert 0 <= D_q - D_opt < 1e-9
    # the published 4-digit values hold for the stored table too
    for qc, ref in zip(q[4:], (0.2451, 0.7560, 1.3440, 2.1520)):
        assert abs(qc - ref) <= 1e-4


def test_gaussian_tail_helpers_against_scipy():
    for lo, hi in [(-np.inf, -1.7), (-1.7, -0.3), (-0.3, 0.4), (0.4, 2.5), (2.5, np.inf), (5.0, 9.0)]:
        p = codebook.cell_probability(lo, hi)
        ref = stats.norm.sf(lo) - stats.norm.sf(hi) if lo >= 0 else stats.norm.cdf(hi) - stats.norm.cdf(lo)
        assert math.isclose(p, ref, rel_tol=1e-12, abs_tol=1e-300)
