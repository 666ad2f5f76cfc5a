"""Pins for the coordinate law and its Lloyd–Max codebook (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, special

from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quad(f, a, b):
    v, _ = integrate.quad(f, a, b, limit=400, epsabs=1e-14, epsrel=1e-12)
    return v


def _dens(d):
    return lambda x: float(O.coord_density(np.array([x]), d)[0])


@pytest.mark.parametrize("d", [3, 4, 16, 128, 200, 1536])
def test_density_normalised_and_unit_second_moment(d):
    f = _dens(d)
    s = 4.0 / math.sqrt(d) if d > 50 else 1.0
    pts = [-s, 0.0, s]
    mass = integrate.quad(f, -1, 1, points=pts, limit=400)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -1, 1, points=pts, limit=400)[0]
    assert mass == pytest.approx(1.0, abs=1e-9)
    assert d * m2 == pytest.approx(1.0, abs=1e-8)


@pytest.mark.parametrize("d", [5, 128, 1536])
def test_cdf_and_first_moment_match_quadrature(d):
    f = _dens(d)
    for a, b in [(-0.05, 0.02), (0.01, 0.09), (0.1, 0.3), (-1.0, -0.02)]:
        assert O.coord_cdf(b, d) - O.coord_cdf(a, d) == pytest.approx(_quad(f, a, b), abs=1e-11)
        assert O.cell_first_moment(a, b, d) == pytest.approx(_quad(lambda x: x * f(x), a, b), abs=1e-11)


@pytest.mark.parametrize("d", [3, 128, 200, 1536, 3072])
def test_one_bit_centroid_closed_form(d):
    lm = O.lloyd_max(d, 1)
    # conditional mean of the positive half by quadrature ...
    f = _dens(d)
    s = min(1.0, 6.0 / math.sqrt(d))
    half_mean = 2.0 * integrate.quad(lambda x: x * f(x), 0.0, 1.0, points=[s], limit=400)[0]
    assert lm.centroids[1] == pytest.approx(half_mean, rel=1e-8)
    # ... and the Gamma-ratio closed form Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2))
    cf = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert lm.centroids[1] == pytest.approx(cf, rel=1e-10)
    assert lm.centroids[0] == -lm.centroids[1]


def test_one_bit_shrinkage_is_about_36_percent():
    # [ttakun]: the 1-bit mse quantizer underestimates inner products by ~36%;
    # the shrinkage d*c_1^2 tends to 2/pi.
    a128 = 128 * O.lloyd_max(128, 1).centroids[1] ** 2
    assert a128 == pytest.approx(0.639111, abs=2e-6)
    assert 1.0 - a128 == pytest.approx(0.36, abs=0.005)
    big = 200000
    assert big * O.lloyd_max(big, 1).centroids[1] ** 2 == pytest.approx(2.0 / math.pi, abs=1e-5)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (200, 3), (1536, 4)])
def test_lloyd_max_optimality_conditions_by_quadrature(d, bits):
    lm = O.lloyd_max(d, bits)
    f = _dens(d)
    c, t = lm.centroids, lm.boundaries
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=1e-15)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        mass = _quad(f, a, b)
        mean = _quad(lambda x: x * f(x), a, b) / mass
        assert mean == pytest.approx(c[k], rel=1e-7, abs=1e-12)
    # distortion by direct quadrature of (x - Q(x))^2
    dist = sum(_quad(lambda x, ck=c[k]: (x - ck) ** 2 * f(x), edges[k], edges[k + 1]) for k in range(len(c)))
    assert d * dist == pytest.approx(lm.distortion, rel=1e-7)


def _gaussian_table():
    out = {}
    with open(os.path.join(GOLDEN, "gaussian_lloyd_max.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            left, right = line.split("|")
            parts = left.split()
            out[int(parts[0])] = ([float(v) for v in parts[1:]], float(right))
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_large_d_limit_is_the_gaussian_lloyd_max_quantizer(bits):
    levels, mse = _gaussian_table()[bits]
    d = 400000
    lm = O.lloyd_max(d, bits)
    pos = lm.centroids[len(lm.centroids) // 2:] * math.sqrt(d)
    assert np.allclose(pos, levels, atol=2e-4)
    assert lm.distortion == pytest.approx(mse, rel=2e-3)


def test_distortion_within_2_7x_of_the_shannon_bound():
    # [ttakun]: the mse is only ~2.7x above the information-theoretic lower
    # bound 4^-b; the ratio stays below sqrt(3)*pi/2 ~ 2.72 for b = 1..4.
    ratios = []
    for bits in (1, 2, 3, 4):
        r = O.lloyd_max(128, bits).distortion * 4 ** bits
        ratios.append(r)
        assert 1.0 < r < math.sqrt(3) * math.pi / 2
    assert all(a < b for a, b in zip(ratios, ratios[1:]))


def test_nearest_index_equals_brute_force_argmin():
    cd = O.make_codec(128, 4, O.MSE, 0)
    rng = np.random.default_rng(3)
    y = rng.normal(0, 1 / math.sqrt(128), 200000)
    t = cd.boundaries
    near = np.concatenate([t, np.nextafter(t, 1), np.nextafter(t, -1), [0.0, -0.0, 0.9, -0.9]])
    y = np.concatenate([y, near])
    got = O.nearest_index(cd, y)
    # brute force: count boundaries strictly below, in pure Python
    for i in range(0, len(y), 997):
        assert got[i] == sum(1 for tk in t if tk < y[i])
    for tk_i, tk in enumerate(t):
        assert O.nearest_index(cd, np.array([tk]))[0] == tk_i          # tie -> lower index
        assert O.nearest_index(cd, np.array([np.nextafter(tk, 1)]))[0] == tk_i + 1
    # away from the boundaries the index is the nearest (f64) centroid
    c = cd.centroids64
    far = np.min(np.abs(y[:, None] - cd.boundaries64[None, :]), axis=1) > 1e-8
    assert np.array_equal(got[far], np.argmin(np.abs(y[far, None] - c[None, :]), axis=1))


@pytest.mark.parametrize("bits", range(1, 9))
def test_three_dimensional_law_is_uniform_and_its_quantizer_is_the_uniform_one(bits):
    """At d = 3 the coordinate of a uniform point on the sphere is uniform on
    [-1, 1] (Archimedes' hat-box theorem: f_3 = 1/2), whose Lloyd–Max
    quantizer is the uniform one: c_k = (2k + 1)/L - 1, t_k = 2(k + 1)/L - 1,
    distortion d (2/L)^2 / 12 = 4^-b."""
    assert np.allclose(O.coord_density(np.linspace(-0.99, 0.99, 7), 3), 0.5, rtol=1e-14)
    lm = O.lloyd_max(3, bits)
    L = 1 << bits
    k = np.arange(L)
    assert np.allclose(lm.centroids, (2 * k + 1) / L - 1.0, atol=1e-14)
    assert np.allclose(lm.boundaries, 2.0 * (k[:-1] + 1) / L - 1.0, atol=1e-14)
    assert lm.distortion == pytest.approx(4.0 ** -bits, rel=1e-12)


def test_two_dimensional_law_is_the_arcsine_law():
    """d = 2: a uniform point on the circle has coordinates cos(theta), whose
    law is the arcsine law 1/(pi sqrt(1 - x^2)) with CDF 1/2 + asin(x)/pi; the
    1-bit centroid is E|cos theta| = 2/pi and its distortion 1 - 8/pi^2."""
    x = np.linspace(-0.999, 0.999, 41)
    assert np.allclose(O.coord_density(x, 2), 1.0 / (math.pi * np.sqrt(1.0 - x * x)), rtol=1e-13)
    assert np.allclose(O.coord_cdf(x, 2), 0.5 + np.arcsin(x) / math.pi, atol=1e-14)
    lm = O.lloyd_max(2, 1)
    assert lm.centroids[1] == pytest.approx(2.0 / math.pi, rel=1e-14)
    assert lm.distortion == pytest.approx(1.0 - 8.0 / math.pi ** 2, rel=1e-12)
    # the 2-bit quantizer by brute force: minimise the distortion of a
    # symmetric (-b, -a, a, b) codebook over a fine grid (boundaries at the
    # midpoints), the mean-square error integrated in closed form
    F = lambda t: 0.5 + np.arcsin(t) / math.pi                       # noqa: E731
    M1 = lambda t: -np.sqrt(1.0 - t * t) / math.pi                   # antiderivative of x f(x)
    M2 = lambda t: (np.arcsin(t) - t * np.sqrt(1.0 - t * t)) / (2 * math.pi)  # of x^2 f(x)

    def mse(a, b):
        m = 0.5 * (a + b)
        inner = (M2(m) - M2(0.0)) - 2 * a * (M1(m) - M1(0.0)) + a * a * (F(m) - F(0.0))
        outer = (M2(1.0) - M2(m)) - 2 * b * (M1(1.0) - M1(m)) + b * b * (F(1.0) - F(m))
        return 2 * 2 * (inner + outer)                               # both halves, d = 2
    grid = np.linspace(0.01, 0.99, 981)
    A, B = np.meshgrid(grid, grid, indexing="ij")
    ok = A < B
    vals = np.where(ok, mse(A, B), np.inf)
    i, j = np.unravel_index(np.argmin(vals), vals.shape)
    lm2 = O.lloyd_max(2, 2)
    assert lm2.centroids[2] == pytest.approx(grid[i], abs=2e-3)
    assert lm2.centroids[3] == pytest.approx(grid[j], abs=2e-3)
    assert lm2.distortion <= vals[i, j] + 1e-12


@pytest.mark.parametrize("d,bits", [(2, 8), (4, 8), (128, 7), (128, 8), (1536, 8)])
def test_many_level_codebooks_are_fixed_points(d, bits):
    """With 128 or 256 levels the returned codebook satisfies both Lloyd–Max
    conditions: applying the map once more moves no centroid by more than
    1e-10, centroids ascend, and the distortion keeps the 4^-b scaling."""
    lm = O.lloyd_max(d, bits)
    c = lm.centroids
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    mass = O.coord_cdf(edges[1:], d) - O.coord_cdf(edges[:-1], d)
    again = O.cell_first_moment(edges[:-1], edges[1:], d) / mass
    assert np.max(np.abs(again - c)) < 1e-10
    assert np.all(np.diff(c) > 0)
    assert 0.3 < lm.distortion * 4 ** bits < 2.72
