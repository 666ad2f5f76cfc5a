"""Pins for the oracle's random source and rotation (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


def test_mix64_matches_published_splitmix64_sequence():
    # SplitMix64 = finaliser applied to a Weyl sequence; its published outputs
    # for state 1234567 pin the finaliser's shifts and multipliers.
    expect = _golden_ints("splitmix64_1234567.txt")
    state = 1234567
    got = []
    for _ in expect:
        state = (state + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        got.append(int(O.mix64(np.uint64(state))))
    assert got == expect


def test_gaussian_stream_is_standard_normal():
    z = O.gaussian_stream(0, 0, O.MAT_PI, np.arange(1 << 20))
    assert abs(z.mean()) < 5.0 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 5.0 * math.sqrt(2.0 / z.size)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # fourth moment of N(0,1) is 3
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_gaussian_streams_are_distinct_and_uncorrelated():
    e = np.arange(200000)
    a = O.gaussian_stream(7, 0, O.MAT_PI, e)
    b = O.gaussian_stream(7, 1, O.MAT_PI, e)
    c = O.gaussian_stream(7, 0, O.MAT_S, e)
    d = O.gaussian_stream(8, 0, O.MAT_PI, e)
    for other in (b, c, d):
        r = np.corrcoef(a, other)[0, 1]
        assert abs(r) < 5.0 / math.sqrt(e.size)
    # reproducible
    assert np.array_equal(a, O.gaussian_stream(7, 0, O.MAT_PI, e))


def test_box_muller_single_value_by_hand():
    # element 0 of stream (seed 0, group 0, Pi) evaluated step by step with
    # Python integers, independently of the vectorised code path
    M = (1 << 64) - 1

    def fin(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    key = fin(0) ^ ((16 * 0 + 0) << 32)
    h0, h1 = fin(key ^ 0), fin(key ^ 1)
    u1 = ((h0 >> 11) + 1) / 2.0 ** 53
    u2 = (h1 >> 11) / 2.0 ** 53
    z = math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2)
    assert O.gaussian_stream(0, 0, O.MAT_PI, [0])[0] == pytest.approx(z, rel=1e-15, abs=1e-15)


def _gram_schmidt(g):
    # classical Gram–Schmidt on the columns, pure Python loops
    d = g.shape[0]
    q = np.zeros_like(g)
    for k in range(d):
        v = g[:, k].copy()
        for j in range(k):
            v -= np.dot(q[:, j], g[:, k]) * q[:, j]
        q[:, k] = v / math.sqrt(float(np.dot(v, v)))
    return q


@pytest.mark.parametrize("d", [3, 8, 17])
def test_rotation_equals_gram_schmidt_of_gaussian(d):
    # diag(R) > 0 makes Q the Gram–Schmidt basis of G's columns
    g = O.gaussian_matrix(11, 2, O.MAT_PI, d, d)
    assert np.allclose(O.rotation(d, 11, 2), _gram_schmidt(g), atol=1e-10)


@pytest.mark.parametrize("d", [2, 128, 200])
def test_rotation_is_orthogonal(d):
    pi = O.rotation(d, 0, 0)
    assert np.max(np.abs(pi.T @ pi - np.eye(d))) < 1e-12
    assert abs(abs(np.linalg.det(pi)) - 1.0) < 1e-9
    p32 = pi.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(p32.T @ p32 - np.eye(d))) < 1e-6


def test_rotation_columns_are_haar_first_column_uniform_on_sphere():
    # Pi e_1 = G[:,0]/||G[:,0]||: over many seeds each coordinate follows f_d
    d = 16
    vals = np.array([O.rotation(d, s, 0)[0, 0] for s in range(3000)])
    assert stats.kstest(vals, lambda x: O.coord_cdf(x, d)).pvalue > 1e-3


def test_rotated_coordinates_follow_the_pages_density():
    # y = Pi x/||x|| for the 4096 seeded N(0,1) vectors of the parity workload:
    # one coordinate per vector against F_d
    import workloads

    d = 128
    x = workloads.parity_vectors().astype(np.float64)
    pi = O.rotation(d, 0, 0)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = u @ pi.T
    for j in (0, 37, 127):
        assert stats.kstest(y[:, j], lambda t: O.coord_cdf(t, d)).pvalue > 1e-3
    # histogram vs density (chi-square style, coarse)
    hist, edges = np.histogram(y.ravel(), bins=40, range=(-0.35, 0.35))
    expect = (O.coord_cdf(edges[1:], d) - O.coord_cdf(edges[:-1], d)) * y.size
    mask = expect > 50
    assert np.max(np.abs(hist[mask] - expect[mask]) / np.sqrt(expect[mask])) < 6.0


@pytest.mark.parametrize("d", [2, 3])
def test_rotated_low_dimensional_coordinates_follow_the_law(d):
    """y = Pi x/||x|| at d = 2 (arcsine law) and d = 3 (uniform law): one
    coordinate of 5000 seeded Gaussian vectors against F_d."""
    x = np.random.default_rng(40 + d).standard_normal((5000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = u @ O.rotation(d, 3, 0).T
    for j in range(d):
        assert stats.kstest(y[:, j], lambda t: O.coord_cdf(t, d)).pvalue > 1e-3
