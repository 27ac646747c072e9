"""Pins of the oracle's rotation and source against what the pages and mathematics fix.

Rotation: [TQ 3.1] (QR of a Gaussian matrix) and [FQ 2.3] (shared Haar
rotation).  Source: [FQ 2.1] and [BSQ key design 1] (block density, polar
split), [TQ 2] (coordinate law).
"""
import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import rotation, source


def test_rotation_orthogonal():
    Pi = rotation.make_rotation(64, 0)
    assert np.max(np.abs(Pi.T @ Pi - np.eye(64))) <= 1e-12
    assert np.max(np.abs(Pi @ Pi.T - np.eye(64))) <= 1e-12
    assert abs(abs(np.linalg.det(Pi)) - 1.0) <= 1e-12


def test_rotation_matches_cholesky_gram_schmidt():
    # The QR factor with a positive-diagonal R is unique: Q = G R^-1 with
    # R^T R = G^T G (Cholesky).  An independent construction of the same matrix.
    G = rotation.gaussian_matrix(64, 0)
    R = np.linalg.cholesky(G.T @ G).T
    Q = np.linalg.solve(R.T, G.T).T
    assert np.max(np.abs(Q - rotation.make_rotation(64, 0))) <= 1e-9


def test_rotation_is_haar_in_distribution():
    # For a Haar rotation, Pi e_0 is uniform on the sphere, so Pi[0, 0] follows
    # the coordinate law f_X of [TQ 2]; (1 + x)/2 ~ Beta((d-1)/2, (d-1)/2).
    # A missing sign fix biases this entry's sign and fails the test.
    d = 16
    vals = np.array([rotation.make_rotation(d, s)[0, 0] for s in range(3000)])
    a = (d - 1) / 2.0
    p = stats.kstest((1 + vals) / 2, stats.beta(a, a).cdf).pvalue
    assert p > 1e-3
    assert abs(np.mean(vals > 0) - 0.5) < 0.05


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
def test_block_density_normalised(k):
    # Integrate f_{d,k} over the unit ball in polar form: area(S^{k-1}) r^{k-1} f(r) dr.
    d = 64
    area = 2 * np.pi ** (k / 2) / special.gamma(k / 2)
    f = lambda r: area * r ** (k - 1) * source.block_density(np.array([[r] + [0.0] * (k - 1)]), d)[0]
    val = integrate.quad(f, 0, 1, epsabs=1e-13, limit=200)[0]
    assert abs(val - 1.0) < 1e-9


def test_coordinate_density_is_k1_block_density():
    x = np.linspace(-0.99, 0.99, 41)
    a = source.coordinate_density(x, 64)
    b = source.block_density(x[:, None], 64)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("k", [2, 3, 4, 8])
def test_sampler_radius_is_beta(k):
    d = 64
    z = source.sample_blocks(d, k, 1 << 15, [7, k])
    r2 = np.sum(z * z, axis=1)
    p = stats.kstest(r2, stats.beta(k / 2, (d - k) / 2).cdf).pvalue
    assert p > 1e-3


@pytest.mark.parametrize("k", [2, 3, 8])
def test_sampler_matches_polar_split(k):
    d = 64
    a = source.sample_blocks(d, k, 1 << 14, [8, k])
    b = source.sample_blocks_polar(d, k, 1 << 14, [9, k])
    for j in range(k):
        assert stats.ks_2samp(a[:, j], b[:, j]).pvalue > 1e-3
    ra = np.sum(a * a, axis=1)
    rb = np.sum(b * b, axis=1)
    assert stats.ks_2samp(ra, rb).pvalue > 1e-3


def test_sampler_angle_uniform_k2():
    z = source.sample_blocks(64, 2, 1 << 15, [10])
    ang = np.mod(np.arctan2(z[:, 1], z[:, 0]), 2 * np.pi)
    assert stats.kstest(ang / (2 * np.pi), "uniform").pvalue > 1e-3


def test_sampler_coordinate_law_k1():
    d = 64
    z = source.sample_blocks(d, 1, 1 << 15, [11])[:, 0]
    a = (d - 1) / 2
    assert stats.kstest((1 + z) / 2, stats.beta(a, a).cdf).pvalue > 1e-3
    # and the density formula itself integrates to that CDF
    cdf_quad = integrate.quad(lambda t: source.coordinate_density(np.array([t]), d)[0], -1, 0.1)[0]
    assert abs(cdf_quad - stats.beta(a, a).cdf(0.55)) < 1e-10
