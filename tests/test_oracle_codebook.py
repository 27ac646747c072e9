"""Pins of the oracle's codebook construction and scalar comparator.

[FQ 2.2] (radii, directions, Lloyd-Max), [FQ 2.3] (rate), [FQ 3.2]
(Theorem 2), [TQ 1.3, 2.1, 3.1, 3.3] (scalar Lloyd-Max, printed D_mse and
centroids, Shannon lower bound).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import gammaln

from oracle import codebook, scalar, source

from conftest import GOLDEN_DIR


# ------------------------------------------------------------------ radii
def test_kronecker_roots():
    assert abs(codebook.kronecker_root(1) - (1 + math.sqrt(5)) / 2) < 1e-15
    assert abs(codebook.kronecker_root(2) - 1.3247179572447460) < 1e-15
    for k in range(1, 10):
        x = codebook.kronecker_root(k)
        assert x > 1 and abs(x ** (k + 1) - x - 1) < 1e-13


def test_k2_radii_closed_form():
    t = (np.arange(256) + 0.5) / 256
    r = codebook.radii_from_levels(t, 64, 2)
    assert np.max(np.abs(r ** 2 - (1 - (1 - t) ** (4 / 64)))) < 1e-13


@pytest.mark.parametrize("k", [2, 3, 4, 8])
def test_radius_law_is_companded_density(k):
    # Bennett-Gersho: point density lambda(z) ~ f_{d,k}(z)^{k/(k+2)}.  The law of
    # s = r^2 for points distributed as lambda is s^{k/2-1} lambda(sqrt s) up to a
    # constant; its ratio to the Beta(a, b) density must be constant in s.
    d = 64
    a, b = codebook.radius_law(d, k)
    s = np.linspace(0.01, 0.5, 50)
    lam = source.block_density(np.sqrt(s)[:, None] * np.eye(k)[0][None, :], d) ** (k / (k + 2))
    law = s ** (k / 2 - 1) * lam
    ratio = law / stats.beta(a, b).pdf(s)
    assert np.max(ratio) / np.min(ratio) - 1 < 1e-10


# ------------------------------------------------------------- directions
@pytest.mark.parametrize("k", [3, 4, 8])
def test_direction_map_is_uniform_on_sphere(k):
    w = np.random.default_rng([12, k]).random((1 << 14, k - 1))
    u = codebook.sphere_direction(w, k)
    assert np.max(np.abs(np.sum(u * u, axis=1) - 1)) < 1e-12
    # every coordinate of a uniform point on S^{k-1}: (1+x)/2 ~ Beta((k-1)/2, (k-1)/2)
    a = (k - 1) / 2
    for j in range(k):
        assert stats.kstest((1 + u[:, j]) / 2, stats.beta(a, a).cdf).pvalue > 1e-4


def test_k2_start_is_golden_spiral():
    C = codebook.initial_codebook(64, 2, 64)
    r = np.linalg.norm(C, axis=1)
    assert np.all(np.diff(r) > 0)                       # radius grows with n
    ang = np.arctan2(C[:, 1], C[:, 0])
    step = np.mod(np.diff(ang), 2 * np.pi)
    golden = 2 * np.pi * (1 / codebook.GOLDEN)          # 2 pi / phi (= -golden angle mod 2 pi)
    assert np.max(np.abs(step - golden)) < 1e-12


def test_k3_start_is_fibonacci_sphere():
    N = 512
    C = codebook.initial_codebook(64, 3, N)
    u = C / np.linalg.norm(C, axis=1, keepdims=True)
    n = np.arange(N)
    assert np.max(np.abs(u[:, 0] - (1 - 2 * (n + 0.5) / N))) < 1e-12
    az = np.mod(np.arctan2(u[:, 2], u[:, 1]) / (2 * np.pi), 1.0)
    assert np.max(np.abs(np.mod(az - n / codebook.GOLDEN + 0.5, 1.0) - 0.5)) < 1e-9


def test_roberts_sequence():
    k = 4
    P = codebook.lowdisc_points(k, 100)
    phi = codebook.kronecker_root(k)
    step = np.mod(P[1] - P[0], 1.0)
    assert np.max(np.abs(step - phi ** -(np.arange(k) + 1.0))) < 1e-12
    assert np.max(np.abs(P[0] - 0.5)) == 0


# ------------------------------------------------------------------ Lloyd
def naive_nearest(C, X):
    out = []
    for x in X:
        best, bi = None, -1
        for i, c in enumerate(C):
            dd = sum((float(a) - float(b)) ** 2 for a, b in zip(x, c))
            if best is None or dd < best:
                best, bi = dd, i
        out.append(bi)
    return np.array(out)


@pytest.mark.parametrize("k,N", [(2, 16), (3, 32), (8, 16)])
def test_nearest_matches_naive_loop(k, N):
    C = codebook.initial_codebook(64, k, N)
    X = source.sample_blocks(64, k, 300, [13, k])
    idx, d2 = codebook.nearest(C, X)
    assert np.array_equal(idx, naive_nearest(C, X))
    assert np.allclose(d2, np.sum((X - C[idx]) ** 2, axis=1), rtol=1e-12, atol=1e-15)


def test_unit_distortion_partial_block_hand_worked():
    # d = 4, k = 3: one full block and a one-coordinate last block [FQ 2.3:
    # blocks of k coordinates, the last one shorter].  Codewords (0,0,0) and
    # (1,0,0); blocks (0.4,5,5) and (0.6,5,5).  Full blocks: both at squared
    # distance 50.16 (0.16 + 25 + 25 from the nearer codeword).  Last block
    # (first coordinate only): 0.4 -> 0 and 0.6 -> 1, both 0.16.  So
    # D = (nb - 1) e_full + e_part = 50.16 + 0.16.
    C = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
    X = np.array([[0.4, 5.0, 5.0], [0.6, 5.0, 5.0]])
    D, e_full, e_part = codebook.unit_distortion(C, 4, X)
    assert math.isclose(e_full, 50.16, rel_tol=1e-14)
    assert math.isclose(e_part, 0.16, rel_tol=1e-12)
    assert math.isclose(D, 50.32, rel_tol=1e-14)
    # d = 7, k = 3: two full blocks, the last one of one coordinate
    D7, _, _ = codebook.unit_distortion(C, 7, X)
    assert math.isclose(D7, 2 * 50.16 + 0.16, rel_tol=1e-14)
    # k divides d: no partial term
    D6, e6, p6 = codebook.unit_distortion(C, 6, X)
    assert p6 is None and math.isclose(D6, 2 * 50.16, rel_tol=1e-14)


def test_lloyd_monotone_and_centroid_condition():
    X = source.sample_blocks(64, 2, 1 << 14, [14])
    C, hist = codebook.lloyd(codebook.initial_codebook(64, 2, 16), X, max_iter=400, tol=1e-13)
    assert all(b <= a * (1 + 1e-14) for a, b in zip(hist, hist[1:]))
    idx, _ = codebook.nearest(C, X)
    for n in range(16):
        cell = X[idx == n]
        assert len(cell) > 0
        assert np.linalg.norm(C[n] - cell.mean(axis=0)) < 1e-6


def test_lloyd_k1_matches_quadrature():
    # MC Lloyd at k = 1 on the source must reproduce the quadrature Lloyd-Max
    # of f_X within Monte Carlo error ([TQ 3.1]).
    d = 64
    X = source.sample_blocks(d, 1, 1 << 18, [15])
    c_q, D_q = scalar.scalar_lloyd_max(d, 2)
    C, hist = codebook.lloyd(np.sort(X[:4], axis=0), X, max_iter=500, tol=1e-12)
    c_mc = np.sort(C[:, 0])
    assert np.max(np.abs(c_mc - c_q)) < 0.01 * np.max(np.abs(c_q))
    assert abs(d * hist[-1] - D_q) < 0.01 * D_q


# ------------------------------------------------------- scalar comparator
@pytest.fixture(scope="module")
def scalar64():
    return {b: scalar.scalar_lloyd_max(64, b) for b in (1, 2, 3, 4)}


def test_scalar_b1_closed_form(scalar64):
    # b = 1: the centroids are +-E[x | x > 0] = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    d = 64
    c1 = math.exp(gammaln(d / 2) - 0.5 * math.log(math.pi) - gammaln((d + 1) / 2))
    c, D = scalar64[1]
    assert np.max(np.abs(np.abs(c) - c1)) < 1e-10
    # and D = d (E x^2 - c1^2) = d (1/d - c1^2)
    assert abs(D - d * (1 / d - c1 ** 2)) < 1e-9


def test_scalar_large_d_limit_matches_printed():
    g = json.load(open(os.path.join(GOLDEN_DIR, "turboquant_printed.json")))
    d = 4096
    for b in (1, 2, 3, 4):
        c, D = scalar.scalar_lloyd_max(d, b)
        printed = g["d_mse_by_bits"][str(b)]
        dec = g["d_mse_printed_decimals"][str(b)]
        assert round(D, dec) == pytest.approx(printed, abs=1e-12), (b, D)
        if b == 1:
            assert abs(c[-1] * math.sqrt(d) - math.sqrt(2 / math.pi)) < 2e-3
        if b == 2:
            pos = c[2:] * math.sqrt(d)
            assert round(pos[0], 3) == pytest.approx(0.453) and round(pos[1], 2) == pytest.approx(1.51)


def test_scalar_within_bounds(scalar64):
    for b, (c, D) in scalar64.items():
        assert D >= 4.0 ** -b                                  # [TQ 3.3] lower bound
        assert D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -b     # [TQ 1.3] upper bound
        assert np.all(np.diff(c) > 0) and np.allclose(c, -c[::-1], atol=1e-12)


def test_scalar_d64_near_printed(scalar64):
    g = json.load(open(os.path.join(GOLDEN_DIR, "turboquant_printed.json")))
    for b in (1, 2, 4):
        assert abs(scalar64[b][1] - g["d_mse_by_bits"][str(b)]) < 0.05 * g["d_mse_by_bits"][str(b)]
