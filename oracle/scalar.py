"""Scalar product specialisation (k = 1): TurboQuant's Lloyd-Max table (oracle).

[TQ 3.1]: quantising one rotated coordinate is a one-dimensional continuous
k-means problem on f_X with 2^b levels; the optimum is a Voronoi partition of
[-1, 1] whose boundaries are midpoints between sorted centroids, and each
centroid is the conditional mean of its cell.  [FQ 3.2] (Theorem 2) compares
the vector code against exactly this product code at matched rate.

Computed here by deterministic quadrature (scipy.integrate.quad) of f_X from
[TQ 2]; the MSE per unit vector is d * E(x - c(x))^2.
"""
import numpy as np
from scipy import integrate
from scipy.special import betaincinv

from .source import coordinate_density


def _cell_moments(a, b, d):
    f = lambda x: coordinate_density(np.array([x]), d)[0]
    opts = dict(epsabs=1e-15, epsrel=1e-13, limit=200)
    m0 = integrate.quad(f, a, b, **opts)[0]
    m1 = integrate.quad(lambda x: x * f(x), a, b, **opts)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), a, b, **opts)[0]
    return m0, m1, m2


def scalar_lloyd_max(d, bits, max_iter=2000, tol=1e-14):
    """Optimal 2^bits-level scalar quantiser of f_X; returns (centroids, D_scalar).

    Start: the quantiles (i+1/2)/L of f_X (its CDF is that of 2*Beta((d-1)/2,
    (d-1)/2) - 1).  Iterate midpoint boundaries / conditional means until the
    largest centroid move is below ``tol``.
    """
    L = 1 << bits
    a = (d - 1) / 2.0
    c = 2.0 * betaincinv(a, a, (np.arange(L) + 0.5) / L) - 1.0
    for _ in range(max_iter):
        edges = np.concatenate([[-1.0], 0.5 * (c[1:] + c[:-1]), [1.0]])
        new = np.empty_like(c)
        for i in range(L):
            m0, m1, _ = _cell_moments(edges[i], edges[i + 1], d)
            new[i] = m1 / m0 if m0 > 0 else c[i]
        move = np.max(np.abs(new - c))
        c = new
        if move < tol:
            break
    edges = np.concatenate([[-1.0], 0.5 * (c[1:] + c[:-1]), [1.0]])
    mse = 0.0
    for i in range(L):
        m0, m1, m2 = _cell_moments(edges[i], edges[i + 1], d)
        mse += m2 - 2.0 * c[i] * m1 + c[i] * c[i] * m0
    return c, d * mse

