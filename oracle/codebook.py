"""Offline FibQuant codebook construction (oracle, float64).

[FQ 2.2]: the shared codebook matches the spherical-Beta source with three
parts -- radii r_n from Bennett-Gersho companding of the radial density
(closed form at k = 2), quasi-uniform directions u_n (planar Fibonacci spiral
at k = 2, Fibonacci sphere at k = 3, Roberts-Kronecker sequence at k >= 4),
and multi-restart Lloyd-Max refinement of that deterministic start for the
finite size N.  [FQ 2.1]: one codebook serves every layer, head and prompt.

Readings (the pages name the parts but not their formulas):

* Radii.  Bennett-Gersho: the MSE-optimal point density in k dimensions is
  proportional to f^{k/(k+2)}.  Applied to f_{d,k}, the induced law of r^2
  is Beta(k/2, 1 + k(d-k-2)/(2(k+2))); radius level t in (0, 1) maps to
  r = sqrt(Q(t)) with Q that law's quantile function.  At k = 2 the law is
  Beta(1, d/4), whose quantile has the closed form r^2 = 1 - (1-t)^{4/d}
  (for d = 64, r^2 = 1 - (1-t)^{1/16}) -- the k = 2 closed form of [FQ 2.2].
* Directions.  One map from a point P in [0,1)^k: coordinate 0 is the radius
  level t, coordinates 1..k-1 give a direction on S^{k-1} through the exact
  inverse-CDF (Rosenblatt) map of the uniform law on the sphere: on S^{m-1}
  the first coordinate x has (1+x)/2 ~ Beta((m-1)/2, (m-1)/2), the rest is
  sqrt(1-x^2) times a uniform point of S^{m-2}, down to the circle, where
  the angle is 2 pi w.
    k = 2: P_n = ((n+1/2)/N, frac(n/phi)) -- the golden-angle spiral.
    k = 3: P_n = (frac(1/2 + n/rho), 1 - (n+1/2)/N, frac(n/phi)) -- the
           Fibonacci sphere, with the radius level decorrelated from the
           height by the plastic number rho.
    k >= 4: Roberts' R_k sequence P_n = frac(1/2 + n alpha),
           alpha_j = phi_k^{-(j+1)}, phi_k the root > 1 of x^{k+1} = x + 1.
* Lloyd-Max.  Restart 0 is the unshifted start; restart r >= 1 applies a
  seeded Cranley-Patterson shift P_n <- frac(P_n + U_r) before the map.
  Each iteration assigns every training sample to its nearest codeword and
  moves each codeword to its cell mean; an empty cell keeps its codeword.
  Stop when the relative MSE decrease is below ``tol`` or after
  ``max_iter`` iterations.  The restart with the lowest training MSE wins.
* Distortion.  D = sum over the nb blocks of E|z_j - c(z_j)|^2 per unit
  vector, i.e. (d/k) E|z - c(z)|^2 when k divides d ([TQ 1.1] defines the
  MSE per unit vector; [BSQ main table] uses the same scale).  When k does
  not divide d the last block keeps only its first r = d - (nb-1) k
  coordinates and is searched with the first r coordinates of each codeword.
* Stored precision (the pages fix how the table is built, not the precision
  it is kept in).  The Lloyd-Max table is rounded, nearest-even, to values
  that IEEE binary16 represents exactly, and kept as float32: the artifact
  stores that table and every later oracle step reads it.  Half-precision
  copies of the table are then exact, so decoders may gather codewords from
  binary16 tables without rounding them; the move is at most 2^-12 of each
  coordinate's size (2^-25 absolute below the binary16 normal range), far
  below the quantisation error.
"""
import math

import numpy as np
from scipy.spatial import cKDTree
from scipy.special import betaincinv

from . import source

GOLDEN = (1.0 + math.sqrt(5.0)) / 2.0


def kronecker_root(k):
    """The unique root > 1 of x^{k+1} = x + 1 (golden ratio at k=1, plastic number at k=2)."""
    x = 2.0
    for _ in range(200):
        f = x ** (k + 1) - x - 1.0
        fp = (k + 1) * x ** k - 1.0
        step = f / fp
        x -= step
        if abs(step) < 1e-17:
            break
    return x


def radius_law(d, k):
    """Parameters (a, b) of the companded law r^2 ~ Beta(a, b) (Bennett-Gersho reading)."""
    return k / 2.0, 1.0 + k * (d - k - 2) / (2.0 * (k + 2))


def radii_from_levels(t, d, k):
    """r = sqrt(Q_{Beta(a,b)}(t)) for radius levels t in (0, 1)."""
    a, b = radius_law(d, k)
    return np.sqrt(betaincinv(a, b, np.asarray(t, dtype=np.float64)))


def sphere_direction(w, k):
    """Map w in [0,1)^{k-1} to a point of S^{k-1} by the inverse-CDF chain.

    w has shape [n, k-1]; returns [n, k].  k = 1 returns +-1 by w < 1/2 is not
    needed (k >= 2 only).
    """
    w = np.asarray(w, dtype=np.float64)
    n = w.shape[0]
    out = np.empty((n, k), dtype=np.float64)
    scale = np.ones(n)
    col = 0
    for m in range(k, 2, -1):  # sphere S^{m-1} in R^m, m >= 3
        a = (m - 1) / 2.0
        x = 2.0 * betaincinv(a, a, w[:, col]) - 1.0
        out[:, col] = scale * x
        scale = scale * np.sqrt(np.maximum(0.0, 1.0 - x * x))
        col += 1
    ang = 2.0 * np.pi * w[:, col]
    out[:, col] = scale * np.cos(ang)
    out[:, col + 1] = scale * np.sin(ang)
    return out


def lowdisc_points(k, N):
    """The deterministic point set P_n in [0,1)^k, n = 0..N-1 (see module docstring)."""
    n = np.arange(N, dtype=np.float64)
    if k == 2:
        return np.stack([(n + 0.5) / N, np.mod(n / GOLDEN, 1.0)], axis=1)
    if k == 3:
        rho = kronecker_root(2)
        return np.stack([np.mod(0.5 + n / rho, 1.0), 1.0 - (n + 0.5) / N,
                         np.mod(n / GOLDEN, 1.0)], axis=1)
    if k >= 4:
        phi = kronecker_root(k)
        alpha = phi ** -(np.arange(k, dtype=np.float64) + 1.0)
        return np.mod(0.5 + n[:, None] * alpha[None, :], 1.0)
    raise ValueError("k must be >= 2")


def initial_codebook(d, k, N, shift=None):
    """Deterministic radial-angular start c_n = r_n u_n, optionally Cranley-Patterson shifted."""
    p = lowdisc_points(k, N)
    if shift is not None:
        p = np.mod(p + np.asarray(shift, dtype=np.float64)[None, :], 1.0)
    # keep radius levels strictly inside (0, 1) so the quantile is finite
    t = np.clip(p[:, 0], 1e-300, 1.0 - 1e-16)
    r = radii_from_levels(t, d, k)
    u = sphere_direction(p[:, 1:], k)
    return r[:, None] * u


def nearest(C, X):
    """Nearest codeword index and squared distance for each row of X (library NN search)."""
    k = C.shape[1]
    if k <= 8:
        dist, idx = cKDTree(C).query(X, k=1, workers=-1)
        return idx.astype(np.int64), dist * dist
    idx = np.empty(X.shape[0], dtype=np.int64)
    d2 = np.empty(X.shape[0], dtype=np.float64)
    cc = np.sum(C * C, axis=1)
    chunk = max(1 << 10, min(1 << 15, (1 << 27) // C.shape[0]))   # <= 1 GB per product
    for s in range(0, X.shape[0], chunk):
        xs = X[s:s + chunk]
        part = cc[None, :] - 2.0 * (xs @ C.T)
        j = np.argmin(part, axis=1)
        idx[s:s + chunk] = j
        diff = xs - C[j]
        d2[s:s + chunk] = np.sum(diff * diff, axis=1)
    return idx, d2


def lloyd(C0, X, max_iter=200, tol=1e-9):
    """Lloyd-Max refinement of C0 on training blocks X.

    Returns (C, history) where history[t] is the training MSE per block of the
    codebook at the start of iteration t, and history[-1] is the MSE of the
    returned C.
    """
    C = np.array(C0, dtype=np.float64, copy=True)
    N, k = C.shape
    history = []
    for it in range(max_iter + 1):
        idx, d2 = nearest(C, X)
        mse = float(np.mean(d2))
        history.append(mse)
        if it == max_iter:
            break
        if it > 0 and history[-2] - mse <= tol * history[-2]:
            break
        counts = np.bincount(idx, minlength=N).astype(np.float64)
        nonempty = counts > 0
        for j in range(k):
            sums = np.bincount(idx, weights=X[:, j], minlength=N)
            C[nonempty, j] = sums[nonempty] / counts[nonempty]
    return C, history


def block_layout(d, k):
    """(nb, r): number of blocks ceil(d/k) and the real size r of the last block."""
    nb = -(-d // k)
    return nb, d - (nb - 1) * k


def unit_distortion(C, d, test_blocks):
    """Per-unit-vector distortion D of codebook C on source blocks (see module docstring).

    ``test_blocks`` are full k-blocks from the source; the partial block of a
    k-not-dividing-d layout uses their first r coordinates (the same
    marginal).
    """
    N, k = C.shape
    nb, r = block_layout(d, k)
    _, d2 = nearest(C, test_blocks)
    e_full = float(np.mean(d2))
    if r == k:
        return nb * e_full, e_full, None
    _, d2p = nearest(C[:, :r], test_blocks[:, :r])
    e_part = float(np.mean(d2p))
    return (nb - 1) * e_full + e_part, e_full, e_part


def mc_seeds(d, k, N):
    """Seed sequences of the training sample, the test sample and the restart shifts."""
    return [d, k, N], [d, k, N, 1], [d, k, N, 2]


def half_grid(C):
    """Round a table to the nearest binary16 values (ties to even), held as float32."""
    with np.errstate(over="ignore"):
        h = np.asarray(C, dtype=np.float64).astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("codeword outside the binary16 range")
    return h.astype(np.float32)


def build_codebook(d, k, N, restarts=8, samples=1 << 20, test_samples=1 << 20,
                   max_iter=200, tol=1e-9, log=None):
    """The full offline build: start points, multi-restart Lloyd-Max, binary16-grid rounding.

    Returns a dict with the table ``C`` (float32 holding binary16 values) and its
    bookkeeping.
    """
    s_train, s_test, s_shift = mc_seeds(d, k, N)
    X = source.sample_blocks(d, k, samples, s_train)
    shifts = np.random.default_rng(s_shift).random((restarts, k))
    best = None
    for r in range(restarts):
        C0 = initial_codebook(d, k, N, None if r == 0 else shifts[r])
        C, hist = lloyd(C0, X, max_iter=max_iter, tol=tol)
        if log:
            log(f"k={k} N={N} restart {r}: {len(hist) - 1} iterations, "
                f"train MSE/block {hist[-1]:.6e}")
        if best is None or hist[-1] < best[1][-1]:
            best = (C, hist, r)
    C, hist, r_best = best
    C32 = half_grid(C)
    T = source.sample_blocks(d, k, test_samples, s_test)
    D_test, e_full, e_part = unit_distortion(C32.astype(np.float64), d, T)
    nb, rr = block_layout(d, k)
    return {
        "C": C32, "d": d, "k": k, "N": N, "nb": nb, "partial": rr,
        "restarts": restarts, "samples": samples, "max_iter": max_iter, "tol": tol,
        "best_restart": r_best, "iterations": len(hist) - 1,
        "D_train_block": hist[-1], "D_test": D_test,
        "E_full_test": e_full, "E_partial_test": e_part,
    }
