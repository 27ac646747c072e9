"""The canonical spherical-Beta block source (oracle, float64).

[FQ 2.1, 3.1] (Theorem 1): after normalisation and a Haar rotation the unit
vector is uniform on S^{d-1}, whatever the input distribution, so any block
of k consecutive coordinates has one fixed density f_{d,k} on the unit ball.
[BSQ key design 1] writes that density out and its polar split: the block is
r * theta with r^2 ~ Beta(k/2, (d-k)/2) and theta uniform on S^{k-1},
independent.  [TQ 2] gives the k = 1 marginal.
"""
import numpy as np
from scipy.special import gammaln


def block_density(z, d):
    """f_{d,k}(z) = Gamma(d/2) / (pi^{k/2} Gamma((d-k)/2)) (1-|z|^2)^{(d-k-2)/2}.

    z has shape [..., k]; zero outside the open unit ball.  [BSQ key design 1]
    """
    z = np.asarray(z, dtype=np.float64)
    k = z.shape[-1]
    r2 = np.sum(z * z, axis=-1)
    logc = gammaln(d / 2.0) - (k / 2.0) * np.log(np.pi) - gammaln((d - k) / 2.0)
    out = np.zeros_like(r2)
    inside = r2 < 1.0
    out[inside] = np.exp(logc + 0.5 * (d - k - 2) * np.log1p(-r2[inside]))
    return out


def coordinate_density(x, d):
    """f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1-x^2)^{(d-3)/2} on [-1, 1].

    The law of one coordinate of a uniform point on S^{d-1}.  [TQ 2, lemma]
    """
    x = np.asarray(x, dtype=np.float64)
    logc = gammaln(d / 2.0) - 0.5 * np.log(np.pi) - gammaln((d - 1) / 2.0)
    out = np.zeros_like(x)
    inside = np.abs(x) < 1.0
    out[inside] = np.exp(logc + 0.5 * (d - 3) * np.log1p(-x[inside] ** 2))
    return out


def sample_blocks(d, k, count, seed):
    """Draw ``count`` blocks from the source by its definition.

    g ~ N(0, I_d); the block is the first k coordinates of g / |g|
    (a uniform point on S^{d-1}, [FQ 2.1]).  Generated in chunks so memory
    stays bounded; the stream depends only on ``seed``.
    """
    rng = np.random.default_rng(seed)
    out = np.empty((count, k), dtype=np.float64)
    chunk = 1 << 16
    for s in range(0, count, chunk):
        m = min(chunk, count - s)
        g = rng.standard_normal((m, d))
        out[s:s + m] = g[:, :k] / np.linalg.norm(g, axis=1, keepdims=True)
    return out


def sample_blocks_polar(d, k, count, seed):
    """Draw blocks through the polar split of [BSQ key design 1].

    r^2 ~ Beta(k/2, (d-k)/2), theta = h/|h| with h ~ N(0, I_k), independent.
    Used only to cross-check ``sample_blocks``.
    """
    rng = np.random.default_rng(seed)
    r = np.sqrt(rng.beta(k / 2.0, (d - k) / 2.0, size=count))
    h = rng.standard_normal((count, k))
    return r[:, None] * h / np.linalg.norm(h, axis=1, keepdims=True)
