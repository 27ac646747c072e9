"""The shared random rotation Pi (oracle, float64).

[FQ 1, 2.3]: the codec applies one shared random orthogonal (Haar) rotation to
every normalised vector.  [TQ 3.1]: such a rotation is obtained from the QR
decomposition of a matrix with i.i.d. standard normal entries.

Reading: the QR factor Q is made unique (and exactly Haar distributed) by
flipping column signs so that the triangular factor has a positive diagonal;
sgn(0) is taken as +1.  The encoder forms z = Pi u and the decoder applies
Pi^T, so Pi is stored row-major with z_j = sum_i Pi[j, i] u_i.
"""
import numpy as np

D_DEFAULT = 64
SEED_ROT = 0


def make_rotation(d=D_DEFAULT, seed=SEED_ROT):
    """Return the d x d Haar rotation Pi built from a seeded Gaussian matrix.

    G has i.i.d. N(0, 1) entries drawn by ``numpy.random.default_rng(seed)``;
    G = Q R (Householder QR, LAPACK); Pi = Q diag(sgn(diag R)).
    """
    g = np.random.default_rng(seed).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def gaussian_matrix(d=D_DEFAULT, seed=SEED_ROT):
    """The Gaussian matrix G that ``make_rotation`` factors (for pins)."""
    return np.random.default_rng(seed).standard_normal((d, d))
