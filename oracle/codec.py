"""FibQuant encode / pack / unpack / decode (oracle, float64).

[FQ 2.3]: the encoder computes the norm nu = |x|_2, rotates the unit vector
Pi x / nu, splits it into d/k blocks of k coordinates and looks up the nearest
codeword of the shared codebook for every block; the decoder fetches the
codewords, rebuilds and concatenates the blocks, applies the inverse rotation
and scales by the norm.  The rate is b = log2(N) / k bits per coordinate.
[FQ 1]: records sit at fixed addresses so any token decodes on its own by
address arithmetic, which forces a fixed-rate code.

Readings:

* The norm is stored as IEEE binary16, rounded to nearest-even from the
  exact float64 norm (overflow to +inf).  Normalisation uses the unrounded
  norm; decoding scales by the stored binary16 value.
* nu = 0: every index is 0, the stored norm is 0 and the vector decodes to 0.
* Block j covers coordinates [j k, min((j+1) k, d)).  When k does not divide
  d the last block keeps its r real coordinates; its distance and its decoded
  value use the first r coordinates of each codeword.
* Distance D_j(n) = sum over the block's real coordinates of (z - c_n)^2,
  evaluated in float64 on the float32 table; ties go to the lowest n.
* Record layout: field j (log2 N bits) occupies bits [j b, (j+1) b) of the
  record, counted from the least significant bit of little-endian 32-bit
  words; a record is W = ceil(nb b / 32) words; unused high bits are 0.
  Norms live in their own array, one binary16 per record.
* Packed records (a second storage form): record r of R = nb b + 16 bits at
  bits [r R, (r+1) R) of one word stream, counted from the least significant
  bit of little-endian 32-bit words -- field j at record bits [j b, (j+1) b),
  then the 16 bits of the binary16 norm; bits past the last record are 0.
  No record is rounded up to whole words, so a k = 64, N = 4096 vector takes
  28 bits (12 + 16), the rate of the code plus its norm.
"""
from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------- binary16 norm
def f16_round(v):
    """Round float64 values to IEEE binary16, nearest-even, overflow to inf.

    Returns the binary16 bit patterns as uint16.  numpy's float64 -> float16
    cast rounds directly from the double (pinned in tests against exact
    rational rounding).
    """
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_value(bits):
    """float64 value of binary16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f16_round_exact(v):
    """binary16 rounding of one float by exact rational arithmetic (pin for ``f16_round``)."""
    q = Fraction(float(v))
    sign = 0x8000 if q < 0 or (q == 0 and np.signbit(v)) else 0
    q = abs(q)
    if q == 0:
        return sign
    # binary16: 5 exponent bits (bias 15), 10 fraction bits, subnormal spacing 2^-24
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    m = q / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * ulp
    if val >= Fraction(65520) or val >= 2 ** 16:
        return sign | 0x7C00
    if val < Fraction(2) ** -14:
        return sign | int(val / Fraction(2) ** -24)
    e2 = val.numerator.bit_length() - val.denominator.bit_length()
    if Fraction(2) ** e2 > val:
        e2 -= 1
    frac = int((val / Fraction(2) ** e2 - 1) * 1024)
    return sign | ((e2 + 15) << 10) | frac


# --------------------------------------------------------------------- encode
def block_bounds(d, k):
    nb = -(-d // k)
    return [(j * k, min((j + 1) * k, d)) for j in range(nb)]


def rotate_units(x, Pi):
    """nu = |x|_2 and z = Pi (x / nu) in float64; z = 0 where nu = 0."""
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    u = np.zeros_like(x)
    nz = nu > 0
    u[nz] = x[nz] / nu[nz, None]
    return nu, u @ Pi.T


def block_distances(z, C, d, k, j):
    """D_j(n) for every vector (rows of z) and codeword n: shape [n_vec, N]."""
    lo, hi = block_bounds(d, k)[j]
    r = hi - lo
    Cb = np.asarray(C, dtype=np.float64)[:, :r]
    diff = z[:, None, lo:hi] - Cb[None, :, :]
    return np.sum(diff * diff, axis=2)


def encode(x, Pi, C, chunk=2048):
    """Indices [n, nb] (int64) and binary16 norm bits [n] of vectors x [n, d]."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    N, k = C.shape
    nb = -(-d // k)
    idx = np.zeros((n, nb), dtype=np.int64)
    nu_all = np.zeros(n)
    # bound the [chunk, N, k] difference array (large codebooks, large k)
    chunk = max(1, min(chunk, (1 << 25) // (N * k)))
    for s in range(0, n, chunk):
        nu, z = rotate_units(x[s:s + chunk], Pi)
        nu_all[s:s + chunk] = nu
        for j in range(nb):
            idx[s:s + chunk, j] = np.argmin(block_distances(z, C, d, k, j), axis=1)
        idx[s:s + chunk][nu == 0] = 0
    return idx, f16_round(nu_all)


def accept_indices(x, Pi, C, got, window=1e-6, chunk=2048):
    """Check candidate indices against the oracle under the near-tie window.

    An index i for block j is accepted when D_j(i) - min_n D_j(n) <= window *
    D_j(i) (with float64 distances); returns (n_exact, n_window, n_bad).
    """
    x = np.asarray(x, dtype=np.float64)
    got = np.asarray(got, dtype=np.int64)
    n, d = x.shape
    N, k = C.shape
    nb = got.shape[1]
    exact = window_ok = bad = 0
    chunk = max(1, min(chunk, (1 << 25) // (N * k)))
    for s in range(0, n, chunk):
        nu, z = rotate_units(x[s:s + chunk], Pi)
        g = got[s:s + chunk]
        for j in range(nb):
            D = block_distances(z, C, d, k, j)
            best = np.argmin(D, axis=1)
            dmin = D[np.arange(len(best)), best]
            dg = D[np.arange(len(best)), g[:, j]]
            same = g[:, j] == best
            zero = nu == 0
            same |= zero & (g[:, j] == 0)
            ok = ~same & ~zero & (dg - dmin <= window * dg)
            exact += int(np.sum(same))
            window_ok += int(np.sum(ok))
            bad += int(np.sum(~same & ~ok))
    return exact, window_ok, bad


# ------------------------------------------------------------------ pack/unpack
def pack(idx, bits):
    """Pack indices [n, nb] into records [n, W] uint32 (layout in the module docstring)."""
    idx = np.asarray(idx, dtype=np.uint64)
    n, nb = idx.shape
    W = -(-(nb * bits) // 32)
    words = np.zeros((n, W), dtype=np.uint64)
    for j in range(nb):
        pos = j * bits
        w, o = pos // 32, pos % 32
        words[:, w] |= (idx[:, j] << np.uint64(o)) & np.uint64(0xFFFFFFFF)
        if o + bits > 32:
            words[:, w + 1] |= idx[:, j] >> np.uint64(32 - o)
    return words.astype(np.uint32)


def unpack(words, nb, bits):
    """Inverse of ``pack``: records [n, W] uint32 -> indices [n, nb] int64."""
    words = np.asarray(words, dtype=np.uint64)
    n = words.shape[0]
    mask = np.uint64((1 << bits) - 1)
    idx = np.zeros((n, nb), dtype=np.int64)
    for j in range(nb):
        pos = j * bits
        w, o = pos // 32, pos % 32
        v = words[:, w] >> np.uint64(o)
        if o + bits > 32:
            v |= words[:, w + 1] << np.uint64(32 - o)
        idx[:, j] = (v & mask).astype(np.int64)
    return idx


# --------------------------------------------------------------------- decode
def codeword_vectors(idx, C, d):
    """Concatenate the codewords of every block (partial last block truncated): [n, d]."""
    idx = np.asarray(idx, dtype=np.int64)
    N, k = C.shape
    Cd = np.asarray(C, dtype=np.float64)
    out = np.empty((idx.shape[0], d), dtype=np.float64)
    for j, (lo, hi) in enumerate(block_bounds(d, k)):
        out[:, lo:hi] = Cd[idx[:, j], :hi - lo]
    return out


def decode(idx, norm_bits, Pi, C):
    """x_hat = nu16 * Pi^T concat(c_{i_j}) in float64, [n, d]."""
    d = Pi.shape[0]
    zhat = codeword_vectors(idx, C, d)
    return f16_value(norm_bits)[:, None] * (zhat @ Pi)


def decode_records(words, norm_bits, Pi, C):
    """Decode straight from packed records."""
    N, k = C.shape
    d = Pi.shape[0]
    nb = -(-d // k)
    bits = int(N).bit_length() - 1
    return decode(unpack(words, nb, bits), norm_bits, Pi, C)


# -------------------------------------------------------------- packed records
def packed_record_bits(nb, bits):
    """R: the fields of one record and its 16-bit norm."""
    return nb * bits + 16


def pack_stream(idx, norm_bits, bits):
    """Indices [n, nb] and binary16 norm bits [n] -> packed stream (uint32 words)."""
    idx = np.asarray(idx, dtype=np.uint64)
    n, nb = idx.shape
    R = packed_record_bits(nb, bits)
    nu = np.asarray(norm_bits, dtype=np.uint64)
    rec = np.zeros((n, R), dtype=np.uint8)            # one bit per entry, LSB first
    for j in range(nb):
        for t in range(bits):
            rec[:, j * bits + t] = (idx[:, j] >> np.uint64(t)) & np.uint64(1)
    for t in range(16):
        rec[:, nb * bits + t] = (nu >> np.uint64(t)) & np.uint64(1)
    words = -(-(n * R) // 32)
    flat = np.zeros(words * 32, dtype=np.uint8)
    flat[:n * R] = rec.reshape(-1)
    return np.packbits(flat, bitorder="little").view("<u4").astype(np.uint32)


def unpack_stream(words, n, nb, bits):
    """Inverse of ``pack_stream``: (indices [n, nb] int64, norm bits [n] uint16)."""
    R = packed_record_bits(nb, bits)
    w = np.ascontiguousarray(words, dtype="<u4")
    flat = np.unpackbits(w.view(np.uint8), bitorder="little")[:n * R].reshape(n, R)
    weights = (np.uint64(1) << np.arange(bits, dtype=np.uint64))
    idx = np.zeros((n, nb), dtype=np.int64)
    for j in range(nb):
        idx[:, j] = (flat[:, j * bits:(j + 1) * bits].astype(np.uint64) @ weights).astype(np.int64)
    w16 = (np.uint64(1) << np.arange(16, dtype=np.uint64))
    nu = (flat[:, nb * bits:].astype(np.uint64) @ w16).astype(np.uint16)
    return idx, nu
