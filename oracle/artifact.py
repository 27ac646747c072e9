"""The shared codebook artifact: writer and reader (oracle side).

[FQ 2.1, 3.1]: one offline codebook serves every layer, head and prompt, and
[FQ 1, 2.3] one shared rotation is applied to every vector.  Reading: the
artifact therefore holds both -- the rotation Pi (float64) and the codebook
table C (float32) -- so no consumer has to re-run QR or the random number
generator.  The GPU library parses this same byte layout with its own code.

Layout (little-endian), 256-byte header then payload then trailer:

  off  type   field
    0  4s     magic b"FQCB"
    4  u32    version (1)
    8  u32    header bytes (256)
   12  u32    d
   16  u32    k
   20  u32    N (a power of two)
   24  u32    nb = ceil(d / k)
   28  u32    index bits = log2 N
   32  u32    record words W = ceil(nb * index bits / 32)
   36  u32    real coordinates of the last block
   40  u32    Lloyd restarts
   44  u32    Lloyd iteration cap
   48  u32    iterations of the kept restart
   52  u32    kept restart
   56  u64    rotation seed
   64  u64    training samples
   72  f64    Lloyd relative-decrease tolerance
   80  f64    training MSE per block of the kept restart
   88  f64    test distortion per unit vector (float32 table)
   96  f64    nominal rate log2(N) / k
  104  f64    actual rate nb * index bits / d
  112  f64    companded radius law parameter a
  120  f64    companded radius law parameter b
  128..255    zero
  256  f64[d*d]  Pi, row-major, z_j = sum_i Pi[j, i] u_i
   ..  f32[N*k]  C, row-major, codeword n = C[n, :]
   ..  u64    FNV-1a 64 of every preceding byte
"""
import struct

import numpy as np

MAGIC = b"FQCB"
VERSION = 1
HEADER_BYTES = 256
_HDR = struct.Struct("<4s13I2Q7d")
FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data):
    """FNV-1a 64-bit hash (byte at a time, as published by Fowler, Noll and Vo)."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def record_words(nb, bits):
    return -(-(nb * bits) // 32)


def write_artifact(Pi, book):
    """Serialise rotation ``Pi`` and a ``codebook.build_codebook`` result to bytes."""
    d, k, N = book["d"], book["k"], book["N"]
    bits = int(N).bit_length() - 1
    assert 1 << bits == N
    nb = book["nb"]
    hdr = _HDR.pack(MAGIC, VERSION, HEADER_BYTES, d, k, N, nb, bits, record_words(nb, bits),
                    book["partial"], book["restarts"], book["max_iter"], book["iterations"],
                    book["best_restart"], book.get("seed_rot", 0), book["samples"], book["tol"],
                    book["D_train_block"], book["D_test"], bits / k, nb * bits / d,
                    book["law_a"], book["law_b"])
    hdr = hdr + b"\0" * (HEADER_BYTES - len(hdr))
    body = hdr + np.ascontiguousarray(Pi, dtype="<f8").tobytes() \
        + np.ascontiguousarray(book["C"], dtype="<f4").tobytes()
    return body + struct.pack("<Q", fnv1a64(body))


def read_artifact(blob):
    """Parse and check an artifact; returns a dict with float64 ``Pi`` and float32 ``C``."""
    blob = bytes(blob)
    if len(blob) < HEADER_BYTES + 8:
        raise ValueError("artifact truncated")
    f = _HDR.unpack_from(blob, 0)
    (magic, version, hbytes, d, k, N, nb, bits, W, partial, restarts, max_iter, iters, best,
     seed_rot, samples, tol, d_train, d_test, rate_nom, rate_act, law_a, law_b) = f
    if magic != MAGIC or version != VERSION or hbytes != HEADER_BYTES:
        raise ValueError("bad artifact header")
    size = HEADER_BYTES + 8 * d * d + 4 * N * k + 8
    if len(blob) != size:
        raise ValueError("artifact size mismatch")
    (h,) = struct.unpack_from("<Q", blob, size - 8)
    if h != fnv1a64(blob[:size - 8]):
        raise ValueError("artifact hash mismatch")
    Pi = np.frombuffer(blob, dtype="<f8", count=d * d, offset=HEADER_BYTES).reshape(d, d)
    C = np.frombuffer(blob, dtype="<f4", count=N * k, offset=HEADER_BYTES + 8 * d * d)
    return {"d": d, "k": k, "N": N, "nb": nb, "bits": bits, "W": W, "partial": partial,
            "restarts": restarts, "max_iter": max_iter, "iterations": iters,
            "best_restart": best, "seed_rot": seed_rot, "samples": samples, "tol": tol,
            "D_train_block": d_train, "D_test": d_test, "rate_nominal": rate_nom,
            "rate_actual": rate_act, "law_a": law_a, "law_b": law_b, "hash": h,
            "Pi": Pi.astype(np.float64), "C": C.reshape(N, k).copy()}
