"""Pins of the oracle's encode / pack / decode / attention.

[FQ 1] fixed-address records, [FQ 2.3] encoder and decoder, [FQ 5] fusion
into attention.  Each pin is chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails it.
"""
import json
import os

import numpy as np
import pytest
from scipy.spatial import cKDTree

from kv_cache_compression_fq_amd import synth
from oracle import attend, codebook, codec, rotation

from conftest import GOLDEN_DIR

PI = rotation.make_rotation(64, 0)


def small_book(k, N, seed=0):
    """A small Lloyd-refined codebook (not an artifact) for fast pins."""
    from oracle import source
    X = source.sample_blocks(64, k, 1 << 13, [16, k, N, seed])
    C, _ = codebook.lloyd(codebook.initial_codebook(64, k, N), X, max_iter=30)
    return C.astype(np.float32)


# ---------------------------------------------------------------- binary16
def test_f16_round_matches_exact_rational():
    rng = np.random.default_rng(17)
    vals = list(10.0 ** rng.uniform(-9, 5.2, 3000))
    # exact midpoints between binary16 neighbours, and values one double-ulp either side
    base = np.arange(0x0001, 0x7BFF, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0x0001, 0x7BFF, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (base + nxt) / 2
    vals += list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, np.inf))
    vals += [0.0, 65504.0, 65519.99, 65520.0, 7e4, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14]
    got = codec.f16_round(np.array(vals))
    want = np.array([codec.f16_round_exact(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


# -------------------------------------------------------------------- pack
def test_pack_hand_examples():
    ex = json.load(open(os.path.join(GOLDEN_DIR, "pack_examples.json")))["examples"]
    for e in ex:
        idx = np.zeros((1, e["nb"]), dtype=np.int64)
        for j, v in e["nonzero"].items():
            idx[0, int(j)] = v
        words = codec.pack(idx, e["bits"])
        assert [f"0x{w:08X}" for w in words[0]] == e["words"], e["why"]
        assert np.array_equal(codec.unpack(words, e["nb"], e["bits"]), idx)


@pytest.mark.parametrize("nb,bits", [(32, 4), (32, 6), (32, 8), (22, 9), (16, 8), (8, 8),
                                     (8, 4), (16, 2), (22, 12)])
def test_pack_roundtrip_and_padding(nb, bits):
    rng = np.random.default_rng([18, nb, bits])
    idx = rng.integers(0, 1 << bits, size=(200, nb))
    words = codec.pack(idx, bits)
    W = -(-(nb * bits) // 32)
    assert words.shape == (200, W)
    assert np.array_equal(codec.unpack(words, nb, bits), idx)
    used = nb * bits - 32 * (W - 1)
    if used < 32:
        assert np.all(words[:, -1] >> np.uint32(used) == 0)


def test_pack_stream_hand_examples():
    ex = json.load(open(os.path.join(GOLDEN_DIR, "packed_stream_examples.json")))["examples"]
    for e in ex:
        idx = np.array(e["fields"], dtype=np.int64)
        nbits = np.array([int(v, 16) for v in e["norms"]], dtype=np.uint16)
        words = codec.pack_stream(idx, nbits, e["bits"])
        assert [f"0x{w:08X}" for w in words] == e["words"], e["why"]
        i2, n2 = codec.unpack_stream(words, len(idx), e["nb"], e["bits"])
        assert np.array_equal(i2, idx) and np.array_equal(n2, nbits)


@pytest.mark.parametrize("nb,bits", [(1, 12), (2, 12), (8, 4), (16, 2), (22, 9), (32, 4)])
def test_pack_stream_roundtrip_and_record_bits(nb, bits):
    """Round trip on ragged counts, and record r's first nb*bits bits are the
    word-aligned record's (same field layout), its next 16 its norm."""
    rng = np.random.default_rng([19, nb, bits])
    for n in (1, 7, 33, 200):
        idx = rng.integers(0, 1 << bits, size=(n, nb))
        nbits = rng.integers(0, 1 << 16, size=n).astype(np.uint16)
        words = codec.pack_stream(idx, nbits, bits)
        R = codec.packed_record_bits(nb, bits)
        assert len(words) == -(-(n * R) // 32)
        i2, n2 = codec.unpack_stream(words, n, nb, bits)
        assert np.array_equal(i2, idx) and np.array_equal(n2, nbits)
        allbits = np.unpackbits(words.view(np.uint8), bitorder="little")
        assert not np.any(allbits[n * R:])                     # padding bits are zero
        aligned = np.unpackbits(codec.pack(idx, bits).view(np.uint8), bitorder="little")
        aligned = aligned.reshape(n, -1)[:, :nb * bits]
        assert np.array_equal(allbits[:n * R].reshape(n, R)[:, :nb * bits], aligned)


# ------------------------------------------------------------------ encode
def naive_encode_one(x, Pi, C):
    """Pure-Python loops: norm, rotation, per-block brute-force argmin."""
    d = len(x)
    N, k = C.shape
    nu = sum(float(v) ** 2 for v in x) ** 0.5
    if nu == 0:
        return [0] * (-(-d // k)), 0.0
    z = [sum(float(Pi[j, i]) * float(x[i]) / nu for i in range(d)) for j in range(d)]
    out = []
    for lo in range(0, d, k):
        hi = min(lo + k, d)
        best, bi = None, 0
        for n in range(N):
            dd = sum((z[lo + t] - float(C[n, t])) ** 2 for t in range(hi - lo))
            if best is None or dd < best:
                best, bi = dd, n
        out.append(bi)
    return out, nu


@pytest.mark.parametrize("k,N", [(2, 16), (3, 8), (4, 4), (8, 16)])
def test_encode_matches_naive_loops(k, N):
    C = small_book(k, N)
    x = np.concatenate([synth.tiny_vectors(24, seed=19), synth.special_vectors(dtype=np.float32)])
    idx, nbits = codec.encode(x, PI, C)
    for r in range(len(x)):
        want, nu = naive_encode_one(x[r], PI, C)
        assert list(idx[r]) == want
        assert nbits[r] == codec.f16_round_exact(nu)


def test_encode_matches_kdtree_full_blocks():
    C = small_book(2, 16)
    x = synth.tiny_vectors(4096)
    idx, _ = codec.encode(x, PI, C)
    nu, z = codec.rotate_units(x, PI)
    _, kd = cKDTree(C.astype(np.float64)).query(z.reshape(-1, 2))
    assert np.mean(idx.reshape(-1) == kd) == 1.0


def test_zero_vector():
    C = small_book(2, 16)
    x = np.zeros((3, 64))
    idx, nbits = codec.encode(x, PI, C)
    assert np.all(idx == 0) and np.all(nbits == 0)
    assert np.all(codec.decode(idx, nbits, PI, C) == 0)


def test_partial_block_uses_first_coordinates():
    # k = 3, d = 64: 22 blocks, the last holds only coordinate 63.
    C = small_book(3, 8)
    x = synth.tiny_vectors(64, seed=20)
    idx, _ = codec.encode(x, PI, C)
    nu, z = codec.rotate_units(x, PI)
    want = np.argmin((z[:, 63:64] - C[None, :, 0].astype(np.float64)) ** 2, axis=1)
    assert np.array_equal(idx[:, 21], want)
    xh = codec.decode(idx, codec.f16_round(nu), PI, C)
    zh = codec.codeword_vectors(idx, C, 64)
    assert np.array_equal(zh[:, 63], C[idx[:, 21], 0].astype(np.float64))
    assert np.allclose(xh, codec.f16_value(codec.f16_round(nu))[:, None] * (zh @ PI))


def test_accept_indices_detects_planted_error():
    C = small_book(2, 16)
    x = synth.tiny_vectors(256, seed=21)
    idx, _ = codec.encode(x, PI, C)
    assert codec.accept_indices(x, PI, C, idx) == (256 * 32, 0, 0)
    bad = idx.copy()
    bad[5, 7] = (bad[5, 7] + 1) % 16
    ex, win, nbad = codec.accept_indices(x, PI, C, bad)
    assert nbad == 1 and ex == 256 * 32 - 1


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("k,N", [(2, 16), (3, 8), (8, 16)])
def test_decode_error_identity(k, N):
    # |x - nu Pi^T z_hat|^2 = nu^2 sum_j |z_j - c_{i_j}|^2 because Pi is orthogonal.
    C = small_book(k, N)
    x = synth.tiny_vectors(128, seed=22).astype(np.float64)
    idx, _ = codec.encode(x, PI, C)
    nu, z = codec.rotate_units(x, PI)
    zh = codec.codeword_vectors(idx, C, 64)
    xh = nu[:, None] * (zh @ PI)
    lhs = np.sum((x - xh) ** 2, axis=1)
    rhs = nu ** 2 * np.sum((z - zh) ** 2, axis=1)
    assert np.max(np.abs(lhs - rhs) / rhs) < 1e-10


def test_decode_records_equals_decode():
    C = small_book(3, 8)
    x = synth.tiny_vectors(50, seed=23)
    idx, nbits = codec.encode(x, PI, C)
    words = codec.pack(idx, 3)
    assert np.array_equal(codec.decode_records(words, nbits, PI, C), codec.decode(idx, nbits, PI, C))


def test_decode_uses_inverse_rotation():
    # One block carries the codeword, the rest are codeword 0 = a chosen zero row:
    # then x_hat = nu * Pi^T e-block, i.e. rows of Pi.
    C = np.zeros((4, 2), dtype=np.float32)
    C[1] = [1.0, 0.0]
    idx = np.zeros((1, 32), dtype=np.int64)
    idx[0, 5] = 1                          # coordinate 10 of z_hat is 1
    nb = codec.f16_round(np.array([2.0]))
    xh = codec.decode(idx, nb, PI, C)
    assert np.allclose(xh[0], 2.0 * PI[10, :], atol=0, rtol=1e-15)


# --------------------------------------------------------------- attention
def attn_case(T, B=2, Hq=4, Hkv=2, k=4, N=16, seed=24):
    C = small_book(k, N)
    W = -(-(16 * 4) // 32)
    kw = synth.random_records((B, Hkv, T), W, 64, seed)
    vw = synth.random_records((B, Hkv, T), W, 64, seed + 1)
    kn = synth.random_norms((B, Hkv, T), seed + 2)
    vn = synth.random_norms((B, Hkv, T), seed + 3)
    q = synth.query(B, Hq, seed=seed + 4)
    return q, kw, kn, vw, vn, C


def test_attend_rotated_equals_direct():
    q, kw, kn, vw, vn, C = attn_case(T=300)
    o = attend.attend(q, kw, kn, vw, vn, PI, C, C, 0.125)
    for b in range(2):
        for h in range(4):
            o2 = attend.attend_rotated(q, kw, kn, vw, vn, PI, C, C, 0.125, b, h)
            assert np.max(np.abs(o[b, h] - o2)) <= 1e-12 * np.max(np.abs(o[b, h]))


def test_attend_single_token_returns_value():
    q, kw, kn, vw, vn, C = attn_case(T=1)
    o = attend.attend(q, kw, kn, vw, vn, PI, C, C, 0.125)
    for b in range(2):
        for h in range(4):
            v = codec.decode_records(vw[b, h // 2], vn[b, h // 2], PI, C)[0]
            assert np.allclose(o[b, h], v, rtol=1e-13, atol=0)


def test_attend_zero_query_is_mean():
    q, kw, kn, vw, vn, C = attn_case(T=37)
    q[:] = 0
    o = attend.attend(q, kw, kn, vw, vn, PI, C, C, 0.125)
    for b in range(2):
        for g in range(2):
            v = codec.decode_records(vw[b, g], vn[b, g], PI, C)
            assert np.allclose(o[b, 2 * g], v.mean(axis=0), rtol=1e-12, atol=1e-12)


def test_attend_gqa_grouping_and_softmax():
    q, kw, kn, vw, vn, C = attn_case(T=64)
    o = attend.attend(q, kw, kn, vw, vn, PI, C, C, 0.125)
    vw2 = vw.copy()
    vw2[:, 1] ^= np.uint32(0x5)       # change KV head 1 only
    o2 = attend.attend(q, kw, kn, vw2, vn, PI, C, C, 0.125)
    assert np.array_equal(o[:, :2], o2[:, :2])
    assert not np.allclose(o[:, 2:], o2[:, 2:])
    K = codec.decode_records(kw[0, 0], kn[0, 0], PI, C)
    V = codec.decode_records(vw[0, 0], vn[0, 0], PI, C)
    out, p = attend.softmax_attend(q[0, 0].astype(np.float64), K, V, 0.125)
    assert abs(p.sum() - 1) < 1e-14 and np.all(p > 0)


def test_attend_queries_causal_limits():
    # query m of M sees the first T - M + m + 1 tokens: with M = 1 it is the
    # single-query form over T tokens; the zero query averages exactly its
    # visible values; a cache longer than T is ignored past T
    q, kw, kn, vw, vn, C = attn_case(T=50)
    T, M = 40, 4
    qm = np.stack([synth.query(2, 4, seed=40 + m) for m in range(M)], axis=2)
    o = attend.attend_queries(qm, kw, kn, vw, vn, PI, C, C, 0.125, T)
    for m in range(M):
        n = T - M + m + 1
        ref = attend.attend(qm[:, :, m], kw[:, :, :n], kn[:, :, :n], vw[:, :, :n], vn[:, :, :n],
                            PI, C, C, 0.125)
        assert np.array_equal(o[:, :, m], ref)
    one = attend.attend_queries(q[:, :, None], kw, kn, vw, vn, PI, C, C, 0.125, 50)
    assert np.array_equal(one[:, :, 0], attend.attend(q, kw, kn, vw, vn, PI, C, C, 0.125))
    qz = np.zeros((2, 4, M, 64), dtype=np.float16)
    oz = attend.attend_queries(qz, kw, kn, vw, vn, PI, C, C, 0.125, T)
    V = codec.decode_records(vw[1, 1], vn[1, 1], PI, C)
    for m in range(M):
        assert np.allclose(oz[1, 3, m], V[:T - M + m + 1].mean(axis=0), rtol=1e-12, atol=1e-12)
