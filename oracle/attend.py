"""Decode-step attention over a compressed KV cache (oracle, float64).

[FQ 5]: the fixed-address, random-access records are what lets decompression
be fused into attention kernels; [FQ-abs]: the cache is read at every decoding
step.  The pages fix no attention variant, so the oracle states the plain one:
decompress every key and value with the codec's decoder, then single-query
softmax attention per query head.

Readings: scores s_t = scale * <q_h, k_hat_t> over all T tokens (no mask);
p = softmax(s); o_h = sum_t p_t v_hat_t.  Grouped-query mapping: query head h
reads KV head floor(h / (Hq / Hkv)).  ``scale`` is passed in (1/sqrt(d) in the
workloads).

``attend_rotated`` is the same quantity computed in the rotated domain
(scores nu_t <Pi q, z_hat_t>, values accumulated as sum p_t nu_t z_hat_t and
rotated back once); Pi being orthogonal, the two agree exactly in exact
arithmetic.  It is a pin of the decompress-then-attend form, not a separate
definition.
"""
import numpy as np

from . import codec


def softmax_attend(q, K, V, scale):
    """o = softmax(scale * K q) V for one query q [d], keys K [T, d], values V [T, d]."""
    s = scale * (K @ q)
    s = s - np.max(s)
    p = np.exp(s)
    p /= np.sum(p)
    return p @ V, p


def attend(q, k_words, k_norms, v_words, v_norms, Pi, Ck, Cv, scale, rows=None):
    """Decompress-then-attend.

    q: [B, Hq, d]; k_words/v_words: [B, Hkv, T, W*] uint32 records;
    k_norms/v_norms: [B, Hkv, T] binary16 bits.  ``rows`` optionally limits the
    output to a list of (b, h) pairs; returns {(b, h): o [d]} then, else an
    array [B, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_words.shape[1]
    group = Hq // Hkv
    pairs = rows if rows is not None else [(b, h) for b in range(B) for h in range(Hq)]
    cache = {}
    out = {}
    for b, h in pairs:
        g = h // group
        if (b, g) not in cache:
            Kh = codec.decode_records(k_words[b, g], k_norms[b, g], Pi, Ck)
            Vh = codec.decode_records(v_words[b, g], v_norms[b, g], Pi, Cv)
            cache = {(b, g): (Kh, Vh)}
        Kh, Vh = cache[(b, g)]
        out[(b, h)] = softmax_attend(q[b, h], Kh, Vh, scale)[0]
    if rows is not None:
        return out
    o = np.empty((B, Hq, d))
    for (b, h), v in out.items():
        o[b, h] = v
    return o


def attend_queries(q, k_words, k_norms, v_words, v_norms, Pi, Ck, Cv, scale, T, rows=None):
    """Several queries per head over the first T cached tokens, causal.

    The pages fix no multi-query variant (a prefill chunk, speculative draft
    tokens); the reading: the M queries of a head are the last M positions, so
    query m sees tokens 0 .. T - M + m, each with the single-query softmax of
    ``attend``.  q: [B, Hq, M, d]; caches [B, Hkv, >= T, W*] / [B, Hkv, >= T].
    ``rows`` optionally limits the output to (b, h, m) triples (returns a dict);
    else an array [B, Hq, M, d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, M, d = q.shape
    Hkv = k_words.shape[1]
    group = Hq // Hkv
    trips = rows if rows is not None else [(b, h, m) for b in range(B) for h in range(Hq)
                                            for m in range(M)]
    cache = {}
    out = {}
    for b, h, m in trips:
        g = h // group
        if (b, g) not in cache:
            Kh = codec.decode_records(k_words[b, g, :T], k_norms[b, g, :T], Pi, Ck)
            Vh = codec.decode_records(v_words[b, g, :T], v_norms[b, g, :T], Pi, Cv)
            cache = {(b, g): (Kh, Vh)}
        Kh, Vh = cache[(b, g)]
        n = T - M + m + 1
        out[(b, h, m)] = softmax_attend(q[b, h, m], Kh[:n], Vh[:n], scale)[0]
    if rows is not None:
        return out
    o = np.empty((B, Hq, M, d))
    for (b, h, m), v in out.items():
        o[b, h, m] = v
    return o


def attend_rotated(q, k_words, k_norms, v_words, v_norms, Pi, Ck, Cv, scale, b, h):
    """The rotated-domain form of ``attend`` for one (b, h) row (pin only)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_words.shape[1]
    g = h // (Hq // Hkv)
    Nk, kk = Ck.shape
    Nv, kv = Cv.shape
    ik = codec.unpack(k_words[b, g], -(-d // kk), int(Nk).bit_length() - 1)
    iv = codec.unpack(v_words[b, g], -(-d // kv), int(Nv).bit_length() - 1)
    zk = codec.codeword_vectors(ik, Ck, d)
    zv = codec.codeword_vectors(iv, Cv, d)
    nk = codec.f16_value(k_norms[b, g])
    nv = codec.f16_value(v_norms[b, g])
    qr = Pi @ q[b, h]
    s = scale * nk * (zk @ qr)
    s = s - np.max(s)
    p = np.exp(s)
    p /= np.sum(p)
    o_rot = (p * nv) @ zv
    return Pi.T @ o_rot
