"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers; it holds none of the codec's
arithmetic.  Both the HIP path and the CPU oracle receive what it returns.

Recipe (a stand-in for real GPT-2-small / TinyLlama KV caches, which need
model weights and text that are not available here):

* A stream is one (config seed, layer, K/V, head) tuple, seeded as
  ``numpy.random.default_rng([cfg_seed, layer, kv, head])``.
* Each stream draws a per-channel scale s_c = 10^U(-1, 1) (log-uniform on
  [0.1, 10]) and, when outliers are on, a per-channel factor o_c = 20 with
  probability 0.01 (else 1); the scales are shared by all batch rows and
  tokens of the stream.
* Values are g * s_c * o_c with g ~ N(0, 1), rounded to the storage type
  (binary16 for the cache-shaped configs, float32 for the tiny one).
* Cache order is [layer][K/V][batch][head][token][channel].
"""
import numpy as np

D = 64


def stream_scales(rng, d=D, outliers=True):
    s = 10.0 ** rng.uniform(-1.0, 1.0, size=d)
    if outliers:
        s = s * np.where(rng.random(d) < 0.01, 20.0, 1.0)
    return s


def kv_stream(cfg_seed, layer, kv, head, shape, outliers=True, dtype=np.float16, d=D):
    """Values of one stream, shape ``shape + (d,)``."""
    rng = np.random.default_rng([cfg_seed, layer, kv, head])
    s = stream_scales(rng, d, outliers)
    g = rng.standard_normal(tuple(shape) + (d,))
    return (g * s).astype(dtype)


def kv_slab(cfg_seed, layer, kv, B, H, T, outliers=True, dtype=np.float16, d=D):
    """One (layer, K/V) slab [B, H, T, d]: head h is stream (cfg_seed, layer, kv, h)."""
    out = np.empty((B, H, T, d), dtype=dtype)
    for h in range(H):
        out[:, h] = kv_stream(cfg_seed, layer, kv, h, (B, T), outliers, dtype, d)
    return out


def kv_cache(cfg_seed, L, B, H, T, outliers=True, dtype=np.float16, d=D):
    """A whole cache [L, 2, B, H, T, d]."""
    out = np.empty((L, 2, B, H, T, d), dtype=dtype)
    for layer in range(L):
        for kv in range(2):
            out[layer, kv] = kv_slab(cfg_seed, layer, kv, B, H, T, outliers, dtype, d)
    return out


def tiny_vectors(n=4096, seed=1, d=D):
    """The tiny CPU-checkable set: n x d float32, one stream, no outliers."""
    return kv_stream(seed, 0, 0, 0, (n,), outliers=False, dtype=np.float32, d=d)


def special_vectors(d=D, dtype=np.float16):
    """Edge-case rows: zero, one-hot, tiny and huge norms, repeated value, negative."""
    rows = [np.zeros(d), np.eye(d)[0], np.eye(d)[d - 1] * -3.0, np.full(d, 1e-3),
            np.full(d, 250.0), np.linspace(-1.0, 1.0, d), np.full(d, -0.5)]
    return np.array(rows).astype(dtype)


def random_rows(n_total, m, seed=33):
    """m row addresses uniform on [0, n_total) with replacement (int64)."""
    return np.random.default_rng(seed).integers(0, n_total, size=m, dtype=np.int64)


def query(B, Hq, seed=5, d=D, dtype=np.float16):
    """Decode-step queries [B, Hq, d] ~ N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((B, Hq, d)).astype(dtype)


def random_records(shape, words, used_bits, seed):
    """Uniform random records [*shape, words] uint32 with bits >= used_bits cleared.

    With N a power of two every field value is a valid index, so uniform bits
    are uniform indices.
    """
    rng = np.random.default_rng(seed)
    r = rng.integers(0, 1 << 32, size=tuple(shape) + (words,), dtype=np.uint64)
    top = used_bits - 32 * (words - 1)
    if top < 32:
        r[..., -1] &= np.uint64((1 << top) - 1)
    return r.astype(np.uint32)


def random_norms(shape, seed, lo=0.5, hi=2.5):
    """binary16 norms 10^U(lo, hi) as uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    return (10.0 ** rng.uniform(lo, hi, size=shape)).astype(np.float16).view(np.uint16)


def kv_slab_device(cfg_seed, layer, kv, B, H, T, device, outliers=True, d=D):
    """Device-side slab [B, H, T, d] binary16 with the same recipe (bench inputs only).

    The per-channel scales come from the same numpy stream as ``kv_slab``; the
    Gaussian draws come from a torch generator seeded from that stream, so the
    values are seeded and reproducible but not bit-identical to ``kv_slab``.
    """
    import torch
    out = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    for h in range(H):
        rng = np.random.default_rng([cfg_seed, layer, kv, h])
        s = torch.from_numpy(stream_scales(rng, d, outliers)).float().to(device)
        gen = torch.Generator(device=device)
        gen.manual_seed(int(rng.integers(0, 2 ** 62)))
        g = torch.randn((B, T, d), generator=gen, device=device, dtype=torch.float32)
        out[:, h] = (g * s).half()
    return out
