"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Contract:
* indices equal the oracle's, or fall in the near-tie window
  D(i) - D_min <= 1e-6 D(i) (float64 distances); out-of-window count must be 0;
* norms bit-exact, except +-1 binary16 ulp where the exact norm lies within
  1e-6 (relative) of a rounding midpoint; unused record bits are 0;
* decode of the oracle's codes: max |y - x_hat| <= 1e-3 * nu16 per vector;
* attention on identical inputs: per (b, h) relative L2 error <= 2e-3;
* outputs end where they should: canary words after them are untouched.
Full-size indices are checked with the compiled float64 oracle
(``oracle/nearest.c``, the same definition as ``oracle.codec``).
Inputs are the seeded synthetic generators of ``kv_cache_compression_fq_amd.synth``.
"""
import numpy as np
import pytest

from kv_cache_compression_fq_amd import fq, synth
from oracle import artifact, attend, codec, native

from conftest import VARIANTS, artifact_path

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("device:", torch.cuda.get_device_name(0), flush=True)
    return torch.device("cuda:0")


_BOOKS = {}


def book(k, N):
    """(oracle artifact dict, GPU codebook) for a variant, loaded once."""
    if (k, N) not in _BOOKS:
        blob = open(artifact_path(k, N), "rb").read()
        _BOOKS[(k, N)] = (artifact.read_artifact(blob), fq.fq_codebook_load(blob, 0))
    return _BOOKS[(k, N)]


def to_dev(a, dev, view=None):
    a = np.ascontiguousarray(a)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to(dev)


def gpu_encode(cb, x, dev):
    codes, norms = fq.fq_encode(cb, to_dev(x, dev))
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32), norms.cpu().numpy().view(np.uint16)


def check_norms(x, norms):
    nu = np.sqrt(np.sum(np.asarray(x, dtype=np.float64) ** 2, axis=1))
    want = codec.f16_round(nu)
    diff = np.nonzero(norms != want)[0]
    for r in diff:
        lo = codec.f16_value(np.array([min(norms[r], want[r])]))[0]
        hi = codec.f16_value(np.array([max(norms[r], want[r])]))[0]
        mid = 0.5 * (lo + hi)
        assert abs(int(norms[r]) - int(want[r])) == 1, (r, norms[r], want[r])
        assert abs(nu[r] - mid) <= 1e-6 * nu[r], (r, nu[r], mid)
    return len(diff)


def check_encode(art, x, codes, norms):
    nb, bits, W = art["nb"], art["bits"], art["W"]
    assert codes.shape == (len(x), W)
    used = nb * bits - 32 * (W - 1)
    if used < 32:
        assert np.all((codes[:, -1] >> np.uint32(used)) == 0), "pad bits not zero"
    idx = codec.unpack(codes, nb, bits)
    ex, win, bad = codec.accept_indices(x, art["Pi"], art["C"], idx)
    assert bad == 0, f"{bad} indices outside the near-tie window ({ex} exact, {win} in window)"
    check_norms(x, norms)
    return ex, win


# ------------------------------------------------------------------ encode
def test_encode_tiny_fp32(dev):
    art, cb = book(2, 16)
    x = np.concatenate([synth.tiny_vectors(4096), synth.tiny_vectors(37, seed=2),
                        synth.special_vectors(dtype=np.float32)])
    codes, norms = gpu_encode(cb, x, dev)
    ex, win = check_encode(art, x, codes, norms)
    print(f"tiny fp32: {ex} exact, {win} in window")


@pytest.mark.parametrize("k,N", VARIANTS)
def test_encode_variants_fp16(dev, k, N):
    art, cb = book(k, N)
    x = np.concatenate([synth.kv_slab(2, 0, 0, 2, 3, 411).reshape(-1, 64),
                        synth.special_vectors()])
    codes, norms = gpu_encode(cb, x, dev)
    ex, win = check_encode(art, x, codes, norms)
    print(f"k{k}N{N}: {ex} exact, {win} in window")


@pytest.mark.parametrize("k,N", [(8, 256), (32, 4096), (64, 4096), (64, 16384)])
def test_encode_large_blocks_fp32_and_tiny(dev, k, N):
    """The matrix-core searches (k = 8 with N = 256; k = 32 / 64 with N = 4096;
    k = 64 with N = 16384):
    float32 input with the special vectors, then inputs shorter than one wave's
    share (5 rows) and one row past a workgroup's share (513 rows)."""
    art, cb = book(k, N)
    x = np.concatenate([synth.tiny_vectors(700, seed=3), synth.special_vectors(dtype=np.float32)])
    codes, norms = gpu_encode(cb, x, dev)
    ex, win = check_encode(art, x, codes, norms)
    for m in (5, 513):
        xs = synth.kv_slab(2, 1, 0, 1, 1, m).reshape(-1, 64)
        c, nn = gpu_encode(cb, xs, dev)
        check_encode(art, xs, c, nn)
    print(f"k{k}N{N} fp32: {ex} exact, {win} in window")


@pytest.mark.parametrize("k,N", [(8, 256), (32, 4096), (64, 4096), (64, 16384)])
def test_encode_large_blocks_many_uncertain(dev, k, N):
    """Runs of zero vectors (every block uncertain: all codewords scanned,
    index 0) between ordinary rows, more than one pass's worth per wave, so
    the list of uncertain blocks is settled early as well as at the end."""
    art, cb = book(k, N)
    xs = synth.kv_slab(2, 3, 1, 1, 1, 9000).reshape(-1, 64).copy()
    xs[100:700] = 0.0
    xs[5000:5100] = 0.0
    codes, norms = gpu_encode(cb, xs, dev)
    ex, win = check_encode(art, xs, codes, norms)
    assert np.all(codes[100:700] == 0) and np.all(norms[100:700] == 0)
    print(f"k{k}N{N} with zero runs: {ex} exact, {win} in window")


@pytest.mark.parametrize("k,N", [(3, 512), (8, 256), (64, 4096)])
def test_encode_strided_rows_and_empty(dev, k, N):
    """Rows read with a stride (x_ld = 72, the extra columns ignored) give the
    records of the packed rows; n = 0 is a no-op (grid, matrix-core k = 8 and
    large-block kernels)."""
    art, cb = book(k, N)
    x = synth.kv_slab(2, 1, 1, 1, 2, 300).reshape(-1, 64)
    wide = np.zeros((len(x), 72), dtype=np.float16)
    wide[:, :64] = x
    wide[:, 64:] = 1000.0                      # must be ignored
    xt = to_dev(wide, dev)
    codes, norms = fq.fq_encode(cb, xt[:, :64])
    torch.cuda.synchronize()
    c2, n2 = gpu_encode(cb, x, dev)
    check_encode(art, x, c2, n2)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), c2)
    assert np.array_equal(norms.cpu().numpy().view(np.uint16), n2)
    e = torch.empty((0, 64), dtype=torch.float16, device=dev)
    fq.fq_encode(cb, e)                        # n == 0: no-op


def test_search_cost_model(dev):
    """fq_search_cost: full scans count N per block, zero vectors scan every
    block, and candidate lists count between 1 and the list capacity per block."""
    x = synth.kv_slab(2, 0, 0, 1, 2, 500).reshape(-1, 64)
    _, c4 = book(4, 4)
    e, f = fq.fq_search_cost(c4, x)
    assert e == 16 * 4 and f == 1.0
    _, c2 = book(2, 16)
    e, f = fq.fq_search_cost(c2, x)
    assert 32 <= e < 32 * 8 and f < 0.05
    e0, f0 = fq.fq_search_cost(c2, np.zeros((3, 64), dtype=np.float16))
    assert e0 == 32 * 16 and f0 == 1.0
    _, c3 = book(3, 4096)
    e, f = fq.fq_search_cost(c3, x.astype(np.float32))
    assert 22 <= e < 22 * 16


def test_encode_rejects_misaligned(dev):
    art, cb = book(2, 16)
    x = torch.zeros((10, 72), dtype=torch.float16, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_encode(cb, x[:, 1:65])
    assert e.value.status == fq.FQ_ERR_INVALID_ARG


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("k,N", VARIANTS)
@pytest.mark.parametrize("ydt", ["f16", "f32"])
def test_decode_variants(dev, k, N, ydt):
    art, cb = book(k, N)
    x = np.concatenate([synth.kv_slab(3, 0, 1, 2, 2, 333).reshape(-1, 64),
                        synth.special_vectors()])
    idx, nbits = codec.encode(x, art["Pi"], art["C"])
    words = codec.pack(idx, art["bits"])
    y = fq.fq_decode(cb, to_dev(words, dev, np.int32), to_dev(nbits, dev, np.int16),
                     y_dtype=torch.float16 if ydt == "f16" else torch.float32)
    torch.cuda.synchronize()
    want = codec.decode(idx, nbits, art["Pi"], art["C"])
    got = y.float().cpu().numpy().astype(np.float64)
    nu16 = codec.f16_value(nbits)
    err = np.max(np.abs(got - want), axis=1)
    assert np.all(err <= 1e-3 * nu16 + 1e-30), float(np.max(err / np.maximum(nu16, 1e-30)))
    print(f"k{k}N{N} {ydt}: max err/nu {np.max(err / np.maximum(nu16, 1e-30)):.2e}")


@pytest.mark.parametrize("kb", [(4, 256), (64, 4096), (3, 512), (64, 16384)])
def test_random_access_decode(dev, kb):
    art, cb = book(*kb)
    x = synth.kv_slab(3, 0, 0, 4, 1, 500).reshape(-1, 64)
    idx, nbits = codec.encode(x, art["Pi"], art["C"])
    words = codec.pack(idx, art["bits"])
    rows = synth.random_rows(len(x), 3001, seed=34)
    rows[:5] = [0, len(x) - 1, 7, 7, 0]
    rows[5], rows[6] = -1, len(x)               # out of range: zero rows
    y = fq.fq_decode(cb, to_dev(words, dev, np.int32), to_dev(nbits, dev, np.int16),
                     rows=to_dev(rows, dev), y_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    full = codec.decode(idx, nbits, art["Pi"], art["C"])
    ok = (rows >= 0) & (rows < len(x))
    want = np.zeros_like(got)
    want[ok] = full[rows[ok]]
    nu16 = np.zeros(len(rows))
    nu16[ok] = codec.f16_value(nbits)[rows[ok]]
    err = np.max(np.abs(got - want), axis=1)
    assert np.all(err <= 1e-3 * nu16)
    assert np.all(got[~ok] == 0)


# ----------------------------------------------------------- packed records
@pytest.mark.parametrize("k,N", [(64, 4096), (32, 4096), (8, 16), (2, 16), (3, 512), (3, 4096),
                                 (64, 16384)])
def test_pack_records_bit_exact(dev, k, N):
    """fq_pack_records of uniform random records and norms equals the oracle's
    packed stream bit for bit (ragged counts), and writes nothing past it."""
    art, cb = book(k, N)
    bits = art["nb"] * art["bits"]
    assert cb.packed_bits == bits + 16
    for n in (1, 13, 1000, 4099):
        w = synth.random_records((n,), cb.W, bits, 41 + n)
        nu = synth.random_norms((n,), 42 + n)
        words = cb.packed_words(n)
        pv, pw = canary_buffer(words, 0, torch.int32, dev)
        fq.fq_pack_records(cb, to_dev(w, dev, np.int32), to_dev(nu, dev, np.int16), packed=pv)
        torch.cuda.synchronize()
        assert canary_intact(pw, words)
        want = codec.pack_stream(codec.unpack(w, art["nb"], art["bits"]), nu, art["bits"])
        assert np.array_equal(host(pv, np.uint32), want), (k, N, n)


@pytest.mark.parametrize("k,N", [(64, 4096), (32, 4096), (8, 16), (3, 4096), (2, 64), (64, 16384)])
def test_decode_packed_contiguous_and_random_access(dev, k, N):
    """Encode, pack, decode from the packed stream: every row equals the
    word-aligned decode of the same codes bit for bit, and the oracle's decode
    within 1e-3 nu16; random access (with out-of-range addresses -> zero rows)."""
    art, cb = book(k, N)
    x = np.concatenate([synth.kv_slab(2, 4, 1, 1, 3, 700).reshape(-1, 64), synth.special_vectors()])
    n = len(x)
    codes, norms = fq.fq_encode(cb, to_dev(x, dev))
    packed = fq.fq_pack_records(cb, codes, norms)
    yv, yw = canary_buffer(n, 64, torch.int16, dev)
    fq.fq_decode_packed(cb, packed, n, y=yv.view(torch.float16))
    y_ref = fq.fq_decode(cb, codes, norms)
    rows = synth.random_rows(n, 3000, seed=43)
    rows[:4] = [-1, n, n - 1, 0]
    rv, rw = canary_buffer(len(rows), 64, torch.int16, dev)
    fq.fq_decode_packed(cb, packed, n, rows=to_dev(rows, dev), y=rv.view(torch.float16))
    torch.cuda.synchronize()
    assert canary_intact(yw, n) and canary_intact(rw, len(rows))
    assert torch.equal(yv, y_ref.view(torch.int16))
    c_np, n_np = host(codes, np.uint32), host(norms, np.uint16)
    i2, n2 = codec.unpack_stream(host(packed, np.uint32), n, art["nb"], art["bits"])
    assert np.array_equal(i2, codec.unpack(c_np, art["nb"], art["bits"])) and np.array_equal(n2, n_np)
    check_decode_full(art, c_np, n_np, host(yv, np.float16), f"packed k{k}N{N}")
    got = host(rv, np.float16).astype(np.float64)
    ok = (rows >= 0) & (rows < n)
    assert np.all(got[~ok] == 0)
    assert np.array_equal(got[ok], host(yv, np.float16).astype(np.float64)[rows[ok]])


# ---------------------------------------------------------------- attention
ATT_CASES = [
    # (B, Hq, Hkv, T, codebook shared by K and V); k = 4, 8 with T a multiple
    # of 8 take the transposed-quarter kernel, the rest the staged-index one
    (2, 8, 1, 1000, (4, 256)),
    (3, 24, 3, 1048, (4, 256)),
    (1, 8, 1, 64, (4, 256)),
    (1, 16, 2, 2056, (8, 256)),
    (1, 1, 1, 8, (8, 256)),
    (2, 4, 1, 512, (8, 16)),
    (1, 3, 3, 264, (4, 4)),
    (1, 4, 1, 1, (4, 256)),
    (2, 8, 1, 300, (4, 256)),
    (2, 32, 4, 1000, (2, 16)),
    (1, 8, 1, 777, (3, 512)),
    (2, 12, 12, 1024, (2, 64)),
    (1, 8, 8, 4099, (8, 16)),
    (1, 16, 2, 2049, (8, 256)),
    (2, 6, 3, 100, (4, 4)),
    (1, 8, 1, 64, (2, 256)),
    (2, 8, 2, 520, (2, 32)),
    # one split per (batch, KV head) (T <= 256, or 512 or more pairs),
    # finished without the merge pass
    (4, 32, 4, 256, (4, 256)),
    (8, 16, 2, 200, (2, 16)),
    (128, 8, 8, 130, (2, 64)),
    (1, 4, 4, 130, (2, 128)),
    # k = 2, N = 16 read as k = 4, N = 256 over codeword pairs: the GPT-2
    # shape (one query head per KV head) and grouped heads
    (4, 12, 12, 1024, (2, 16)),
    (2, 16, 2, 2056, (2, 16)),
]


def run_attention(dev, q, kw, kn, vw, vn, ck, cv, scale=0.125):
    o = fq.fq_attend_decode(ck, cv, to_dev(q, dev), to_dev(kw, dev, np.int32),
                            to_dev(kn, dev, np.int16), to_dev(vw, dev, np.int32),
                            to_dev(vn, dev, np.int16), scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", ATT_CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}T{c[3]}k{c[4][0]}N{c[4][1]}")
def test_attention(dev, case):
    B, Hq, Hkv, T, kb = case
    art, cb = book(*kb)
    seed = B * 1000 + T
    bits = cb.nb * cb.info["idx_bits"]
    kw = synth.random_records((B, Hkv, T), cb.W, bits, seed)
    vw = synth.random_records((B, Hkv, T), cb.W, bits, seed + 1)
    kn = synth.random_norms((B, Hkv, T), seed + 2)
    vn = synth.random_norms((B, Hkv, T), seed + 3)
    q = synth.query(B, Hq, seed=seed + 4)
    got = run_attention(dev, q, kw, kn, vw, vn, cb, cb)
    ref = attend.attend(q, kw, kn, vw, vn, art["Pi"], art["C"], art["C"], 0.125)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    print(f"{case}: max rel {np.max(rel):.2e}")
    assert np.max(rel) <= 2e-3


QUERY_CASES = [
    # (B, Hq, Hkv, T, T_ld, M, codebook): M causal queries per head over the
    # first T of T_ld cached tokens (slots past T hold other records)
    (2, 4, 4, 300, 320, 4, (2, 16)),
    (2, 8, 4, 512, 520, 4, (4, 256)),     # transposed-quarter kernel, 8 columns
    (1, 8, 1, 1000, 1000, 1, (4, 256)),
    (3, 2, 2, 77, 100, 8, (8, 256)),      # T not a multiple of 8: staged kernel
    (2, 4, 2, 2048, 4096, 3, (3, 512)),
    (1, 4, 1, 8, 64, 2, (8, 16)),
    (4, 16, 4, 2000, 2048, 2, (4, 256)),
]


@pytest.mark.parametrize("case", QUERY_CASES,
                         ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}T{c[3]}ld{c[4]}M{c[5]}k{c[6][0]}N{c[6][1]}")
def test_attend_queries(dev, case):
    B, Hq, Hkv, T, T_ld, M, kb = case
    art, cb = book(*kb)
    seed = B * 1000 + T + M
    bits = cb.nb * cb.info["idx_bits"]
    kw = synth.random_records((B, Hkv, T_ld), cb.W, bits, seed)
    vw = synth.random_records((B, Hkv, T_ld), cb.W, bits, seed + 1)
    kn = synth.random_norms((B, Hkv, T_ld), seed + 2)
    vn = synth.random_norms((B, Hkv, T_ld), seed + 3)
    q = np.stack([synth.query(B, Hq, seed=seed + 4 + m) for m in range(M)], axis=2)
    o = fq.fq_attend_queries(cb, cb, to_dev(q, dev), to_dev(kw, dev, np.int32),
                             to_dev(kn, dev, np.int16), to_dev(vw, dev, np.int32),
                             to_dev(vn, dev, np.int16), T, 0.125)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    ref = attend.attend_queries(q, kw, kn, vw, vn, art["Pi"], art["C"], art["C"], 0.125, T)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    print(f"{case}: max rel {np.max(rel):.2e}")
    assert np.max(rel) <= 2e-3


STEP_CASES = [
    # (codebook, M, pos, separate K and V handles); pos + M a multiple of 8
    # with k = 4, 8 (and k = 2, N = 16 over codeword pairs) takes the direct
    # kernel, which encodes the appended tokens on all four waves; the rest
    # encode them one wave per vector inside the staged kernel
    ((4, 256), 1, 101, False), ((4, 256), 3, 101, False), ((2, 16), 1, 101, False),
    ((2, 64), 4, 101, False), ((4, 256), 1, 103, False), ((8, 256), 8, 96, False),
    ((4, 256), 2, 62, True), ((2, 16), 2, 5, True), ((8, 16), 1, 0, False),
    ((2, 16), 1, 103, False), ((2, 16), 3, 61, True),
]


@pytest.mark.parametrize("kb,M,pos,two", STEP_CASES)
def test_decode_step_appends_and_attends(dev, kb, M, pos, two):
    """Encode-on-append: the M new keys and values land in slots pos .. pos + M - 1
    as the oracle encodes them, no other slot changes, and the output is the
    oracle's causal attention over the pos + M cached tokens."""
    art, cb = book(*kb)
    cbv = fq.fq_codebook_load(open(artifact_path(*kb), "rb").read(), 0) if two else cb
    B, Hq, Hkv, T_ld = 2, 8, 4, 264
    Hq = min(Hq, Hkv * (8 // M))
    bits = cb.nb * cb.info["idx_bits"]
    kw = synth.random_records((B, Hkv, T_ld), cb.W, bits, 71)
    vw = synth.random_records((B, Hkv, T_ld), cb.W, bits, 72)
    kn = synth.random_norms((B, Hkv, T_ld), 73)
    vn = synth.random_norms((B, Hkv, T_ld), 74)
    k_new = synth.kv_slab(3, 5, 0, B, Hkv, M)          # [B, Hkv, M, 64]
    v_new = synth.kv_slab(3, 5, 1, B, Hkv, M)
    q = np.stack([synth.query(B, Hq, seed=80 + m) for m in range(M)], axis=2)
    tk = [to_dev(kw, dev, np.int32), to_dev(kn, dev, np.int16), to_dev(vw, dev, np.int32),
          to_dev(vn, dev, np.int16)]
    o = fq.fq_decode_step(cb, cbv, to_dev(q, dev), to_dev(k_new, dev), to_dev(v_new, dev), *tk,
                          pos, 0.125)
    torch.cuda.synchronize()
    kw2, kn2, vw2, vn2 = [t.cpu().numpy() for t in tk]
    kw2, vw2 = kw2.view(np.uint32), vw2.view(np.uint32)
    kn2, vn2 = kn2.view(np.uint16), vn2.view(np.uint16)
    new = slice(pos, pos + M)
    for old, got in ((kw, kw2), (kn, kn2), (vw, vw2), (vn, vn2)):
        keep = np.ones(T_ld, dtype=bool)
        keep[new] = False
        assert np.array_equal(old[:, :, keep], got[:, :, keep])
    for x, c, nn in ((k_new, kw2, kn2), (v_new, vw2, vn2)):
        check_encode(art, x.reshape(-1, 64), c[:, :, new].reshape(-1, cb.W),
                     nn[:, :, new].reshape(-1))
    got = o.float().cpu().numpy().astype(np.float64)
    ref = attend.attend_queries(q, kw2, kn2, vw2, vn2, art["Pi"], art["C"], art["C"], 0.125,
                                pos + M)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    print(f"k{kb[0]}N{kb[1]} M{M}: max rel {np.max(rel):.2e}")
    assert np.max(rel) <= 2e-3


def test_decode_step_off_grid_codebook(dev):
    """A codebook whose table is not on the binary16 grid (the shipped ones
    are): the appended tokens go through the separate float64 append launch
    and the attention through the hi / lo table path."""
    art = artifact.read_artifact(open(artifact_path(2, 16), "rb").read())
    C = art["C"].astype(np.float64)
    C = (C * (1.0 + 1e-4 * np.sin(np.arange(C.size)).reshape(C.shape))).astype(np.float32)
    assert not np.array_equal(C.astype(np.float16).astype(np.float32), C)
    art2 = dict(art)
    art2["C"] = C
    art2["d"] = 64
    blob = artifact.write_artifact(art["Pi"], art2)
    ref_art = artifact.read_artifact(blob)
    cb = fq.fq_codebook_load(blob, 0)
    B, Hq, Hkv, T_ld, M, pos = 2, 8, 4, 128, 2, 40
    bits = cb.nb * cb.info["idx_bits"]
    kw = synth.random_records((B, Hkv, T_ld), cb.W, bits, 61)
    vw = synth.random_records((B, Hkv, T_ld), cb.W, bits, 62)
    kn = synth.random_norms((B, Hkv, T_ld), 63)
    vn = synth.random_norms((B, Hkv, T_ld), 64)
    k_new = synth.kv_slab(3, 7, 0, B, Hkv, M)
    v_new = synth.kv_slab(3, 7, 1, B, Hkv, M)
    q = np.stack([synth.query(B, Hq, seed=66 + m) for m in range(M)], axis=2)
    tk = [to_dev(kw, dev, np.int32), to_dev(kn, dev, np.int16), to_dev(vw, dev, np.int32),
          to_dev(vn, dev, np.int16)]
    o = fq.fq_decode_step(cb, cb, to_dev(q, dev), to_dev(k_new, dev), to_dev(v_new, dev), *tk,
                          pos, 0.125)
    torch.cuda.synchronize()
    kw2, kn2, vw2, vn2 = [t.cpu().numpy() for t in tk]
    kw2, vw2, kn2, vn2 = kw2.view(np.uint32), vw2.view(np.uint32), kn2.view(np.uint16), vn2.view(np.uint16)
    new = slice(pos, pos + M)
    for x, c, nn in ((k_new, kw2, kn2), (v_new, vw2, vn2)):
        check_encode(ref_art, x.reshape(-1, 64), c[:, :, new].reshape(-1, cb.W),
                     nn[:, :, new].reshape(-1))
    got = o.float().cpu().numpy().astype(np.float64)
    ref = attend.attend_queries(q, kw2, kn2, vw2, vn2, ref_art["Pi"], ref_art["C"], ref_art["C"],
                                0.125, pos + M)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert np.max(rel) <= 2e-3


OFF_GRID = [(2, 64), (3, 512), (4, 256), (8, 256), (8, 16), (4, 4), (3, 4096)]


@pytest.mark.parametrize("k,N", OFF_GRID)
def test_off_grid_codebooks(dev, k, N):
    """Tables that are not on the binary16 grid (the shipped ones are, reading
    of the table precision): each shipped table scaled by 1 + 1e-4 sin(i) per
    entry.  Encode (candidate lists rebuilt for the new table; for k = 8 with
    N = 256 the vector-unit scan instead of the matrix-core search, which
    needs a binary16 table) against the oracle on the same float32 table,
    decode (binary16 copy of the table: within the 1e-3 nu bar) and, where
    the attention kernels take the variant, attention over random records
    (hi / lo table path) against the oracle's decompress-then-attend."""
    art = artifact.read_artifact(open(artifact_path(k, N), "rb").read())
    C = art["C"].astype(np.float64)
    C = (C * (1.0 + 1e-4 * np.sin(np.arange(C.size)).reshape(C.shape))).astype(np.float32)
    assert not np.array_equal(C.astype(np.float16).astype(np.float32), C)
    art2 = dict(art)
    art2["C"] = C
    blob = artifact.write_artifact(art["Pi"], art2)
    ref = artifact.read_artifact(blob)
    cb = fq.fq_codebook_load(blob, 0)
    x = np.concatenate([synth.kv_slab(3, 5, 0, 2, 3, 400).reshape(-1, 64), synth.special_vectors()])
    codes, norms = gpu_encode(cb, x, dev)
    ex, win = check_encode(ref, x, codes, norms)
    y = fq.fq_decode(cb, to_dev(codes, dev, np.int32), to_dev(norms, dev, np.int16))
    torch.cuda.synchronize()
    check_decode_full(ref, codes, norms, y.cpu().numpy(), f"off-grid k{k}N{N}")
    if (k, N) != (3, 4096):      # the 4096-entry table exceeds the attention kernels' LDS
        B, Hq, Hkv, T = 2, 8, 2, 520
        bits = cb.nb * cb.info["idx_bits"]
        kw = synth.random_records((B, Hkv, T), cb.W, bits, 71)
        vw = synth.random_records((B, Hkv, T), cb.W, bits, 72)
        kn = synth.random_norms((B, Hkv, T), 73)
        vn = synth.random_norms((B, Hkv, T), 74)
        q = synth.query(B, Hq, seed=75)
        got = run_attention(dev, q, kw, kn, vw, vn, cb, cb)
        want = attend.attend(q, kw, kn, vw, vn, ref["Pi"], ref["C"], ref["C"], 0.125)
        rel = np.linalg.norm(got - want, axis=-1) / np.linalg.norm(want, axis=-1)
        assert np.max(rel) <= 2e-3, float(np.max(rel))
    print(f"off-grid k{k}N{N}: {ex} exact, {win} in window", flush=True)


def test_decode_step_large_append(dev):
    """A prefill-sized append (64 x 32 heads x 8 tokens per cache, past the
    small-append kernel's range) into an empty cache, then causal attention."""
    art, cb = book(2, 64)
    B, Hkv, M, T_ld = 64, 32, 8, 16
    Hq = Hkv
    kw = np.zeros((B, Hkv, T_ld, cb.W), dtype=np.uint32)
    kn = np.zeros((B, Hkv, T_ld), dtype=np.uint16)
    k_new = synth.kv_slab(3, 6, 0, B, Hkv, M)
    v_new = synth.kv_slab(3, 6, 1, B, Hkv, M)
    q = np.stack([synth.query(B, Hq, seed=90 + m) for m in range(M)], axis=2)
    tk = [to_dev(kw, dev, np.int32), to_dev(kn, dev, np.int16), to_dev(kw, dev, np.int32),
          to_dev(kn, dev, np.int16)]
    o = fq.fq_decode_step(cb, cb, to_dev(q, dev), to_dev(k_new, dev), to_dev(v_new, dev), *tk, 0,
                          0.125)
    torch.cuda.synchronize()
    kw2, kn2, vw2, vn2 = [t.cpu().numpy() for t in tk]
    kw2, vw2, kn2, vn2 = kw2.view(np.uint32), vw2.view(np.uint32), kn2.view(np.uint16), vn2.view(np.uint16)
    assert np.all(kw2[:, :, M:] == 0) and np.all(vn2[:, :, M:] == 0)
    for x, c, nn in ((k_new, kw2, kn2), (v_new, vw2, vn2)):
        check_encode(art, x.reshape(-1, 64), c[:, :, :M].reshape(-1, cb.W), nn[:, :, :M].reshape(-1))
    got = o.float().cpu().numpy().astype(np.float64)
    ref = attend.attend_queries(q, kw2, kn2, vw2, vn2, art["Pi"], art["C"], art["C"], 0.125, M)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert np.max(rel) <= 2e-3


def test_queries_and_step_reject_bad_shapes(dev):
    _, c4 = book(4, 256)
    kw = torch.zeros((1, 2, 64, c4.W), dtype=torch.int32, device=dev)
    nn = torch.zeros((1, 2, 64), dtype=torch.int16, device=dev)
    q = torch.zeros((1, 8, 3, 64), dtype=torch.float16, device=dev)    # 4 heads x 3 queries per KV head
    with pytest.raises(fq.FQError) as e:
        fq.fq_attend_queries(c4, c4, q, kw, nn, kw, nn, 32, 0.125)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED
    q2 = torch.zeros((1, 2, 2, 64), dtype=torch.float16, device=dev)
    with pytest.raises(fq.FQError) as e:                                  # T > T_ld
        fq.fq_attend_queries(c4, c4, q2, kw, nn, kw, nn, 65, 0.125)
    assert e.value.status == fq.FQ_ERR_INVALID_ARG
    kn = torch.zeros((1, 2, 2, 64), dtype=torch.float16, device=dev)
    with pytest.raises(fq.FQError) as e:                                  # pos + M > T_ld
        fq.fq_decode_step(c4, c4, q2, kn, kn, kw, nn, kw, nn, 63, 0.125)
    assert e.value.status == fq.FQ_ERR_INVALID_ARG


def test_attention_rejects_unsupported(dev):
    _, c4 = book(4, 256)
    _, c2 = book(2, 16)
    q = torch.zeros((1, 16, 64), dtype=torch.float16, device=dev)
    kw = torch.zeros((1, 1, 8, c4.W), dtype=torch.int32, device=dev)
    nn = torch.zeros((1, 1, 8), dtype=torch.int16, device=dev)
    with pytest.raises(fq.FQError) as e:            # 16 query heads per KV head
        fq.fq_attend_decode(c4, c4, q, kw, nn, kw, nn, 0.125)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED
    with pytest.raises((fq.FQError, ValueError)):   # K and V codebooks of different variants
        fq.fq_attend_decode(c4, c2, q[:, :8], kw, nn, kw, nn, 0.125)
    _, c64 = book(64, 4096)                          # table larger than LDS
    q8 = torch.zeros((1, 8, 64), dtype=torch.float16, device=dev)
    k1 = torch.zeros((1, 1, 8, c64.W), dtype=torch.int32, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_attend_decode(c64, c64, q8, k1, nn, k1, nn, 0.125)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED


def test_attention_rejects_keys_and_values_under_different_rotations(dev):
    """Two valid artifacts that differ only in the rotation: scores and values
    live in one rotated domain, so attention, multi-query attention and the
    decode step refuse the pair (FibQuant technical summary, sections 1 and
    2.3: one shared rotation)."""
    from oracle import rotation
    art, c4 = book(4, 256)
    other = dict(art)
    other["d"] = 64
    cb_b = fq.fq_codebook_load(artifact.write_artifact(rotation.make_rotation(64, 1), other), 0)
    same = fq.fq_codebook_load(artifact.write_artifact(art["Pi"], other), 0)
    B, Hq, Hkv, T = 1, 8, 1, 64
    q = torch.zeros((B, Hq, 64), dtype=torch.float16, device=dev)
    kw = torch.zeros((B, Hkv, T, c4.W), dtype=torch.int32, device=dev)
    nn = torch.zeros((B, Hkv, T), dtype=torch.int16, device=dev)
    for call in (lambda v: fq.fq_attend_decode(c4, v, q, kw, nn, kw, nn, 0.125),
                 lambda v: fq.fq_attend_queries(c4, v, q.view(B, Hq, 1, 64), kw, nn, kw, nn, T,
                                                0.125),
                 lambda v: fq.fq_decode_step(c4, v, q.view(B, Hq, 1, 64),
                                             q.view(B, Hq, 1, 64)[:, :Hkv],
                                             q.view(B, Hq, 1, 64)[:, :Hkv], kw, nn, kw, nn,
                                             T - 1, 0.125)):
        with pytest.raises(fq.FQError) as e:
            call(cb_b)
        assert e.value.status == fq.FQ_ERR_UNSUPPORTED
        call(same)                    # a second handle with the same rotation is fine
    torch.cuda.synchronize()


def test_attention_tinyllama_sampled(dev):
    """Decode step at batch 16, 32 query / 4 KV heads, 32768 tokens, k4N256.

    Sampled (batch, KV head) streams carry oracle-encoded synthetic keys and
    values (per-channel log-uniform scales, 1% x20 outlier channels); the rest
    carry uniform random records.  Checked row by row on the sampled streams.
    """
    B, Hq, Hkv, T = 16, 32, 4, 32768
    art, cb = book(4, 256)
    bits = cb.nb * cb.info["idx_bits"]
    kw = synth.random_records((B, Hkv, T), cb.W, bits, 51)
    vw = synth.random_records((B, Hkv, T), cb.W, bits, 52)
    kn = synth.random_norms((B, Hkv, T), 53)
    vn = synth.random_norms((B, Hkv, T), 54)
    sampled = [(0, 0), (7, 2), (15, 3)]
    for (b, g) in sampled:
        for kv, (w_, n_) in enumerate(((kw, kn), (vw, vn))):
            x = synth.kv_stream(3, b, kv, g, (T,))
            idx, nb = codec.encode(x, art["Pi"], art["C"])
            w_[b, g] = codec.pack(idx, art["bits"])
            n_[b, g] = nb
    q = synth.query(B, Hq, seed=5)
    got = run_attention(dev, q, kw, kn, vw, vn, cb, cb)
    rows = [(b, h) for (b, g) in sampled for h in range(8 * g, 8 * g + 8)]
    ref = attend.attend(q, kw, kn, vw, vn, art["Pi"], art["C"], art["C"], 0.125, rows=rows)
    worst = 0.0
    for (b, h), o in ref.items():
        rel = np.linalg.norm(got[b, h] - o) / np.linalg.norm(o)
        worst = max(worst, rel)
    print(f"tinyllama sampled rows: max rel {worst:.2e}")
    assert worst <= 2e-3


# ------------------------------------------------- full-size configurations
# Coverage at the configurations' real sizes, in the launch configuration the
# bench times, every row of every set: the GPT-2-small-shaped cache for every
# variant, the TinyLlama-shaped cache (plus every one of 2^20 random-access
# decodes) and the 2^24-vector stress set -- every index against the compiled
# float64 oracle, every norm, every pad bit, every decoded vector.  Every
# output buffer is followed by canary words that must survive.
TAIL = 64                          # canary rows after every output
CANARY32 = -0x5A5A5A5B             # 0xA5A5A5A5 as int32
CANARY16 = 0x5A5A


def canary_buffer(n, cols, dtype, dev):
    """(view of the first n rows, the whole buffer) with TAIL canary rows after them."""
    fill = CANARY32 if dtype == torch.int32 else CANARY16
    shape = (n + TAIL,) + ((cols,) if cols else ())
    whole = torch.full(shape, fill, dtype=dtype, device=dev)
    return whole[:n], whole


def canary_intact(whole, n):
    fill = CANARY32 if whole.dtype == torch.int32 else CANARY16
    return bool(torch.all(whole[n:] == fill).item())


def canary_codec_outputs(cb, n, dev):
    codes, cw = canary_buffer(n, cb.W, torch.int32, dev)
    norms, nw = canary_buffer(n, 0, torch.int16, dev)
    return codes, norms, (cw, nw)


def check_norms_from_nu(nu, norms):
    want = codec.f16_round(nu)
    diff = np.nonzero(norms != want)[0]
    for r in diff:
        lo = codec.f16_value(np.array([min(norms[r], want[r])]))[0]
        hi = codec.f16_value(np.array([max(norms[r], want[r])]))[0]
        assert abs(int(norms[r]) - int(want[r])) == 1, (r, norms[r], want[r])
        assert abs(nu[r] - 0.5 * (lo + hi)) <= 1e-6 * nu[r], (r, nu[r])
    return len(diff)


def check_rows_full(art, x, codes, norms, label, chunk=1 << 18):
    """Every index of every row against the compiled float64 oracle (near-tie
    window 1e-6), every norm, every pad bit; x, codes, norms host arrays."""
    nb, bits, W = art["nb"], art["bits"], art["W"]
    n = len(x)
    assert codes.shape == (n, W)
    used = nb * bits - 32 * (W - 1)
    if used < 32:
        assert np.all((codes[:, -1] >> np.uint32(used)) == 0), "pad bits not zero"
    ex = win = bad = 0
    first = -1
    near_mid = 0
    for s in range(0, n, chunk):
        xs = x[s:s + chunk]
        e_, w_, b_, f_ = native.accept(xs, art["Pi"], art["C"],
                                       codec.unpack(codes[s:s + chunk], nb, bits))
        ex, win, bad = ex + e_, win + w_, bad + b_
        if first < 0 and f_ >= 0:
            first = s + f_
        xd = xs.astype(np.float64)
        near_mid += check_norms_from_nu(np.sqrt(np.sum(xd * xd, axis=1)), norms[s:s + chunk])
    print(f"PARITY {label} rows={n} indices exact={ex} in_window={win} out_of_window={bad} "
          f"norms_off_by_one_ulp_at_midpoint={near_mid}", flush=True)
    assert bad == 0, f"{label}: {bad} indices outside the near-tie window (first row {first})"
    return ex, win


def check_decode_full(art, codes, norms, y, label, chunk=1 << 18):
    """Every decoded row against the oracle's float64 decode of the same record:
    max |y - x_hat| <= 1e-3 nu16 per row."""
    worst = 0.0
    for s in range(0, len(codes), chunk):
        idx = codec.unpack(codes[s:s + chunk], art["nb"], art["bits"])
        want = codec.decode(idx, norms[s:s + chunk], art["Pi"], art["C"])
        got = y[s:s + chunk].astype(np.float64)
        nu16 = codec.f16_value(norms[s:s + chunk])
        err = np.max(np.abs(got - want), axis=1)
        bad = np.nonzero(err > 1e-3 * nu16 + 1e-30)[0]
        assert len(bad) == 0, f"{label}: row {s + bad[0]} decode error {err[bad[0]]}"
        worst = max(worst, float(np.max(err / np.maximum(nu16, 1e-30))))
    print(f"PARITY {label} decoded rows={len(codes)} max_err_over_nu={worst:.3e}", flush=True)
    return worst


def host(t, dt):
    return t.cpu().numpy().view(dt)


_GPT2 = []


def gpt2_cache():
    if not _GPT2:
        _GPT2.append(synth.kv_cache(2, 12, 4, 12, 1024).reshape(-1, 64))
    return _GPT2[0]


@pytest.mark.parametrize("k,N", [(2, 16), (2, 64), (2, 256), (3, 512)])
def test_gpt2_cache_full_size(dev, k, N):
    """GPT-2-small-shaped cache (1,179,648 vectors), encoded and decoded on the
    GPU in the bench's launch configuration: every index, norm, pad bit and
    decoded vector checked against the oracle; no write past any output."""
    print(f"gpt2 cache k{k}N{N}", flush=True)
    art, cb = book(k, N)
    x = gpt2_cache()
    n = len(x)
    xd = to_dev(x, dev)
    codes, norms, (cw, nw) = canary_codec_outputs(cb, n, dev)
    fq.fq_encode(cb, xd, codes, norms)
    yv, yw = canary_buffer(n, 64, torch.int16, dev)
    fq.fq_decode(cb, codes, norms, y=yv.view(torch.float16))
    torch.cuda.synchronize()
    assert canary_intact(cw, n) and canary_intact(nw, n) and canary_intact(yw, n)
    c_np, n_np = host(codes, np.uint32), host(norms, np.uint16)
    check_rows_full(art, x, c_np, n_np, f"gpt2 k{k}N{N}")
    check_decode_full(art, c_np, n_np, host(yv, np.float16), f"gpt2 k{k}N{N}")


@pytest.mark.parametrize("k,N", [(32, 4096), (64, 4096), (64, 16384)])
def test_large_blocks_gpt2_cache_full_size(dev, k, N):
    """k = 32 / 64 with N = 4096 and k = 64 with N = 16384 on the whole
    GPT-2-small-shaped cache: every row against the oracle (each costs N * 64
    float64 multiply-adds there), every norm and pad bit, every decoded vector."""
    print(f"gpt2 cache k{k}N{N}", flush=True)
    art, cb = book(k, N)
    x = gpt2_cache()
    n = len(x)
    codes, norms, (cw, nw) = canary_codec_outputs(cb, n, dev)
    fq.fq_encode(cb, to_dev(x, dev), codes, norms)
    yv, yw = canary_buffer(n, 64, torch.int16, dev)
    fq.fq_decode(cb, codes, norms, y=yv.view(torch.float16))
    torch.cuda.synchronize()
    assert canary_intact(cw, n) and canary_intact(nw, n) and canary_intact(yw, n)
    c_np, n_np = host(codes, np.uint32), host(norms, np.uint16)
    check_rows_full(art, x, c_np, n_np, f"gpt2 k{k}N{N} (all rows)")
    check_decode_full(art, c_np, n_np, host(yv, np.float16), f"gpt2 k{k}N{N}")


@pytest.mark.parametrize("k,N", [(32, 4096), (64, 4096), (64, 16384)])
def test_packed_records_gpt2_cache_full_size(dev, k, N):
    """The 25.6x (k = 32), 36.6x (k = 64, N = 4096) and 34.1x (k = 64,
    N = 16384) packed forms of the whole GPT-2-shaped cache: packed stream equal
    to the oracle's packing of the GPU's codes, every vector decoded from it
    equal to the word-aligned decode bit for bit."""
    print(f"gpt2 cache k{k}N{N} packed", flush=True)
    art, cb = book(k, N)
    x = gpt2_cache()
    n = len(x)
    codes, norms = fq.fq_encode(cb, to_dev(x, dev))
    words = cb.packed_words(n)
    pv, pw = canary_buffer(words, 0, torch.int32, dev)
    fq.fq_pack_records(cb, codes, norms, packed=pv)
    y1 = fq.fq_decode(cb, codes, norms)
    y2 = fq.fq_decode_packed(cb, pv, n)
    torch.cuda.synchronize()
    assert canary_intact(pw, words)
    want = codec.pack_stream(codec.unpack(host(codes, np.uint32), art["nb"], art["bits"]),
                             host(norms, np.uint16), art["bits"])
    assert np.array_equal(host(pv, np.uint32), want)
    assert torch.equal(y1, y2)
    print(f"PARITY gpt2 k{k}N{N} packed rows={n} bits_per_vector={cb.packed_bits} "
          f"compression={1024 / cb.packed_bits:.1f}x", flush=True)


@pytest.mark.parametrize("k,N", [(4, 256), (8, 256)])
def test_tinyllama_cache_encode_and_random_access(dev, k, N):
    """TinyLlama-shaped cache (22 layers x {K,V} x batch 8 x 4 heads x 2048
    tokens, generated on the device): full encode, every row against the
    oracle, then 2^20 uniformly drawn addresses decoded by address, every one
    of them checked against the oracle's decode of the record it names."""
    print(f"tinyllama cache k{k}N{N}", flush=True)
    art, cb = book(k, N)
    L, B, H, T = 22, 8, 4, 2048
    slabs = [synth.kv_slab_device(3, layer, kv, B, H, T, dev).reshape(-1, 64)
             for layer in range(L) for kv in range(2)]
    xd = torch.cat(slabs)
    del slabs
    n = xd.shape[0]
    codes, norms, (cw, nw) = canary_codec_outputs(cb, n, dev)
    fq.fq_encode(cb, xd, codes, norms)
    addr = synth.random_rows(n, 1 << 20, seed=33)
    yv, yw = canary_buffer(len(addr), 64, torch.int16, dev)
    fq.fq_decode(cb, codes, norms, rows=to_dev(addr, dev), y=yv.view(torch.float16))
    torch.cuda.synchronize()
    assert canary_intact(cw, n) and canary_intact(nw, n) and canary_intact(yw, len(addr))
    c_np, n_np = host(codes, np.uint32), host(norms, np.uint16)
    check_rows_full(art, xd.cpu().numpy(), c_np, n_np, f"tinyllama k{k}N{N} (all rows)")
    check_decode_full(art, c_np[addr], n_np[addr], host(yv, np.float16),
                      f"tinyllama k{k}N{N} random access (2^20 addresses)")


_STRESS = {}


def stress_outputs(k, N, dev):
    """2^24 vectors (256 streams x 65536 tokens, generated on the device),
    encoded and decoded in the bench's launch configuration, with canaries
    after every output; host copies of inputs and outputs (kept for the
    parts of one code)."""
    if _STRESS.get("key") != (k, N):
        _STRESS.clear()
        art, cb = book(k, N)
        xd = synth.kv_slab_device(4, 0, 0, 1, 256, 65536, dev).reshape(-1, 64)
        n = xd.shape[0]
        codes, norms, (cw, nw) = canary_codec_outputs(cb, n, dev)
        fq.fq_encode(cb, xd, codes, norms)
        yv, yw = canary_buffer(n, 64, torch.int16, dev)
        fq.fq_decode(cb, codes, norms, y=yv.view(torch.float16))
        torch.cuda.synchronize()
        assert canary_intact(cw, n) and canary_intact(nw, n) and canary_intact(yw, n)
        used = art["nb"] * art["bits"] - 32 * (art["W"] - 1)
        if used < 32:
            assert not bool(torch.any((codes[:, -1] >> used) != 0).item()), "pad bits not zero"
        _STRESS.update(key=(k, N), x=xd.cpu().numpy(), codes=host(codes, np.uint32),
                       norms=host(norms, np.uint16), y=host(yv, np.float16))
        del xd, codes, norms, yv
    return _STRESS


@pytest.mark.parametrize("k,N,part,parts", [(8, 16, 0, 1), (4, 4, 0, 1)] +
                         [(3, 4096, p, 4) for p in range(4)])
def test_stress_set_2_24(dev, k, N, part, parts):
    """The 2^24-vector set: every row checked against the oracle (indices,
    norms, decoded vectors), every pad bit, no write past any output; the
    k3N4096 rows in four parts (its brute-force search compares 4096
    codewords per block), each its own test."""
    print(f"stress set k{k}N{N} part {part + 1}/{parts}", flush=True)
    art, _ = book(k, N)
    st = stress_outputs(k, N, dev)
    n = len(st["x"])
    lo, hi = n * part // parts, n * (part + 1) // parts
    what = "all rows" if parts == 1 else f"rows {lo}..{hi - 1}"
    check_rows_full(art, st["x"][lo:hi], st["codes"][lo:hi], st["norms"][lo:hi],
                    f"stress k{k}N{N} ({what})")
    check_decode_full(art, st["codes"][lo:hi], st["norms"][lo:hi], st["y"][lo:hi],
                      f"stress k{k}N{N} ({what})")
    if part == parts - 1:
        _STRESS.clear()


@pytest.mark.parametrize("layer", [0, 21])
def test_attention_tinyllama_layer_full(dev, layer):
    """One TinyLlama decode-step layer in full: batch 16, 32 query / 4 KV heads,
    32768 tokens, k4N256 keys and values generated and encoded on the device;
    every (b, h) output checked against the oracle's decompress-then-attend of
    the same records."""
    print(f"attention layer {layer}", flush=True)
    art, cb = book(4, 256)
    B, Hq, Hkv, T = 16, 32, 4, 32768
    enc = []
    for kv in range(2):
        x = synth.kv_slab_device(3, layer, kv, B, Hkv, T, dev).reshape(-1, 64)
        c, nn = fq.fq_encode(cb, x)
        enc.append((c.view(B, Hkv, T, cb.W), nn.view(B, Hkv, T)))
        del x
    q = synth.query(B, Hq, seed=5)
    out = fq.fq_attend_decode(cb, cb, to_dev(q, dev), enc[0][0], enc[0][1], enc[1][0],
                              enc[1][1], 0.125)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    kw = enc[0][0].cpu().numpy().view(np.uint32)
    kn = enc[0][1].cpu().numpy().view(np.uint16)
    vw = enc[1][0].cpu().numpy().view(np.uint32)
    vn = enc[1][1].cpu().numpy().view(np.uint16)
    ref = attend.attend(q, kw, kn, vw, vn, art["Pi"], art["C"], art["C"], 0.125)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    glob = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"layer {layer}: max rel {np.max(rel):.2e}, global {glob:.2e}")
    assert np.max(rel) <= 2e-3


def test_attention_fidelity_rises_with_rate(dev):
    """Attention over the compressed cache against exact attention over the
    uncompressed binary16 cache (float64 on the host): the mean cosine over
    (batch, query head) rises with the rate in the k = 2 family."""
    B, Hq, Hkv, T = 2, 32, 4, 2048
    G = Hq // Hkv
    q = synth.query(B, Hq, seed=7)
    means = []
    for N in (16, 64, 256):
        _, cb = book(2, N)
        cos = []
        for layer in (0, 21):
            K = synth.kv_slab(3, layer, 0, B, Hkv, T)
            V = synth.kv_slab(3, layer, 1, B, Hkv, T)
            kc, kn = fq.fq_encode(cb, to_dev(K.reshape(-1, 64), dev))
            vc, vn = fq.fq_encode(cb, to_dev(V.reshape(-1, 64), dev))
            o = fq.fq_attend_decode(cb, cb, to_dev(q, dev), kc.view(B, Hkv, T, cb.W),
                                    kn.view(B, Hkv, T), vc.view(B, Hkv, T, cb.W),
                                    vn.view(B, Hkv, T), 0.125).float().cpu().numpy()
            qd = q.astype(np.float64).reshape(B, Hkv, G, 64)
            s = np.einsum("bgxd,bgtd->bgxt", qd, K.astype(np.float64)) * 0.125
            p = np.exp(s - s.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            ref = np.einsum("bgxt,bgtd->bgxd", p, V.astype(np.float64)).reshape(B, Hq, 64)
            cos.append((o * ref).sum(-1) / (np.linalg.norm(o, axis=-1) * np.linalg.norm(ref, axis=-1)))
        means.append(float(np.mean(cos)))
    print("mean attention cosine at 2, 3, 4 bits:", means)
    assert means[0] < means[1] < means[2]
    assert means[2] > 0.8
