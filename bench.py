#!/usr/bin/env python3
"""Throughput of the FibQuant hot path on one MI355X.

One step is one pass of the whole path over the GPT-2-small-shaped KV cache
(12 layers x {K, V} x batch 4 x 12 heads x 1024 tokens, d = 64, binary16,
seeded synthetic values with per-channel log-uniform scales and 1% x20
outlier channels):

  for each rate variant k2N16, k2N64, k2N256, k3N512:
      encode every vector (norm, rotation, block search, packing)
      decode every record (gather, inverse rotation, rescale) to binary16
  random-access decode of 2^20 uniformly drawn records (k2N16 codes)
  decode-step attention over the compressed cache, all 12 layers (k2N16)

``value`` is vectors encoded and decoded per second over the whole step.  The
same run also times fused attention at the TinyLlama-shaped decode step
(batch 16, 32 query / 4 KV heads, 32768 tokens, 22 layers, k4N256) and
reports its HBM bandwidth, and times the CPU oracle on a bounded sample.

Each (variant, op) works on its own buffers (four input replicas of 151 MB)
so that reads are served from HBM rather than the 256 MB Infinity Cache.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV vectors/s encode+decode (d=64) and attend HBM GB/s, % of MI355X peak"
HBM_PEAK_GBS = 8000.0
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12     # non-packed lane-ops/s: 39.3 T
MFMA_F16_PEAK_TFLOPS = 2500.0                      # dense binary16 matrix cores
VARIANTS = [(2, 16), (2, 64), (2, 256), (3, 512)]
LARGE_VARIANTS = [(32, 4096), (64, 4096)]
L, B, H, T = 12, 4, 12, 1024
N_RAND = 1 << 20
COPY_BYTES = 1 << 28


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def enc_ops_per_vector(k, N):
    """Op-count model of encode: 4096 rotation MACs + nb*N*(k+2) search lane-ops."""
    nb = -(-64 // k)
    return 4096 + nb * N * (k + 2)


def record_bytes(k, N):
    nb = -(-64 // k)
    bits = N.bit_length() - 1
    return 4 * (-(-(nb * bits) // 32))


class Timer:
    """Per-op HIP event pairs on the launch stream (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.ms = {}

    def run(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.pending.append((name, ev0, ev1))

    def collect(self):
        self.torch.cuda.synchronize()
        for name, a, b in self.pending:
            self.ms.setdefault(name, []).append(a.elapsed_time(b))
        self.pending = []

    def reset(self):
        self.collect()
        self.ms = {}


def cpu_baseline(n_sample):
    """Time the oracle on a bounded sample of the same workload (BLAS held to 1 thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from kv_cache_compression_fq_amd import fq, synth
    from oracle import artifact, codec
    x = synth.kv_slab(2, 0, 0, 1, 1, n_sample).reshape(-1, 64)
    total = 0.0
    with threadpool_limits(limits=1):
        for k, N in VARIANTS:
            art = artifact.read_artifact(fq.read_codebook_bytes(k, N))
            t0 = time.perf_counter()
            idx, nb = codec.encode(x, art["Pi"], art["C"])
            codec.decode(idx, nb, art["Pi"], art["C"])
            total += time.perf_counter() - t0
    return {"value": len(VARIANTS) * n_sample / total, "unit": "vectors/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_sample} vectors of layer 0 / K / head 0 of the same cache, encode + "
                      f"decode at each of the 4 variants ({total:.1f} s, numpy float64, "
                      f"BLAS limited to 1 thread)"}


def source_digest():
    """SHA-256 over the library's sources and header, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_compression_fq_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".hip", ".cpp", ".h")))
    files.append(os.path.join(ROOT, "include", "fq.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


# bench op name -> kernel label used in the counter summaries under profiles/
_KERNEL_LABEL = {"encode_k2N16": "encode_kernel<2,4,f16,grid>",
                 "encode_k2N64": "encode_kernel<2,6,f16,grid>",
                 "encode_k2N256": "encode_kernel<2,8,f16,grid>",
                 "encode_k3N512": "encode_kernel<3,9,f16,grid>",
                 "decode_k2N16": "decode_kernel<2,4,f16>", "decode_k2N64": "decode_kernel<2,6,f16>",
                 "decode_k2N256": "decode_kernel<2,8,f16>",
                 "decode_k3N512": "decode_kernel<3,9,f16>",
                 "random_decode_k2N16": "decode_kernel<2,4,f16,gather>"}


def measured_traffic(op):
    """HBM bytes per launch of `op` from the committed counter summary, or None when
    there is none or the library sources changed since the counters were taken.  The
    summary lists each kernel once per grid size; the step's launch is the largest grid."""
    path = os.path.join(ROOT, "profiles", "fq_kernels_gpt2_small_step_and_tinyllama_attend.txt")
    label = _KERNEL_LABEL.get(op)
    if label is None or not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    if f"source-sha256: {source_digest()}" not in text:
        return None
    best = None
    in_counters = False
    for line in text:
        if line.startswith("HBM traffic"):
            in_counters = True
        f = line.split()
        if not in_counters or len(f) != 7 or f[0] != label:
            continue
        try:
            wg, total = int(f[1]), (float(f[5]) + float(f[6])) * 1e6
        except ValueError:
            continue
        if best is None or wg > best[0]:
            best = (wg, total)
    return None if best is None else best[1]


def measured_utilisation(op):
    """VALU and MFMA utilisation of `op`'s kernel from the committed counter summary
    (rocprofv3 VALUBusy, VALUUtilization, MfmaUtil; the largest grid, which is the
    step's launch), or None when there is none or the library sources changed."""
    path = os.path.join(ROOT, "profiles", "fq_search_utilisation_valu_mfma_bench.txt")
    label = _KERNEL_LABEL.get(op)
    if label is None or not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    if f"source-sha256: {source_digest()}" not in text:
        return None
    best = None
    for line in text:
        f = line.split()
        if len(f) != 8 or f[0] != label:
            continue
        try:
            wg, busy, lanes, mfma = int(f[1]), float(f[3]), float(f[4]), float(f[5])
        except ValueError:
            continue
        if best is None or wg > best[0]:
            best = (wg, {"valu_busy_pct": busy, "valu_lanes_pct": lanes, "mfma_busy_pct": mfma})
    return None if best is None else best[1]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=16384)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy three times, so that a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known size")
    ap.add_argument("--no-fidelity", action="store_true",
                    help="skip the attention-fidelity sweep over the rates")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timing of the tiny, TinyLlama-cache and 2^24-vector sets")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the large-block (k = 32, 64; N = 4096) encode / decode timing")
    ap.add_argument("--attend-layers", type=int, default=22)
    ap.add_argument("--attend-steps", type=int, default=10)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the codec shards by (layer, head) or token range "
              "with no exchange, so no multi-GPU figure is produced; run with --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from kv_cache_compression_fq_amd import fq, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"device {torch.cuda.get_device_name(0)}")

    # ---------------------------------------------------------------- inputs
    n = L * 2 * B * H * T
    t0 = time.time()
    x_host = synth.kv_cache(2, L, B, H, T).reshape(n, 64)
    x0 = torch.from_numpy(x_host).to(dev)
    xs = [x0] + [x0.clone() for _ in VARIANTS[1:]]
    del x_host
    cbs = [fq.load_codebook(k, N) for k, N in VARIANTS]
    codes = [torch.empty((n, cb.W), dtype=torch.int32, device=dev) for cb in cbs]
    norms = [torch.empty((n,), dtype=torch.int16, device=dev) for _ in cbs]
    ys = [torch.empty((n, 64), dtype=torch.float16, device=dev) for _ in cbs]
    rows = torch.from_numpy(synth.random_rows(n, N_RAND, seed=33)).to(dev)
    y_rand = torch.empty((N_RAND, 64), dtype=torch.float16, device=dev)
    q = torch.from_numpy(synth.query(B, H, seed=5)).to(dev)
    per_slab = B * H * T
    ws_bytes = fq.fq_attend_workspace_size(cbs[0], B, H, H, T)
    ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=dev)
    att_out = torch.empty((B, H, 64), dtype=torch.float16, device=dev)
    log(f"inputs ready: {n} vectors ({time.time() - t0:.1f} s)")

    if a.copy_calibration:
        src = torch.empty((COPY_BYTES,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 copies of {COPY_BYTES} bytes")

    timer = Timer(torch)

    def step():
        # all encodes first: by the time a variant's records are decoded, three
        # 151 MB input reads have passed through the 256 MB Infinity Cache
        for v, cb in enumerate(cbs):
            timer.run(f"encode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_encode(cb, xs[v], codes[v], norms[v]))
        for v, cb in enumerate(cbs):
            timer.run(f"decode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_decode(cb, codes[v], norms[v], y=ys[v]))
        timer.run("random_decode_k2N16",
                  lambda: fq.fq_decode(cbs[0], codes[0], norms[0], rows=rows, y=y_rand))
        W = cbs[0].W
        for layer in range(L):
            kc = codes[0][(2 * layer) * per_slab:(2 * layer + 1) * per_slab].view(B, H, T, W)
            vc = codes[0][(2 * layer + 1) * per_slab:(2 * layer + 2) * per_slab].view(B, H, T, W)
            kn = norms[0][(2 * layer) * per_slab:(2 * layer + 1) * per_slab].view(B, H, T)
            vn = norms[0][(2 * layer + 1) * per_slab:(2 * layer + 2) * per_slab].view(B, H, T)
            timer.run("attend_gpt2_k2N16",
                      lambda kc=kc, vc=vc, kn=kn, vn=vn: fq.fq_attend_decode(
                          cbs[0], cbs[0], q, kc, kn, vc, vn, 0.125, workspace=ws, out=att_out))

    for _ in range(a.warmup):
        step()
    timer.reset()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    timer.collect()
    ms_per_step = 1e3 * elapsed / a.steps
    vectors = 2 * n * len(VARIANTS)               # each vector encoded and decoded
    value = vectors / (elapsed / a.steps)

    ops = {}
    for name, lst in timer.ms.items():
        ops[name] = {"ms_avg": float(np.mean(lst)), "launches": len(lst)}
    for k, N in VARIANTS:
        e = ops[f"encode_k{k}N{N}"]
        e["vectors_per_s"] = n / (e["ms_avg"] * 1e-3)
        e["ops_per_vector"] = enc_ops_per_vector(k, N)
        e["alu_tops"] = e["vectors_per_s"] * e["ops_per_vector"] / 1e12
        e["alu_frac"] = e["alu_tops"] / VALU_PEAK_TOPS
        e["utilisation"] = measured_utilisation(f"encode_k{k}N{N}")
        d = ops[f"decode_k{k}N{N}"]
        d["vectors_per_s"] = n / (d["ms_avg"] * 1e-3)
        d["bytes_per_vector"] = record_bytes(k, N) + 2 + 128
        d["gbs"] = d["vectors_per_s"] * d["bytes_per_vector"] / 1e9
        d["hbm_frac"] = d["gbs"] / HBM_PEAK_GBS
    r = ops["random_decode_k2N16"]
    r["vectors_per_s"] = N_RAND / (r["ms_avg"] * 1e-3)
    r["bytes_per_vector"] = 8 + record_bytes(2, 16) + 2 + 128
    r["gbs"] = r["vectors_per_s"] * r["bytes_per_vector"] / 1e9
    at = ops["attend_gpt2_k2N16"]
    at["bytes_per_call"] = per_slab * 2 * (record_bytes(2, 16) + 2) + 2 * B * H * 64 * 2
    at["gbs"] = at["bytes_per_call"] / (at["ms_avg"] * 1e-3) / 1e9

    # dominant kernel of the step
    totals = {k: v["ms_avg"] * v["launches"] for k, v in ops.items()}
    dom = max(totals, key=totals.get)
    traffic = measured_traffic(dom)
    if dom.startswith("encode"):
        ach = ops[dom]["alu_tops"]
        roof = {"kernel": dom, "bound": "alu", "achieved": ach, "peak": VALU_PEAK_TOPS,
                "unit": "Tops/s", "frac": ach / VALU_PEAK_TOPS, "traffic": traffic,
                "note": "op model = exhaustive search, nb*N*(k+2) lane-ops per vector; the "
                        "exact candidate-list search does less work, so frac > 1 is its "
                        "gain over an exhaustive search at the VALU peak"}
    else:
        ach = ops[dom].get("gbs", 0.0)
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic}

    # ------------------------------------ large blocks (k = 32, 64; N = 4096)
    large = None if a.no_large else bench_large(torch, fq, xs[0], ys[0], a.steps, a.warmup)

    # ---------------------------------------------- TinyLlama-shaped attention
    attend = None
    if a.attend_layers > 0:
        for t in (xs, codes, norms, ys):
            t.clear()
        torch.cuda.empty_cache()
        attend = bench_attend(torch, fq, synth, dev, a.attend_layers, a.attend_steps, a.warmup)

    fid = None if a.no_fidelity else fidelity(torch, fq, synth, dev)

    cfgs = None if a.no_configs else bench_configs(torch, fq, synth, dev)

    cpu = None if a.no_cpu_baseline else cpu_baseline(a.cpu_sample)

    out = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gpt2-small-kv-cache: 12 layers x {K,V} x batch 4 x 12 heads x "
                               "seq 1024, d=64, fp16; FibQuant k2N16, k2N64, k2N256, k3N512; "
                               "+ 2^20 random-access decodes + 12-layer decode-step attention",
                   "vectors": n, "variants": [f"k{k}N{N}" for k, N in VARIANTS],
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ops": ops,
        "attend_tinyllama": attend,
        "large_k": large,
        "configs": cfgs,
        "fidelity": fid,
    }
    print(json.dumps(out))
    return 0


FIDELITY_VARIANTS = [(8, 16), (4, 4), (8, 256), (4, 256), (2, 16), (2, 32), (3, 512), (2, 64),
                     (2, 128), (2, 256)]   # k3N4096's tables exceed the attention kernel's LDS


def fidelity(torch, fq, synth, dev, B=2, Hq=32, Hkv=4, T=4096, layers=(0, 11, 21)):
    """Attention-output fidelity against the compression ratio (quality context).

    TinyLlama-shaped seeded caches (per-channel log-uniform scales, 1 % x20
    outlier channels), three layers, batch 2, 32 query / 4 KV heads, 4096
    tokens: the fused attention over the compressed cache against exact
    softmax attention over the uncompressed binary16 cache (float32), cosine
    per (batch, query head).  The compression ratio counts the stored record
    and norm against 64 binary16 values.  With N(0, 1) queries and these
    channel scales the scores spread over tens of units, so attention is
    close to an argmax over keys and key errors that swap the top tokens
    change a head's output entirely: the sweep is a stress case for the rate
    axis, not a model-quality figure.
    """
    import math
    G = Hq // Hkv
    n = B * Hkv * T
    q = torch.from_numpy(synth.query(B, Hq, seed=7)).to(dev)
    caches = []
    for layer in layers:
        K = synth.kv_slab_device(3, layer, 0, B, Hkv, T, dev)
        V = synth.kv_slab_device(3, layer, 1, B, Hkv, T, dev)
        qf = q.float().view(B, Hkv, G, 64)
        s = torch.matmul(qf, K.float().transpose(-1, -2).contiguous()) * 0.125
        o = torch.matmul(torch.softmax(s, dim=-1), V.float()).reshape(B, Hq, 64)
        caches.append((K, V, o))
    rows = []
    for k, N in FIDELITY_VARIANTS + LARGE_VARIANTS:
        cb = fq.load_codebook(k, N)
        cos = []
        for K, V, o_ref in caches:
            kc, kn = fq.fq_encode(cb, K.reshape(n, 64))
            vc, vn = fq.fq_encode(cb, V.reshape(n, 64))
            if k < 32:
                o = fq.fq_attend_decode(cb, cb, q, kc.view(B, Hkv, T, cb.W), kn.view(B, Hkv, T),
                                        vc.view(B, Hkv, T, cb.W), vn.view(B, Hkv, T), 0.125)
            else:
                # no fused attention for tables larger than LDS: decode, then the
                # same float32 attention as the reference
                Kd = fq.fq_decode(cb, kc, kn).float().view(B, Hkv, T, 64)
                Vd = fq.fq_decode(cb, vc, vn).float().view(B, Hkv, T, 64)
                sd = torch.matmul(q.float().view(B, Hkv, G, 64),
                                  Kd.transpose(-1, -2).contiguous()) * 0.125
                o = torch.matmul(torch.softmax(sd, dim=-1), Vd).reshape(B, Hq, 64)
            cos.append(torch.nn.functional.cosine_similarity(o.float(), o_ref, dim=-1).flatten())
        c = torch.cat(cos)
        rows.append({"variant": f"k{k}N{N}", "bits_per_coord": math.log2(N) / k,
                     "compression": 128.0 / (4 * cb.W + 2),
                     "attn_cos_mean": float(c.mean()),
                     "attn_cos_p10": float(torch.quantile(c, 0.1)),
                     "share_cos_ge_0.9": float((c >= 0.9).float().mean())})
    log("fidelity sweep done")
    return {"workload": f"tinyllama-shaped caches, layers {list(layers)}, batch {B}, "
                        f"{Hq} q / {Hkv} kv heads, {T} tokens; exact attention in float32 on "
                        "the binary16 cache as reference", "rows": rows}


def bench_large(torch, fq, x, y, steps, warmup):
    """Encode and decode of the GPT-2-shaped cache with the k = 32 and k = 64, N = 4096 codes.

    The block search is a dense contraction here (4096 codewords of k
    coordinates per block, 64 * 4096 multiply-adds per vector at either k), run
    on the matrix cores: its roofline is the binary16 MFMA peak.  The kernel
    forms every product twice (z split into binary16 hi and lo parts), so
    the algorithmic fraction reported here is at most one half.
    """
    import numpy as np
    n = x.shape[0]
    out = {}
    for k, N in LARGE_VARIANTS:
        cb = fq.load_codebook(k, N)
        codes = torch.empty((n, cb.W), dtype=torch.int32, device=x.device)
        norms = torch.empty((n,), dtype=torch.int16, device=x.device)
        timer = Timer(torch)
        for i in range(warmup + steps):
            if i == warmup:
                timer.reset()
            timer.run("encode", lambda: fq.fq_encode(cb, x, codes, norms))
            timer.run("decode", lambda: fq.fq_decode(cb, codes, norms, y=y))
        timer.collect()
        te = float(np.median(timer.ms["encode"])) * 1e-3
        td = float(np.median(timer.ms["decode"])) * 1e-3
        flops = 2.0 * 64 * N * n                  # one multiply-add per codeword coordinate
        dec_bytes = n * (record_bytes(k, N) + 2 + 128)
        out[f"k{k}N{N}"] = {
            "bits_per_coord": math.log2(N) / k, "compression": 128.0 / (4 * cb.W + 2),
            "encode_ms": te * 1e3, "encode_vectors_per_s": n / te,
            "encode_mfma_tflops": flops / te / 1e12,
            "encode_mfma_frac": flops / te / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "decode_ms": td * 1e3, "decode_gbs": dec_bytes / td / 1e9,
            "decode_hbm_frac": dec_bytes / td / 1e9 / HBM_PEAK_GBS}
        del codes, norms
    log("large-block timing done")
    return {"workload": f"gpt2-small-kv-cache, {n} vectors, fp16; median of {steps} launches",
            "peak_mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS, "codes": out}


def bench_configs(torch, fq, synth, dev, reps=5):
    """The other configurations' throughput, each op timed with HIP events (median).

    tiny: 4096 float32 vectors, k2N16 encode + decode (a latency figure);
    tinyllama cache: 22 layers x {K,V} x batch 8 x 4 heads x 2048 tokens,
      full encode at k4N256 and k8N256, then 2^20 uniformly drawn addresses
      decoded by address;
    stress set: 2^24 vectors (256 streams x 65536 tokens) at k8N16, k4N4
      (0.5 bit per coordinate) and k3N4096, encode and decode.
    Algorithmic bytes: encode 128 B read + record + norm written; decode the
    reverse; random access adds the 8-byte address.
    """
    import numpy as np

    def timed(fn, n_rep):
        ts = []
        for i in range(n_rep + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i:
                ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    def codec_rows(cb, x, n, with_decode=True, rows=None):
        codes = torch.empty((n, cb.W), dtype=torch.int32, device=dev)
        norms = torch.empty((n,), dtype=torch.int16, device=dev)
        rb = record_bytes(cb.k, cb.N) + 2
        te = timed(lambda: fq.fq_encode(cb, x, codes, norms), reps)
        r = {"encode_ms": te * 1e3, "encode_vectors_per_s": n / te,
             "encode_gbs": n * (128 + rb) / te / 1e9}
        if with_decode:
            y = torch.empty((n, 64), dtype=torch.float16, device=dev)
            td = timed(lambda: fq.fq_decode(cb, codes, norms, y=y), reps)
            r.update({"decode_ms": td * 1e3, "decode_vectors_per_s": n / td,
                      "decode_gbs": n * (128 + rb) / td / 1e9,
                      "decode_hbm_frac": n * (128 + rb) / td / 1e9 / HBM_PEAK_GBS})
            del y
        if rows is not None:
            m = rows.shape[0]
            y = torch.empty((m, 64), dtype=torch.float16, device=dev)
            tr = timed(lambda: fq.fq_decode(cb, codes, norms, rows=rows, y=y), reps)
            r.update({"random_decode_ms": tr * 1e3, "random_decodes_per_s": m / tr,
                      "random_decode_gbs": m * (8 + 128 + rb) / tr / 1e9})
            del y
        return r

    out = {}
    cb = fq.load_codebook(2, 16)
    xt = torch.from_numpy(synth.tiny_vectors(4096)).to(dev)
    out["tiny_4096_fp32_k2N16"] = codec_rows(cb, xt, 4096)

    L3, B3, H3, T3 = 22, 8, 4, 2048
    x3 = torch.cat([synth.kv_slab_device(3, l, kv, B3, H3, T3, dev).reshape(-1, 64)
                    for l in range(L3) for kv in range(2)])
    n3 = x3.shape[0]
    rows = torch.from_numpy(synth.random_rows(n3, 1 << 20, seed=33)).to(dev)
    for k, N in ((4, 256), (8, 256)):
        out[f"tinyllama_cache_{n3}_k{k}N{N}"] = codec_rows(fq.load_codebook(k, N), x3, n3,
                                                            with_decode=False, rows=rows)
    del x3, rows
    torch.cuda.empty_cache()

    x4 = synth.kv_slab_device(4, 0, 0, 1, 256, 65536, dev).reshape(-1, 64)
    n4 = x4.shape[0]
    for k, N in ((8, 16), (4, 4), (3, 4096)):
        out[f"stress_{n4}_k{k}N{N}"] = codec_rows(fq.load_codebook(k, N), x4, n4)
    del x4
    torch.cuda.empty_cache()
    log("configuration timing done")
    return out


def bench_attend(torch, fq, synth, dev, layers, steps, warmup):
    """Fused attention at batch 16, 32 query / 4 KV heads, 32768 tokens, k4N256, per layer."""
    Bq, Hq, Hkv, Tq = 16, 32, 4, 32768
    cb = fq.load_codebook(4, 256)
    per = Bq * Hkv * Tq
    kc = [torch.empty((Bq, Hkv, Tq, cb.W), dtype=torch.int32, device=dev) for _ in range(layers)]
    vc = [torch.empty((Bq, Hkv, Tq, cb.W), dtype=torch.int32, device=dev) for _ in range(layers)]
    kn = [torch.empty((Bq, Hkv, Tq), dtype=torch.int16, device=dev) for _ in range(layers)]
    vn = [torch.empty((Bq, Hkv, Tq), dtype=torch.int16, device=dev) for _ in range(layers)]
    t0 = time.time()
    for layer in range(layers):
        for kv, (c, nn) in enumerate(((kc, kn), (vc, vn))):
            x = synth.kv_slab_device(3, layer, kv, Bq, Hkv, Tq, dev).reshape(per, 64)
            fq.fq_encode(cb, x, c[layer].view(per, cb.W), nn[layer].view(per))
            del x
    torch.cuda.synchronize()
    log(f"attention cache ready: {layers} layers ({time.time() - t0:.1f} s)")
    q = torch.from_numpy(synth.query(Bq, Hq, seed=5)).to(dev)
    ws = torch.empty((fq.fq_attend_workspace_size(cb, Bq, Hq, Hkv, Tq),), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((Bq, Hq, 64), dtype=torch.float16, device=dev)
    timer = Timer(torch)

    def one():
        for layer in range(layers):
            timer.run("attend", lambda layer=layer: fq.fq_attend_decode(
                cb, cb, q, kc[layer], kn[layer], vc[layer], vn[layer], 0.125, workspace=ws,
                out=out))

    for _ in range(warmup):
        one()
    timer.reset()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    timer.collect()
    import numpy as np
    ms = float(np.mean(timer.ms["attend"]))
    bytes_layer = per * 2 * (cb.W * 4 + 2) + 2 * Bq * Hq * 64 * 2

    # the same step with encode-on-append: the new token's key and value are
    # encoded into the last slot, then attention reads all 32768 tokens
    k_new = synth.kv_slab_device(3, 0, 0, Bq, Hkv, 1, dev)
    v_new = synth.kv_slab_device(3, 0, 1, Bq, Hkv, 1, dev)
    q4 = q.view(Bq, Hq, 1, 64)
    out4 = out.view(Bq, Hq, 1, 64)
    timer.reset()
    for i in range(warmup + steps):
        if i == warmup:
            timer.reset()
        for layer in range(layers):
            timer.run("step", lambda layer=layer: fq.fq_decode_step(
                cb, cb, q4, k_new, v_new, kc[layer], kn[layer], vc[layer], vn[layer], Tq - 1, 0.125,
                workspace=ws, out=out4))
    timer.collect()
    ms_step = float(np.mean(timer.ms["step"]))
    return {"workload": "tinyllama decode step: batch 16, 32 q / 4 kv heads, seq 32768, d=64, "
                        f"k4N256 K and V, {layers} layers",
            "ms_per_layer_event": ms, "ms_per_layer_wall": 1e3 * el / (steps * layers),
            "bytes_per_layer": bytes_layer, "gbs": bytes_layer / (ms * 1e-3) / 1e9,
            "hbm_frac": bytes_layer / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_step_with_append_ms_per_layer": ms_step}


if __name__ == "__main__":
    sys.exit(main())
