#!/usr/bin/env python3
"""Throughput of the FibQuant hot path on one MI355X.

One step is one pass of the whole path over the 2^24-vector stress set
(256 streams x 65536 tokens, d = 64, binary16, seeded synthetic values with
per-channel log-uniform scales and 1 % x20 outlier channels), the largest
configuration that one GPU holds:

  for each code k8N16 (0.5 bit), k4N4 (0.5 bit), k3N4096 (4 bits):
      encode every vector (norm, rotation, block search, packing)
  decode every record of each code (gather, inverse rotation, rescale) to binary16
  random-access decode of 2^20 uniformly drawn records (k3N4096 codes)
  fused decode-step attention over the k4N4-coded set read as a cache
      (keys = first half, values = second half: batch 32, 4 KV heads,
      65536 tokens, 32 query heads)

``value`` is vectors encoded and decoded per second over the whole step
(6 x 2^24 per step).  The same run times, outside the step: the GPT-2-small-
shaped cache (the rate sweep k2N16 / k2N64 / k2N256 / k3N512), the
TinyLlama-shaped decode-step attention (22 layers, k4N256), the other
configurations, a device copy (the achievable-bandwidth ceiling), and the CPU
oracle on a bounded sample.
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
STEP_VARIANTS = [(8, 16), (4, 4), (3, 4096)]
STRESS_STREAMS, STRESS_T = 256, 65536
GPT2_VARIANTS = [(2, 16), (2, 64), (2, 256), (3, 512)]
LARGE_VARIANTS = [(32, 4096), (64, 4096), (64, 16384)]
L2, B2, H2, T2 = 12, 4, 12, 1024
N_RAND = 1 << 20
COPY_BYTES = 1 << 28


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def record_bytes(k, N):
    nb = -(-64 // k)
    bits = N.bit_length() - 1
    return 4 * (-(-(nb * bits) // 32))


def codec_bytes(k, N):
    """Algorithmic bytes per vector of encode or decode: 128 B of binary16 values
    one way, the record and the binary16 norm the other."""
    return 128 + record_bytes(k, N) + 2


class Timer:
    """Per-op HIP event pairs on the launch stream (torch's current stream, which
    the binding passes to every call)."""

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


COUNTERS = os.path.join(ROOT, "profiles", "fq_kernels_stress_step_counters.txt")


def measured_counters(op):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated) and VALU / MFMA
    utilisation of `op`'s kernel from the committed counter summary, or None when
    there is none or the library sources changed since it was taken."""
    if not os.path.exists(COUNTERS):
        return None
    text = open(COUNTERS).read().splitlines()
    if f"source-sha256: {source_digest()}" not in text:
        return None
    for line in text:
        f = line.split()
        if len(f) >= 6 and f[0] == "op" and f[1] == op:
            try:
                vals = [None if v in ("-", "nan") else float(v) for v in f[2:7]]
            except ValueError:
                return None
            out = {"traffic_bytes": vals[0], "valu_busy_pct": vals[1],
                   "valu_lanes_pct": vals[2], "mfma_busy_pct": vals[3]}
            if len(vals) > 4 and vals[4] is not None:
                out["executed_lane_ops_per_vector"] = vals[4]
            return out
    return None


def copy_ceiling(torch, dev, reps=5):
    """Achievable device bandwidth: a 1 GiB copy (read + write) and a 1 GiB fill."""
    import numpy as np
    nbytes = 1 << 30
    src = torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def timed(fn):
        ts = []
        for i in range(reps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i:
                ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    tc = timed(lambda: dst.copy_(src))
    tf = timed(lambda: dst.fill_(3))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": 2 * nbytes / tc / 1e9, "fill_gbs": nbytes / tf / 1e9,
            "copy_frac_of_peak": 2 * nbytes / tc / 1e9 / HBM_PEAK_GBS,
            "what": "torch device copy of 1 GiB (bytes read + written) and fill of 1 GiB, "
                    f"median of {reps}"}


def encode_roofline(k, N, vps, entries):
    """Limits of one encode: HBM (algorithmic bytes) and VALU (the search's own
    work, `entries` codewords compared per vector at k + 2 operations each); the
    lower limit is the bound and frac = achieved / bound."""
    ops = entries * (k + 2)
    lim_valu = VALU_PEAK_TOPS * 1e12 / ops
    lim_hbm = HBM_PEAK_GBS * 1e9 / codec_bytes(k, N)
    if lim_valu < lim_hbm:
        return {"bound": "alu", "achieved": vps * ops / 1e12, "peak": VALU_PEAK_TOPS,
                "unit": "T lane-ops/s", "frac": vps / lim_valu, "search_lane_ops_per_vector": ops,
                "valu_limit_vectors_per_s": lim_valu, "hbm_limit_vectors_per_s": lim_hbm}
    return {"bound": "hbm", "achieved": vps * codec_bytes(k, N) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": vps / lim_hbm, "search_lane_ops_per_vector": ops,
            "valu_limit_vectors_per_s": lim_valu, "hbm_limit_vectors_per_s": lim_hbm}


# the configurations timed outside the step, in the order they run
EXTRAS = ["copy_ceiling", "gpt2_step", "large_k", "attend_tinyllama", "configs"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy three times, so that a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known size")
    ap.add_argument("--no-fidelity", action="store_true",
                    help="skip the attention-fidelity sweep over the rates")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only (no other configurations, no copy ceiling)")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated subset of the other configurations to time: "
                         + ", ".join(EXTRAS))
    ap.add_argument("--attend-layers", type=int, default=22)
    ap.add_argument("--attend-steps", type=int, default=10)
    ap.add_argument("--cost-sample", type=int, default=1 << 15,
                    help="vectors copied to the host for the search-work model")
    a = ap.parse_args()
    chosen = set() if a.no_extras else {e.strip() for e in a.extras.split(",") if e.strip()}
    unknown = chosen - set(EXTRAS)
    if unknown:
        raise SystemExit(f"unknown --extras {sorted(unknown)}; choose from {EXTRAS}")
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

    if a.copy_calibration:
        src = torch.empty((COPY_BYTES,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 copies of {COPY_BYTES} bytes")

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    x = synth.kv_slab_device(4, 0, 0, 1, STRESS_STREAMS, STRESS_T, dev).reshape(-1, 64)
    n = x.shape[0]
    cbs = [fq.load_codebook(k, N) for k, N in STEP_VARIANTS]
    codes = [torch.empty((n, cb.W), dtype=torch.int32, device=dev) for cb in cbs]
    norms = [torch.empty((n,), dtype=torch.int16, device=dev) for _ in cbs]
    ys = [torch.empty((n, 64), dtype=torch.float16, device=dev) for _ in cbs]
    rows = torch.from_numpy(synth.random_rows(n, N_RAND, seed=33)).to(dev)
    y_rand = torch.empty((N_RAND, 64), dtype=torch.float16, device=dev)
    ia = [v for v, kb in enumerate(STEP_VARIANTS) if kb == (4, 4)][0]    # attention code
    ir = [v for v, kb in enumerate(STEP_VARIANTS) if kb == (3, 4096)][0]  # random access
    Ba, Hkv_a, Ta, Hq_a = n // 2 // (4 * STRESS_T), 4, STRESS_T, 32
    cba = cbs[ia]
    kc_a = codes[ia][:n // 2].view(Ba, Hkv_a, Ta, cba.W)
    vc_a = codes[ia][n // 2:].view(Ba, Hkv_a, Ta, cba.W)
    kn_a = norms[ia][:n // 2].view(Ba, Hkv_a, Ta)
    vn_a = norms[ia][n // 2:].view(Ba, Hkv_a, Ta)
    q_a = torch.from_numpy(synth.query(Ba, Hq_a, seed=5)).to(dev)
    ws_a = torch.empty((fq.fq_attend_workspace_size(cba, Ba, Hq_a, Hkv_a, Ta),),
                       dtype=torch.uint8, device=dev)
    out_a = torch.empty((Ba, Hq_a, 64), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready: {n} vectors ({time.time() - t0:.1f} s)")

    timer = Timer(torch)

    def step():
        for v, cb in enumerate(cbs):
            timer.run(f"encode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_encode(cb, x, codes[v], norms[v]))
        for v, cb in enumerate(cbs):
            timer.run(f"decode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_decode(cb, codes[v], norms[v], y=ys[v]))
        cbr = cbs[ir]
        timer.run(f"random_decode_k{cbr.k}N{cbr.N}",
                  lambda: fq.fq_decode(cbr, codes[ir], norms[ir], rows=rows, y=y_rand))
        timer.run(f"attend_k{cba.k}N{cba.N}",
                  lambda: fq.fq_attend_decode(cba, cba, q_a, kc_a, kn_a, vc_a, vn_a, 0.125,
                                              workspace=ws_a, out=out_a))

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
    vectors = 2 * n * len(STEP_VARIANTS)         # each vector encoded and decoded per code
    value = vectors / (elapsed / a.steps)
    log(f"step: {ms_per_step:.3f} ms, {value:.4g} vectors/s")

    # search-work model of each encode, from a host sample of the inputs
    x_sample = x[:a.cost_sample].cpu().numpy()
    ops = {}
    for name, lst in timer.ms.items():
        ops[name] = {"ms_avg": float(np.mean(lst)), "ms_min": float(np.min(lst)),
                     "ms_max": float(np.max(lst)), "launches": len(lst)}
    for (k, N), cb in zip(STEP_VARIANTS, cbs):
        e = ops[f"encode_k{k}N{N}"]
        e["vectors_per_s"] = n / (e["ms_avg"] * 1e-3)
        e["bytes_per_vector"] = codec_bytes(k, N)
        e["gbs"] = e["vectors_per_s"] * e["bytes_per_vector"] / 1e9
        entries, scan = fq.fq_search_cost(cb, x_sample)
        e["search_entries_per_vector"] = entries
        e["full_scan_block_share"] = scan
        e["roofline"] = encode_roofline(k, N, e["vectors_per_s"], entries)
        e["counters"] = measured_counters(f"encode_k{k}N{N}")
        if e["counters"] and "executed_lane_ops_per_vector" in e["counters"]:
            # executed VALU work (counters) over the search's own work model
            e["counters"]["executed_over_search_lane_ops"] = (
                e["counters"]["executed_lane_ops_per_vector"] /
                e["roofline"]["search_lane_ops_per_vector"])
        d = ops[f"decode_k{k}N{N}"]
        d["vectors_per_s"] = n / (d["ms_avg"] * 1e-3)
        d["bytes_per_vector"] = codec_bytes(k, N)
        d["gbs"] = d["vectors_per_s"] * d["bytes_per_vector"] / 1e9
        d["hbm_frac"] = d["gbs"] / HBM_PEAK_GBS
        d["counters"] = measured_counters(f"decode_k{k}N{N}")
    cbr = cbs[ir]
    r = ops[f"random_decode_k{cbr.k}N{cbr.N}"]
    r["vectors_per_s"] = N_RAND / (r["ms_avg"] * 1e-3)
    r["bytes_per_vector"] = 8 + codec_bytes(cbr.k, cbr.N)
    r["gbs"] = r["vectors_per_s"] * r["bytes_per_vector"] / 1e9
    r["note"] = ("scattered records: each costs a whole memory sector, so the HBM fraction "
                 "is not claimed for this op")
    at = ops[f"attend_k{cba.k}N{cba.N}"]
    at["bytes_per_call"] = (n // 2) * 2 * (cba.W * 4 + 2) + 2 * Ba * Hq_a * 64 * 2
    at["gbs"] = at["bytes_per_call"] / (at["ms_avg"] * 1e-3) / 1e9
    at["hbm_frac"] = at["gbs"] / HBM_PEAK_GBS
    at["counters"] = measured_counters(f"attend_k{cba.k}N{cba.N}")

    # dominant kernel of the step: its roofline is the headline one
    totals = {k: v["ms_avg"] * v["launches"] for k, v in ops.items()}
    dom = max(totals, key=totals.get)
    cnt = measured_counters(dom)
    traffic = cnt["traffic_bytes"] if cnt else None
    if dom.startswith("encode"):
        rf = ops[dom]["roofline"]
        roof = {"kernel": dom, "bound": rf["bound"], "achieved": rf["achieved"],
                "peak": rf["peak"], "unit": rf["unit"], "frac": rf["frac"], "traffic": traffic,
                "algorithmic_bytes": n * ops[dom]["bytes_per_vector"],
                "note": "encode limits: HBM = 8 TB/s over 128 B read + record + norm written "
                        "per vector; VALU = 39.3 T lane-ops/s over the search's own work, "
                        "(k + 2) x the codewords the candidate-list search compares per vector "
                        "(fq_search_cost on a host sample); bound = the lower limit"}
    else:
        ach = ops[dom].get("gbs", 0.0)
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic}
    del x_sample

    # free the step's buffers before the other configurations
    for t in (codes, norms, ys):
        t.clear()
    del x, rows, y_rand, kc_a, vc_a, kn_a, vn_a, ws_a
    torch.cuda.empty_cache()

    extras = {}
    if "copy_ceiling" in chosen:
        extras["copy_ceiling"] = copy_ceiling(torch, dev)
    if "gpt2_step" in chosen:
        extras["gpt2_step"] = bench_gpt2(torch, fq, synth, dev, a.steps, a.warmup)
    if "large_k" in chosen:
        extras["large_k"] = bench_large(torch, fq, synth, dev, a.steps, a.warmup)
    if "attend_tinyllama" in chosen and a.attend_layers > 0:
        extras["attend_tinyllama"] = bench_attend(torch, fq, synth, dev, a.attend_layers,
                                                  a.attend_steps, a.warmup)
    if "configs" in chosen:
        extras["configs"] = bench_configs(torch, fq, synth, dev)
    if not a.no_fidelity:
        extras["fidelity"] = fidelity(torch, fq, synth, dev)

    cpu = None if a.no_cpu_baseline else cpu_baseline(value)

    out = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "stress set 2^24 vectors (256 streams x 65536 tokens), d=64, "
                               "fp16; FibQuant k8N16, k4N4, k3N4096 encode + decode, 2^20 "
                               "random-access decodes (k3N4096), decode-step attention over the "
                               "k4N4 set (batch 32, 32 q / 4 kv heads, 65536 tokens)",
                   "vectors": n, "variants": [f"k{k}N{N}" for k, N in STEP_VARIANTS],
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ops": ops,
        **extras,
    }
    print(json.dumps(out))
    return 0


def cpu_baseline(gpu_value):
    """The oracle on the host cores, on a bounded sample of the step's workload.

    Encode = the oracle's nearest-codeword search (the compiled float64 brute
    force, OpenMP over the host threads) + its binary16 norm and packing
    (numpy); decode = the oracle's float64 decode (numpy, BLAS threads).
    Per code, a sample of the stress set is encoded and decoded; the rate is
    extrapolated to the step's mix (every vector encoded and decoded in each of
    the three codes), once with all threads and once with one.  Attention:
    the oracle's decompress-then-attend of a few (batch, query head) rows of
    the TinyLlama decode step (32768 tokens each).
    """
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from kv_cache_compression_fq_amd import fq, synth
    from oracle import artifact, attend, codec, native
    samples = {(8, 16): 1 << 17, (4, 4): 1 << 17, (3, 4096): 1 << 15}
    x = synth.kv_slab(4, 0, 0, 1, 1, max(samples.values())).reshape(-1, 64)
    blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
    omp_all = native.threads()

    def run(threads):
        native.threads(threads)
        secs = 0.0
        per = {}
        with threadpool_limits(limits=threads, user_api="blas"):
            for (k, N), m in samples.items():
                art = artifact.read_artifact(fq.read_codebook_bytes(k, N))
                xs = x[:m]
                t0 = time.perf_counter()
                idx = native.nearest(xs, art["Pi"], art["C"])
                xd = xs.astype(np.float64)
                nb = codec.f16_round(np.sqrt(np.sum(xd * xd, axis=1)))
                words = codec.pack(idx, art["bits"])
                t1 = time.perf_counter()
                codec.decode(codec.unpack(words, art["nb"], art["bits"]), nb, art["Pi"], art["C"])
                t2 = time.perf_counter()
                per[f"k{k}N{N}"] = {"encode_vectors_per_s": m / (t1 - t0),
                                    "decode_vectors_per_s": m / (t2 - t1), "sample": m}
                secs += t2 - t0
        # seconds per vector of the step's mix: encode + decode in each code
        spv = sum(1 / p["encode_vectors_per_s"] + 1 / p["decode_vectors_per_s"]
                  for p in per.values())
        return 2 * len(samples) / spv, per, secs

    v_all, per_all, s_all = run(omp_all)
    v_one, per_one, s_one = run(1)
    native.threads(omp_all)
    # attention rows of the TinyLlama decode step
    art = artifact.read_artifact(fq.read_codebook_bytes(4, 256))
    T, nrows = 32768, 8
    kw = synth.random_records((1, 1, T), 4, 128, 81)
    vw = synth.random_records((1, 1, T), 4, 128, 82)
    kn = synth.random_norms((1, 1, T), 83)
    vn = synth.random_norms((1, 1, T), 84)
    q = synth.query(1, nrows, seed=85)
    t0 = time.perf_counter()
    attend.attend(q, kw, kn, vw, vn, art["Pi"], art["C"], art["C"], 0.125,
                  rows=[(0, h) for h in range(nrows)])
    ta = time.perf_counter() - t0
    return {"value": v_all, "unit": "vectors/s", "cores": omp_all, "kind": "oracle",
            "sample": f"encode + decode of {samples[(8, 16)]} / {samples[(4, 4)]} / "
                      f"{samples[(3, 4096)]} stress-set vectors at k8N16 / k4N4 / k3N4096, "
                      f"extrapolated to the step's mix ({s_all:.1f} s with {omp_all} threads, "
                      f"{s_one:.1f} s with 1)",
            "host_cpu_count": os.cpu_count(), "blas_threads": blas, "openmp_threads": omp_all,
            "value_1_thread": v_one, "per_code": per_all, "per_code_1_thread": per_one,
            "gpu_over_cpu": gpu_value / v_all,
            "attention_rows_per_s": nrows / ta,
            "attention_sample": f"{nrows} (batch, query head) rows of 32768 k4N256 tokens, "
                                f"decompress-then-attend ({ta:.1f} s; one KV head decoded)"}


def bench_gpt2(torch, fq, synth, dev, steps, warmup):
    """The GPT-2-small-shaped cache (12 layers x {K,V} x batch 4 x 12 heads x 1024
    tokens, 1,179,648 vectors): encode and decode at k2N16 / k2N64 / k2N256 / k3N512,
    2^20 random-access decodes (k2N16) and 12 layers of decode-step attention (k2N16).
    Four input replicas of 151 MB, so reads come from HBM rather than the 256 MB
    Infinity Cache."""
    import numpy as np
    n = L2 * 2 * B2 * H2 * T2
    x0 = torch.from_numpy(synth.kv_cache(2, L2, B2, H2, T2).reshape(n, 64)).to(dev)
    xs = [x0] + [x0.clone() for _ in GPT2_VARIANTS[1:]]
    cbs = [fq.load_codebook(k, N) for k, N in GPT2_VARIANTS]
    codes = [torch.empty((n, cb.W), dtype=torch.int32, device=dev) for cb in cbs]
    norms = [torch.empty((n,), dtype=torch.int16, device=dev) for _ in cbs]
    ys = [torch.empty((n, 64), dtype=torch.float16, device=dev) for _ in cbs]
    rows = torch.from_numpy(synth.random_rows(n, N_RAND, seed=33)).to(dev)
    y_rand = torch.empty((N_RAND, 64), dtype=torch.float16, device=dev)
    q = torch.from_numpy(synth.query(B2, H2, seed=5)).to(dev)
    per_slab = B2 * H2 * T2
    ws = torch.empty((max(fq.fq_attend_workspace_size(cbs[0], B2, H2, H2, T2), 256),),
                     dtype=torch.uint8, device=dev)
    att_out = torch.empty((B2, H2, 64), dtype=torch.float16, device=dev)
    timer = Timer(torch)

    def one():
        for v, cb in enumerate(cbs):
            timer.run(f"encode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_encode(cb, xs[v], codes[v], norms[v]))
        for v, cb in enumerate(cbs):
            timer.run(f"decode_k{cb.k}N{cb.N}",
                      lambda v=v, cb=cb: fq.fq_decode(cb, codes[v], norms[v], y=ys[v]))
        timer.run("random_decode_k2N16",
                  lambda: fq.fq_decode(cbs[0], codes[0], norms[0], rows=rows, y=y_rand))
        W = cbs[0].W
        for layer in range(L2):
            sl = slice((2 * layer) * per_slab, (2 * layer + 1) * per_slab)
            sv = slice((2 * layer + 1) * per_slab, (2 * layer + 2) * per_slab)
            kc, vc = codes[0][sl].view(B2, H2, T2, W), codes[0][sv].view(B2, H2, T2, W)
            kn, vn = norms[0][sl].view(B2, H2, T2), norms[0][sv].view(B2, H2, T2)
            timer.run("attend_k2N16", lambda kc=kc, vc=vc, kn=kn, vn=vn: fq.fq_attend_decode(
                cbs[0], cbs[0], q, kc, kn, vc, vn, 0.125, workspace=ws, out=att_out))

    for _ in range(warmup):
        one()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    timer.collect()
    out = {}
    for name, lst in timer.ms.items():
        ms = float(np.mean(lst))
        r = {"ms_avg": ms, "launches": len(lst)}
        if name.startswith(("encode", "decode")):
            k, N = [int(v) for v in name.split("_k")[1].split("N")]
            r["vectors_per_s"] = n / (ms * 1e-3)
            r["gbs"] = r["vectors_per_s"] * codec_bytes(k, N) / 1e9
            r["hbm_frac"] = r["gbs"] / HBM_PEAK_GBS
        elif name.startswith("random"):
            r["vectors_per_s"] = N_RAND / (ms * 1e-3)
            r["gbs"] = r["vectors_per_s"] * (8 + codec_bytes(2, 16)) / 1e9
        else:
            b = per_slab * 2 * (record_bytes(2, 16) + 2) + 2 * B2 * H2 * 64 * 2
            r["gbs"] = b / (ms * 1e-3) / 1e9
            r["hbm_frac"] = r["gbs"] / HBM_PEAK_GBS
        out[name] = r
    log("gpt2-shaped cache timing done")
    return {"workload": "gpt2-small-kv-cache: 12 layers x {K,V} x batch 4 x 12 heads x seq 1024, "
                        "d=64, fp16 (1,179,648 vectors); k2N16/64/256, k3N512 encode + decode, "
                        "2^20 random-access decodes, 12-layer decode-step attention (k2N16)",
            "ms_per_pass": el * 1e3, "vectors_per_s": 2 * n * len(GPT2_VARIANTS) / el,
            "ops": out}


FIDELITY_VARIANTS = [(8, 16), (4, 4), (8, 256), (4, 256), (2, 16), (2, 32), (3, 512), (2, 64),
                     (2, 128), (2, 256)]   # k3N4096's tables exceed the attention kernel's LDS


def fidelity(torch, fq, synth, dev, B=2, Hq=32, Hkv=4, T=4096, layers=(0, 11, 21)):
    """Attention-output fidelity against the compression ratio (quality context).

    TinyLlama-shaped seeded caches (per-channel log-uniform scales, 1 % x20
    outlier channels), three layers, batch 2, 32 query / 4 KV heads, 4096
    tokens: the fused attention over the compressed cache against exact
    softmax attention over the uncompressed binary16 cache (float32), cosine
    per (batch, query head).  Two query sets: N(0, 1) queries (scores spread
    over tens of units: attention is close to an argmax over keys), and
    queries scaled per stream so that the scores have a standard deviation of
    about 1.5 (a softer attention, closer to a trained model's).  The
    compression ratio counts the stored record and norm against 64 binary16
    values.
    """
    G = Hq // Hkv
    n = B * Hkv * T
    q_raw = torch.from_numpy(synth.query(B, Hq, seed=7)).to(dev)
    caches = []
    for layer in layers:
        K = synth.kv_slab_device(3, layer, 0, B, Hkv, T, dev)
        V = synth.kv_slab_device(3, layer, 1, B, Hkv, T, dev)
        qsets = {}
        qf = q_raw.float().view(B, Hkv, G, 64)
        for name in ("gaussian", "score_sd_1.5"):
            qq = qf
            if name != "gaussian":
                s = torch.matmul(qf, K.float().transpose(-1, -2).contiguous()) * 0.125
                qq = qf * (1.5 / s.std(dim=-1, keepdim=True))
            s = torch.matmul(qq, K.float().transpose(-1, -2).contiguous()) * 0.125
            o = torch.matmul(torch.softmax(s, dim=-1), V.float()).reshape(B, Hq, 64)
            qsets[name] = (qq.reshape(B, Hq, 64).half().contiguous(), o)
        caches.append((K, V, qsets))
    rows = []
    for k, N in FIDELITY_VARIANTS + LARGE_VARIANTS:
        cb = fq.load_codebook(k, N)
        cos = {"gaussian": [], "score_sd_1.5": []}
        for K, V, qsets in caches:
            kc, kn = fq.fq_encode(cb, K.reshape(n, 64))
            vc, vn = fq.fq_encode(cb, V.reshape(n, 64))
            for name, (qq, o_ref) in qsets.items():
                if k < 32:
                    o = fq.fq_attend_decode(cb, cb, qq, kc.view(B, Hkv, T, cb.W),
                                            kn.view(B, Hkv, T), vc.view(B, Hkv, T, cb.W),
                                            vn.view(B, Hkv, T), 0.125)
                else:
                    # no fused attention for tables larger than LDS: decode, then the
                    # same float32 attention as the reference
                    Kd = fq.fq_decode(cb, kc, kn).float().view(B, Hkv, T, 64)
                    Vd = fq.fq_decode(cb, vc, vn).float().view(B, Hkv, T, 64)
                    sd = torch.matmul(qq.float().view(B, Hkv, G, 64),
                                      Kd.transpose(-1, -2).contiguous()) * 0.125
                    o = torch.matmul(torch.softmax(sd, dim=-1), Vd).reshape(B, Hq, 64)
                cos[name].append(torch.nn.functional.cosine_similarity(
                    o.float(), o_ref, dim=-1).flatten())
        row = {"variant": f"k{k}N{N}", "bits_per_coord": math.log2(N) / k,
               "compression": 128.0 / (4 * cb.W + 2),
               "compression_packed": 1024.0 / cb.packed_bits}
        for name, lst in cos.items():
            c = torch.cat(lst)
            row[f"{name}_cos_mean"] = float(c.mean())
            row[f"{name}_cos_p10"] = float(torch.quantile(c, 0.1))
        rows.append(row)
    log("fidelity sweep done")
    return {"workload": f"tinyllama-shaped caches, layers {list(layers)}, batch {B}, "
                        f"{Hq} q / {Hkv} kv heads, {T} tokens; exact attention in float32 on "
                        "the binary16 cache as reference; N(0,1) queries, and queries rescaled "
                        "per (batch, query head) to a score standard deviation of 1.5",
            "rows": rows}


def bench_large(torch, fq, synth, dev, steps, warmup):
    """Encode and decode of the GPT-2-shaped cache with the large-block codes:
    k = 32 and k = 64 with N = 4096, and k = 64 with N = 16384 (30-bit packed
    records, the 34.1x point).

    The block search is a dense contraction here (N codewords of k coordinates
    per block, 64 * N multiply-adds per vector at either k), run on the matrix
    cores: its roofline is the binary16 MFMA peak.  The kernel
    forms every product twice (z split into binary16 hi and lo parts), so
    the algorithmic fraction reported here is at most one half.
    """
    import numpy as np
    n = L2 * 2 * B2 * H2 * T2
    x = torch.from_numpy(synth.kv_cache(2, L2, B2, H2, T2).reshape(n, 64)).to(dev)
    y = torch.empty((n, 64), dtype=torch.float16, device=dev)
    out = {}
    for k, N in LARGE_VARIANTS:
        cb = fq.load_codebook(k, N)
        codes = torch.empty((n, cb.W), dtype=torch.int32, device=dev)
        norms = torch.empty((n,), dtype=torch.int16, device=dev)
        timer = Timer(torch)
        for i in range(warmup + steps):
            if i == warmup:
                timer.reset()
            timer.run("encode", lambda: fq.fq_encode(cb, x, codes, norms))
            timer.run("decode", lambda: fq.fq_decode(cb, codes, norms, y=y))
        timer.collect()
        te = float(np.median(timer.ms["encode"])) * 1e-3
        td = float(np.median(timer.ms["decode"])) * 1e-3
        packed = torch.empty((cb.packed_words(n),), dtype=torch.int32, device=x.device)
        fq.fq_pack_records(cb, codes, norms, packed=packed)
        tp = Timer(torch)
        for i in range(warmup + steps):
            if i == warmup:
                tp.reset()
            tp.run("decode_packed", lambda: fq.fq_decode_packed(cb, packed, n, y=y))
        tp.collect()
        tdp = float(np.median(tp.ms["decode_packed"])) * 1e-3
        pk_bytes = n * (cb.packed_bits / 8 + 128)
        flops = 2.0 * 64 * N * n                  # one multiply-add per codeword coordinate
        dec_bytes = n * codec_bytes(k, N)
        out[f"k{k}N{N}"] = {
            "bits_per_coord": math.log2(N) / k, "compression": 128.0 / (4 * cb.W + 2),
            "encode_ms": te * 1e3, "encode_vectors_per_s": n / te,
            "encode_mfma_tflops": flops / te / 1e12,
            "encode_mfma_frac": flops / te / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "decode_ms": td * 1e3, "decode_gbs": dec_bytes / td / 1e9,
            "decode_hbm_frac": dec_bytes / td / 1e9 / HBM_PEAK_GBS,
            "packed_bits_per_vector": cb.packed_bits, "packed_compression": 1024.0 / cb.packed_bits,
            "decode_packed_ms": tdp * 1e3, "decode_packed_gbs": pk_bytes / tdp / 1e9,
            "decode_packed_hbm_frac": pk_bytes / tdp / 1e9 / HBM_PEAK_GBS}
        del codes, norms, packed
    log("large-block timing done")
    return {"workload": f"gpt2-small-kv-cache, {n} vectors, fp16; median of {steps} launches",
            "peak_mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS, "codes": out}


def bench_configs(torch, fq, synth, dev, reps=5):
    """The tiny and TinyLlama-cache configurations, each op timed with HIP events (median).

    tiny: 4096 float32 vectors, k2N16 encode + decode (a latency figure);
    tinyllama cache: 22 layers x {K,V} x batch 8 x 4 heads x 2048 tokens,
      full encode at k4N256 and k8N256, then 2^20 uniformly drawn addresses
      decoded by address.
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
                      "decode_gbs": n * (128 + rb) / td / 1e9})
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
    log("configuration timing done")
    return out


def bench_attend(torch, fq, synth, dev, layers, steps, warmup):
    """Fused attention at batch 16, 32 query / 4 KV heads, 32768 tokens, k4N256, per layer."""
    import numpy as np
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
            xx = synth.kv_slab_device(3, layer, kv, Bq, Hkv, Tq, dev).reshape(per, 64)
            fq.fq_encode(cb, xx, c[layer].view(per, cb.W), nn[layer].view(per))
            del xx
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
    log("tinyllama attention timing done")
    return {"workload": "tinyllama decode step: batch 16, 32 q / 4 kv heads, seq 32768, d=64, "
                        f"k4N256 K and V, {layers} layers",
            "ms_per_layer_event": ms, "ms_per_layer_wall": 1e3 * el / (steps * layers),
            "bytes_per_layer": bytes_layer, "gbs": bytes_layer / (ms * 1e-3) / 1e9,
            "hbm_frac": bytes_layer / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_step_with_append_ms_per_layer": ms_step}


if __name__ == "__main__":
    sys.exit(main())
