"""Offline build of the shared codebook artifacts (calls only ``oracle``).

Writes one ``.fqcb`` file per (k, N) variant into
``kv_cache_compression_fq_amd/codebooks/``.  Every artifact carries the same
rotation Pi (seed 0): one shared rotation for keys, values, layers and heads
([FQ 1, 2.3]) and one codebook per rate ([FQ 2.1]).

Usage:  python -m oracle.build_codebooks [k:N ...] [--samples S] [--restarts R]
"""
import argparse
import os
import sys
import time

from . import artifact, codebook, rotation

VARIANTS = [(2, 16), (2, 64), (2, 256), (3, 512), (4, 256), (8, 256), (8, 16), (4, 4),
            (3, 4096), (2, 32), (2, 128), (32, 4096), (64, 4096), (64, 16384)]
# Large-k codebooks (k = d/2 and k = d, N = 4096): one Lloyd assignment pass
# over 2^20 samples is a 2^20 x 64 x 4096 float64 product (about 24 s on an
# 8-core host), so the full 8-restart, 200-iteration recipe would take hours
# per table.  They train on the full 2^20 samples (256 per cell) with 2
# restarts and at most 30 iterations (recorded in the artifact header).  The
# 14-bit whole-vector code (k = 64, N = 16384: a 30-bit record with its norm,
# the extreme point of the pages' rate sweep) costs four times as much per
# pass and trains with one restart and at most 20 iterations (64 samples per
# cell).
LARGE = {(32, 4096): dict(samples=1 << 20, restarts=2, max_iter=30),
         (64, 4096): dict(samples=1 << 20, restarts=2, max_iter=30),
         (64, 16384): dict(samples=1 << 20, restarts=1, max_iter=20)}
D = 64
OUT_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "kv_cache_compression_fq_amd", "codebooks")


def artifact_name(k, N):
    return f"fq_d{D}_k{k}_N{N}.fqcb"


def build_one(k, N, samples, restarts, out_dir, log):
    Pi = rotation.make_rotation(D, rotation.SEED_ROT)
    t0 = time.time()
    opts = dict(samples=samples, restarts=restarts)
    opts.update(LARGE.get((k, N), {}))
    book = codebook.build_codebook(D, k, N, test_samples=opts["samples"], log=log, **opts)
    book["seed_rot"] = rotation.SEED_ROT
    book["law_a"], book["law_b"] = codebook.radius_law(D, k)
    blob = artifact.write_artifact(Pi, book)
    path = os.path.join(out_dir, artifact_name(k, N))
    with open(path, "wb") as f:
        f.write(blob)
    log(f"wrote {path}: D_test={book['D_test']:.6f} restart={book['best_restart']} "
        f"iters={book['iterations']} ({time.time() - t0:.0f} s)")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("variants", nargs="*", help="k:N pairs (default: all)")
    ap.add_argument("--samples", type=int, default=1 << 20)
    ap.add_argument("--restarts", type=int, default=8)
    ap.add_argument("--out", default=OUT_DIR)
    a = ap.parse_args(argv)
    todo = VARIANTS if not a.variants else [tuple(map(int, v.split(":"))) for v in a.variants]
    os.makedirs(a.out, exist_ok=True)

    def log(msg):
        print(msg, flush=True)

    for k, N in todo:
        build_one(k, N, a.samples, a.restarts, a.out, log)
    return 0


if __name__ == "__main__":
    sys.exit(main())
