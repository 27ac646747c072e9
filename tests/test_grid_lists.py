"""The encoder's candidate-list grids are complete, and the host code is clean
under AddressSanitizer / UndefinedBehaviorSanitizer.

``tests/native/grid_check.cpp`` links the library's own host sources
(``fq_grid.cpp``: grid_plan + build_grid; ``fq_artifact.cpp``: the artifact
parser) with g++, no HIP, and checks every listed cell against a brute-force
float64 nearest-codeword search (FibQuant technical summary, section 2.3;
Block Sphere VQ notes, key design 2).  The sanitizer build runs the same
checks on fewer points plus a parser fuzz (truncated, bit-flipped, rehashed
and random blobs).
"""
import os
import re
import subprocess

import pytest

from conftest import CODEBOOK_DIR, ROOT

CSRC = os.path.join(ROOT, "kv_cache_compression_fq_amd", "csrc")
SRC = [os.path.join(ROOT, "tests", "native", "grid_check.cpp"),
       os.path.join(CSRC, "fq_grid.cpp"), os.path.join(CSRC, "fq_artifact.cpp")]
OUT = os.path.join(ROOT, "_build", "native")
# every shipped codebook with candidate lists (k = 2, 3, and 4 with N >= 64)
GRID_BOOKS = [(2, 16), (2, 32), (2, 64), (2, 128), (2, 256), (3, 512), (3, 4096), (4, 256)]
ALL_BOOKS = GRID_BOOKS + [(4, 4), (8, 16), (8, 256), (32, 4096), (64, 4096)]
LINE = re.compile(r"k(\d+)N(\d+) dims=(\d+) G=(\d+) points=(\d+) lookups=(\d+) listed=(\d+) "
                  r"scanned=(\d+) misses=(\d+) mean_list=([\d.]+) max_list=(\d+) "
                  r"overflow_cells=(\d+) bad_records=(\d+)")


def compile_checker(name, flags):
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, name)
    cmd = ["g++", "-std=c++17", "-fopenmp", "-Wall", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC] + flags + SRC + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run_checker(exe, points, books, extra=(), env=None, timeout=900):
    paths = [os.path.join(CODEBOOK_DIR, f"fq_d64_k{k}_N{N}.fqcb") for k, N in books]
    r = subprocess.run([exe, str(points)] + paths + list(extra), capture_output=True, text=True,
                       env=env, timeout=timeout)
    return r


def parse_lines(stdout):
    rows = {}
    for m in LINE.finditer(stdout):
        k, N, dims = int(m.group(1)), int(m.group(2)), int(m.group(3))
        rows[(k, N, dims)] = {"points": int(m.group(5)), "lookups": int(m.group(6)),
                              "listed": int(m.group(7)), "misses": int(m.group(9)),
                              "mean_list": float(m.group(10)), "bad_records": int(m.group(13))}
    return rows


def expected_grids():
    want = []
    for k, N in GRID_BOOKS:
        want.append((k, N, k))
        if 64 % k:
            want.append((k, N, 1))      # the one-coordinate last block of k = 3
    return want


def test_candidate_lists_hold_the_nearest_codeword():
    """10^6 source blocks (plus 5 * 10^5 boundary and uniform points) per shipped
    grid, each looked up from two float32 views: no listed cell misses the
    float64 nearest codeword."""
    exe = compile_checker("grid_check", ["-O2"])
    r = run_checker(exe, 1_000_000, GRID_BOOKS)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    rows = parse_lines(r.stdout)
    assert sorted(rows) == sorted(expected_grids())
    for key, row in rows.items():
        assert row["points"] == 1_500_000 and row["misses"] == 0 and row["bad_records"] == 0, key
        # most source blocks fall in listed cells, so the lists are what the encoder uses
        assert row["listed"] > 0.8 * row["lookups"], key


def test_grid_checker_detects_a_planted_miss():
    """The checker is not vacuous: with one candidate dropped from every list of
    two or more entries (the mistake a wrong margin or dominance test in
    build_grid would make), it reports misses and fails."""
    exe = compile_checker("grid_check", ["-O2"])
    r = run_checker(exe, 50_000, [(2, 64), (3, 512)], extra=["--drop-last"])
    rows = parse_lines(r.stdout)
    assert r.returncode == 1
    assert rows[(2, 64, 2)]["misses"] > 0 and rows[(3, 512, 3)]["misses"] > 0


def test_host_code_under_address_and_undefined_sanitizers():
    """fq_grid.cpp and fq_artifact.cpp under ASan + UBSan: every shipped grid
    (fewer points) and a parser fuzz over every shipped artifact."""
    exe = compile_checker("grid_check_san", ["-O1", "-g", "-fno-omit-frame-pointer",
                                             "-fsanitize=address,undefined",
                                             "-fno-sanitize-recover=all"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    r = run_checker(exe, 20_000, ALL_BOOKS, extra=["--fuzz"], env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.stdout.count("parser-fuzz bad=0") == len(ALL_BOOKS)
    assert sorted(parse_lines(r.stdout)) == sorted(expected_grids())
