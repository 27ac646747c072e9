import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CODEBOOK_DIR = os.path.join(ROOT, "kv_cache_compression_fq_amd", "codebooks")
GOLDEN_DIR = os.path.join(ROOT, "tests", "golden")
VARIANTS = [(2, 16), (2, 64), (2, 256), (3, 512), (4, 256), (8, 256), (8, 16), (4, 4), (3, 4096),
            (2, 32), (2, 128), (32, 4096), (64, 4096), (64, 16384)]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def artifact_path(k, N):
    return os.path.join(CODEBOOK_DIR, f"fq_d64_k{k}_N{N}.fqcb")


@pytest.fixture(scope="session")
def artifacts():
    from oracle import artifact
    out = {}
    for k, N in VARIANTS:
        with open(artifact_path(k, N), "rb") as f:
            blob = f.read()
        a = artifact.read_artifact(blob)
        a["blob"] = blob
        out[(k, N)] = a
    return out
