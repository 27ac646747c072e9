"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad artifacts and arguments before touching a device.
No compute call is made here, so these run without a GPU."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

from kv_cache_compression_fq_amd import fq
from oracle import artifact, rotation

from conftest import ROOT, VARIANTS, artifact_path


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "fq.h")).read()
    return sorted(set(re.findall(r"\b(fq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fq.library()
    syms = declared_symbols()
    assert set(syms) == set(fq.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings():
    for s in range(7):
        assert fq.fq_status_string(s)
    assert fq.fq_status_string(99) == "unknown status"


@pytest.mark.parametrize("k,N", VARIANTS)
def test_committed_artifacts_pass_library_check(k, N):
    blob = open(artifact_path(k, N), "rb").read()
    st, info = fq.fq_artifact_check(blob)
    assert st == fq.FQ_OK
    a = artifact.read_artifact(blob)
    assert (info["k"], info["N"], info["nb"], info["idx_bits"], info["record_words"]) == \
        (k, N, a["nb"], a["bits"], a["W"])
    assert info["artifact_hash"] == a["hash"]
    assert info["rate_nominal"] == a["bits"] / k
    assert info["packed_bits"] == a["nb"] * a["bits"] + 16


def make_book(k, N, C=None, Pi=None, d=64):
    nb = -(-d // k)
    if C is None:
        C = np.random.default_rng([k, N]).standard_normal((N, k)).astype(np.float32) * 0.1
    book = {"C": C, "d": d, "k": k, "N": N, "nb": nb, "partial": d - (nb - 1) * k,
            "restarts": 1, "max_iter": 1, "iterations": 1, "best_restart": 0, "samples": 1,
            "tol": 0.0, "D_train_block": 0.0, "D_test": 0.0, "law_a": 1.0, "law_b": 1.0}
    return artifact.write_artifact(rotation.make_rotation(d, 0) if Pi is None else Pi, book)


def rehash(blob):
    body = bytes(blob[:-8])
    return body + struct.pack("<Q", artifact.fnv1a64(body))


def test_bad_artifacts_rejected():
    good = make_book(4, 256)
    assert fq.fq_artifact_check(good)[0] == fq.FQ_OK
    BAD = fq.FQ_ERR_BAD_ARTIFACT
    assert fq.fq_artifact_check(b"")[0] == BAD
    assert fq.fq_artifact_check(good[:-1])[0] == BAD                 # truncated
    assert fq.fq_artifact_check(good + b"\0")[0] == BAD              # trailing byte
    b = bytearray(good); b[0] = ord("X")
    assert fq.fq_artifact_check(bytes(b))[0] == BAD                  # magic
    b = bytearray(good); b[4] = 2
    assert fq.fq_artifact_check(rehash(b))[0] == BAD                 # version
    b = bytearray(good); b[400] ^= 0x10
    assert fq.fq_artifact_check(bytes(b))[0] == BAD                  # payload vs hash
    b = bytearray(good); b[24] = 17                                  # nb inconsistent
    assert fq.fq_artifact_check(rehash(b))[0] == BAD
    b = bytearray(good); b[200] = 1                                  # reserved header byte
    assert fq.fq_artifact_check(rehash(b))[0] == BAD
    C = np.zeros((256, 4), dtype=np.float32); C[3, 1] = np.nan
    assert fq.fq_artifact_check(make_book(4, 256, C=C))[0] == BAD    # non-finite codeword
    Pi = rotation.make_rotation(64, 0).copy(); Pi[0, 0] += 1e-6
    assert fq.fq_artifact_check(make_book(4, 256, Pi=Pi))[0] == BAD  # not orthogonal


def test_unsupported_but_valid_artifacts():
    UNS = fq.FQ_ERR_UNSUPPORTED
    st, info = fq.fq_artifact_check(make_book(5, 8))
    assert st == UNS and info["nb"] == 13
    st, info = fq.fq_artifact_check(make_book(2, 8192))
    assert st == UNS
    # 14-bit indices are built for k = 64 only; 15 bits for none
    assert fq.fq_artifact_check(make_book(32, 16384))[0] == UNS
    st, info = fq.fq_artifact_check(make_book(64, 32768))
    assert st == UNS and info["idx_bits"] == 15


def test_null_arguments_rejected_without_device():
    lib = fq.library()
    INV = fq.FQ_ERR_INVALID_ARG
    assert lib.fq_artifact_check(None, 10, None) == INV
    assert lib.fq_codebook_load(None, 0, 0, None) == INV
    out = ctypes.c_void_p()
    assert lib.fq_codebook_load(None, 0, 0, ctypes.byref(out)) == INV
    assert lib.fq_codebook_info(None, None) == INV
    lib.fq_codebook_free(None)
    assert lib.fq_encode(None, None, 1, 10, 64, None, None, None) == INV
    assert lib.fq_decode(None, None, None, None, 0, 10, None, 1, 64, None) == INV
    sz = ctypes.c_size_t()
    assert lib.fq_attend_workspace_size(None, 1, 1, 1, 1, ctypes.byref(sz)) == INV
    assert lib.fq_attend_decode(None, None, None, None, None, None, None, 1, 1, 1, 1,
                                ctypes.c_float(1.0), None, 0, None, None) == INV
    assert lib.fq_attend_decode_static(None, None, None, None, None, None, None, 1, 1, 1, 1,
                                       ctypes.c_float(1.0), None, None) == INV
    assert lib.fq_pack_records(None, None, None, 10, None, None) == INV
    assert lib.fq_decode_packed(None, None, None, 0, 10, None, 1, 64, None) == INV
    e, f = ctypes.c_double(), ctypes.c_double()
    assert lib.fq_search_cost(None, None, 1, 10, 64, ctypes.byref(e), ctypes.byref(f)) == INV


def test_load_without_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    blob = open(artifact_path(2, 16), "rb").read()
    with pytest.raises(fq.FQError) as e:
        fq.fq_codebook_load(blob, 0)
    assert e.value.status == fq.FQ_ERR_DEVICE
