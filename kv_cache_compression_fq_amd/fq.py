"""ctypes binding of ``libfq.so`` with the C names (argument marshalling only).

Every step of the codec runs in the HIP kernels behind the C ABI declared in
``include/fq.h``.  This module only turns torch tensors into device pointers,
picks up the current HIP stream, allocates outputs with torch when the caller
does not pass them, and turns status codes into exceptions.  If the library
is not built it raises; there is no fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfq.so")
CODEBOOK_DIR = os.path.join(PKG, "codebooks")

FQ_F16, FQ_F32 = 1, 2
FQ_OK, FQ_ERR_INVALID_ARG, FQ_ERR_BAD_ARTIFACT, FQ_ERR_UNSUPPORTED, FQ_ERR_NO_MEMORY, \
    FQ_ERR_DEVICE, FQ_ERR_SCRATCH = range(7)
FQ_STATIC_SCRATCH_BYTES = 4 << 20

EXPORTS = ["fq_status_string", "fq_artifact_check", "fq_codebook_load", "fq_codebook_info",
           "fq_search_cost", "fq_codebook_free", "fq_encode", "fq_decode", "fq_pack_records",
           "fq_decode_packed", "fq_attend_workspace_size",
           "fq_attend_decode", "fq_attend_decode_static", "fq_attend_queries",
           "fq_decode_step"]


class FQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {fq_status_string(status)} (status {status})")
        self.status = status


class fq_info(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("k", ctypes.c_int32), ("N", ctypes.c_int32),
                ("nb", ctypes.c_int32), ("idx_bits", ctypes.c_int32),
                ("record_words", ctypes.c_int32), ("last_block", ctypes.c_int32),
                ("packed_bits", ctypes.c_int32), ("rate_nominal", ctypes.c_double),
                ("rate_actual", ctypes.c_double), ("distortion", ctypes.c_double),
                ("artifact_hash", ctypes.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def library(path=LIB_PATH):
    """Load libfq.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m kv_cache_compression_fq_amd.build`")
    lib = ctypes.CDLL(path)
    lib.fq_status_string.argtypes = [ctypes.c_int]
    lib.fq_status_string.restype = ctypes.c_char_p
    lib.fq_artifact_check.argtypes = [_P, ctypes.c_size_t, ctypes.POINTER(fq_info)]
    lib.fq_codebook_load.argtypes = [_P, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(_P)]
    lib.fq_codebook_info.argtypes = [_P, ctypes.POINTER(fq_info)]
    lib.fq_search_cost.argtypes = [_P, _P, ctypes.c_int, _I64, _I64,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.fq_codebook_free.argtypes = [_P]
    lib.fq_codebook_free.restype = None
    lib.fq_encode.argtypes = [_P, _P, ctypes.c_int, _I64, _I64, _P, _P, _P]
    lib.fq_decode.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P]
    lib.fq_pack_records.argtypes = [_P, _P, _P, _I64, _P, _P]
    lib.fq_decode_packed.argtypes = [_P, _P, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P]
    lib.fq_attend_workspace_size.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _I64,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.fq_attend_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, _I64, ctypes.c_float, _P, ctypes.c_size_t, _P,
                                     _P]
    lib.fq_attend_decode_static.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, _I64, ctypes.c_float,
                                            _P, _P]
    lib.fq_attend_queries.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _I64, _I64, ctypes.c_int, ctypes.c_float, _P,
                                      ctypes.c_size_t, _P, _P]
    lib.fq_decode_step.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, _I64, _I64, ctypes.c_int, ctypes.c_float, _P,
                                   ctypes.c_size_t, _P, _P]
    for name in EXPORTS:
        if name not in ("fq_status_string", "fq_codebook_free"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def fq_status_string(status):
    return library().fq_status_string(int(status)).decode()


def _check(status, what):
    if status != FQ_OK:
        raise FQError(status, what)


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# --------------------------------------------------------------------- codebooks
def codebook_path(k, N, d=64):
    return os.path.join(CODEBOOK_DIR, f"fq_d{d}_k{k}_N{N}.fqcb")


def read_codebook_bytes(k, N):
    with open(codebook_path(k, N), "rb") as f:
        return f.read()


def fq_artifact_check(blob):
    """Host-only validation; returns (status, info dict or None)."""
    info = fq_info()
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    st = library().fq_artifact_check(buf, len(blob), ctypes.byref(info))
    return st, (info.as_dict() if st in (FQ_OK, FQ_ERR_UNSUPPORTED) else None)


class Codebook:
    """An fq_codebook handle (device tables owned by the library)."""

    def __init__(self, handle, device):
        self.handle = handle
        self.device = device
        info = fq_info()
        _check(library().fq_codebook_info(handle, ctypes.byref(info)), "fq_codebook_info")
        self.info = info.as_dict()

    def free(self):
        if self.handle:
            library().fq_codebook_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    @property
    def k(self):
        return self.info["k"]

    @property
    def N(self):
        return self.info["N"]

    @property
    def W(self):
        return self.info["record_words"]

    @property
    def nb(self):
        return self.info["nb"]

    @property
    def packed_bits(self):
        return self.info["packed_bits"]

    def packed_words(self, n):
        return -(-(n * self.packed_bits) // 32)


def fq_codebook_load(blob, device=0):
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    _check(library().fq_codebook_load(buf, len(blob), int(device), ctypes.byref(h)),
           "fq_codebook_load")
    return Codebook(h, device)


def load_codebook(k, N, device=0):
    return fq_codebook_load(read_codebook_bytes(k, N), device)


def fq_search_cost(cb, x_host):
    """Search work model for host vectors x_host (numpy [n, >=64] float16 or
    float32): (codewords compared per vector, share of blocks scanning all N)."""
    import numpy as np
    x_host = np.ascontiguousarray(x_host)
    dt = FQ_F16 if x_host.dtype == np.float16 else FQ_F32
    if x_host.dtype not in (np.float16, np.float32) or x_host.ndim != 2:
        raise ValueError("x_host must be a 2-D float16 or float32 array")
    e, f = ctypes.c_double(), ctypes.c_double()
    _check(library().fq_search_cost(cb.handle, x_host.ctypes.data_as(_P), dt, x_host.shape[0],
                                    x_host.shape[1], ctypes.byref(e), ctypes.byref(f)),
           "fq_search_cost")
    return e.value, f.value


def fq_codebook_free(cb):
    cb.free()


# ------------------------------------------------------------------------ codec
def _dtype_code(dt):
    import torch
    if dt == torch.float16:
        return FQ_F16
    if dt == torch.float32:
        return FQ_F32
    raise ValueError(f"unsupported dtype {dt}")


def fq_encode(cb, x, codes=None, norms=None, stream=None):
    """Encode rows of x [n, >=64] (row stride x.stride(0)); returns (codes, norms)."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] < 64:
        raise ValueError("x must be [n, >=64] with unit column stride")
    n = x.shape[0]
    if codes is None:
        codes = torch.empty((n, cb.W), dtype=torch.int32, device=x.device)
    if norms is None:
        norms = torch.empty((n,), dtype=torch.int16, device=x.device)
    if codes.shape != (n, cb.W) or not codes.is_contiguous() or norms.shape != (n,):
        raise ValueError("codes must be [n, W] contiguous and norms [n]")
    _check(library().fq_encode(cb.handle, _ptr(x), _dtype_code(x.dtype), n, x.stride(0),
                               _ptr(codes), _ptr(norms), _stream(stream, x.device)), "fq_encode")
    return codes, norms


def fq_decode(cb, codes, norms, rows=None, y=None, y_dtype=None, stream=None):
    """Decode all records (rows=None) or records rows[i]; returns y [n, 64]."""
    import torch
    if codes.dim() != 2 or codes.shape[1] != cb.W or not codes.is_contiguous():
        raise ValueError("codes must be [n_records, W] contiguous")
    n_records = codes.shape[0]
    n = n_records if rows is None else rows.shape[0]
    if rows is not None and (rows.dtype != torch.int64 or not rows.is_contiguous()):
        raise ValueError("rows must be contiguous int64")
    if y is None:
        y = torch.empty((n, 64), dtype=y_dtype or torch.float16, device=codes.device)
    if y.dim() != 2 or y.shape[0] != n or y.stride(1) != 1:
        raise ValueError("y must be [n, >=64] with unit column stride")
    _check(library().fq_decode(cb.handle, _ptr(codes), _ptr(norms), _ptr(rows), n_records, n,
                               _ptr(y), _dtype_code(y.dtype), y.stride(0),
                               _stream(stream, codes.device)), "fq_decode")
    return y


def fq_pack_records(cb, codes, norms, packed=None, stream=None):
    """Word-aligned records [n, W] + norms [n] -> packed stream [ceil(n R / 32)] int32."""
    import torch
    if codes.dim() != 2 or codes.shape[1] != cb.W or not codes.is_contiguous():
        raise ValueError("codes must be [n, W] contiguous")
    n = codes.shape[0]
    if norms.shape != (n,) or not norms.is_contiguous():
        raise ValueError("norms must be [n] contiguous")
    if packed is None:
        packed = torch.empty((cb.packed_words(n),), dtype=torch.int32, device=codes.device)
    if packed.numel() < cb.packed_words(n) or not packed.is_contiguous():
        raise ValueError("packed must hold ceil(n R / 32) words")
    _check(library().fq_pack_records(cb.handle, _ptr(codes), _ptr(norms), n, _ptr(packed),
                                     _stream(stream, codes.device)), "fq_pack_records")
    return packed


def fq_decode_packed(cb, packed, n_records, rows=None, y=None, y_dtype=None, stream=None):
    """Decode n_records packed records (rows=None) or records rows[i]; returns y [n, 64]."""
    import torch
    if packed.dim() != 1 or not packed.is_contiguous() or packed.numel() < cb.packed_words(n_records):
        raise ValueError("packed must be a contiguous stream of ceil(n_records R / 32) words")
    n = n_records if rows is None else rows.shape[0]
    if rows is not None and (rows.dtype != torch.int64 or not rows.is_contiguous()):
        raise ValueError("rows must be contiguous int64")
    if y is None:
        y = torch.empty((n, 64), dtype=y_dtype or torch.float16, device=packed.device)
    if y.dim() != 2 or y.shape[0] != n or y.stride(1) != 1:
        raise ValueError("y must be [n, >=64] with unit column stride")
    _check(library().fq_decode_packed(cb.handle, _ptr(packed), _ptr(rows), n_records, n, _ptr(y),
                                      _dtype_code(y.dtype), y.stride(0),
                                      _stream(stream, packed.device)), "fq_decode_packed")
    return y


def fq_attend_workspace_size(cb_k, B, Hq, Hkv, T):
    out = ctypes.c_size_t()
    _check(library().fq_attend_workspace_size(cb_k.handle, B, Hq, Hkv, T, ctypes.byref(out)),
           "fq_attend_workspace_size")
    return out.value


def fq_attend_decode(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, scale, workspace=None,
                     out=None, stream=None):
    """Decode-step attention; q [B, Hq, 64] fp16, caches [B, Hkv, T, W] / [B, Hkv, T]."""
    import torch
    B, Hq, d = q.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_codes, k_norms, v_codes, v_norms):
        if not t.is_contiguous():
            raise ValueError("attention inputs must be contiguous")
    if k_codes.shape != (B, Hkv, T, cb_k.W) or v_codes.shape != (B, Hkv, T, cb_v.W):
        raise ValueError("cache code shapes do not match the codebooks")
    if k_norms.shape != (B, Hkv, T) or v_norms.shape != (B, Hkv, T):
        raise ValueError("norm shapes must be [B, Hkv, T]")
    if workspace is None:
        nbytes = fq_attend_workspace_size(cb_k, B, Hq, Hkv, T)
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, 64), dtype=torch.float16, device=q.device)
    _check(library().fq_attend_decode(cb_k.handle, cb_v.handle, _ptr(q), _ptr(k_codes),
                                      _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), B, Hq, Hkv, T,
                                      float(scale), _ptr(workspace), workspace.numel(), _ptr(out),
                                      _stream(stream, q.device)), "fq_attend_decode")
    return out


def fq_attend_decode_static(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, scale, out=None,
                            stream=None):
    """fq_attend_decode with the library's static per-device scratch (no workspace;
    for callers that cannot allocate; calls overlapping on one device race)."""
    import torch
    B, Hq, d = q.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_codes, k_norms, v_codes, v_norms):
        if not t.is_contiguous():
            raise ValueError("attention inputs must be contiguous")
    if k_codes.shape != (B, Hkv, T, cb_k.W) or v_codes.shape != (B, Hkv, T, cb_v.W):
        raise ValueError("cache code shapes do not match the codebooks")
    if k_norms.shape != (B, Hkv, T) or v_norms.shape != (B, Hkv, T):
        raise ValueError("norm shapes must be [B, Hkv, T]")
    if out is None:
        out = torch.empty((B, Hq, 64), dtype=torch.float16, device=q.device)
    _check(library().fq_attend_decode_static(cb_k.handle, cb_v.handle, _ptr(q), _ptr(k_codes),
                                             _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), B, Hq,
                                             Hkv, T, float(scale), _ptr(out),
                                             _stream(stream, q.device)), "fq_attend_decode_static")
    return out


def _check_cache(cb, codes, norms, B, Hkv, name):
    if codes.dim() != 4 or codes.shape[0] != B or codes.shape[1] != Hkv or codes.shape[3] != cb.W:
        raise ValueError(f"{name} codes must be [B, Hkv, T_ld, W]")
    if norms.shape != codes.shape[:3]:
        raise ValueError(f"{name} norms must be [B, Hkv, T_ld]")
    if not codes.is_contiguous() or not norms.is_contiguous():
        raise ValueError(f"{name} cache must be contiguous")


def fq_attend_queries(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, T, scale,
                      workspace=None, out=None, stream=None):
    """Causal attention of M queries per head; q [B, Hq, M, 64] fp16, caches
    [B, Hkv, T_ld, W] / [B, Hkv, T_ld] of which the first T tokens are read."""
    import torch
    B, Hq, M, d = q.shape
    if d != 64 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, M, 64]")
    Hkv, T_ld = k_codes.shape[1], k_codes.shape[2]
    _check_cache(cb_k, k_codes, k_norms, B, Hkv, "key")
    _check_cache(cb_v, v_codes, v_norms, B, Hkv, "value")
    if v_codes.shape[2] != T_ld:
        raise ValueError("key and value caches must have the same capacity")
    if workspace is None:
        nbytes = fq_attend_workspace_size(cb_k, B, Hq * M, Hkv, T)
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, M, 64), dtype=torch.float16, device=q.device)
    _check(library().fq_attend_queries(cb_k.handle, cb_v.handle, _ptr(q), _ptr(k_codes),
                                       _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), B, Hq, Hkv, T,
                                       T_ld, M, float(scale), _ptr(workspace), workspace.numel(),
                                       _ptr(out), _stream(stream, q.device)), "fq_attend_queries")
    return out


def fq_decode_step(cb_k, cb_v, q, k_new, v_new, k_codes, k_norms, v_codes, v_norms, pos, scale,
                   workspace=None, out=None, stream=None):
    """Encode k_new / v_new [B, Hkv, M, 64] fp16 into cache slots pos .. pos + M - 1,
    then causal attention of q [B, Hq, M, 64] over the pos + M cached tokens."""
    import torch
    B, Hq, M, d = q.shape
    Hkv, T_ld = k_codes.shape[1], k_codes.shape[2]
    for t in (q, k_new, v_new):
        if not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError("q, k_new and v_new must be contiguous binary16")
    if k_new.shape != (B, Hkv, M, 64) or v_new.shape != (B, Hkv, M, 64):
        raise ValueError("k_new and v_new must be [B, Hkv, M, 64]")
    _check_cache(cb_k, k_codes, k_norms, B, Hkv, "key")
    _check_cache(cb_v, v_codes, v_norms, B, Hkv, "value")
    if v_codes.shape[2] != T_ld:
        raise ValueError("key and value caches must have the same capacity")
    if workspace is None:
        nbytes = fq_attend_workspace_size(cb_k, B, Hq * M, Hkv, pos + M)
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, M, 64), dtype=torch.float16, device=q.device)
    _check(library().fq_decode_step(cb_k.handle, cb_v.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                    _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), B,
                                    Hq, Hkv, T_ld, pos, M, float(scale), _ptr(workspace),
                                    workspace.numel(), _ptr(out), _stream(stream, q.device)),
           "fq_decode_step")
    return out
