"""FibQuant random-access KV-cache codec for MI355X (gfx950).

The codec's hot path (encode, decode, random-access decode and fused
decode-step attention over the compressed cache) runs in hand-written HIP
kernels behind the C ABI of ``include/fq.h`` (``libfq.so``, built by
``kv_cache_compression_fq_amd.build``).  ``fq`` is the thin ctypes binding
with the same names; ``synth`` draws the seeded synthetic inputs.
"""
from . import fq, synth  # noqa: F401
