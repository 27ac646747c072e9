/*
 * fq.h -- C ABI of the FibQuant random-access KV-cache codec for MI355X (gfx950).
 *
 * Sources cited below:
 *   [FQ]     "FibQuant: Universal Vector Quantization for Random-Access KV-Cache
 *            Compression", technical summary (gist.science), by section:
 *            1 problem statement, 2.1 canonical source, 2.2 codebook
 *            construction, 2.3 encoding and decoding, 5 significance.
 *   [FQ-abs] the authors' abstract of the same paper.
 *
 * Conventions for every call:
 *   - Pure C: plain pointers and sizes.  Every data pointer is HIP device
 *     memory owned by the caller, except the artifact bytes given to
 *     fq_codebook_load / fq_artifact_check, which are host memory.
 *   - Every call returns an fq_status; no exception crosses the boundary.
 *     Arguments are checked on the host before any device work is queued;
 *     an argument error leaves every output untouched.
 *   - Work is queued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream).  A fault inside a kernel surfaces at
 *     the caller's next synchronisation, not as a return code.
 *   - Only fq_codebook_load allocates device memory.  fq_encode, fq_decode
 *     and fq_attend_decode allocate nothing; attention scratch comes from a
 *     caller-provided workspace, or (fq_attend_decode_static) from a static
 *     per-device array of the library.
 *   - A codebook handle is immutable after load and may be used from several
 *     host threads and streams at once.
 *   - Vectors have d = 64 coordinates.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fq_codebook fq_codebook; /* opaque */

typedef enum { FQ_F16 = 1, FQ_F32 = 2 } fq_dtype;

typedef enum {
  FQ_OK = 0,
  FQ_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size or stride */
  FQ_ERR_BAD_ARTIFACT = 2, /* malformed, truncated or corrupt artifact */
  FQ_ERR_UNSUPPORTED = 3, /* well-formed but outside what the kernels handle */
  FQ_ERR_NO_MEMORY = 4,   /* device allocation failed (load only) */
  FQ_ERR_DEVICE = 5,      /* HIP runtime error, or no usable device */
  FQ_ERR_SCRATCH = 6      /* shape exceeds the static scratch of fq_attend_decode_static */
} fq_status;

/* Bytes of the per-device static attention scratch of fq_attend_decode_static. */
#define FQ_STATIC_SCRATCH_BYTES (4u << 20)

typedef struct {
  int32_t d;            /* vector length (64) */
  int32_t k;            /* block size */
  int32_t N;            /* codebook size, a power of two */
  int32_t nb;           /* blocks per vector, ceil(d / k) */
  int32_t idx_bits;     /* bits per index, log2 N */
  int32_t record_words; /* uint32 words per record, ceil(nb * idx_bits / 32) */
  int32_t last_block;   /* real coordinates in the last block */
  int32_t packed_bits;  /* bits per packed record (fq_pack_records): nb * idx_bits + 16 */
  double rate_nominal;  /* log2(N) / k bits per coordinate [FQ 2.3] */
  double rate_actual;   /* nb * idx_bits / d */
  double distortion;    /* test distortion per unit vector recorded in the artifact */
  uint64_t artifact_hash; /* FNV-1a 64 of the artifact body */
} fq_info;

/* Human-readable name of a status code (static storage). */
const char* fq_status_string(fq_status s);

/*
 * Parse and validate an artifact on the host only (no device is touched).
 *
 * The artifact holds the shared rotation Pi (float64, d x d, row-major,
 * z = Pi u) and the shared codebook C (float32, N x k): one offline codebook
 * for every layer and head [FQ 2.1] and one shared Haar rotation [FQ 1, 2.3].
 * Checks: magic, version, header size, 1 <= d <= 4096, 1 <= k <= d, N a power
 * of two with 2 <= N <= 2^20, nb / idx_bits / record_words / last_block
 * consistent, total size, FNV-1a hash, finite values, max |Pi^T Pi - I| <=
 * 1e-9.  Returns FQ_ERR_BAD_ARTIFACT for a malformed or corrupt blob,
 * FQ_ERR_UNSUPPORTED for a valid blob the kernels are not built for (d != 64
 * or a (k, N) outside this list).  Built (k, N): k = 2 with N in {16, 32, 64,
 * 128, 256}; k = 3 with N in {512, 4096}; k = 4 with N in {4, 256}; k = 8
 * with N in {16, 256}; k = 32 with N = 4096; k = 64 with N in {4096, 16384}
 * (the k = 32 and 64 tables must hold binary16 values; fq_codebook_load
 * returns FQ_ERR_UNSUPPORTED otherwise).  `out` may be NULL.
 */
fq_status fq_artifact_check(const void* artifact, size_t nbytes, fq_info* out);

/*
 * Validate an artifact (as fq_artifact_check) and upload its tables to
 * `device`.  The blob is copied; the caller may free it on return.  On
 * success *out receives a handle to release with fq_codebook_free.
 */
fq_status fq_codebook_load(const void* artifact, size_t nbytes, int device, fq_codebook** out);

/* Describe a loaded codebook. */
fq_status fq_codebook_info(const fq_codebook* cb, fq_info* out);

/*
 * Work model of the encoder's block search, for reporting its compute
 * roofline (host only; reads host memory; no device work).  For n vectors of
 * x (host memory, layout as fq_encode), counts the codewords the search
 * compares each block with: the entries of the block's candidate list where
 * the codebook has lists and the block's cell carries one, else all N (a
 * full scan, as for codebooks without lists).  *entries_per_vector receives
 * the mean over the vectors of the sum over their blocks; *full_scan_share
 * (may be NULL) the share of blocks searched over all N.  Each entry costs
 * about k + 2 vector operations (k fused multiply-adds, a compare, a select).
 */
fq_status fq_search_cost(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                         int64_t x_ld, double* entries_per_vector, double* full_scan_share);

/* Release a codebook.  The caller guarantees no queued work still uses it.  NULL is a no-op. */
void fq_codebook_free(fq_codebook* cb);

/*
 * Encode n vectors [FQ 2.3]: nu = |x|_2; z = Pi (x / nu); for each of the nb
 * blocks of z, the index of the nearest codeword (squared Euclidean distance
 * over the block's real coordinates, ties to the lowest index); pack the
 * indices at fixed rate and store the norm [FQ 1].
 *
 *   x      [n rows, stride x_ld elements] of x_dtype (FQ_F16 or FQ_F32), row r at
 *          x + r * x_ld; x_ld >= 64 and x_ld * element size a multiple of 16 bytes
 *          (x_ld a multiple of 8 for F16, of 4 for F32); x 16-byte aligned.
 *          Other strides or alignments return FQ_ERR_INVALID_ARG.
 *   codes  [n, record_words] uint32 out, 4-byte aligned: field j (idx_bits bits)
 *          at bits [j*idx_bits, (j+1)*idx_bits) of the record, counted from the
 *          least significant bit of little-endian words; unused bits are 0.
 *   norms  [n] binary16 out (bit patterns), 2-byte aligned, nu rounded to nearest-even.
 *   A zero vector gets all-zero indices and norm 0.  n == 0 is a no-op.
 *   Indices agree with a float64 evaluation of the same distances except
 *   where two distances lie within a relative 1e-6 of each other.
 */
fq_status fq_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                    int64_t x_ld, uint32_t* codes, uint16_t* norms, void* stream);

/*
 * Decode [FQ 2.3]: fetch the codewords of a record, concatenate them (the last
 * block truncated to its real coordinates), apply Pi^T and scale by the stored
 * norm.  Random access [FQ 1]: when `rows` is non-NULL, output row i decodes
 * record rows[i] (0 <= rows[i] < n_records, checked on the device: an
 * out-of-range address decodes to a zero row); when NULL, row i decodes
 * record i and n_records is ignored.
 *
 *   codes [n_records, record_words] uint32 (4-byte aligned), norms [n_records] binary16
 *         (2-byte aligned), the layout of fq_encode
 *   rows  [n] int64 or NULL, 8-byte aligned; with rows, the record array may span at
 *         most 2^31 - 1 bytes (n_records * record_words * 4), else FQ_ERR_UNSUPPORTED
 *   y     [n rows, stride y_ld elements] of y_dtype out (F16 rounded to
 *         nearest-even, or F32); y 16-byte aligned, y_ld >= 64 and y_ld * element
 *         size a multiple of 16 bytes (else FQ_ERR_INVALID_ARG), y_ld <= 2^22
 *         (else FQ_ERR_UNSUPPORTED)
 */
fq_status fq_decode(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, void* y,
                    fq_dtype y_dtype, int64_t y_ld, void* stream);

/*
 * Packed records: the fixed-rate indices and the binary16 norm of a vector in
 * one bit stream, without rounding records up to whole words, so that the
 * stored size is the code's own rate plus the norm [FQ 1: fixed-rate records
 * at fixed addresses; the norm is stored with the code, 2.3].  Record r
 * occupies bits [r R, (r + 1) R) of `packed` (uint32 words, bits counted from
 * the least significant bit of little-endian words), R = packed_bits =
 * nb * idx_bits + 16: field j at record bits [j idx_bits, (j+1) idx_bits),
 * then the norm's 16 bits.  n records take ceil(n R / 32) words; bits past
 * the last record are 0.  Any record still decodes by address arithmetic
 * alone (bit offset r R).  For k = 64, R = 28 bits at N = 4096 (1024 / 28 =
 * 36.6 times smaller than the binary16 vector) and 30 bits at N = 16384
 * (34.1 times [FQ 4.2]); the word-aligned layout plus the separate norm
 * stores 48 bits (21.3 times).
 *
 * fq_pack_records converts n word-aligned records and their norms (the
 * layout of fq_encode) into the packed stream.  codes 4-byte, norms 2-byte,
 * packed 4-byte aligned; n == 0 is a no-op.
 */
fq_status fq_pack_records(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                          int64_t n, uint32_t* packed, void* stream);

/*
 * fq_decode reading packed records (see fq_pack_records): row i decodes
 * record i (rows NULL; n records in `packed`) or record rows[i] of the
 * n_records in `packed` (an address outside [0, n_records) decodes to a zero
 * row; with rows, the stream may span at most 2^31 - 1 bytes, else
 * FQ_ERR_UNSUPPORTED).  packed 4-byte aligned; y, rows, y_dtype and y_ld as
 * fq_decode.
 */
fq_status fq_decode_packed(const fq_codebook* cb, const uint32_t* packed, const int64_t* rows,
                           int64_t n_records, int64_t n, void* y, fq_dtype y_dtype, int64_t y_ld,
                           void* stream);

/*
 * Bytes of device workspace fq_attend_decode needs for this shape.
 */
fq_status fq_attend_workspace_size(const fq_codebook* cb_k, int B, int Hq, int Hkv, int64_t T,
                                   size_t* bytes);

/*
 * Fused decode-step attention over a compressed cache, the kernel fusion the
 * fixed-address records allow [FQ 5]; the cache is read at every decoding
 * step [FQ-abs].  For batch b and query head h (KV head g = h / (Hq / Hkv)):
 *   s_t = scale * <q[b,h], k_hat[b,g,t]>,  p = softmax_t(s),  out[b,h] = sum_t p_t v_hat[b,g,t]
 * where k_hat / v_hat are the fq_decode reconstructions.  Computed without
 * materialising them: scores nu_t <Pi q, z_hat_t> and values accumulated as
 * sum p_t nu_t z_hat_t in the rotated domain, rotated back once.
 *
 *   q        [B, Hq, 64] binary16
 *   k_codes  [B, Hkv, T, Wk] uint32,  k_norms [B, Hkv, T] binary16  (cb_k layout)
 *   v_codes  [B, Hkv, T, Wv] uint32,  v_norms [B, Hkv, T] binary16  (cb_v layout)
 *   out      [B, Hq, 64] binary16
 *   Hq % Hkv == 0, Hq / Hkv <= 8, T >= 1; workspace of at least
 *   fq_attend_workspace_size bytes, 256-byte aligned, contents need not be
 *   initialised.  cb_k and cb_v may be the same handle; they must be on the
 *   same device (else FQ_ERR_INVALID_ARG) and hold the same (k, N) variant and
 *   the same rotation Pi (one shared codebook and one shared rotation serve
 *   keys and values [FQ 1, 2.1, 2.3]; else FQ_ERR_UNSUPPORTED, since scores
 *   and values are formed in one rotated domain); the k = 3, N = 4096 tables
 *   and the k = 32, 64 tables exceed the kernel's LDS budget
 *   (FQ_ERR_UNSUPPORTED).  All pointers 16-byte aligned.
 */
fq_status fq_attend_decode(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                           const uint32_t* k_codes, const uint16_t* k_norms,
                           const uint32_t* v_codes, const uint16_t* v_norms, int B, int Hq,
                           int Hkv, int64_t T, float scale, void* workspace,
                           size_t workspace_bytes, uint16_t* out, void* stream);

/*
 * fq_attend_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same computation and kernels; the split-K partials live in a library-owned
 * static device array of FQ_STATIC_SCRATCH_BYTES per device instead of a
 * caller workspace.  The array is part of the library's device code (each
 * device holds its own copy until the process ends); its address is looked up
 * when a codebook is first loaded on the device.  This call allocates nothing.
 *
 *   Arguments, requirements and errors as fq_attend_decode, without the
 *   workspace.  A shape whose fq_attend_workspace_size exceeds
 *   FQ_STATIC_SCRATCH_BYTES returns FQ_ERR_SCRATCH (use fq_attend_decode).
 *   Every call on one device shares that device's array: calls that overlap
 *   in time on one device (on different streams, or from host threads with no
 *   ordering between them) race and give undefined outputs; calls ordered on
 *   one stream are safe.  The array needs no clearing between calls.
 */
fq_status fq_attend_decode_static(const fq_codebook* cb_k, const fq_codebook* cb_v,
                                  const uint16_t* q, const uint32_t* k_codes,
                                  const uint16_t* k_norms, const uint32_t* v_codes,
                                  const uint16_t* v_norms, int B, int Hq, int Hkv, int64_t T,
                                  float scale, uint16_t* out, void* stream);

/*
 * Attention of several queries per head over a compressed cache: the steps on
 * either side of decode-step attention in a serving loop [FQ 5] (a prefill
 * chunk, or the draft tokens of speculative decoding).  The M queries of
 * every head are the last M positions: query m of head h sees tokens
 * 0 .. T - M + m (causal), with the same scores and softmax as
 * fq_attend_decode (which is the case M = 1).  Computed by the same kernels,
 * the M queries of a head taking M of the query columns of its KV head.
 *
 *   q        [B, Hq, M, 64] binary16;  out [B, Hq, M, 64] binary16
 *   k_codes  [B, Hkv, T_ld, Wk], k_norms [B, Hkv, T_ld]: token t of (b, g) is
 *            record (b Hkv + g) T_ld + t; the first T of each row are read.
 *   v_codes / v_norms likewise.
 *   1 <= M <= 8, M <= T <= T_ld < 2^31, (Hq / Hkv) * M <= 8; workspace of at
 *   least fq_attend_workspace_size(cb_k, B, Hq * M, Hkv, T) bytes.  Other
 *   requirements and errors as fq_attend_decode.
 */
fq_status fq_attend_queries(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                            const uint32_t* k_codes, const uint16_t* k_norms,
                            const uint32_t* v_codes, const uint16_t* v_norms, int B, int Hq,
                            int Hkv, int64_t T, int64_t T_ld, int M, float scale, void* workspace,
                            size_t workspace_bytes, uint16_t* out, void* stream);

/*
 * One decode step with encode-on-append [FQ 1, 2.3, 5]: encode the M new keys
 * and values of every (batch, KV head) into cache slots pos .. pos + M - 1
 * (the float64 nearest codewords and binary16 norms fq_encode computes, with
 * its near-tie allowance), then attend as fq_attend_queries over the
 * T = pos + M tokens now in the cache.  Kernels queued on `stream`: the
 * attention workgroups holding the new tokens encode them before reading
 * their tiles (codebooks whose tables hold binary16 values, as the shipped
 * ones do), otherwise an append launch precedes the attention; no host
 * synchronisation and no intermediate buffers.  Keys and values share the
 * rotation of cb_k, which must equal cb_v's (the one shared rotation).
 *
 *   k_new, v_new  [B, Hkv, M, 64] binary16
 *   caches        as fq_attend_queries, capacity T_ld tokens; slots >= pos + M
 *                 are neither read nor written
 *   0 <= pos <= T_ld - M; other arguments as fq_attend_queries.
 */
fq_status fq_decode_step(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                         const uint16_t* k_new, const uint16_t* v_new, uint32_t* k_codes,
                         uint16_t* k_norms, uint32_t* v_codes, uint16_t* v_norms, int B, int Hq,
                         int Hkv, int64_t T_ld, int64_t pos, int M, float scale, void* workspace,
                         size_t workspace_bytes, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
