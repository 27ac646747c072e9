// Internal declarations shared by the library's own translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <vector>

#include "fq.h"
#include "fq_host.h"

namespace fq {

// Per-codebook device tables, all inside one allocation.
struct DeviceTables {
  double* pi64;      // [64][64] Pi, row-major (z = Pi u)
  double* pi64t;     // [64][64] Pi^T, row-major
  float* pi32;       // [64][64] Pi rounded to float32
  float* pi32t;      // [64][64] Pi^T rounded to float32
  float* enc;        // [N + 1][S] search table: -2 c_0 .. -2 c_{k-1}, |c|^2, zero pad; S =
                     // enc_stride; row N is a sentinel (zero codeword, infinite norm)
  _Float16* cb16hi;  // [N][k]   codewords rounded to binary16
  _Float16* cb16lo;  // [N][k]   (c - hi) * 2^11 rounded to binary16
  _Float16* pi16hi;  // [64][64] Pi rounded to binary16, row-major
  _Float16* pi16lo;  // [64][64] (Pi - hi) * 2^11 rounded to binary16
  _Float16* pifrag;  // Pi as v_mfma_f32_16x16x32_f16 B fragments (decode), see fq_api.hip
  _Float16* encfrag; // Pi hi / lo as v_mfma_f32_16x16x16_f16 A fragments (encode)
  uint16_t* grid;     // k = 2, 3: candidate records of the block grid (fq_grid.cpp)
  uint16_t* grid1;    // k = 3: candidate records of the one-coordinate last block
  _Float16* lfrag;    // k >= 32: codebook as v_mfma_f32_16x16x32_f16 A fragments,
                      // [tile][kc][lane][8] = C[16 tile + lane % 16][32 kc + 8 (lane / 16) + e]
  float* hnorm;       // k >= 32: -|c_n|^2 / 2 in float32
  _Float16* pair16;   // k = 2, N = 16, binary16-exact: [256][4] codeword pairs, entry
                      // i0 + 16 i1 = (c_i0, c_i1), so a record reads as k = 4, N = 256
};

}  // namespace fq

struct fq_codebook {
  int device;
  int d, k, N, nb, bits, W, last;
  int enc_stride;
  double rate_nominal, rate_actual, distortion;
  uint64_t hash;
  uint64_t pi_digest;   // FNV-1a 64 of Pi's float64 bytes: keys and values must share Pi
  float enc_ez16;   // encode: bound on |z~ - z| per coordinate, binary16 input
  float enc_ez32;   // the same for float32 input
  int grid_G;       // cells per dimension of the block grid (0: no grid, full scan)
  int grid1_G;      // cells of the last-block grid (k = 3)
  bool half_exact;  // every codeword coordinate is a binary16 number
  double cmax;      // largest codeword norm
  double hshift;    // constant added to every score of the matrix-core k = 8 search
  std::vector<uint16_t> grid_host, grid1_host;   // host copies of the candidate grids
  std::vector<double> pi;  // host copy of Pi
  std::vector<float> c;    // host copy of C
  void* dev_block;         // the single device allocation
  size_t dev_bytes;
  fq::DeviceTables t;
};

namespace fq {

// Launchers (return hipSuccess or the launch error).  Shapes are validated by
// the caller; pointers are device pointers.
// Where encoded row r is stored: record r (inner == 0), or record
// (r / inner) * stride + pos + r % inner (appending to caches of row stride
// `stride` records).
struct OutRows {
  int64_t inner = 0, stride = 0, pos = 0;
};
// A second input encoded by the same launch (same codebook, dtype, row stride
// and OutRows map), its rows following the first input's.
struct SecondInput {
  const void* x = nullptr;
  int64_t n = 0;
  uint32_t* codes = nullptr;
  uint16_t* norms = nullptr;
};
hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n,
                         int64_t ld, uint32_t* codes, uint16_t* norms, hipStream_t s,
                         OutRows rows = OutRows(), SecondInput second = SecondInput());
// Exact float64 encode of a few binary16 rows into cache slots (decode-step
// appends): rows < n1 from x1 into codes1 / norms1, the rest from x2 into
// codes2 / norms2, each mapped by `rows` (inner > 0).
hipError_t launch_append(const fq_codebook* cb, const uint16_t* x1, const uint16_t* x2,
                         int64_t n1, int64_t n, uint32_t* codes1, uint16_t* norms1,
                         uint32_t* codes2, uint16_t* norms2, OutRows rows, hipStream_t s);
hipError_t launch_encode_large(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n,
                               int64_t ld, uint32_t* codes, uint16_t* norms, hipStream_t s);
// k = 8, N = 256 on the matrix cores (binary16-exact codebooks; plain row-major
// records of two words)
bool encode_k8_applies(const fq_codebook* cb);
hipError_t launch_encode_k8(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n,
                            int64_t ld, uint32_t* codes, uint16_t* norms, hipStream_t s);
// `packed`: codes is a packed record stream (norms unused), see fq_pack_records
hipError_t launch_decode(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                         const int64_t* rows, int64_t n_records, int64_t n, void* y,
                         fq_dtype yt, int64_t ld, hipStream_t s, bool packed = false);
// word-aligned records + norms -> packed stream
hipError_t launch_pack(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                       int64_t n, uint32_t* packed, hipStream_t s);
int packed_record_bits(const fq_codebook* cb);
bool attend_supported(const fq_codebook* cb);  // the codebooks fit the kernel's LDS
size_t attend_workspace_bytes(const fq_codebook* cb_k, int B, int Hq, int Hkv, int64_t T);
// Tokens a decode step appends (the last M of the T attended tokens), to be
// encoded into the caches before they are read.
struct AppendIn {
  const uint16_t* k_new = nullptr;   // [B, Hkv, M, 64] binary16
  const uint16_t* v_new = nullptr;
  int M = 0;                         // 0: nothing to append
  const double* pi64t = nullptr;     // Pi^T, float64 (the key codebook's)
  uint32_t* kc = nullptr;            // the caches, written
  uint16_t* kn = nullptr;
  uint32_t* vc = nullptr;
  uint16_t* vn = nullptr;
};

// Attention over T tokens of caches whose per-(b, KV head) rows are Tld
// records apart; with Mq > 1 every Mq consecutive query heads are the Mq
// queries of one head, query m seeing tokens 0 .. T - Mq + m (causal).  With
// app.M > 0 the appended tokens are encoded first: inside the attention
// kernel, by the workgroups whose split holds them, where that kernel runs;
// else by launch_append ahead of it.
hipError_t launch_attend(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                         const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                         const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, int64_t Tld,
                         int Mq, float scale, void* ws, uint16_t* out, hipStream_t s,
                         const AppendIn& app = AppendIn());

// Workgroups of `kern` that fit on the current device at once (CUs x blocks per CU),
// or 0 if the runtime cannot say.
inline int64_t resident_blocks(const void* kern, int threads, size_t shm) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, shm) != hipSuccess)
    return 0;
  return (int64_t)cus * (per_cu < 1 ? 1 : per_cu);
}

// resident_blocks of one kernel per device, computed on first use.  Safe to
// share between host threads: each slot is an atomic, and two threads that
// race on an empty slot both store the same value.
struct DeviceCache {
  static constexpr int MAX_DEVICES = 64;
  std::atomic<int64_t> slot[MAX_DEVICES] = {};
  int64_t get(const void* kern, int threads, size_t shm) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
      return resident_blocks(kern, threads, shm);
    int64_t v = slot[dev].load(std::memory_order_relaxed);
    if (v == 0) {
      v = resident_blocks(kern, threads, shm);
      slot[dev].store(v, std::memory_order_relaxed);
    }
    return v;
  }
};

// Binary16 helpers usable on host and device.
__host__ __device__ inline uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

}  // namespace fq
