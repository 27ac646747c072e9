// Host-side declarations of the library that need no HIP headers: variant
// table, artifact parsing, and the candidate-list grids of the block search.
// The grid cell arithmetic is written once, as functions the HIP compiler
// builds for both host and device, so the encoder and the host build of the
// grid checks evaluate the very same float32 expressions.
#pragma once

#if defined(__HIP__)
#define FQ_HD __host__ __device__
#else
#define FQ_HD
#endif

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "fq.h"

namespace fq {

constexpr int D = 64;             // vector length handled by the kernels
constexpr int MAX_N = 16384;      // largest codebook (k = 64)
constexpr int MAX_WORDS = 12;     // record words for k >= 2, N <= 4096: ceil(32*12/32)
constexpr int MAX_QUERIES = 8;    // queries per head in one attention call

// (k, index bits) pairs the kernels are built for: the configurations' rates
// (k=2: N 16 / 64 / 256, k=3: N 512 / 4096, k=4: N 4 / 256, k=8: N 16 / 256)
// plus the fractional k=2 rates 2.5 and 3.5 (N 32 / 128).  X(k, bits).
#define FQ_VARIANTS(X) \
  X(2, 4) X(2, 5) X(2, 6) X(2, 7) X(2, 8) X(3, 9) X(3, 12) X(4, 2) X(4, 8) X(8, 4) X(8, 8)

// Large blocks (k = d/2 and k = d with N = 4096, and k = d with N = 16384):
// the table exceeds LDS, so they have their own encode kernel
// (fq_encode_large.hip) and a decode that gathers codewords from the
// L2-resident table.
#define FQ_VARIANTS_LARGE(X) X(32, 12) X(64, 12) X(64, 14)

inline bool variant_supported(int k, int bits) {
#define FQ_IS(KK, BB) if (k == KK && bits == BB) return true;
  FQ_VARIANTS(FQ_IS)
  FQ_VARIANTS_LARGE(FQ_IS)
#undef FQ_IS
  return false;
}

constexpr bool large_block(int k) { return k >= 32; }

// ------------------------------------------------------------------ artifact
// The codebook artifact: a 256-byte header (this struct, then zero bytes),
// Pi as d x d float64 (row-major, z = Pi u), the codebook as N x k float32,
// and an FNV-1a 64 hash of everything before it.
struct ArtifactHeader {
  char magic[4];
  uint32_t version, header_bytes, d, k, N, nb, bits, W, last, restarts, max_iter, iters, best;
  uint64_t seed_rot, samples;
  double tol, d_train, d_test, rate_nom, rate_act, law_a, law_b;
};
static_assert(sizeof(ArtifactHeader) == 128, "header layout");
constexpr uint32_t ARTIFACT_HEADER_BYTES = 256;
constexpr uint32_t ARTIFACT_VERSION = 1;

uint64_t fnv1a64(const unsigned char* p, size_t n);

// Parse and validate a blob (checks listed at fq_artifact_check in fq.h).  On
// FQ_OK or FQ_ERR_UNSUPPORTED fills *hdr; on FQ_OK also points *pi and *cw at
// the payload inside the blob (possibly unaligned: read through memcpy).
fq_status parse_artifact(const void* blob, size_t nbytes, ArtifactHeader* hdr,
                         const unsigned char** pi, const unsigned char** cw);

// --------------------------------------------------- candidate-list grids
// uint16 entries per cell record: count + up to 7 (k = 2) or 15 (k = 3) or
// 31 (k = 4) candidates
constexpr int grid_record_entries(int k) { return k == 2 ? 8 : (k == 3 ? 16 : 32); }
constexpr uint16_t GRID_OVERFLOW = 0xFFFF;
constexpr double GRID_MARGIN = 1e-4;     // box widening: rotation error + float32 cell arithmetic
constexpr double GRID_R = 0.5;           // the grid covers [-R, R]^dims
constexpr double GRID_REACH = 0.3;       // distance searched when building a cell's list

struct GridTable {
  int dims = 0, G = 0, re = 0;
  double R = 0.0;
  int max_len = 0, overflow = 0;
  std::vector<uint16_t> rec;             // [G^dims][re]
};

// Candidate lists of the first `dims` coordinates of the N x k codebook `cw`
// over a G^dims grid on [-R, R]^dims, records of `re` entries, unused slots
// set to `pad`.
void build_grid(const float* cw, int N, int k, int dims, int G, double R, int re, uint16_t pad,
                GridTable* out);

// Which grids a codebook gets: *G cells per dimension of the k-dimensional
// block grid, *G1 cells of the one-coordinate last-block grid (0: none).
// Returns false when the block search scans the whole codebook instead.
bool grid_plan(int k, int N, int last, int* G, int* G1);

// Cells per unit length of a grid with G cells per dimension, in float32.
inline float grid_scale(int G) { return (float)(G / (2.0 * GRID_R)); }

// Position of a float32 coordinate along one axis of a grid with G cells per
// dimension (scale = grid_scale(G)), in cells from the grid's lower edge:
// v * scale + R * scale with one rounding (a fused multiply-add).  The
// coordinate lies inside the grid when the position is in [0, G) (false for
// NaN), and then its cell is the position truncated to an integer.  The
// encoder's cell of a block is sum_t cell(z_t) G^t, taken only when every
// coordinate is inside.  Host and device evaluate the same correctly rounded
// operations.
FQ_HD inline float grid_pos(float v, float scale) {
  return __builtin_fmaf(v, scale, (float)GRID_R * scale);
}
FQ_HD inline bool grid_pos_inside(float u, int G) { return u >= 0.f && u < (float)G; }

}  // namespace fq
