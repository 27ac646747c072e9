// Parsing and validation of the codebook artifact (host only).
//
// The artifact carries the codec's two shared objects: the rotation Pi, one
// Haar rotation used for every vector (FibQuant technical summary, sections 1
// and 2.3), and the codebook, one offline table for every layer and head
// (section 2.1).  Nothing here touches a device.
#include <math.h>
#include <string.h>

#include <vector>

#include "fq_host.h"

namespace fq {

// FNV-1a, 64-bit: offset basis and prime of the published definition.
uint64_t fnv1a64(const unsigned char* p, size_t n) {
  uint64_t h = 0xCBF29CE484222325ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

static bool is_pow2(uint32_t v) { return v && !(v & (v - 1)); }

fq_status parse_artifact(const void* blob, size_t nbytes, ArtifactHeader* hdr,
                         const unsigned char** pi, const unsigned char** cw) {
  if (!blob || !hdr) return FQ_ERR_INVALID_ARG;
  if (nbytes < ARTIFACT_HEADER_BYTES + 8) return FQ_ERR_BAD_ARTIFACT;
  const unsigned char* b = static_cast<const unsigned char*>(blob);
  memcpy(hdr, b, sizeof(ArtifactHeader));
  if (memcmp(hdr->magic, "FQCB", 4) != 0 || hdr->version != ARTIFACT_VERSION ||
      hdr->header_bytes != ARTIFACT_HEADER_BYTES)
    return FQ_ERR_BAD_ARTIFACT;
  for (size_t i = sizeof(ArtifactHeader); i < ARTIFACT_HEADER_BYTES; ++i)
    if (b[i] != 0) return FQ_ERR_BAD_ARTIFACT;
  const uint32_t d = hdr->d, k = hdr->k, N = hdr->N;
  if (d < 1 || d > 4096 || k < 1 || k > d || !is_pow2(N) || N < 2 || N > (1u << 20))
    return FQ_ERR_BAD_ARTIFACT;
  const uint64_t want = ARTIFACT_HEADER_BYTES + 8ull * d * d + 4ull * N * k + 8;
  if (nbytes != want) return FQ_ERR_BAD_ARTIFACT;
  uint32_t bits = 0;
  while ((1u << bits) < N) ++bits;
  const uint32_t nb = (d + k - 1) / k;
  if (hdr->nb != nb || hdr->bits != bits || hdr->W != (nb * bits + 31) / 32 ||
      hdr->last != d - (nb - 1) * k)
    return FQ_ERR_BAD_ARTIFACT;
  uint64_t h;
  memcpy(&h, b + want - 8, 8);
  if (h != fnv1a64(b, want - 8)) return FQ_ERR_BAD_ARTIFACT;
  const unsigned char* pp = b + ARTIFACT_HEADER_BYTES;
  const unsigned char* cp = pp + 8ull * d * d;
  // the payload is not guaranteed aligned inside the caller's blob: read through memcpy
  std::vector<double> P((size_t)d * d);
  memcpy(P.data(), pp, 8ull * d * d);
  for (double v : P)
    if (!isfinite(v)) return FQ_ERR_BAD_ARTIFACT;
  for (uint64_t i = 0; i < (uint64_t)N * k; ++i) {
    float v;
    memcpy(&v, cp + 4 * i, 4);
    if (!isfinite(v)) return FQ_ERR_BAD_ARTIFACT;
  }
  // orthogonality of Pi
  double worst = 0;
  for (uint32_t i = 0; i < d; ++i)
    for (uint32_t j = i; j < d; ++j) {
      double s = 0;
      for (uint32_t r = 0; r < d; ++r) s += P[(size_t)r * d + i] * P[(size_t)r * d + j];
      worst = fmax(worst, fabs(s - (i == j ? 1.0 : 0.0)));
    }
  if (worst > 1e-9) return FQ_ERR_BAD_ARTIFACT;
  if (d != (uint32_t)D || N > (uint32_t)MAX_N || !variant_supported(k, bits))
    return FQ_ERR_UNSUPPORTED;
  if (pi) *pi = pp;
  if (cw) *cw = cp;
  return FQ_OK;
}

}  // namespace fq
