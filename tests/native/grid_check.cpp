// Host-only check of the encoder's candidate-list grids (test program).
//
// The block search of the encode kernel looks for the nearest codeword of a
// block only among the codewords listed for the block's grid cell (FibQuant
// technical summary, section 2.3: every block goes to its nearest codeword;
// Block Sphere VQ notes, key design 2: a cell of the block space maps to a
// short list of codewords).  That is exact only if every list holds the
// nearest codeword of every point that can land in its cell.  This program
// builds the grids exactly as the library does (grid_plan + build_grid from
// fq_grid.cpp, the artifact parsed by fq_artifact.cpp) and checks, against a
// brute-force float64 search over all N codewords:
//
//   * blocks of random unit vectors (the canonical spherical source: the
//     first coordinates of a normalised N(0, I_64) vector),
//   * points on and next to cell boundaries (jitter 0, 1e-7, 1e-6, 1e-5),
//   * uniform points of the whole grid box,
//
// each looked up twice, from its float32 rounding and from a float32 value
// moved by up to 1e-5 per coordinate (ten times the encoder's bound on its
// rotation error), with the encoder's own float32 cell arithmetic
// (grid_pos / grid_pos_inside from fq_host.h).  A cell without a list is fine
// (the encoder then scans the whole codebook); a listed cell that misses the
// nearest codeword is a failure.  It also checks the record layout and, when
// asked, feeds corrupted artifacts to the parser (the sanitizer build).
// --drop-last removes the last candidate of every list of two or more before
// the check, to show that the check detects incomplete lists.
//
// Usage: grid_check <points per grid> <artifact>... [--fuzz] [--drop-last]
// Prints one line per grid; exit status 0 when no check failed.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "fq_host.h"

namespace {

// splitmix64: a counter-based generator, one stream per (seed, index)
uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(mix64(seed)) {}
  uint64_t next() { return mix64(s++); }
  double uniform() { return (next() >> 11) * 0x1p-53; }   // [0, 1)
  double normal() {                                        // Box-Muller
    double u1 = uniform();
    while (u1 <= 0.0) u1 = uniform();
    return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * uniform());
  }
};

std::vector<unsigned char> read_file(const char* path) {
  std::vector<unsigned char> b;
  FILE* f = fopen(path, "rb");
  if (!f) return b;
  unsigned char buf[65536];
  size_t r;
  while ((r = fread(buf, 1, sizeof buf, f)) > 0) b.insert(b.end(), buf, buf + r);
  fclose(f);
  return b;
}

// brute-force nearest codeword of a point over the first `dims` coordinates
int nearest(const double* z, const std::vector<float>& C, int N, int k, int dims) {
  int best = 0;
  double bd = INFINITY;
  for (int n = 0; n < N; ++n) {
    double s = 0.0;
    for (int t = 0; t < dims; ++t) {
      const double df = z[t] - (double)C[(size_t)n * k + t];
      s += df * df;
    }
    if (s < bd) {
      bd = s;
      best = n;
    }
  }
  return best;
}

struct Stats {
  long points = 0, lookups = 0, listed = 0, scanned = 0, misses = 0;
  double list_sum = 0.0;
};

// record layout: count (or overflow), increasing indices < N, pads == N
long check_records(const fq::GridTable& g, int N) {
  long bad = 0;
  const size_t cells = g.rec.size() / g.re;
  for (size_t c = 0; c < cells; ++c) {
    const uint16_t* r = g.rec.data() + c * g.re;
    if (r[0] == fq::GRID_OVERFLOW) continue;
    const int cnt = r[0];
    if (cnt < 1 || cnt > g.re - 1) {
      ++bad;
      continue;
    }
    for (int e = 1; e <= cnt; ++e)
      if (r[e] >= N || (e > 1 && r[e] <= r[e - 1])) ++bad;
    for (int e = cnt + 1; e < g.re; ++e)
      if (r[e] != N) ++bad;
  }
  return bad;
}

// one grid: `npts` source blocks plus a quarter as many boundary and uniform points
Stats check_grid(const fq::GridTable& g, const std::vector<float>& C, int N, int k, long npts,
                 uint64_t seed) {
  const int dims = g.dims, G = g.G;
  const float scale = fq::grid_scale(G);
  const double h = 2.0 * fq::GRID_R / G;
  const long n_src = npts, n_edge = npts / 4, n_uni = npts / 4, total = n_src + n_edge + n_uni;
  const double jit[4] = {0.0, 1e-7, 1e-6, 1e-5};
  long lookups = 0, listed = 0, scanned = 0, misses = 0;
  double list_sum = 0.0;
#pragma omp parallel for schedule(dynamic, 4096) reduction(+ : lookups, listed, scanned, misses, list_sum)
  for (long p = 0; p < total; ++p) {
    Rng rng(seed * 0x100000001B3ull + (uint64_t)p);
    double z[4] = {0, 0, 0, 0};
    if (p < n_src) {
      double g64[64], ss = 0.0;
      for (int i = 0; i < 64; ++i) {
        g64[i] = rng.normal();
        ss += g64[i] * g64[i];
      }
      for (int t = 0; t < dims; ++t) z[t] = g64[t] / sqrt(ss);
    } else if (p < n_src + n_edge) {
      for (int t = 0; t < dims; ++t) {
        const int cell = (int)(rng.uniform() * G);
        const double lo = -fq::GRID_R + cell * h;
        if (rng.uniform() < 0.5) {
          const double side = rng.uniform() < 0.5 ? lo : lo + h;
          const double dj = jit[(int)(rng.uniform() * 4)] * (rng.uniform() < 0.5 ? -1.0 : 1.0);
          z[t] = side + dj;
        } else {
          z[t] = lo + rng.uniform() * h;
        }
      }
    } else {
      for (int t = 0; t < dims; ++t) z[t] = -fq::GRID_R + 2.0 * fq::GRID_R * rng.uniform();
    }
    const int want = nearest(z, C, N, k, dims);
    for (int view = 0; view < 2; ++view) {
      float zf[4];
      for (int t = 0; t < dims; ++t)
        zf[t] = (float)(view == 0 ? z[t] : z[t] + 1e-5 * (2.0 * rng.uniform() - 1.0));
      bool inside = true;
      int cell = 0, mul = 1;
      for (int t = 0; t < dims; ++t) {
        const float u = fq::grid_pos(zf[t], scale);
        const bool in = fq::grid_pos_inside(u, G);
        inside = inside && in;
        if (in) cell += (int)u * mul;
        mul *= G;
      }
      ++lookups;
      const uint16_t* r = g.rec.data() + (size_t)cell * g.re;
      if (!inside || r[0] == fq::GRID_OVERFLOW) {
        ++scanned;
        continue;
      }
      ++listed;
      list_sum += r[0];
      bool found = false;
      for (int e = 1; e <= r[0]; ++e) found = found || r[e] == want;
      if (!found) {
        ++misses;
#pragma omp critical
        if (misses <= 5) fprintf(stderr, "  miss: point %ld (%.9g %.9g %.9g %.9g) view %d cell %d nearest %d\n", p,
                z[0], z[1], z[2], z[3], view, cell, want);
      }
    }
  }
  Stats s;
  s.points = total;
  s.lookups = lookups;
  s.listed = listed;
  s.scanned = scanned;
  s.misses = misses;
  s.list_sum = list_sum;
  return s;
}

// corrupted artifacts: every outcome must be a status, never a crash or a read
// outside the blob (the sanitizer build checks the latter)
long fuzz_parser(const std::vector<unsigned char>& blob, uint64_t seed) {
  long bad = 0;
  fq::ArtifactHeader h;
  auto ok_status = [](fq_status s) {
    return s == FQ_OK || s == FQ_ERR_BAD_ARTIFACT || s == FQ_ERR_UNSUPPORTED;
  };
  // truncations (the heap copy has exactly n bytes, so an overread is caught)
  if (fq::parse_artifact(blob.data(), 0, &h, nullptr, nullptr) != FQ_ERR_BAD_ARTIFACT) ++bad;
  for (size_t n = 1; n < blob.size(); n += (n < 300 ? 1 : 997)) {
    std::vector<unsigned char> b(blob.begin(), blob.begin() + n);
    if (fq::parse_artifact(b.data(), n, &h, nullptr, nullptr) != FQ_ERR_BAD_ARTIFACT) ++bad;
  }
  // one flipped byte, then the same with the trailing hash recomputed
  Rng rng(seed);
  for (int it = 0; it < 400; ++it) {
    std::vector<unsigned char> b(blob);
    const size_t pos = it < 128 ? (size_t)it : (size_t)(rng.uniform() * (b.size() - 8));
    b[pos] ^= (unsigned char)(1 + (rng.next() % 255));
    if (fq::parse_artifact(b.data(), b.size(), &h, nullptr, nullptr) != FQ_ERR_BAD_ARTIFACT)
      ++bad;
    const uint64_t hh = fq::fnv1a64(b.data(), b.size() - 8);
    memcpy(b.data() + b.size() - 8, &hh, 8);
    const unsigned char *pi = nullptr, *cw = nullptr;
    if (!ok_status(fq::parse_artifact(b.data(), b.size(), &h, &pi, &cw))) ++bad;
  }
  // random bytes of random lengths
  for (int it = 0; it < 200; ++it) {
    std::vector<unsigned char> b(1 + (size_t)(rng.uniform() * 5000));
    for (auto& c : b) c = (unsigned char)rng.next();
    if (b.size() >= 4) memcpy(b.data(), "FQCB", 4);
    if (!ok_status(fq::parse_artifact(b.data(), b.size(), &h, nullptr, nullptr))) ++bad;
  }
  if (fq::parse_artifact(nullptr, 100, &h, nullptr, nullptr) != FQ_ERR_INVALID_ARG) ++bad;
  return bad;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s <points per grid> <artifact>... [--fuzz]\n", argv[0]);
    return 2;
  }
  const long npts = atol(argv[1]);
  bool fuzz = false, drop = false;
  int failures = 0;
  for (int a = 2; a < argc; ++a) {
    if (strcmp(argv[a], "--fuzz") == 0) fuzz = true;
    if (strcmp(argv[a], "--drop-last") == 0) drop = true;
  }
  for (int a = 2; a < argc; ++a) {
    if (argv[a][0] == '-' && argv[a][1] == '-') continue;
    const std::vector<unsigned char> blob = read_file(argv[a]);
    fq::ArtifactHeader h;
    const unsigned char *pp = nullptr, *cp = nullptr;
    const fq_status st = fq::parse_artifact(blob.data(), blob.size(), &h, &pp, &cp);
    if (st != FQ_OK) {
      printf("%s: parse status %d\n", argv[a], (int)st);
      ++failures;
      continue;
    }
    const int N = (int)h.N, k = (int)h.k;
    std::vector<float> C((size_t)N * k);
    memcpy(C.data(), cp, 4ull * N * k);
    if (fuzz) {
      const long fb = fuzz_parser(blob, 1000 + k * 10000 + N);
      printf("k%dN%d parser-fuzz bad=%ld\n", k, N, fb);
      if (fb) ++failures;
    }
    int G = 0, G1 = 0;
    if (!fq::grid_plan(k, N, (int)h.last, &G, &G1)) continue;
    for (int which = 0; which < 2; ++which) {
      const int dims = which == 0 ? k : 1, g = which == 0 ? G : G1;
      if (g <= 0) continue;
      fq::GridTable grid;
      fq::build_grid(C.data(), N, k, dims, g, fq::GRID_R, fq::grid_record_entries(k), (uint16_t)N,
                     &grid);
      const long rb = check_records(grid, N);
      if (drop)
        for (size_t c = 0; c < grid.rec.size() / grid.re; ++c) {
          uint16_t* r = grid.rec.data() + c * grid.re;
          if (r[0] != fq::GRID_OVERFLOW && r[0] >= 2) r[r[0]--] = (uint16_t)N;
        }
      const Stats s = check_grid(grid, C, N, k, npts, 7 + which + 2 * (uint64_t)N + 8192ull * k);
      printf("k%dN%d dims=%d G=%d points=%ld lookups=%ld listed=%ld scanned=%ld misses=%ld "
             "mean_list=%.3f max_list=%d overflow_cells=%d bad_records=%ld\n",
             k, N, dims, g, s.points, s.lookups, s.listed, s.scanned, s.misses,
             s.listed ? s.list_sum / s.listed : 0.0, grid.max_len, grid.overflow, rb);
      if (s.misses || rb) ++failures;
    }
  }
  fflush(stdout);
  return failures ? 1 : 0;
}
