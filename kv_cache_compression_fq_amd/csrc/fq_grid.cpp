// Exact candidate lists for the block search of low-dimensional codebooks.
//
// The encoder's block search is an exact nearest-codeword problem (FibQuant
// technical summary, section 2.3: each block goes to its nearest codeword).
// For block sizes k = 2, 3 and 4 the blocks live in a low-dimensional ball, so
// the search can be cut down without changing a single index: cover [-R, R]^dims
// with a uniform grid and give every cell the list of codewords that can be
// nearest to *some* point of the cell (widened by a margin that covers the
// encoder's rotation error and float32 cell arithmetic).  A point's nearest
// codeword is then always in its cell's list.
//
// A codeword i is kept for box B when both hold:
//   1. min_{z in B} |z - c_i|^2 <= min_j max_{z in B} |z - c_j|^2, and
//   2. no codeword j beats i on all of B, i.e. the largest value over B of
//      |z - c_j|^2 - |z - c_i|^2 = 2 <z, c_i - c_j> + |c_j|^2 - |c_i|^2 (linear
//      in z, so largest at a corner) is not negative.
// Each test only removes codewords that are nearest nowhere in B, so the list
// is a superset of the true candidates.  Both are evaluated in float64 with a
// relative slack in the keeping direction.
//
// Records: `re` uint16 per cell, entry 0 the count (GRID_OVERFLOW when the
// list does not fit or the cell is far outside the codebook), then the indices
// in increasing order; unused entries hold `pad` (the encoder's sentinel row).
#include <math.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "fq_host.h"

namespace fq {

// Grid sizes per codebook: cells of about a quarter (k = 2) or a third
// (k = 3) of the codeword spacing keep lists short; the one-coordinate last
// block of k = 3 gets 4N cells; k = 4 gets 14^4 cells, which holds the lists
// of a 256-codeword table within 31 entries.  Other codebooks scan.
bool grid_plan(int k, int N, int last, int* G, int* G1) {
  *G = 0;
  *G1 = 0;
  if (k == 2)
    *G = N <= 64 ? 32 : 64;
  else if (k == 3)
    *G = N <= 512 ? 32 : 64;
  else if (k == 4 && N >= 64)
    *G = 14;
  else
    return false;
  if (last < k) *G1 = 4 * N;
  return true;
}

void build_grid(const float* cw, int N, int k, int dims, int G, double R, int re, uint16_t pad,
                GridTable* out) {
  const double h = 2.0 * R / G, mu = GRID_MARGIN;
  int ncell = 1;
  for (int t = 0; t < dims; ++t) ncell *= G;
  out->dims = dims;
  out->G = G;
  out->re = re;
  out->R = R;
  out->max_len = 0;
  out->overflow = 0;
  out->rec.assign((size_t)ncell * re, pad);

  // codeword coordinates (first `dims`), norms, bucket = clamped cell
  std::vector<double> P((size_t)N * dims), cc(N);
  std::vector<int> bucket(N), start(ncell + 1, 0), members(N);
  for (int i = 0; i < N; ++i) {
    double s = 0.0;
    int b = 0, mul = 1;
    for (int t = 0; t < dims; ++t) {
      const double v = cw[(size_t)i * k + t];
      P[(size_t)i * dims + t] = v;
      s += v * v;
      int u = (int)floor((v + R) / h);
      u = u < 0 ? 0 : (u >= G ? G - 1 : u);
      b += u * mul;
      mul *= G;
    }
    cc[i] = s;
    bucket[i] = b;
    ++start[b + 1];
  }
  for (int b = 0; b < ncell; ++b) start[b + 1] += start[b];
  {
    std::vector<int> fill(start.begin(), start.end() - 1);
    for (int i = 0; i < N; ++i) members[fill[bucket[i]]++] = i;
  }

  // search radius in cells: a fixed distance, tighter in three dimensions
  // where a ring holds many buckets
  const int max_rings = dims < 3 ? (int)ceil(GRID_REACH / h) : std::max(6, (int)ceil(0.5 * GRID_REACH / h));
  std::vector<int> cand, kept;
  std::vector<std::pair<double, int>> order;
  int u[4] = {0, 0, 0, 0};
  double lo[4], hi[4];
  auto dmax = [&](int j) {
    double s = 0.0;
    for (int t = 0; t < dims; ++t) {
      const double a = lo[t] - P[(size_t)j * dims + t], b = hi[t] - P[(size_t)j * dims + t];
      s += fmax(a * a, b * b);
    }
    return s;
  };
  auto dmin = [&](int j) {
    double s = 0.0;
    for (int t = 0; t < dims; ++t) {
      const double v = P[(size_t)j * dims + t];
      const double g = v < lo[t] ? lo[t] - v : (v > hi[t] ? v - hi[t] : 0.0);
      s += g * g;
    }
    return s;
  };
  // visit the codewords of the buckets at Chebyshev distance exactly r from
  // cell u: the shell of the cube [u - r, u + r]^dims, one face layer at a time
  auto ring = [&](int r, auto&& fn) {
    auto bucket_row = [&](int a0lo, int a0hi, int a0step, int a1, int a2) {
      for (int a0 = a0lo; a0 <= a0hi; a0 += a0step) {
        if (a0 < 0 || a0 >= G) continue;
        const int b = a0 + G * (a1 + G * a2);
        for (int m = start[b]; m < start[b + 1]; ++m) fn(members[m]);
      }
    };
    const int r1 = dims > 1 ? r : 0, r2 = dims > 2 ? r : 0;
    for (int a2 = u[2] - r2; a2 <= u[2] + r2; ++a2) {
      if (a2 < 0 || a2 >= G) continue;
      const bool e2 = dims > 2 && (a2 == u[2] - r || a2 == u[2] + r);
      for (int a1 = u[1] - r1; a1 <= u[1] + r1; ++a1) {
        if (a1 < 0 || a1 >= G) continue;
        const bool e1 = dims > 1 && (a1 == u[1] - r || a1 == u[1] + r);
        if (e1 || e2 || r == 0)
          bucket_row(u[0] - r, u[0] + r, 1, a1, a2);
        else
          bucket_row(u[0] - r, u[0] + r, 2 * r, a1, a2);
      }
    }
  };

  // keep codewords of the candidate set `cand` that no other codeword beats on
  // the whole box; write the cell's record
  auto finish_cell = [&](uint16_t* rec) {
    // 2. drop codewords beaten on the whole box by another one; trying the
    //    candidates with the smallest worst-case distance first ends most
    //    checks after a few comparisons
    order.clear();
    for (int j : cand) order.push_back({dmax(j), j});
    std::sort(order.begin(), order.end());
    kept.clear();
    for (int i : cand) {
      bool beaten = false;
      for (const auto& oj : order) {
        const int j = oj.second;
        if (j == i) continue;
        double f = cc[j] - cc[i];
        for (int t = 0; t < dims; ++t) {
          const double g = 2.0 * (P[(size_t)i * dims + t] - P[(size_t)j * dims + t]);
          f += fmax(g * lo[t], g * hi[t]);
        }
        if (f < -1e-12 * (1.0 + cc[i] + cc[j])) {
          beaten = true;
          break;
        }
      }
      if (!beaten) kept.push_back(i);
    }
    std::sort(kept.begin(), kept.end());
    out->max_len = std::max(out->max_len, (int)kept.size());
    if ((int)kept.size() > re - 1) {
      rec[0] = GRID_OVERFLOW;
      ++out->overflow;
    } else {
      rec[0] = (uint16_t)kept.size();
      for (size_t m = 0; m < kept.size(); ++m) rec[1 + m] = (uint16_t)kept[m];
    }
  };

  for (int cell = 0; cell < ncell; ++cell) {
    int rem = cell;
    for (int t = 0; t < dims; ++t) {
      u[t] = rem % G;
      rem /= G;
      lo[t] = -R + u[t] * h - mu;
      hi[t] = -R + (u[t] + 1) * h + mu;
    }
    if (dims >= 4) {
      // four dimensions: test every codeword (G^4 cells of a few hundred
      // codewords each take well under a second)
      uint16_t* rec = out->rec.data() + (size_t)cell * re;
      double best = INFINITY;
      for (int j = 0; j < N; ++j) best = fmin(best, dmax(j));
      const double lim = best * (1.0 + 1e-9) + 1e-18;
      cand.clear();
      for (int j = 0; j < N; ++j)
        if (dmin(j) <= lim) cand.push_back(j);
      finish_cell(rec);
      continue;
    }
    // 1. smallest worst-case distance over the box; codewords in rings beyond r
    //    are at least r h - mu away from the box
    //    Cells that would need rings beyond max_rings lie far outside the
    //    codebook, where blocks almost never fall: they get no list and the
    //    encoder searches the whole codebook there.
    uint16_t* rec = out->rec.data() + (size_t)cell * re;
    double best = INFINITY;
    bool done = false;
    for (int r = 0; r <= max_rings; ++r) {
      ring(r, [&](int j) { best = fmin(best, dmax(j)); });
      const double lb = r * h - mu;
      if (lb > 0.0 && best <= lb * lb) {
        done = true;
        break;
      }
    }
    const double lim = best * (1.0 + 1e-9) + 1e-18;
    cand.clear();
    for (int r = 0; done; ++r) {
      const double lb = (r - 1) * h - mu;
      if (r >= 1 && lb > 0.0 && lb * lb > lim) break;
      if (r > max_rings) {
        done = false;
        break;
      }
      ring(r, [&](int j) {
        if (dmin(j) <= lim) cand.push_back(j);
      });
    }
    if (!done) {
      rec[0] = GRID_OVERFLOW;
      ++out->overflow;
      continue;
    }
    finish_cell(rec);
  }
}

}  // namespace fq
