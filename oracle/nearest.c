/*
 * Brute-force nearest codewords in float64 -- oracle, TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and bench.py's cpu_baseline leg load this
 * library; the product path never does, and it shares no code with the HIP
 * kernels.  It computes exactly what oracle/codec.py `encode` and
 * `accept_indices` compute, in plain compiled loops, so that whole caches
 * (millions of vectors) can be checked in seconds:
 *
 * FibQuant technical summary, section 2.3 (encoding): the norm
 * nu = |x|_2; the unit vector x / nu is rotated by the shared rotation,
 * z = Pi (x / nu); z is cut into blocks of k coordinates, block j covering
 * coordinates [j k, min((j + 1) k, d)); each block goes to the codeword of
 * the shared codebook nearest to it.  Readings (the same as codec.py):
 *   - distance D_j(n) = sum over the block's real coordinates t of
 *     (z_{jk+t} - C[n][t])^2, so a partial last block compares only its
 *     real coordinates with the first coordinates of each codeword;
 *   - ties go to the lowest index;
 *   - nu = 0: every index is 0;
 *   - near-tie acceptance: an index i is accepted when
 *     D_j(i) - min_n D_j(n) <= window * D_j(i).
 * No pruning, blocking or reordering: every codeword of every block is
 * evaluated.  Vectors are independent, so they are split over OpenMP threads.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* Threads the searches below use (OpenMP); n < 1 leaves the setting alone. */
int fqo_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
}

/* z = Pi u with u = x / nu, of one vector (u is scratch of d doubles); returns nu. */
static double rotate_unit(const double* x, int d, const double* Pi, double* u, double* z) {
  double ss = 0.0;
  for (int j = 0; j < d; ++j) ss += x[j] * x[j];
  const double nu = sqrt(ss);
  for (int j = 0; j < d; ++j) u[j] = nu > 0.0 ? x[j] / nu : 0.0;
  for (int i = 0; i < d; ++i) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += Pi[(int64_t)i * d + j] * u[j];
    z[i] = s;
  }
  return nu;
}

/* D_j(n) of block [lo, lo + r) of z against codeword n. */
static double block_distance(const double* z, int lo, int r, const float* C, int k, int n) {
  double s = 0.0;
  for (int t = 0; t < r; ++t) {
    const double df = z[lo + t] - (double)C[(int64_t)n * k + t];
    s += df * df;
  }
  return s;
}

/* Nearest codeword of one block: index of the smallest distance (lowest index
 * on ties) and that distance. */
static int block_argmin(const double* z, int lo, int r, const float* C, int N, int k,
                        double* dmin) {
  int best = 0;
  double bd = INFINITY;
  for (int n = 0; n < N; ++n) {
    const double dd = block_distance(z, lo, r, C, k, n);
    if (dd < bd) {
      bd = dd;
      best = n;
    }
  }
  *dmin = bd;
  return best;
}

/*
 * Indices of n vectors x [n][d] (float64): idx [n][nb], nb = ceil(d / k).
 * Returns 0, or -1 on a bad argument.
 */
int fqo_nearest(const double* x, int64_t n, int d, const double* Pi, const float* C, int N, int k,
                int64_t* idx) {
  if (!x || !Pi || !C || !idx || n < 0 || d < 1 || d > 4096 || k < 1 || k > d || N < 1)
    return -1;
  const int nb = (d + k - 1) / k;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * 2 * (size_t)d);
    double* u = z + d;
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
      const double nu = rotate_unit(x + v * d, d, Pi, u, z);
      for (int j = 0; j < nb; ++j) {
        const int lo = j * k, r = (lo + k <= d) ? k : d - lo;
        double dm;
        idx[v * nb + j] = nu > 0.0 ? block_argmin(z, lo, r, C, N, k, &dm) : 0;
      }
    }
    free(z);
  }
  return 0;
}

/*
 * Check candidate indices got [n][nb] under the near-tie window.
 * counts[0] = indices equal to the oracle's (or 0 for a zero vector),
 * counts[1] = other indices inside the window, counts[2] = the rest;
 * *first_bad = the first vector holding an index of the third kind, or -1.
 * Returns 0, or -1 on a bad argument.
 */
int fqo_accept(const double* x, int64_t n, int d, const double* Pi, const float* C, int N, int k,
               const int64_t* got, double window, int64_t* counts, int64_t* first_bad) {
  if (!x || !Pi || !C || !got || !counts || !first_bad || n < 0 || d < 1 || d > 4096 || k < 1 ||
      k > d || N < 1)
    return -1;
  const int nb = (d + k - 1) / k;
  int64_t ex = 0, win = 0, bad = 0, fb = n;
#pragma omp parallel reduction(+ : ex, win, bad) reduction(min : fb)
  {
    double* z = (double*)malloc(sizeof(double) * 2 * (size_t)d);
    double* u = z + d;
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
      const double nu = rotate_unit(x + v * d, d, Pi, u, z);
      for (int j = 0; j < nb; ++j) {
        const int64_t g = got[v * nb + j];
        if (nu == 0.0) {
          if (g == 0) {
            ++ex;
          } else {
            ++bad;
            if (v < fb) fb = v;
          }
          continue;
        }
        const int lo = j * k, r = (lo + k <= d) ? k : d - lo;
        double dmin;
        const int best = block_argmin(z, lo, r, C, N, k, &dmin);
        if (g == best) {
          ++ex;
        } else if (g >= 0 && g < N) {
          const double dg = block_distance(z, lo, r, C, k, (int)g);
          if (dg - dmin <= window * dg) {
            ++win;
          } else {
            ++bad;
            if (v < fb) fb = v;
          }
        } else {
          ++bad;
          if (v < fb) fb = v;
        }
      }
    }
    free(z);
  }
  counts[0] = ex;
  counts[1] = win;
  counts[2] = bad;
  *first_bad = fb < n ? fb : -1;
  return 0;
}
