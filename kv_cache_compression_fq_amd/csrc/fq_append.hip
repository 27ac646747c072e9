// Encode-on-append for a decode step (FibQuant technical summary, sections
// 1, 2.3 and 5): the few new keys and values of a step are encoded straight
// into their cache slots.
//
// A step appends only B * Hkv * M vectors, so the bulk encoder's machinery
// (candidate grids, a float32 certificate, its float64 re-check) is mostly
// latency here.  This kernel takes one wave per vector and computes the
// definition directly in float64: the norm, z = Pi x / |x| (lane t forms
// z_t from coalesced rows of Pi^T, all loaded at once), then for every block
// the nearest codeword by float64 squared distance over all N codewords of
// the search table staged in LDS (the blocks side by side, a few lanes per
// block; ties to the lowest index), the fields packed LSB-first and the
// binary16 norm rounded once from the float64 norm.  It gives the bulk
// encoder's result (the same float64 argmin; see fq_encode for near-ties).
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int AP_WAVES = 4;

struct AppendArgs {
  const uint16_t* x1;   // [n1][64] binary16
  const uint16_t* x2;   // [n - n1][64] binary16 (may be null when n == n1)
  int64_t n1, n;
  uint32_t* codes1;
  uint16_t* norms1;
  uint32_t* codes2;
  uint16_t* norms2;
  OutRows rows;
  const double* pi64t;  // Pi^T, float64
  const float* enc;     // [N + 1][S]: -2 c, |c|^2
  int S, k, N, nb, bits, W;
};

__device__ inline double shfl_xor_d(double v, int m) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = __shfl_xor(p.x, m, 64);
  p.y = __shfl_xor(p.y, m, 64);
  return __builtin_bit_cast(double, p);
}

template <int K>
__global__ __launch_bounds__(AP_WAVES * 64) void append_kernel(AppendArgs a) {
  constexpr int S = ((K + 1) + 3) / 4 * 4;   // search-table row (floats)
  __shared__ double sX[AP_WAVES][D];
  __shared__ double sZ[AP_WAVES][D];
  __shared__ uint32_t sIdx[AP_WAVES][D];
  extern __shared__ __align__(16) float sEnc[];   // [N][S] search table
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * AP_WAVES + wave;
  const bool live = r < a.n;   // every wave reaches the barrier below
  const bool first = r < a.n1;
  const int64_t rr = !live ? 0 : (first ? r : r - a.n1);
  const uint16_t* xr = (first || !live ? a.x1 : a.x2) + rr * D;

  // all loads first: the table for the workgroup, x, the rows of Pi^T
  for (int i = threadIdx.x; i < a.N * S / 4; i += AP_WAVES * 64)
    reinterpret_cast<floatx4*>(sEnc)[i] = reinterpret_cast<const floatx4*>(a.enc)[i];
  const double xv = (double)f16_bits_to_f32(xr[lane]);
  double pv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) pv[i] = a.pi64t[i * D + lane];
  __syncthreads();
  if (!live) return;   // no barriers below

  // norm and z = Pi x / |x| in float64
  double ss = xv * xv;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor_d(ss, m);
  const double nu = sqrt(ss);
  sX[wave][lane] = xv;
  wave_lds_sync();
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < D; ++i) acc = fma(pv[i], sX[wave][i], acc);
  sZ[wave][lane] = acc / nu;   // a zero vector gives NaN: every distance is NaN, index 0
  wave_lds_sync();

  // nearest codeword of every block: P = 64 / nb (rounded down to a power of
  // two) lanes per block, lane p of block b taking codewords p, p + P, ...
  constexpr int NB = (D + K - 1) / K;
  constexpr int P = NB <= 8 ? 8 : (NB <= 16 ? 4 : 2);   // NB = 8, 16, 22 or 32
  const int b = lane / P, p = lane % P;
  double best = INFINITY;
  int bi = 0;
  if (b < NB) {
    const int c0 = b * K;
    const int rd = D - c0 < K ? D - c0 : K;   // real coordinates of the block
    double zb[K];
#pragma unroll
    for (int t = 0; t < K; ++t) zb[t] = t < rd ? sZ[wave][c0 + t] : 0.0;
#pragma unroll 4
    for (int cn = p; cn < a.N; cn += P) {
      const float* er = sEnc + cn * S;
      float ev[S];
#pragma unroll
      for (int q = 0; q < S / 4; ++q) {
        const floatx4 v4 = *reinterpret_cast<const floatx4*>(er + 4 * q);
        ev[4 * q] = v4[0];
        ev[4 * q + 1] = v4[1];
        ev[4 * q + 2] = v4[2];
        ev[4 * q + 3] = v4[3];
      }
      double dd = 0.0;
#pragma unroll
      for (int t = 0; t < K; ++t) {
        const double df = t < rd ? zb[t] + 0.5 * (double)ev[t] : 0.0;   // c = -enc / 2, exact
        dd = fma(df, df, dd);
      }
      if (dd < best) {
        best = dd;
        bi = cn;
      }
    }
  }
#pragma unroll
  for (int m = P >> 1; m >= 1; m >>= 1) {   // within the block's lanes
    const double ob = shfl_xor_d(best, m);
    const int oi = __shfl_xor(bi, m, 64);
    if (ob < best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (b < NB && p == 0) sIdx[wave][b] = (uint32_t)bi;
  wave_lds_sync();

  // the record (lane w builds word w) and the norm, in their cache slot
  const int64_t rec = (rr / a.rows.inner) * a.rows.stride + a.rows.pos + rr % a.rows.inner;
  if (lane < a.W) {
    uint32_t word = 0;
    for (int j = 0; j < a.nb; ++j) {
      const int p0 = j * a.bits - 32 * lane;   // field start relative to this word
      if (p0 >= 32 || p0 + a.bits <= 0) continue;
      const uint32_t f = sIdx[wave][j];
      word |= p0 >= 0 ? (f << p0) : (f >> (-p0));
    }
    (first ? a.codes1 : a.codes2)[rec * a.W + lane] = word;
  }
  if (lane == 0) (first ? a.norms1 : a.norms2)[rec] = f64_to_f16_bits(nu);
}

}  // namespace

hipError_t launch_append(const fq_codebook* cb, const uint16_t* x1, const uint16_t* x2,
                         int64_t n1, int64_t n, uint32_t* codes1, uint16_t* norms1,
                         uint32_t* codes2, uint16_t* norms2, OutRows rows, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (rows.inner <= 0) return hipErrorInvalidValue;
  AppendArgs a;
  a.x1 = x1;
  a.x2 = x2;
  a.n1 = n1;
  a.n = n;
  a.codes1 = codes1;
  a.norms1 = norms1;
  a.codes2 = codes2;
  a.norms2 = norms2;
  a.rows = rows;
  a.pi64t = cb->t.pi64t;
  a.enc = cb->t.enc;
  a.S = cb->enc_stride;
  a.k = cb->k;
  a.N = cb->N;
  a.nb = cb->nb;
  a.bits = cb->bits;
  a.W = cb->W;
  const int64_t blocks = (n + AP_WAVES - 1) / AP_WAVES;
  const size_t shm = (size_t)cb->N * cb->enc_stride * 4;   // at most 64 KB (k = 3, N = 4096)
  auto go = [&](auto kern) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(AP_WAVES * 64), shm, s, a);
    return hipGetLastError();
  };
  if (cb->enc_stride != ((cb->k + 1) + 3) / 4 * 4) return hipErrorInvalidValue;
  switch (cb->k) {
    case 2: return go(append_kernel<2>);
    case 3: return go(append_kernel<3>);
    case 4: return go(append_kernel<4>);
    case 8: return go(append_kernel<8>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fq
