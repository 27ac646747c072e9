// FibQuant encode (FibQuant technical summary, section 2.3): norm, shared
// rotation, per-block nearest codeword, fixed-rate packing (section 1).
//
// One thread per vector.  The rotation is taken in float64 (Pi held in LDS),
// so z is exact to float64 rounding; z is then rounded to float32 and every
// block is searched over the whole codebook with d'(n) = |c_n|^2 - 2 <z, c_n>
// in float32, keeping the best and the second-best value.  The float32 value of
// d'(n) is within eps of the exact one (bound below), so whenever the
// best-vs-second gap exceeds 2 eps the float32 winner is the exact argmin.
// Otherwise the block is re-searched in float64 with the distance
// sum_t (z_t - c_t)^2, ties to the lowest index.
//
// eps: z_t is rounded once (relative 2^-24), -2c_t is exact, |c|^2 is rounded
// once, and the k fused multiply-adds of the chain each round once with a
// partial result bounded by |c|^2 + 2 |c| |z|; so
//   |d'_f32 - d'| <= 2^-24 (k + 3) (cmax^2 + 2 cmax |z_j|)
// with cmax the largest codeword norm.  A 25% margin covers the float64
// error of z.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int ENC_THREADS = 256;

template <int K>
struct EncShape {
  static constexpr int NB = (D + K - 1) / K;
  static constexpr int LAST = D - (NB - 1) * K;
  static constexpr int S = ((K + 1) + 3) / 4 * 4;
};

template <typename TX>
__device__ inline void load_row(const TX* xr, float (&xv)[D]);

template <>
__device__ inline void load_row<_Float16>(const _Float16* xr, float (&xv)[D]) {
  const uint4* p = reinterpret_cast<const uint4*>(xr);
#pragma unroll
  for (int q = 0; q < D / 8; ++q) {
    uint4 v = p[q];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[8 * q + 2 * e] = f16_bits_to_f32((uint16_t)(w[e] & 0xFFFFu));
      xv[8 * q + 2 * e + 1] = f16_bits_to_f32((uint16_t)(w[e] >> 16));
    }
  }
}

template <>
__device__ inline void load_row<float>(const float* xr, float (&xv)[D]) {
  const float4* p = reinterpret_cast<const float4*>(xr);
#pragma unroll
  for (int q = 0; q < D / 4; ++q) {
    float4 v = p[q];
    xv[4 * q] = v.x;
    xv[4 * q + 1] = v.y;
    xv[4 * q + 2] = v.z;
    xv[4 * q + 3] = v.w;
  }
}

template <int K, typename TX>
__global__ __launch_bounds__(ENC_THREADS) void encode_ref_kernel(
    const TX* __restrict__ x, int64_t n, int64_t ld, const double* __restrict__ pi64,
    const float* __restrict__ enc, const double* __restrict__ cb64, int N, int bits, int W,
    float cmax, float cmax_last, uint32_t* __restrict__ codes, uint16_t* __restrict__ norms) {
  using Sh = EncShape<K>;
  constexpr int S = Sh::S;
  extern __shared__ __align__(16) unsigned char smem[];
  double* sPi = reinterpret_cast<double*>(smem);
  float* sEnc = reinterpret_cast<float*>(smem + sizeof(double) * D * D);
  for (int i = threadIdx.x; i < D * D; i += blockDim.x) sPi[i] = pi64[i];
  for (int i = threadIdx.x; i < N * S; i += blockDim.x) sEnc[i] = enc[i];
  __syncthreads();

  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  float xv[D];
  load_row<TX>(x + r * ld, xv);
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < D; ++i) ss = fma((double)xv[i], (double)xv[i], ss);
  const double nu = sqrt(ss);
  uint32_t* out = codes + r * W;
  norms[r] = f64_to_f16_bits(nu);
  if (!(nu > 0.0)) {
    for (int w = 0; w < W; ++w) out[w] = 0u;
    return;
  }
  const double inv = 1.0 / nu;
  uint64_t acc = 0;
  int nacc = 0, wi = 0;
  for (int j = 0; j < Sh::NB; ++j) {
    const int rj = (j == Sh::NB - 1) ? Sh::LAST : K;
    double zd[K];
    float zf[K];
    float zz = 0.f;
#pragma unroll
    for (int t = 0; t < K; ++t) {
      double a = 0.0;
      if (t < rj) {
        const double* prow = sPi + (j * K + t) * D;
#pragma unroll
        for (int i = 0; i < D; ++i) a = fma(prow[i], (double)xv[i], a);
        a *= inv;
      }
      zd[t] = a;
      zf[t] = (float)a;
      zz = fmaf(zf[t], zf[t], zz);
    }
    float m1 = INFINITY, m2 = INFINITY;
    int i1 = 0;
    if (rj == K) {
      for (int c = 0; c < N; ++c) {
        const float* e = sEnc + c * S;
        float dv = e[K];
#pragma unroll
        for (int t = 0; t < K; ++t) dv = fmaf(zf[t], e[t], dv);
        if (dv < m1) {
          m2 = m1;
          m1 = dv;
          i1 = c;
        } else if (dv < m2) {
          m2 = dv;
        }
      }
    } else {
      for (int c = 0; c < N; ++c) {
        const float* e = sEnc + c * S;
        float ccr = 0.f, dv = 0.f;
#pragma unroll
        for (int t = 0; t < K; ++t)
          if (t < rj) ccr = fmaf(0.5f * e[t], 0.5f * e[t], ccr);
        dv = ccr;
#pragma unroll
        for (int t = 0; t < K; ++t)
          if (t < rj) dv = fmaf(zf[t], e[t], dv);
        if (dv < m1) {
          m2 = m1;
          m1 = dv;
          i1 = c;
        } else if (dv < m2) {
          m2 = dv;
        }
      }
    }
    const float cm = (rj == K) ? cmax : cmax_last;
    const float eps = 1.25f * 5.9604645e-8f * (float)(K + 3) * (cm * cm + 2.f * cm * sqrtf(zz));
    if (!(m2 - m1 > 2.f * eps)) {
      double best = INFINITY;
      int bi = 0;
      for (int c = 0; c < N; ++c) {
        double dd = 0.0;
#pragma unroll
        for (int t = 0; t < K; ++t)
          if (t < rj) {
            const double df = zd[t] - cb64[c * K + t];
            dd = fma(df, df, dd);
          }
        if (dd < best) {
          best = dd;
          bi = c;
        }
      }
      i1 = bi;
    }
    acc |= (uint64_t)(uint32_t)i1 << nacc;
    nacc += bits;
    if (nacc >= 32) {
      out[wi++] = (uint32_t)acc;
      acc >>= 32;
      nacc -= 32;
    }
  }
  if (nacc > 0) out[wi++] = (uint32_t)acc;
}

template <int K, typename TX>
hipError_t launch_ref(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                      uint16_t* norms, hipStream_t s) {
  const size_t shm = sizeof(double) * D * D + sizeof(float) * cb->N * cb->enc_stride;
  auto kern = encode_ref_kernel<K, TX>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + ENC_THREADS - 1) / ENC_THREADS;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(ENC_THREADS), shm, s, x, n, ld,
                     cb->t.pi64, cb->t.enc, cb->t.cb64, cb->N, cb->bits, cb->W, cb->cmax,
                     cb->cmax_last, codes, norms);
  return hipGetLastError();
}

template <typename TX>
hipError_t dispatch_k(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                      uint16_t* norms, hipStream_t s) {
  switch (cb->k) {
    case 2: return launch_ref<2, TX>(cb, x, n, ld, codes, norms, s);
    case 3: return launch_ref<3, TX>(cb, x, n, ld, codes, norms, s);
    case 4: return launch_ref<4, TX>(cb, x, n, ld, codes, norms, s);
    case 8: return launch_ref<8, TX>(cb, x, n, ld, codes, norms, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n, int64_t ld,
                         uint32_t* codes, uint16_t* norms, hipStream_t s) {
  if (xt == FQ_F16)
    return dispatch_k<_Float16>(cb, static_cast<const _Float16*>(x), n, ld, codes, norms, s);
  return dispatch_k<float>(cb, static_cast<const float*>(x), n, ld, codes, norms, s);
}

}  // namespace fq
