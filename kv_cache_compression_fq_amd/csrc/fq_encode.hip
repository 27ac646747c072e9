// FibQuant encode (FibQuant technical summary, section 2.3): norm, shared
// rotation, per-block nearest codeword, fixed-rate packing (section 1).
//
// One wave encodes a chunk of 16 vectors at a time:
//
//  1. norm: nu = |x|_2 in float64 from the exact input values; the stored
//     norm is nu rounded once to binary16.
//  2. rotation on the matrix cores: Pi = Pi_hi + 2^-11 Pi_lo (both binary16),
//     y = Pi_hi x + 2^-11 Pi_lo x with v_mfma_f32_16x16x32_f16 (binary16 input
//     is exact; float32 input is scaled by a power of two and split the same
//     way), z~ = y / nu in float32, staged in LDS.
//  3. block search: every (vector, block) column looks for
//     argmin_n t(n) = |c_n|^2 - 2 <z~, c_n> (the distance without |z|^2) over
//     the codebook, in float32, keeping the best and second-best value.
//  4. certification: with D = t + |z|^2, the computed t of every codeword is
//     within gv (sqrt D + 3|z|)^2 of its exact value at z~ (a chain of k
//     float32 fused multiply-adds, each rounded once), and z~ is within ez of
//     the exact z per coordinate, which moves a difference t(n) - t(m) by at
//     most 2 ez sqrt(k) (sqrt D_n + sqrt D_m).  Both bounds grow more slowly
//     than the gap as D_n grows, so when the second-best gap exceeds their sum
//     for the runner-up, the float32 winner is the exact argmin for the exact
//     z and the result is final.
//  5. otherwise (near ties, non-finite data) the block is redone exactly by
//     the whole wave: z's block in float64 from x and the float64 Pi, then all
//     N codewords with sum_t (z_t - c_t)^2 in float64, ties to the lowest index.
//  6. the chunk's indices are packed LSB-first into fixed-size records and
//     written with coalesced word stores, norms beside them.
//
// ez covers the binary16 split of Pi (and of x), the float32 accumulation on
// the matrix cores (taken as at most one rounding of 2^-23 relative per
// accumulated term, 130 terms) and the final scaling; it is computed on the
// host from the actual split residuals.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int EV = 16;          // vectors per wave chunk
constexpr int ENC_WAVES = 8;    // waves per workgroup
constexpr int ZP = 68;          // floats per staged z row
constexpr int ROT_BYTES = 2 * 4 * 2 * 64 * 8 * 2;   // Pi fragments, [part][ot][ks][lane][8]
constexpr float SLACK = 1e-5f;  // covers |D~ - D| inside the square roots of the bound

template <int K, int BITS>
struct EncShape {
  static constexpr int NB = (D + K - 1) / K;
  static constexpr int LAST = D - (NB - 1) * K;
  static constexpr int S = ((K + 1) + 3) / 4 * 4;   // search-table stride (floats)
  static constexpr int W = (NB * BITS + 31) / 32;
  static constexpr int IP = (NB + 2) / 2 * 2;       // u16 per staged index row
  static constexpr int NCOL = EV * NB;              // columns per chunk
  static constexpr int CPL = (NCOL + 63) / 64;      // columns per lane
  static constexpr size_t WAVE_BYTES =
      ((size_t)EV * ZP * 4 + EV * 8 + (size_t)EV * IP * 2 + (size_t)NCOL * 2 + 15) / 16 * 16;
};

struct EncArgs {
  const void* x;
  int64_t n, ld;
  uint32_t* codes;
  uint16_t* norms;
  const _Float16* rotfrag;
  const float* enc;
  const double* pi64;
  int N;
  float ez;   // bound on |z~ - z| per coordinate of a unit vector
  float gv;   // relative rounding bound of the float32 search value
};

__host__ __device__ inline size_t enc_table_bytes(int N, int S) {
  return ((size_t)N * S * 4 + 15) / 16 * 16;
}

__device__ inline double shfl_xor_f64(double v, int m) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = __shfl_xor(p.x, m, 64);
  p.y = __shfl_xor(p.y, m, 64);
  return __builtin_bit_cast(double, p);
}

// x fragments of one vector (lane's vector j = lane % 16, coordinates
// 32 ks + 8 (lane / 16) .. + 7) as binary16 hi parts (and lo parts, scaled by
// 2^11, for float32 input), the float64 sum of squares, and for float32 input
// the power of two the fragments were scaled by.
template <typename TX>
struct XFrag {
  half8 hi[2], lo[2];
  double ss;
  float escale;   // the fragments hold x * 2^-e; escale = 2^e
};

template <typename TX>
__device__ inline void load_x(const TX* xr, int g, XFrag<TX>& f);

template <>
__device__ inline void load_x<_Float16>(const _Float16* xr, int g, XFrag<_Float16>& f) {
  double ss = 0.0;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 32 * ks + 8 * g);
    f.hi[ks] = __builtin_bit_cast(half8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double t = (double)(float)f.hi[ks][e];
      ss = fma(t, t, ss);
    }
  }
  ss += shfl_xor_f64(ss, 16);
  ss += shfl_xor_f64(ss, 32);
  f.ss = ss;
  f.escale = 1.f;
}

template <>
__device__ inline void load_x<float>(const float* xr, int g, XFrag<float>& f) {
  float v[2][8];
  double ss = 0.0;
  float mx = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(xr + 32 * ks + 8 * g);
    const floatx4 b = *reinterpret_cast<const floatx4*>(xr + 32 * ks + 8 * g + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[ks][e] = a[e];
      v[ks][4 + e] = b[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss = fma((double)v[ks][e], (double)v[ks][e], ss);
      mx = fmaxf(mx, fabsf(v[ks][e]));
    }
  }
  ss += shfl_xor_f64(ss, 16);
  ss += shfl_xor_f64(ss, 32);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // scale so that |x| <= 1: binary16 then holds every element without overflow
  int e = 0;
  if (mx > 0.f && mx <= 3.0e38f) (void)frexpf(mx, &e);
  const float down = ldexpf(1.f, -e);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = v[ks][i] * down;
      const _Float16 h = (_Float16)s;
      f.hi[ks][i] = h;
      f.lo[ks][i] = (_Float16)((s - (float)h) * 2048.f);
    }
  f.ss = ss;
  f.escale = ldexpf(1.f, e);
}

// Word w of a record from the staged indices of one vector.
template <int BITS>
__device__ inline uint32_t pack_word(const uint16_t* idx, int nb, int w) {
  const int j0 = (32 * w) / BITS;
  int j1 = (32 * w + 31) / BITS;
  if (j1 > nb - 1) j1 = nb - 1;
  uint32_t v = 0;
  for (int jj = j0; jj <= j1; ++jj) {
    const int s = jj * BITS - 32 * w;
    const uint32_t f = idx[jj];
    v |= s >= 0 ? (f << s) : (f >> (-s));
  }
  return v;
}

template <int K, int BITS, typename TX>
__global__ __launch_bounds__(ENC_WAVES * 64) void encode_kernel(EncArgs a) {
  using Sh = EncShape<K, BITS>;
  constexpr int NB = Sh::NB, S = Sh::S, IP = Sh::IP;
  extern __shared__ __align__(16) unsigned char smem[];
  const int N = a.N;
  _Float16* sRot = reinterpret_cast<_Float16*>(smem);
  float* sEnc = reinterpret_cast<float*>(smem + ROT_BYTES);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  unsigned char* wb = smem + ROT_BYTES + enc_table_bytes(N, S) + wave * Sh::WAVE_BYTES;
  float* sZ = reinterpret_cast<float*>(wb);
  double* sNu = reinterpret_cast<double*>(wb + EV * ZP * 4);
  uint16_t* sIdx = reinterpret_cast<uint16_t*>(wb + EV * ZP * 4 + EV * 8);
  uint16_t* sFb = sIdx + EV * IP;

  for (int i = threadIdx.x; i < ROT_BYTES / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(sRot)[i] = reinterpret_cast<const u32x4*>(a.rotfrag)[i];
  for (int i = threadIdx.x; i < N * S / 4; i += blockDim.x)
    reinterpret_cast<floatx4*>(sEnc)[i] = reinterpret_cast<const floatx4*>(a.enc)[i];
  __syncthreads();

  const TX* __restrict__ x = static_cast<const TX*>(a.x);
  const int64_t nchunks = (a.n + EV - 1) / EV;
  const int64_t tw = (int64_t)gridDim.x * ENC_WAVES;
  const int j = lane & 15, g = lane >> 4;
  const float ez2 = 2.f * a.ez;

  for (int64_t ch = (int64_t)blockIdx.x * ENC_WAVES + wave; ch < nchunks; ch += tw) {
    const int64_t base = ch * EV;
    const int nv = (int)((a.n - base) < EV ? (a.n - base) : EV);
    const int jr = j < nv ? j : nv - 1;

    // ---- 1. load + norm
    XFrag<TX> xf;
    load_x<TX>(x + (base + jr) * a.ld, g, xf);
    const double nu = sqrt(xf.ss);
    const uint16_t nbits = f64_to_f16_bits(nu);
    const float inv = nu > 0.0 ? (float)((double)xf.escale / nu) : 0.f;
    if (g == 0) sNu[j] = nu;

    // ---- 2. rotation: lane holds z~[vector j][16 ot + 4 g + r]
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
      floatx4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8 ph = *reinterpret_cast<const half8*>(sRot + (((0 * 4 + ot) * 2 + ks) * 64 + lane) * 8);
        const half8 pl = *reinterpret_cast<const half8*>(sRot + (((1 * 4 + ot) * 2 + ks) * 64 + lane) * 8);
        ah = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, xf.hi[ks], ah, 0, 0, 0);
        al = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, xf.hi[ks], al, 0, 0, 0);
        if constexpr (sizeof(TX) == 4)
          al = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, xf.lo[ks], al, 0, 0, 0);
      }
      floatx4 zv;
#pragma unroll
      for (int r = 0; r < 4; ++r) zv[r] = fmaf(al[r], 0x1p-11f, ah[r]) * inv;
      *reinterpret_cast<floatx4*>(sZ + j * ZP + 16 * ot + 4 * g) = zv;
    }
    wave_lds_sync();

    // ---- 3-4. search + certification, one column per lane at a time
    int nfb = 0;
    for (int q = 0; q < Sh::CPL; ++q) {
      const int c = lane + 64 * q;
      const int v = c / NB, b = c - v * NB;
      const bool live = c < Sh::NCOL && v < nv;
      const bool partial = (K * (b + 1) > D);
      float z[K];
      float zz = 0.f;
#pragma unroll
      for (int t = 0; t < K; ++t) {
        const bool real = live && (!partial || t < Sh::LAST);
        z[t] = real ? sZ[v * ZP + K * b + t] : 0.f;
        zz = fmaf(z[t], z[t], zz);
      }
      float m1 = INFINITY, m2 = INFINITY;
      int i1 = 0;
#pragma unroll 4
      for (int i = 0; i < N; ++i) {
        const float* e = sEnc + i * S;
        float t = partial ? 0.25f * e[0] * e[0] : e[K];
#pragma unroll
        for (int tt = 0; tt < K; ++tt) t = fmaf(e[tt], z[tt], t);
        const bool p = t < m1;
        m2 = __builtin_amdgcn_fmed3f(m1, m2, t);
        m1 = p ? t : m1;
        i1 = p ? i : i1;
      }
      const float zn = sqrtf(zz);
      const float r1 = sqrtf(fmaxf(m1 + zz, 0.f) + SLACK), r2 = sqrtf(fmaxf(m2 + zz, 0.f) + SLACK);
      const float keff = partial ? 1.f : (float)K;
      const float A1 = r1 + 3.f * zn, A2 = r2 + 3.f * zn;
      const float thr = a.gv * (A1 * A1 + A2 * A2) + ez2 * sqrtf(keff) * (r1 + r2) + 1e-12f;
      const bool zero = live && !(sNu[v] > 0.0);
      const bool certain = (m2 - m1) > thr;
      if (live) sIdx[v * IP + b] = (uint16_t)(zero ? 0 : i1);
      const bool fb = live && !zero && !certain;
      const uint64_t m = __builtin_amdgcn_ballot_w64(fb);
      if (fb) {
        const int pos = nfb + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        sFb[pos] = (uint16_t)c;
      }
      nfb += __builtin_popcountll(m);
    }
    wave_lds_sync();

    // ---- 5. exact float64 redo of uncertified columns, by the whole wave
    for (int e = 0; e < nfb; ++e) {
      const int c = sFb[e];
      const int v = c / NB, b = c - v * NB;
      const int rj = (K * (b + 1) > D) ? Sh::LAST : K;
      const double nuv = sNu[v];
      const double xj = (double)x[(base + v) * a.ld + lane];
      double zd[K];
#pragma unroll
      for (int t = 0; t < K; ++t) {
        double s = 0.0;
        if (t < rj) {
          s = a.pi64[(K * b + t) * D + lane] * xj;
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) s += shfl_xor_f64(s, m);
        }
        zd[t] = s / nuv;
      }
      double best = INFINITY;
      int bi = 0;
      for (int i = lane; i < N; i += 64) {
        const float* ee = sEnc + i * S;
        double dd = 0.0;
#pragma unroll
        for (int t = 0; t < K; ++t)
          if (t < rj) {
            const double df = zd[t] + 0.5 * (double)ee[t];   // c = -e / 2, exact
            dd = fma(df, df, dd);
          }
        if (dd < best) {
          best = dd;
          bi = i;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ob = shfl_xor_f64(best, m);
        const int oi = __shfl_xor(bi, m, 64);
        if (ob < best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      if (lane == 0) sIdx[v * IP + b] = (uint16_t)bi;
      wave_lds_sync();
    }
    wave_lds_sync();

    // ---- 6. pack + store
    uint32_t* __restrict__ out = a.codes + base * Sh::W;
    for (int t = lane; t < nv * Sh::W; t += 64) {
      const int v = t / Sh::W, w = t - v * Sh::W;
      out[t] = pack_word<BITS>(sIdx + v * IP, NB, w);
    }
    if (g == 0 && j < nv) a.norms[base + j] = nbits;
    wave_lds_sync();
  }
}

template <int K, int BITS, typename TX>
hipError_t launch_k(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                    uint16_t* norms, hipStream_t s) {
  using Sh = EncShape<K, BITS>;
  const size_t shm = ROT_BYTES + enc_table_bytes(cb->N, Sh::S) + ENC_WAVES * Sh::WAVE_BYTES;
  auto kern = encode_kernel<K, BITS, TX>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  static int64_t cap = 0;
  if (cap == 0) cap = resident_blocks(reinterpret_cast<const void*>(kern), ENC_WAVES * 64, shm);
  const int64_t chunks = (n + EV - 1) / EV;
  int64_t blocks = (chunks + ENC_WAVES - 1) / ENC_WAVES;
  if (cap > 0 && blocks > cap) blocks = cap;
  EncArgs a;
  a.x = x;
  a.n = n;
  a.ld = ld;
  a.codes = codes;
  a.norms = norms;
  a.rotfrag = cb->t.encfrag;
  a.enc = cb->t.enc;
  a.pi64 = cb->t.pi64;
  a.N = cb->N;
  a.ez = sizeof(TX) == 2 ? cb->enc_ez16 : cb->enc_ez32;
  a.gv = (float)((K + 2) * 0x1p-24 * 1.01);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(ENC_WAVES * 64), shm, s, a);
  return hipGetLastError();
}

template <typename TX>
hipError_t dispatch(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                    uint16_t* norms, hipStream_t s) {
#define FQ_ENC_CASE(KK, BB) \
  if (cb->k == KK && cb->bits == BB) return launch_k<KK, BB, TX>(cb, x, n, ld, codes, norms, s);
  FQ_VARIANTS(FQ_ENC_CASE)
#undef FQ_ENC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n, int64_t ld,
                         uint32_t* codes, uint16_t* norms, hipStream_t s) {
  if (xt == FQ_F16)
    return dispatch<_Float16>(cb, static_cast<const _Float16*>(x), n, ld, codes, norms, s);
  return dispatch<float>(cb, static_cast<const float*>(x), n, ld, codes, norms, s);
}

}  // namespace fq
