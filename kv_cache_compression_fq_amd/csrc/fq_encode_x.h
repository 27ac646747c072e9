// Encode steps shared by the block-search kernels (FibQuant technical summary,
// section 2.3): loading a 16-vector chunk, its norm, and the shared rotation
// on the matrix cores, with z~ = Pi x / |x| staged in LDS.
#pragma once

#include <type_traits>

#include "fq_common.h"

namespace fq {
namespace encx {

constexpr int EV = 16;          // vectors per wave chunk
constexpr int ZP = 68;          // floats per staged z row
constexpr int ROT_BYTES = 2 * 4 * 4 * 64 * 4 * 2;   // Pi fragments, [part][ot][kq][lane][4]

__device__ inline double shfl_xor_f64(double v, int m) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = __shfl_xor(p.x, m, 64);
  p.y = __shfl_xor(p.y, m, 64);
  return __builtin_bit_cast(double, p);
}

// x fragments of one vector for v_mfma_f32_16x16x16_f16 (lane's vector
// j = lane % 16, coordinates 16 kq + 4 (lane / 16) .. + 3) as binary16 hi parts
// (and lo parts, scaled by 2^11, for float32 input), the float64 sum of
// squares, and for float32 input the power of two the fragments were scaled by.
template <typename TX>
struct XFrag {
  half4 hi[4], lo[4];
  float ss;       // sum of squares of the (scaled) vector, pairwise in float32
  float escale;   // the fragments hold x * 2^-e; escale = 2^e
};

// Pairwise float32 sum of the 16 squares a lane holds, then across the four
// lanes of the vector: six rounding levels, so the relative error of the
// (positive) sum is below 6 * 2^-24, well inside the norm's tolerance.
__device__ inline float pairwise_squares(const float (&v)[16]) {
  float t8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t8[i] = fmaf(v[2 * i], v[2 * i], v[2 * i + 1] * v[2 * i + 1]);
  const float t4[4] = {t8[0] + t8[1], t8[2] + t8[3], t8[4] + t8[5], t8[6] + t8[7]};
  float ss = (t4[0] + t4[1]) + (t4[2] + t4[3]);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  return ss;
}

// Raw loads of one lane's x elements (issued one chunk ahead).
template <typename TX>
struct XRaw;
template <>
struct XRaw<_Float16> {
  u32x2 q[4];
};
template <>
struct XRaw<float> {
  floatx4 q[4];
};

// Each input row is read exactly once.  NT = true marks the loads
// non-temporal, so the input stream does not evict other data from L2.
template <typename TX, bool NT = false>
__device__ inline void load_raw(const TX* xr, int g, XRaw<TX>& r) {
  using Q = std::remove_reference_t<decltype(r.q[0])>;
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    const Q* p = reinterpret_cast<const Q*>(xr + 16 * kq + 4 * g);
    if constexpr (NT)
      r.q[kq] = __builtin_nontemporal_load(p);
    else
      r.q[kq] = *p;
  }
}

template <typename TX>
__device__ inline void finish_x(const XRaw<TX>& r, XFrag<TX>& f);

template <>
__device__ inline void finish_x<_Float16>(const XRaw<_Float16>& r, XFrag<_Float16>& f) {
  float v[16];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    f.hi[kq] = __builtin_bit_cast(half4, r.q[kq]);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * kq + e] = (float)f.hi[kq][e];   // squares exact in float32
  }
  f.ss = pairwise_squares(v);
  f.escale = 1.f;
}

template <>
__device__ inline void finish_x<float>(const XRaw<float>& r, XFrag<float>& f) {
  float mx = 0.f;
#pragma unroll
  for (int kq = 0; kq < 4; ++kq)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(r.q[kq][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // scale so that |x| <= 1: binary16 then holds every element without overflow,
  // and the squares cannot overflow float32
  int e = 0;
  if (mx > 0.f && mx <= 3.0e38f) (void)frexpf(mx, &e);
  const float down = ldexpf(1.f, -e);
  float v[16];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sv = r.q[kq][i] * down;
      v[4 * kq + i] = sv;
      const _Float16 h = (_Float16)sv;
      f.hi[kq][i] = h;
      f.lo[kq][i] = (_Float16)((sv - (float)h) * 2048.f);
    }
  f.ss = pairwise_squares(v);
  f.escale = ldexpf(1.f, e);
}

// z~ of the chunk into sZ: row j (= lane % 16) gets coordinates
// 16 ot + 4 (lane / 16) + r.  Pi = Pi_hi + 2^-11 Pi_lo as A fragments of
// v_mfma_f32_16x16x16_f16 in sRot ([part][ot][kq][lane][4]).  Every
// 16-product group of the hi part is accumulated from zero and the groups are
// summed in float32, which keeps the rounding bound small; the lo products
// (Pi_lo x, and Pi_hi x_lo for float32 input) carry a weight of 2^-11, so
// their roundings hardly count and they are chained in one accumulator.  inv
// is 1 / |x|.
template <typename TX>
__device__ inline void rotate_to_lds(const XFrag<TX>& xf, const _Float16* sRot, float inv, float* sZ,
                                     int lane) {
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ot = 0; ot < 4; ++ot) {
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    floatx4 ph4[4];
    floatx4 lo = zero;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const half4 ph = *reinterpret_cast<const half4*>(sRot + (((0 * 4 + ot) * 4 + kq) * 64 + lane) * 4);
      const half4 pl = *reinterpret_cast<const half4*>(sRot + (((1 * 4 + ot) * 4 + kq) * 64 + lane) * 4);
      ph4[kq] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, xf.hi[kq], zero, 0, 0, 0);
      lo = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, xf.hi[kq], lo, 0, 0, 0);
      if constexpr (sizeof(TX) == 4) lo = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, xf.lo[kq], lo, 0, 0, 0);
    }
    floatx4 zv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float zh = (ph4[0][r] + ph4[1][r]) + (ph4[2][r] + ph4[3][r]);
      zv[r] = fmaf(lo[r], 0x1p-11f, zh) * inv;
    }
    *reinterpret_cast<floatx4*>(sZ + j * ZP + 16 * ot + 4 * g) = zv;
  }
}

}  // namespace encx
}  // namespace fq
