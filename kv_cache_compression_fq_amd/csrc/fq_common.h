// Device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

// binary16 bit pattern -> float
__device__ inline float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// float64 -> binary16 with one rounding to nearest-even: truncate into float32,
// mark inexactness in the last bit (round-to-odd), then round float32 -> binary16.
// float32 carries 13 more fraction bits than binary16, so the second rounding
// sees the sticky bit and the result equals a direct rounding of the double.
__device__ inline uint16_t f64_to_f16_bits(double v) {
  float f = __double2float_rz(v);
  if ((double)f != v) f = __uint_as_float(__float_as_uint(f) | 1u);
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ inline uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Field j (bits wide) of a record: bits [j*bits, (j+1)*bits), LSB-first over
// little-endian 32-bit words.
__device__ inline uint32_t record_field(const uint32_t* rec, int j, int bits) {
  const int pos = j * bits;
  const int w = pos >> 5, o = pos & 31;
  uint32_t v = rec[w] >> o;
  if (o + bits > 32) v |= rec[w + 1] << (32 - o);
  return v & ((1u << bits) - 1u);
}

// Order LDS traffic between the lanes of one wave (no workgroup barrier).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace fq
