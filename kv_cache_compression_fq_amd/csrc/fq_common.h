// Device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BUF_DWORD3 = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)
constexpr int CPOL_NT_SC1 = 2 | 16;      // buffer cache policy: non-temporal (nt) at system scope (sc1)

// Compile-time record shape of a (k, index bits) variant for d = 64.
template <int K, int BITS>
struct Shape {
  static constexpr int NB = (64 + K - 1) / K;                 // blocks per vector
  static constexpr int W = (NB * BITS + 31) / 32;             // record words
  static constexpr int IDX_PITCH = (NB + 7) / 8 * 8 + 4;      // u16 per staged index row
};

// W words at byte offset `off` of a buffer, with the widest loads the record
// alignment allows (records of 1, 2, 4 or 8 words sit on their own size).
template <int W>
__device__ inline void load_record(uint32_t (&w)[W], __amdgpu_buffer_rsrc_t rc, uint32_t off) {
  if constexpr (W == 4 || W == 8) {
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, off + 16 * q, 0, 0);
      w[4 * q] = v.x;
      w[4 * q + 1] = v.y;
      w[4 * q + 2] = v.z;
      w[4 * q + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, off + 4 * i, 0, 0);
  }
}

// Unpack one record into 16-bit indices at dst[0 .. NB) (static shifts).
template <int K, int BITS, int W>
__device__ inline void unpack_record(const uint32_t (&w)[W], uint16_t* dst) {
  constexpr int NB = Shape<K, BITS>::NB;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  uint32_t f[NB + 1];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int pos = j * BITS, wi = pos >> 5, o = pos & 31;
    uint32_t v = w[wi] >> o;
    if (o + BITS > 32) v |= w[wi + 1] << (32 - o);
    f[j] = v & MASK;
  }
  f[NB] = 0u;
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
  if constexpr (BITS == 8 && NB % 4 == 0) {
    // byte fields: one byte permute per pair of indices
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) {
      d32[2 * i] = __builtin_amdgcn_perm(0u, w[i], 0x0c010c00u);
      d32[2 * i + 1] = __builtin_amdgcn_perm(0u, w[i], 0x0c030c02u);
    }
  } else if constexpr (BITS == 4 && NB % 8 == 0) {
    // nibble fields: even and odd nibbles into bytes, then one byte permute
    // per pair of indices (field 2 p from the even bytes, 2 p + 1 from the odd)
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const uint32_t ev = w[i] & 0x0F0F0F0Fu, od = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        d32[4 * i + p] = __builtin_amdgcn_perm(od, ev, 0x0c000c00u | (uint32_t)p | ((uint32_t)(4 + p) << 16));
    }
  } else {
#pragma unroll
    for (int j = 0; j < NB; j += 2) d32[j >> 1] = f[j] | (f[j + 1] << 16);
  }
}

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
