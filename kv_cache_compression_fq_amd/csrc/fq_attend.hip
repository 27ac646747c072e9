// Fused decode-step attention over the compressed cache (FibQuant technical
// summary, section 5: fixed-address records let decompression be fused into
// attention).  Scores and the value sum are taken in the rotated domain:
//   <q, nu Pi^T z_hat> = nu <Pi q, z_hat>,   sum_t p_t nu_t Pi^T z_hat_t = Pi^T sum_t p_t nu_t z_hat_t
// so only the query is rotated on the way in and the output once on the way out.
//
// Split-K over the context: kernel A computes, for each (batch, KV head, split),
// the running max m, the sum l and the unnormalised rotated output of every
// query head of the group; kernel B merges the splits (log-sum-exp), applies
// Pi^T and writes binary16.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int ATT_THREADS = 256;
constexpr int ATT_TILE = 64;      // tokens per tile
constexpr int MAX_G = 16;         // query heads per KV head
constexpr int PART = D + 2;       // floats per partial: m, l, o[64]

struct SplitPlan {
  int S;
  int64_t chunk;
};

SplitPlan plan_splits(int B, int Hkv, int64_t T) {
  const int64_t pairs = (int64_t)B * Hkv;
  int64_t S = (1024 + pairs - 1) / pairs;
  const int64_t max_s = (T + 255) / 256;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  int64_t chunk = (T + S - 1) / S;
  chunk = (chunk + ATT_TILE - 1) / ATT_TILE * ATT_TILE;
  S = (T + chunk - 1) / chunk;
  return {(int)S, chunk};
}

template <int KK, int KV>
__global__ __launch_bounds__(ATT_THREADS) void attend_split_ref_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kc,
    const uint16_t* __restrict__ kn, const uint32_t* __restrict__ vc,
    const uint16_t* __restrict__ vn, int Hq, int Hkv, int64_t T, int64_t chunk, float scale,
    const float* __restrict__ pi32, const float* __restrict__ cbk, int Nk, int bitsk, int Wk,
    const float* __restrict__ cbv, int Nv, int bitsv, int Wv, float* __restrict__ ws, int S) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)split * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;

  extern __shared__ __align__(16) unsigned char smem[];
  float* sQ = reinterpret_cast<float*>(smem);             // [G][64] rotated, scaled queries
  float* sPart = sQ + MAX_G * D;                           // [4][G][TILE] partial scores
  float* sP = sPart + 4 * MAX_G * ATT_TILE;                // [G][TILE] p * nu_v
  float* sAlpha = sP + MAX_G * ATT_TILE;                   // [G]
  float* sCbK = sAlpha + MAX_G;                            // [Nk][KK]
  float* sCbV = sCbK + Nk * KK;                            // [Nv][KV]

  for (int e = tid; e < Nk * KK; e += ATT_THREADS) sCbK[e] = cbk[e];
  for (int e = tid; e < Nv * KV; e += ATT_THREADS) sCbV[e] = cbv[e];
  // q_rot[h][c] = scale * sum_i Pi[c][i] q[b, g*G + h][i]
  for (int e = tid; e < G * D; e += ATT_THREADS) {
    const int h = e / D, c = e % D;
    const uint16_t* qr = q + ((int64_t)b * Hq + (int64_t)g * G + h) * D;
    float a = 0.f;
    for (int i = 0; i < D; ++i) a = fmaf(pi32[c * D + i], f16_bits_to_f32(qr[i]), a);
    sQ[h * D + c] = a * scale;
  }
  __syncthreads();

  const int64_t base = ((int64_t)b * Hkv + g) * T;
  // per-head running state: wave w owns heads w, w+4, ...
  float m_run[MAX_G / 4], l_run[MAX_G / 4];
#pragma unroll
  for (int u = 0; u < MAX_G / 4; ++u) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }
  // value accumulators: thread owns coordinate c = lane for heads wave, wave+4, ...
  float o_acc[MAX_G / 4];
#pragma unroll
  for (int u = 0; u < MAX_G / 4; ++u) o_acc[u] = 0.f;

  for (int64_t tt = t0; tt < t1; tt += ATT_TILE) {
    const int64_t t = tt + lane;
    const bool valid = t < t1;
    // ---- scores: part `wave` covers coordinates [16 wave, 16 wave + 16)
    {
      float zk[16];
      float nuk = 0.f;
      if (valid) {
        const uint32_t* rec = kc + (base + t) * Wk;
        nuk = f16_bits_to_f32(kn[base + t]);
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
          const int c = wave * 16 + cc;
          const int j = c / KK, tq = c % KK;
          zk[cc] = sCbK[record_field(rec, j, bitsk) * KK + tq];
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) zk[cc] = 0.f;
      }
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) a = fmaf(sQ[h * D + wave * 16 + cc], zk[cc], a);
        sPart[(wave * MAX_G + h) * ATT_TILE + lane] = a * nuk;
      }
    }
    __syncthreads();
    // ---- online softmax: wave w handles heads w, w+4, ...; lane = token
    {
      const float nuv = valid ? f16_bits_to_f32(vn[base + t]) : 0.f;
#pragma unroll
      for (int u = 0; u < MAX_G / 4; ++u) {
        const int h = wave + 4 * u;
        if (h < G) {
          float s = sPart[(0 * MAX_G + h) * ATT_TILE + lane] + sPart[(1 * MAX_G + h) * ATT_TILE + lane] +
                    sPart[(2 * MAX_G + h) * ATT_TILE + lane] + sPart[(3 * MAX_G + h) * ATT_TILE + lane];
          if (!valid) s = -INFINITY;
          const float mt = wave_max(s);
          const float mn = fmaxf(m_run[u], mt);
          const float p = valid ? __expf(s - mn) : 0.f;
          const float ps = wave_sum(p);
          const float alpha = __expf(m_run[u] - mn);
          l_run[u] = l_run[u] * alpha + ps;
          m_run[u] = mn;
          sP[h * ATT_TILE + lane] = p * nuv;
          if (lane == 0) sAlpha[h] = alpha;
        }
      }
    }
    __syncthreads();
    // ---- values: thread owns coordinate c = lane, heads wave, wave+4, ...
    {
      const int c = lane;
      const int j = c / KV, tq = c % KV;
#pragma unroll
      for (int u = 0; u < MAX_G / 4; ++u) {
        const int h = wave + 4 * u;
        if (h < G) o_acc[u] *= sAlpha[h];
      }
      const int64_t nt = (t1 - tt) < ATT_TILE ? (t1 - tt) : ATT_TILE;
      for (int e = 0; e < nt; ++e) {
        const uint32_t* rec = vc + (base + tt + e) * Wv;
        const float zv = sCbV[record_field(rec, j, bitsv) * KV + tq];
#pragma unroll
        for (int u = 0; u < MAX_G / 4; ++u) {
          const int h = wave + 4 * u;
          if (h < G) o_acc[u] = fmaf(sP[h * ATT_TILE + e], zv, o_acc[u]);
        }
      }
    }
    __syncthreads();
  }
  // ---- write partials
#pragma unroll
  for (int u = 0; u < MAX_G / 4; ++u) {
    const int h = wave + 4 * u;
    if (h < G) {
      float* dst = ws + (((int64_t)b * Hq + (int64_t)g * G + h) * S + split) * PART;
      if (lane == 0) {
        dst[0] = m_run[u];
        dst[1] = l_run[u];
      }
      dst[2 + lane] = o_acc[u];
    }
  }
}

__global__ __launch_bounds__(64) void attend_merge_kernel(const float* __restrict__ ws, int S,
                                                          int Hq, const float* __restrict__ pi32,
                                                          uint16_t* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const float* src = ws + ((int64_t)b * Hq + h) * S * PART;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, src[s * PART]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = __expf(src[s * PART] - M);
    L = fmaf(w, src[s * PART + 1], L);
    o = fmaf(w, src[s * PART + 2 + c], o);
  }
  __shared__ float sO[D];
  sO[c] = o / L;
  __syncthreads();
  // out = Pi^T o_rot: out[c] = sum_j Pi[j][c] o_rot[j]
  float a = 0.f;
  for (int j = 0; j < D; ++j) a = fmaf(pi32[j * D + c], sO[j], a);
  out[((int64_t)b * Hq + h) * D + c] = f32_to_f16_rne(a);
}

template <int KK, int KV>
hipError_t launch_ref(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                      const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                      const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, float scale,
                      float* ws, uint16_t* out, hipStream_t s) {
  const SplitPlan p = plan_splits(B, Hkv, T);
  const size_t shm = sizeof(float) * (MAX_G * D + 4 * MAX_G * ATT_TILE + MAX_G * ATT_TILE +
                                      MAX_G + ck->N * KK + cv->N * KV);
  auto kern = attend_split_ref_kernel<KK, KV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.S, Hkv, B), dim3(ATT_THREADS), shm, s, q, kc, kn, vc, vn, Hq,
                     Hkv, T, p.chunk, scale, ck->t.pi32, ck->t.cb32, ck->N, ck->bits, ck->W,
                     cv->t.cb32, cv->N, cv->bits, cv->W, ws, p.S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(Hq, B), dim3(64), 0, s, ws, p.S, Hq, ck->t.pi32,
                     out);
  return hipGetLastError();
}

template <int KK>
hipError_t dispatch_v(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                      const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                      const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, float scale,
                      float* ws, uint16_t* out, hipStream_t s) {
  switch (cv->k) {
    case 2: return launch_ref<KK, 2>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, ws, out, s);
    case 3: return launch_ref<KK, 3>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, ws, out, s);
    case 4: return launch_ref<KK, 4>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, ws, out, s);
    case 8: return launch_ref<KK, 8>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, ws, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t attend_workspace_bytes(const fq_codebook* /*cb_k*/, int B, int Hq, int Hkv, int64_t T) {
  const SplitPlan p = plan_splits(B, Hkv, T);
  return ((size_t)B * Hq * p.S * PART * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_attend(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                         const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                         const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, float scale,
                         void* ws, uint16_t* out, hipStream_t s) {
  float* w = static_cast<float*>(ws);
  switch (ck->k) {
    case 2: return dispatch_v<2>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, w, out, s);
    case 3: return dispatch_v<3>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, w, out, s);
    case 4: return dispatch_v<4>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, w, out, s);
    case 8: return dispatch_v<8>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, w, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fq
