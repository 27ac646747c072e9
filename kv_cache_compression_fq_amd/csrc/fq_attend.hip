// Fused decode-step attention over the compressed cache (FibQuant technical
// summary, section 5: fixed-address records let decompression be fused into
// attention).  Scores and the value sum are taken in the rotated domain:
//   <q, nu Pi^T z_hat> = nu <Pi q, z_hat>,   sum_t p_t nu_t Pi^T z_hat_t = Pi^T sum_t p_t nu_t z_hat_t
// so only the query is rotated on the way in and the output once on the way out.
//
// Kernel A, one wave per (batch, KV head, split of the context), G = Hq / Hkv <= 8
// query heads per wave, tiles of 64 tokens:
//  * lane t loads the K and V records and norms of token t (unconditional
//    buffer loads, next two tiles in flight) and unpacks them into 16-bit index
//    tables in LDS (value indices permuted so that the four a lane needs sit
//    together);
//  * scores on v_mfma_f32_16x16x32_f16 as one product over a stacked
//    contraction: A = [Z_hi | Z_hi | Z_lo] (the tile's key codewords gathered
//    from the LDS codebook, lo = (c - hi) 2^11), B = [Q_hi ; Q_lo ; Q_hi 2^-11]
//    (the rotated, scaled queries of the group in columns 0..G-1, lo = q - hi),
//    so every product has weight one and a single accumulator holds
//    z_hi q_hi + z_hi q_lo + z_lo q_hi: ~22 bits, which the outlier-heavy caches
//    need (rounding only the key codebook to binary16 moves attention outputs
//    by up to 1e-2 relative);
//  * online softmax in registers: lane (h, g) owns head h and tokens
//    4g..4g+3 of every 16-token sub-tile;
//  * values O^T = Z_v^T P'^T (P' = p * nu_v in binary16): the A operand is
//    fetched with ds_read_tr16_b64 transpose reads pointed straight at the
//    value codewords in LDS (k = 4 or 8), or at value rows expanded into LDS
//    (k = 2 or 3), again as hi and lo parts (binary16 value codewords alone
//    leave errors near 1e-3 relative on outlier-heavy caches); the lo part
//    enters the same accumulator through a second K-step with P' 2^-11;
//  * for k = 4 and 8 both products use v_mfma_f32_16x16x16_f16, whose A
//    operand is one codeword row per lane (scores) or one transpose read
//    (values), and whose B operand for the values is the lane's own four
//    weights, so nothing is repacked;
//  * scores are kept in the log2 domain (the query carries scale * log2 e), so
//    every softmax weight is one exp2;
//  * the wave writes its (m, l, o) partial per query head.
// Kernel B merges the splits (log-sum-exp), applies Pi^T and writes binary16.
#include <type_traits>

#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int ATT_WAVES = 4;
constexpr int ATT_THREADS = 64 * ATT_WAVES;
constexpr int TILE = 64;           // tokens per wave iteration (one lane per token)
constexpr int MAX_G = 8;           // query heads per KV head
constexpr int PART = D + 2;        // floats per partial: m, l, o[64]
constexpr int Q_PITCH = D + 8;     // binary16 row pitch of the query table
constexpr int Z_PITCH = D + 4;     // binary16 row pitch of expanded value rows
constexpr float NEG_BIG = -3.0e38f;

struct SplitPlan {
  int S;          // workgroup splits per (batch, KV head)
  int64_t chunk;  // tokens per workgroup split, a multiple of ATT_WAVES * TILE
};

// About `target` workgroups over the device; each wave gets at least one
// tile.  The four waves of a workgroup take interleaved tiles of its split.
constexpr int64_t SPLIT_TARGET = 512;          // kernel A: two workgroups per compute unit
constexpr int64_t SPLIT_TARGET_DIRECT = 768;   // kernel A': three
SplitPlan plan_splits(int B, int Hkv, int64_t T, int64_t target) {
  constexpr int64_t STEP = (int64_t)ATT_WAVES * TILE;
  const int64_t pairs = (int64_t)B * Hkv;
  int64_t S = (target + pairs - 1) / pairs;
  const int64_t max_s = (T + STEP - 1) / STEP;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  int64_t chunk = (T + S - 1) / S;
  chunk = (chunk + STEP - 1) / STEP * STEP;
  S = (T + chunk - 1) / chunk;
  return {(int)S, chunk};
}

template <int K, int BITS>
struct AttShape {
  using Sh = Shape<K, BITS>;
  static constexpr bool EXPAND = !(K == 4 || K == 8);   // value rows expanded into LDS
  __host__ __device__ static constexpr size_t wave_lds() {
    return (size_t)2 * TILE * Sh::IDX_PITCH * 2 + 2 * TILE * 4 +
           (EXPAND ? (size_t)2 * TILE * Z_PITCH * 2 : 0);
  }
};

template <int W>
struct TileRegs {
  uint32_t kw[W], vw[W];
  uint32_t kn, vn;   // raw binary16 norms
};

// Key codebook layout in LDS.  k = 2, 4, 8: one interleaved row per codeword,
// hi part then lo part (2k binary16), so one read fetches both; k = 3: two
// separate [N][3] tables (gathered a coordinate at a time).
template <int K>
struct KeyTable {
  static constexpr bool INTERLEAVED = (K == 2 || K == 4 || K == 8);
};

// Coordinates [c0, c0 + 8) of one key row, hi and lo parts (c0 multiple of 8).
template <int K>
__device__ inline void gather8_hl(const uint16_t* idx, const _Float16* tab, const _Float16* tab_lo,
                                  int c0, half8& hi, half8& lo) {
  if constexpr (K == 8) {
    const uint32_t i0 = idx[c0 >> 3];
    hi = *reinterpret_cast<const half8*>(tab + i0 * 16);
    lo = *reinterpret_cast<const half8*>(tab + i0 * 16 + 8);
  } else if constexpr (K == 4) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(idx + (c0 >> 2));
    const u32x4 a = *reinterpret_cast<const u32x4*>(tab + (pair & 0xFFFFu) * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(tab + (pair >> 16) * 8);
    const u32x4 hv = {a.x, a.y, b.x, b.y}, lv = {a.z, a.w, b.z, b.w};
    hi = __builtin_bit_cast(half8, hv);
    lo = __builtin_bit_cast(half8, lv);
  } else if constexpr (K == 2) {
    const uint2 q = *reinterpret_cast<const uint2*>(idx + (c0 >> 1));
    const uint2* t = reinterpret_cast<const uint2*>(tab);
    const uint2 a = t[q.x & 0xFFFFu], b = t[q.x >> 16], c = t[q.y & 0xFFFFu], d = t[q.y >> 16];
    const u32x4 hv = {a.x, b.x, c.x, d.x}, lv = {a.y, b.y, c.y, d.y};
    hi = __builtin_bit_cast(half8, hv);
    lo = __builtin_bit_cast(half8, lv);
  } else {  // K = 3: one coordinate at a time; the last block may be partial
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const int j = c / K, t = c - j * K;
      const uint32_t i0 = idx[j];
      hi[e] = tab[i0 * K + t];
      lo[e] = tab_lo[i0 * K + t];
    }
  }
}

// ds_read_tr16_b64: within each 16-lane group, output lane i element m is
// element i % 4 of the 64-bit row addressed by lane 4 m + i / 4 of the group.
__device__ inline half4 read_tr(const _Float16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));  // address-space cast
  return __builtin_bit_cast(half4, v);
}

__device__ inline float rot8(float x) {   // value of lane (l +- 8) within its 16-lane row
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Value record of one token into LDS with the indices permuted for the value
// pass: block b = (16 / K) mt + q goes to position 4 q + mt (k = 4, 8), so a
// lane reads the four blocks of its coordinate quarter with one 8-byte load.
template <int K, int BITS, int W>
__device__ inline void unpack_record_vperm(const uint32_t (&w)[W], uint16_t* dst) {
  constexpr int NB = Shape<K, BITS>::NB;
  constexpr int QB = 16 / K;
  static_assert(NB == 4 * QB, "four blocks per coordinate quarter");
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  uint32_t f[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int pos = j * BITS, wi = pos >> 5, o = pos & 31;
    uint32_t v = w[wi] >> o;
    if (o + BITS > 32) v |= w[wi + 1] << (32 - o);
    f[j] = v & MASK;
  }
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
  for (int i = 0; i < NB / 2; ++i) {
    const int p0 = 2 * i, p1 = 2 * i + 1;              // positions 4 q + mt
    const int b0 = QB * (p0 & 3) + (p0 >> 2), b1 = QB * (p1 & 3) + (p1 >> 2);
    d32[i] = f[b0] | (f[b1] << 16);
  }
}

constexpr int MERGE_PITCH = PART + 2;   // floats per wave partial in the LDS merge area

template <int K, int BITS>
struct AttLds {
  using Sh = Shape<K, BITS>;
  __host__ __device__ static size_t key_bytes(int N) {   // key table(s)
    return ((size_t)N * 2 * K * 2 + 15) / 16 * 16;
  }
  __host__ __device__ static size_t val_bytes(int N) {   // value hi and lo tables
    return 2 * (((size_t)N * K * 2 + 15) / 16 * 16);
  }
  __host__ __device__ static size_t total(int N) {
    return key_bytes(N) + val_bytes(N) + 48 * Q_PITCH * 2 + MAX_G * D * 4 +
           ATT_WAVES * AttShape<K, BITS>::wave_lds() + ATT_WAVES * MAX_G * MERGE_PITCH * 4;
  }
};

// Merge the four waves' partials of each head (held in LDS) and write either
// the workgroup's partial (m, l, o_rot) for the merge kernel or, when the
// context has a single split, the head's output out = Pi^T o_rot / l in
// binary16 (row c of Pi^T from the transposed table).
__device__ inline void finish_heads(const float* sMerge, int G, int Hq, int b, int g, int S, int sw,
                                    float* ws, const float* pi32t, uint16_t* out) {
  __shared__ float sO[MAX_G * D];
  for (int e = threadIdx.x; e < G * D; e += ATT_THREADS) {
    const int h = e / D, c = e % D;
    float M = NEG_BIG;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) M = fmaxf(M, sMerge[(w * MAX_G + h) * MERGE_PITCH]);
    float Ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) {
      const float* pw = sMerge + (w * MAX_G + h) * MERGE_PITCH;
      const float wt = pw[1] > 0.f ? __builtin_amdgcn_exp2f(pw[0] - M) : 0.f;
      Ls = fmaf(wt, pw[1], Ls);
      o = fmaf(wt, pw[2 + c], o);
    }
    if (S > 1) {
      float* dst = ws + (((int64_t)b * Hq + (int64_t)g * G + h) * S + sw) * PART;
      if (c == 0) {
        dst[0] = M;
        dst[1] = Ls;
      }
      dst[2 + c] = o;
    } else {
      sO[e] = o / Ls;
    }
  }
  if (S > 1) return;
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += ATT_THREADS) {
    const int h = e / D, c = e % D;
    const float4* pr = reinterpret_cast<const float4*>(pi32t + c * D);
    float a = 0.f;
#pragma unroll 4
    for (int i = 0; i < D / 4; ++i) {
      const float4 p = pr[i];
      a = fmaf(p.x, sO[h * D + 4 * i], a);
      a = fmaf(p.y, sO[h * D + 4 * i + 1], a);
      a = fmaf(p.z, sO[h * D + 4 * i + 2], a);
      a = fmaf(p.w, sO[h * D + 4 * i + 3], a);
    }
    out[((int64_t)b * Hq + (int64_t)g * G + h) * D + c] = f32_to_f16_rne(a);
  }
}

// One appended vector, encoded by one wave from the float64 definition: the
// norm, z = Pi x / |x| (lane t forms z_t from coalesced rows of Pi^T), then
// for every block the nearest codeword of the binary16 table in LDS (exact:
// the table holds binary16 values) by float64 squared distance, ties to the
// lowest index; the record (LSB-first fields) and the binary16 norm, rounded
// once from the float64 norm.  scratch: 2 * 64 doubles + 64 words per wave.
template <int K, int BITS, int RB>
__device__ void append_one(const uint16_t* x, const _Float16* sTab, int tstride, int N,
                           const double* pi64t, uint32_t* rec, uint16_t* nrm, double* scratch,
                           int lane) {
  // P lanes per block (a power of two, P * NB <= 64); the last block of k = 3
  // has one real coordinate
  constexpr int NB = (D + K - 1) / K, W = Shape<K, BITS>::W;
  constexpr int P = NB <= 8 ? 8 : (NB <= 16 ? 4 : 2);
  double* sX = scratch;
  double* sZ = scratch + D;
  uint32_t* sI = reinterpret_cast<uint32_t*>(scratch + 2 * D);
  // the encode is latency-bound: x and the first RB rows of Pi^T are loaded
  // before the norm's reduction, each further batch of RB rows once the
  // previous one is used (D / RB round trips to memory; RB is what the
  // calling kernel's register budget allows)
  const double xv = (double)f16_bits_to_f32(x[lane]);
  double pv[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) pv[i] = pi64t[i * D + lane];
  double ss = xv * xv;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    int2 v = __builtin_bit_cast(int2, ss);
    v.x = __shfl_xor(v.x, m, 64);
    v.y = __shfl_xor(v.y, m, 64);
    ss += __builtin_bit_cast(double, v);
  }
  const double nu = sqrt(ss);
  sX[lane] = xv;
  wave_lds_sync();
  double acc = 0.0;
#pragma unroll 1
  for (int h = 0; h < D / RB; ++h) {
    if (h > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i) pv[i] = pi64t[(RB * h + i) * D + lane];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) acc = fma(pv[i], sX[RB * h + i], acc);
  }
  sZ[lane] = acc / nu;   // a zero vector gives NaN: every distance is NaN, index 0
  wave_lds_sync();
  const int b = lane / P, p = lane % P;
  const int rd = b < NB ? (D - b * K < K ? D - b * K : K) : 0;   // real coordinates
  double zb[K];
#pragma unroll
  for (int t = 0; t < K; ++t) zb[t] = t < rd ? sZ[b * K + t] : 0.0;
  double best = INFINITY;
  int bi = 0;
  if (b < NB) {
    for (int cn = p; cn < N; cn += P) {
      double dd = 0.0;
#pragma unroll
      for (int t = 0; t < K; ++t) {
        const double df = t < rd ? zb[t] - (double)(float)sTab[cn * tstride + t] : 0.0;
        dd = fma(df, df, dd);
      }
      if (dd < best) {
        best = dd;
        bi = cn;
      }
    }
  }
#pragma unroll
  for (int m = P >> 1; m >= 1; m >>= 1) {
    int2 v = __builtin_bit_cast(int2, best);
    v.x = __shfl_xor(v.x, m, 64);
    v.y = __shfl_xor(v.y, m, 64);
    const double ob = __builtin_bit_cast(double, v);
    const int oi = __shfl_xor(bi, m, 64);
    if (ob < best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (b < NB && p == 0) sI[b] = (uint32_t)bi;
  wave_lds_sync();
  if (lane < W) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p0 = j * BITS - 32 * lane;
      if (p0 >= 32 || p0 + BITS <= 0) continue;
      word |= p0 >= 0 ? (sI[j] << p0) : (sI[j] >> (-p0));
    }
    rec[lane] = word;
  }
  if (lane == 0) *nrm = f64_to_f16_bits(nu);
  wave_lds_sync();
}

// The appended tokens of one (batch, KV head) that fall in a workgroup's
// split, key and value of a token at a time with all four waves (k = 4 or 8,
// binary16 tables in LDS): wave w forms the partial rotation of both vectors
// over coordinates 16 w .. 16 w + 15 (its 16 rows of Pi^T, loaded once for
// all tokens) and its share of both sums of squares; after a barrier, waves
// 0 and 1 search half of the key's blocks each, waves 2 and 3 the value's;
// after a second barrier waves 0 and 2 pack the records and store the norms.
// The definition is append_one's (float64 norm, rotation and distances, ties
// to the lowest index); only the order of the float64 sums differs.
// scratch: 12 * 64 + 8 doubles and 2 * d / k words.
template <int K, int BITS>
__device__ void append_pairs(const AppendIn& app, int64_t stream, int64_t T, int64_t Tld, int64_t ap0,
                             int64_t t1, const _Float16* sK, const _Float16* sV, int N, double* scr,
                             int wave, int lane) {
  constexpr int NB = D / K, W = Shape<K, BITS>::W;
  constexpr int HB = NB / 2;    // blocks per searching wave
  constexpr int P = 64 / HB;    // lanes per block: 8 (k = 4) or 16 (k = 8)
  static_assert(K == 4 || K == 8, "k = 4 or 8");
  double* sP = scr;                              // [wave][vector][64] partial rotations
  double* sS = scr + 8 * D;                      // [wave][vector] partial sums of squares
  double* sZ = scr + 8 * D + 8 + wave * D;       // this wave's z
  uint32_t* sI = reinterpret_cast<uint32_t*>(scr + 12 * D + 8);   // [vector][NB] indices
  double pv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pv[i] = app.pi64t[(16 * wave + i) * D + lane];
  const int v = wave >> 1, hb = wave & 1;
  const _Float16* tab = v ? sV : sK;
  // x of token t (key and value; lane = coordinate), one token ahead
  auto xload = [&](int64_t t, int& xk, int& xv) {
    const int64_t row = stream * app.M + (t - (T - app.M));
    xk = app.k_new[row * D + lane];
    xv = app.v_new[row * D + lane];
  };
  int nk = 0, nv = 0;
  if (ap0 < t1) xload(ap0, nk, nv);
  for (int64_t t = ap0; t < t1; ++t) {
    const int xk = nk, xv = nv;
    if (t + 1 < t1) xload(t + 1, nk, nv);
    double ak = 0.0, av = 0.0, sk = 0.0, sv = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double a = (double)f16_bits_to_f32((uint16_t)__builtin_amdgcn_readlane(xk, 16 * wave + i));
      const double c = (double)f16_bits_to_f32((uint16_t)__builtin_amdgcn_readlane(xv, 16 * wave + i));
      ak = fma(pv[i], a, ak);
      av = fma(pv[i], c, av);
      sk = fma(a, a, sk);
      sv = fma(c, c, sv);
    }
    sP[(2 * wave) * D + lane] = ak;
    sP[(2 * wave + 1) * D + lane] = av;
    if (lane == 0) {
      sS[2 * wave] = sk;
      sS[2 * wave + 1] = sv;
    }
    __syncthreads();
    const double nu = sqrt(((sS[v] + sS[2 + v]) + sS[4 + v]) + sS[6 + v]);
    // a zero vector gives NaN: every distance is NaN, index 0
    sZ[lane] = (((sP[v * D + lane] + sP[(2 + v) * D + lane]) + sP[(4 + v) * D + lane]) +
                sP[(6 + v) * D + lane]) / nu;
    wave_lds_sync();
    const int b = hb * HB + lane / P, p = lane % P;
    double zb[K];
#pragma unroll
    for (int e = 0; e < K; ++e) zb[e] = sZ[b * K + e];
    double best = INFINITY;
    int bi = 0;
    for (int cn = p; cn < N; cn += P) {
      const _Float16* cr = tab + cn * K;
      double dd = 0.0;
#pragma unroll
      for (int e = 0; e < K; ++e) {
        const double df = zb[e] - (double)(float)cr[e];
        dd = fma(df, df, dd);
      }
      if (dd < best) {
        best = dd;
        bi = cn;
      }
    }
#pragma unroll
    for (int m = P >> 1; m >= 1; m >>= 1) {
      int2 q = __builtin_bit_cast(int2, best);
      q.x = __shfl_xor(q.x, m, 64);
      q.y = __shfl_xor(q.y, m, 64);
      const double ob = __builtin_bit_cast(double, q);
      const int oi = __shfl_xor(bi, m, 64);
      if (ob < best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (p == 0) sI[v * NB + b] = (uint32_t)bi;
    __syncthreads();
    if (hb == 0) {
      const int64_t r = stream * Tld + t;
      if (lane < W) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int p0 = j * BITS - 32 * lane;
          if (p0 >= 32 || p0 + BITS <= 0) continue;
          const uint32_t f = sI[v * NB + j];
          word |= p0 >= 0 ? (f << p0) : (f >> (-p0));
        }
        (v ? app.vc : app.kc)[r * W + lane] = word;
      }
      if (lane == 0) (v ? app.vn : app.kn)[r] = f64_to_f16_bits(nu);
    }
  }
}

template <int K, int BITS>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void attend_split_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kc,
    const uint16_t* __restrict__ kn, const uint32_t* __restrict__ vc,
    const uint16_t* __restrict__ vn, int Hq, int Hkv, int64_t T, int64_t Tld, int Mq,
    int64_t chunk, int S,
    float scale, const float* __restrict__ pi32, const _Float16* __restrict__ kh_g,
    const _Float16* __restrict__ kl_g, const _Float16* __restrict__ vh_g,
    const _Float16* __restrict__ vl_g, int N, float* __restrict__ ws,
    const float* __restrict__ pi32t, uint16_t* __restrict__ out, AppendIn app) {
  using Sh = Shape<K, BITS>;
  using AS = AttShape<K, BITS>;
  using L = AttLds<K, BITS>;
  constexpr int W = Sh::W, IP = Sh::IDX_PITCH;
  const int G = Hq / Hkv;
  const int sw = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;

  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* sK = reinterpret_cast<_Float16*>(smem);                      // key table(s)
  _Float16* sKlo = sK + (size_t)N * K;                                   // k = 3 lo table
  _Float16* sVh = reinterpret_cast<_Float16*>(smem + L::key_bytes(N));
  _Float16* sVl = reinterpret_cast<_Float16*>(smem + L::key_bytes(N) + L::val_bytes(N) / 2);
  _Float16* sQ = reinterpret_cast<_Float16*>(smem + L::key_bytes(N) + L::val_bytes(N));
  float* sQf = reinterpret_cast<float*>(sQ + 48 * Q_PITCH);             // [MAX_G][D] raw q
  unsigned char* wbase = reinterpret_cast<unsigned char*>(sQf + MAX_G * D) +
                         (size_t)wave * AS::wave_lds();
  float* sMerge = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(sQf + MAX_G * D) +
                                           ATT_WAVES * AS::wave_lds());   // [wave][h][MERGE_PITCH]
  uint16_t* sKi = reinterpret_cast<uint16_t*>(wbase);            // [TILE][IP]
  uint16_t* sVi = sKi + TILE * IP;                               // [TILE][IP]
  float* sNk = reinterpret_cast<float*>(sVi + TILE * IP);        // [TILE]
  float* sNv = sNk + TILE;                                       // [TILE]
  _Float16* sZh = reinterpret_cast<_Float16*>(sNv + TILE);       // [TILE][Z_PITCH] (expand)
  _Float16* sZl = sZh + TILE * Z_PITCH;

  for (int e = threadIdx.x; e < N * K; e += ATT_THREADS) {
    const int n = e / K, t = e - n * K;
    if constexpr (KeyTable<K>::INTERLEAVED) {
      sK[n * 2 * K + t] = kh_g[e];
      sK[n * 2 * K + K + t] = kl_g[e];
    } else {
      sK[e] = kh_g[e];
      sKlo[e] = kl_g[e];
    }
    if constexpr (AS::EXPAND) {
      sVh[e] = vh_g[e];
      sVl[e] = vl_g[e];
    } else {   // interleaved rows [hi | lo] like the key table
      sVh[n * 2 * K + t] = vh_g[e];
      sVh[n * 2 * K + K + t] = vl_g[e];
    }
  }
  for (int e = threadIdx.x; e < MAX_G * D; e += ATT_THREADS) {
    const int h = e / D;
    sQf[e] = h < G ? f16_bits_to_f32(q[((int64_t)b * Hq + (int64_t)g * G + h) * D + (e % D)]) : 0.f;
  }
  __syncthreads();
  // rotated, scaled queries, three parts of 16 rows (heads; rows >= G are
  // zero): part 0 = hi, part 1 = lo = q - hi, part 2 = hi 2^-11; thread (c, hq)
  // forms coordinate c of heads hq and hq + 4
  {
    const int c = threadIdx.x & 63, hq = threadIdx.x >> 6;
    const float4* prow = reinterpret_cast<const float4*>(pi32 + c * D);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 4
    for (int i4 = 0; i4 < D / 4; ++i4) {
      const float4 p = prow[i4];
      const float4 x0 = *reinterpret_cast<const float4*>(sQf + hq * D + 4 * i4);
      const float4 x1 = *reinterpret_cast<const float4*>(sQf + (hq + 4) * D + 4 * i4);
      a0 = fmaf(p.x, x0.x, fmaf(p.y, x0.y, fmaf(p.z, x0.z, fmaf(p.w, x0.w, a0))));
      a1 = fmaf(p.x, x1.x, fmaf(p.y, x1.y, fmaf(p.z, x1.z, fmaf(p.w, x1.w, a1))));
    }
    a0 *= scale * 1.4426950408889634f;   // scores in log2 units
    a1 *= scale * 1.4426950408889634f;
    const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
    sQ[hq * Q_PITCH + c] = h0;
    sQ[(hq + 4) * Q_PITCH + c] = h1;
    sQ[(16 + hq) * Q_PITCH + c] = (_Float16)(a0 - (float)h0);
    sQ[(16 + hq + 4) * Q_PITCH + c] = (_Float16)(a1 - (float)h1);
    sQ[(32 + hq) * Q_PITCH + c] = (_Float16)((float)h0 * 0x1p-11f);
    sQ[(32 + hq + 4) * Q_PITCH + c] = (_Float16)((float)h1 * 0x1p-11f);
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      sQ[(16 * part + 8 + hq) * Q_PITCH + c] = (_Float16)0.f;
      sQ[(16 * part + 12 + hq) * Q_PITCH + c] = (_Float16)0.f;
    }
  }
  __syncthreads();

  const int64_t t0 = (int64_t)sw * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
  const int64_t stream = (int64_t)b * Hkv + g;
  constexpr int64_t WSTEP = (int64_t)ATT_WAVES * TILE;

  // appended tokens in this split: encoded before any tile is read, from the
  // binary16 tables in LDS (hi parts; the launcher sends codebooks whose
  // tables are binary16 values), the merge area as scratch
  {
    const int64_t ap0 = T - app.M > t0 ? T - app.M : t0;
    if (app.M > 0 && ap0 < t1) {
      const int nv = 2 * (int)(t1 - ap0);
      constexpr int KST = KeyTable<K>::INTERLEAVED ? 2 * K : K;   // key table row
      constexpr int VST = AS::EXPAND ? K : 2 * K;                  // value table row
      for (int v = wave; v < nv; v += ATT_WAVES) {
        const int64_t t = ap0 + v / 2;
        const bool isv = v & 1;
        const uint16_t* x =
            (isv ? app.v_new : app.k_new) + (stream * app.M + (t - (T - app.M))) * D;
        const int64_t r = stream * Tld + t;
        append_one<K, BITS, 8>(x, isv ? sVh : sK, isv ? VST : KST, N, app.pi64t,
                            (isv ? app.vc : app.kc) + r * W, (isv ? app.vn : app.kn) + r,
                            reinterpret_cast<double*>(sMerge) + wave * (2 * D + D / 2), lane);
      }
      __threadfence_block();   // the new records are stored before any wave reads them
      __syncthreads();
    }
  }

  // B operands of the score product, K-steps 0..5: part s / 2, coordinates
  // 32 (s % 2) + 8 grp + e, column (head) col
  half8 qf[AS::EXPAND ? 6 : 1];
  half4 q16[AS::EXPAND ? 1 : 3][AS::EXPAND ? 1 : 4];   // direct path: [part][K-step of 16]
  if constexpr (AS::EXPAND) {
#pragma unroll
    for (int s = 0; s < 6; ++s)
      qf[s] = *reinterpret_cast<const half8*>(sQ + (16 * (s >> 1) + col) * Q_PITCH +
                                              32 * (s & 1) + 8 * grp);
  } else {
#pragma unroll
    for (int part = 0; part < 3; ++part)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        q16[part][m] = *reinterpret_cast<const half4*>(sQ + (16 * part + col) * Q_PITCH + 16 * m +
                                                       4 * grp);
  }

  float m_run = NEG_BIG, l_run = 0.f;
  floatx4 oh[4], ol[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    oh[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    ol[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto load = [&](TileRegs<W>& t, int64_t tb) __attribute__((always_inline)) {
    const int64_t left = t1 - tb;
    const int cnt = left <= 0 ? 0 : (left < TILE ? (int)left : TILE);
    const int64_t rec0 = stream * Tld + (left <= 0 ? 0 : tb);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(kc + rec0 * W), (short)0, cnt * W * 4, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(vc + rec0 * W), (short)0, cnt * W * 4, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kn + rec0), (short)0, cnt * 2, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vn + rec0), (short)0, cnt * 2, BUF_DWORD3);
    load_record<W>(t.kw, rk, (uint32_t)(lane * W * 4));
    load_record<W>(t.vw, rv, (uint32_t)(lane * W * 4));
    t.kn = __builtin_amdgcn_raw_buffer_load_b16(rkn, lane * 2, 0, 0);
    t.vn = __builtin_amdgcn_raw_buffer_load_b16(rvn, lane * 2, 0, 0);
  };
  auto stage = [&](const TileRegs<W>& t) __attribute__((always_inline)) {
    if constexpr (AS::EXPAND)
      unpack_record<K, BITS, W>(t.kw, sKi + lane * IP);
    else
      unpack_record_vperm<K, BITS, W>(t.kw, sKi + lane * IP);
    if constexpr (AS::EXPAND)
      unpack_record<K, BITS, W>(t.vw, sVi + lane * IP);
    else
      unpack_record_vperm<K, BITS, W>(t.vw, sVi + lane * IP);
    sNk[lane] = f16_bits_to_f32((uint16_t)t.kn);
    sNv[lane] = f16_bits_to_f32((uint16_t)t.vn);
    if constexpr (AS::EXPAND) {
      // the lane writes its own value row (hi and lo) for the transpose reads
      const uint16_t* vi = sVi + lane * IP;
#pragma unroll
      for (int c0 = 0; c0 < D; c0 += 8) {
        half8 hh, ll;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e, j = c / K;
          hh[e] = sVh[vi[j] * K + (c - j * K)];
          ll[e] = sVl[vi[j] * K + (c - j * K)];
        }
        *reinterpret_cast<half4*>(sZh + lane * Z_PITCH + c0) = half4{hh[0], hh[1], hh[2], hh[3]};
        *reinterpret_cast<half4*>(sZh + lane * Z_PITCH + c0 + 4) = half4{hh[4], hh[5], hh[6], hh[7]};
        *reinterpret_cast<half4*>(sZl + lane * Z_PITCH + c0) = half4{ll[0], ll[1], ll[2], ll[3]};
        *reinterpret_cast<half4*>(sZl + lane * Z_PITCH + c0 + 4) = half4{ll[4], ll[5], ll[6], ll[7]};
      }
    }
  };

  // k = 4, 8: v_mfma_f32_16x16x16_f16 throughout.  Scores: lane (col, grp)
  // gives A = key row of token 16 sub + col, coordinates 16 m + 4 grp .. + 3
  // (one codeword row for k = 4, half of one for k = 8; hi and lo from one
  // interleaved table row).  Values: A = value coordinates 16 mt + col of
  // tokens 16 sub + 4 grp + 0..3 (transpose reads), B = the lane's own four
  // weights p * nu of sub-tile sub, so no operand needs repacking.
  auto process_direct = [&](int64_t tb, auto partial_tag) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    constexpr int QB = 16 / K;                          // blocks per 16 coordinates
    const int qs = grp / (4 / QB), cs = (4 * grp) % K;  // score: index slot, offset in row
    const int qv = (col & 3) / (4 / QB), cv = (4 * (col & 3)) % K;   // value: same
    float sc[4][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const u32x2 ix = *reinterpret_cast<const u32x2*>(sKi + (16 * sub + col) * IP + 4 * qs);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t wd = m < 2 ? ix.x : ix.y;
        const uint32_t i = (m & 1) ? (wd >> 16) : (wd & 0xFFFFu);
        const _Float16* row = sK + i * (2 * K) + cs;
        const half4 zh = *reinterpret_cast<const half4*>(row);
        const half4 zl = *reinterpret_cast<const half4*>(row + K);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(zh, q16[0][m], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(zh, q16[1][m], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(zl, q16[2][m], acc, 0, 0, 0);
      }
      const float4 nk4 = *reinterpret_cast<const float4*>(sNk + 16 * sub + 4 * grp);
      sc[sub][0] = acc[0] * nk4.x;
      sc[sub][1] = acc[1] * nk4.y;
      sc[sub][2] = acc[2] * nk4.z;
      sc[sub][3] = acc[3] * nk4.w;
    }
    if constexpr (PARTIAL) {
      // past the split's end, or past this query's causal limit
      const int valid = (int)(t1 - tb);
      const int64_t lim = T - Mq + (col % MAX_G) % Mq - tb;   // last token this query sees
      const int vq = lim + 1 < (int64_t)valid ? (int)(lim + 1) : valid;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * sub + 4 * grp + r >= vq) sc[sub][r] = NEG_BIG;
    }
    float mx = NEG_BIG;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oh[mt] *= alpha;
    }
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const float4 nv4 = *reinterpret_cast<const float4*>(sNv + 16 * sub + 4 * grp);
      const float nvv[4] = {nv4.x, nv4.y, nv4.z, nv4.w};
      half4 pw, pwl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[sub][r] - m_new);
        ps += p;
        const float w = p * nvv[r];
        pw[r] = (_Float16)w;
        pwl[r] = (_Float16)(w * 0x1p-11f);
      }
      // values of tokens 16 sub + 4 grp + 0..3; lane (col, grp) addresses token
      // 16 sub + 4 grp + col / 4 for the transpose reads
      const u32x2 ixv = *reinterpret_cast<const u32x2*>(sVi + (16 * sub + 4 * grp + (col >> 2)) * IP +
                                                        4 * qv);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t wd = mt < 2 ? ixv.x : ixv.y;
        const uint32_t i = (mt & 1) ? (wd >> 16) : (wd & 0xFFFFu);
        const _Float16* row = sVh + i * (2 * K) + cv;
        const half4 vh = read_tr(row), vl = read_tr(row + K);
        oh[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vh, pw, oh[mt], 0, 0, 0);
        oh[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vl, pwl, oh[mt], 0, 0, 0);
      }
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run += ps;
  };

  auto process = [&](int64_t tb, auto partial_tag) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    // ---- scores for the 4 sub-tiles of 16 tokens (lanes of columns >= G hold
    //      zeros)
    float sc[4][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const uint16_t* ki = sKi + (16 * sub + col) * IP;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        half8 zh, zl;
        gather8_hl<K>(ki, sK, sKlo, 32 * s2 + 8 * grp, zh, zl);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zh, qf[s2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zh, qf[2 + s2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zl, qf[4 + s2], acc, 0, 0, 0);
      }
      const float4 nk4 = *reinterpret_cast<const float4*>(sNk + 16 * sub + 4 * grp);
      sc[sub][0] = acc[0] * nk4.x;
      sc[sub][1] = acc[1] * nk4.y;
      sc[sub][2] = acc[2] * nk4.z;
      sc[sub][3] = acc[3] * nk4.w;
    }
    if constexpr (PARTIAL) {
      // past the split's end, or past this query's causal limit
      const int valid = (int)(t1 - tb);
      const int64_t lim = T - Mq + (col % MAX_G) % Mq - tb;   // last token this query sees
      const int vq = lim + 1 < (int64_t)valid ? (int)(lim + 1) : valid;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * sub + 4 * grp + r >= vq) sc[sub][r] = NEG_BIG;
    }
    // ---- online softmax (lane owns head col; its group lanes share the head)
    float mx = NEG_BIG;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    // rescale the accumulators only when some head's running max moved
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        oh[mt] *= alpha;
        ol[mt] *= alpha;
      }
    }
    m_run = m_new;
    float ps = 0.f;
    half8 pb[2];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const float4 nv4 = *reinterpret_cast<const float4*>(sNv + 16 * sub + 4 * grp);
      const float nv[4] = {nv4.x, nv4.y, nv4.z, nv4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[sub][r] - m_new);
        ps += p;
        pb[sub >> 1][4 * (sub & 1) + r] = (_Float16)(p * nv[r]);
      }
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run += ps;
    // ---- values: K slot (grp, e) holds token 32 ks + 4 grp + (e & 3) + 16 (e >> 2)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int tok_a = 32 * ks + 4 * grp + (col >> 2);
      const int tok_b = tok_a + 16;
      // value indices of blocks (16 / K) mt + q for mt = 0..3 (permuted layout)
      constexpr int QB = 16 / (K < 16 ? K : 16);
      const int qv = (4 * (col & 3)) / K, cin = (4 * (col & 3)) % K;
      u32x2 ixa = {0u, 0u}, ixb = {0u, 0u};
      if constexpr (!AS::EXPAND) {
        ixa = *reinterpret_cast<const u32x2*>(sVi + tok_a * IP + 4 * qv);
        ixb = *reinterpret_cast<const u32x2*>(sVi + tok_b * IP + 4 * qv);
      }
      (void)QB;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int c = 16 * mt + 4 * (col & 3);
        const _Float16 *pah, *pal, *pbh, *pbl;
        if constexpr (AS::EXPAND) {
          pah = sZh + tok_a * Z_PITCH + c;
          pal = sZl + tok_a * Z_PITCH + c;
          pbh = sZh + tok_b * Z_PITCH + c;
          pbl = sZl + tok_b * Z_PITCH + c;
        } else {
          const uint32_t wa = (mt < 2) ? ixa.x : ixa.y, wb = (mt < 2) ? ixb.x : ixb.y;
          const uint32_t ia = (mt & 1) ? (wa >> 16) : (wa & 0xFFFFu);
          const uint32_t ib = (mt & 1) ? (wb >> 16) : (wb & 0xFFFFu);
          pah = sVh + ia * K + cin;
          pal = sVl + ia * K + cin;
          pbh = sVh + ib * K + cin;
          pbl = sVl + ib * K + cin;
        }
        const half4 ha = read_tr(pah), hb = read_tr(pbh), la = read_tr(pal), lb = read_tr(pbl);
        const half8 zh = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
        const half8 zl = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3]};
        oh[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(zh, pb[ks], oh[mt], 0, 0, 0);
        ol[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(zl, pb[ks], ol[mt], 0, 0, 0);
      }
    }
  };

  // wave w takes tiles t0 + (w + 4 i) TILE of the workgroup's split; four tiles
  // of records are in flight per wave (HBM latency needs the bytes in flight)
  int64_t tb = t0 + (int64_t)wave * TILE;
  if (tb < t1) {
    // masked tiles: a partial last tile, or (several queries per head) a
    // tile reaching past T - Mq, where later queries see more tokens
    auto run = [&](int64_t t) __attribute__((always_inline)) {
      const bool plain = t1 - t >= TILE && t + TILE <= T - Mq + 1;
      if constexpr (AS::EXPAND) {
        if (plain)
          process(t, std::false_type());
        else
          process(t, std::true_type());
      } else {
        if (plain)
          process_direct(t, std::false_type());
        else
          process_direct(t, std::true_type());
      }
    };
    // Every path through the loop issues the same loads (a tile past the end
    // is a zero-length buffer read that touches no memory), so the compiler's
    // load counter stays exact across iterations and the waits stay partial;
    // only the load-free compute is skipped for such tiles.
    constexpr int DEPTH = AS::EXPAND ? 2 : 4;
    TileRegs<W> rr[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load(rr[d], tb + d * WSTEP);
    for (;;) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        stage(rr[d]);
        wave_lds_sync();
        load(rr[d], tb + DEPTH * WSTEP);
        if (tb < t1) run(tb);
        wave_lds_sync();
        tb += WSTEP;
      }
      if (tb >= t1) break;
    }
  }

  // ---- merge the four waves' partials of each head in LDS, write one partial
  if (col < G) {
    float* mine = sMerge + (wave * MAX_G + col) * MERGE_PITCH;
    if (grp == 0) {
      mine[0] = m_run;
      mine[1] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mine[2 + 16 * mt + 4 * grp + r] = fmaf(ol[mt][r], 0x1p-11f, oh[mt][r]);
  }
  __syncthreads();
  finish_heads(sMerge, G, Hq, b, g, S, sw, ws, pi32t, out);
}

// One workgroup of 256 per (batch, query head): log-sum-exp merge of the S
// split partials, then out = Pi^T o_rot in binary16.  Thread (c, part) merges
// the splits s = part (mod 4) for coordinate c and forms the part's quarter
// of the rotation; every global load is issued before the first barrier, so
// the whole merge waits on memory once.
__global__ __launch_bounds__(256) void attend_merge_kernel(const float* __restrict__ ws, int S,
                                                           const float* __restrict__ pi32t,
                                                           uint16_t* __restrict__ out) {
  const int64_t bh = blockIdx.x;   // b * Hq + h
  const int c = threadIdx.x & 63, part = threadIdx.x >> 6;
  float4 pr[4];   // Pi^T row c, entries 16 part .. 16 part + 15
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = reinterpret_cast<const float4*>(pi32t + c * D + 16 * part)[i];
  // the head's partials as a buffer: loads past the end read zero (and are
  // then masked), so each batch of four splits loads with no branch
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ws + bh * S * PART), (short)0, S * PART * 4, BUF_DWORD3);
  float m = NEG_BIG, l = 0.f, o = 0.f;
  for (int s0 = 0; s0 < S; s0 += 16) {   // online merge of this part's splits
    float ms[4], ls[4], os[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + part + 4 * k;
      const uint32_t off = (uint32_t)s * PART * 4;
      ms[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
      ls[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 4, 0, 0));
      os[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 8 + 4 * c, 0, 0));
      if (s >= S) ms[k] = NEG_BIG;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float mn = fmaxf(m, ms[k]);
      const float a = __builtin_amdgcn_exp2f(m - mn), w = __builtin_amdgcn_exp2f(ms[k] - mn);
      l = fmaf(l, a, ls[k] * w);
      o = fmaf(o, a, os[k] * w);
      m = mn;
    }
  }
  __shared__ float sm[4], sl[4], so[4][D], sd[4][D];
  if (c == 0) {
    sm[part] = m;
    sl[part] = l;
  }
  so[part][c] = o;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float L = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) L = fmaf(sl[q], __builtin_amdgcn_exp2f(sm[q] - M), L);
  // this thread's quarter of the rotation: coordinates j = 16 part .. + 15
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 16 * part + 4 * i + e;
      float oj = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) oj = fmaf(so[q][j], __builtin_amdgcn_exp2f(sm[q] - M), oj);
      acc = fmaf(pr[i][e], oj, acc);
    }
  }
  sd[part][c] = acc;
  __syncthreads();
  if (part == 0)
    out[bh * D + c] = f32_to_f16_rne((sd[0][c] + sd[1][c] + sd[2][c] + sd[3][c]) / L);
}

// ---------------------------------------------------------------------------
// Kernel A', used when both codebooks hold binary16-exact values (binary16
// tables then lose nothing), k = 4 or 8, and T is a multiple of 8 (every norm
// row 16-byte aligned).  Per wave and 64-token tile:
//  * four loads, each one contiguous span: key records and value records (a
//    record per lane, lanes permuted), key and value norms (8 tokens per lane);
//  * a record's 64 coordinates split into four quarters of 16 (16 / k whole
//    blocks); quarters are redistributed in registers -- a 4 x 4 transpose
//    across the wave's 16-lane rows (permlane swaps) for keys, within lane
//    quads (DPP) for values -- so no index goes through LDS and the token
//    loop has no barrier;
//  * scores on v_mfma_f32_16x16x32_f16, tokens as rows: row i of sub-tile s
//    is token 16 (i / 4) + 4 s + i % 4, and lane (col, grp) supplies quarter
//    grp of its row's token; the B operand holds the query hi parts of the
//    group's heads in columns 0..7 and their lo parts (q - hi, binary16) in
//    columns 8..15, so score = D[., h] + D[., h + 8] (one row rotation);
//  * the softmax runs on distinct work per lane: lane (col, grp) takes head
//    col % 8 and tokens 16 grp + 8 (col / 8) + 0..7;
//  * values O^T = Z^T P'^T on the same instruction, P' = p nu_v in binary16:
//    K-step ks covers tokens 16 grp + 8 ks + 0..7, its A operand comes from
//    transpose reads of 4-coordinate codeword pieces (output row i of slice
//    mt is coordinate 16 (i / 4) + 4 mt + i % 4) and its B operand holds the
//    weights of lane (col % 8) + 8 ks of the row; columns 8..15 of the
//    product are not used.
template <int K, int BITS>
struct DirectCfg {
  static constexpr int W = Shape<K, BITS>::W;
  static constexpr int QB = 16 / K;              // blocks in a quarter
  static constexpr int QBITS = QB * BITS;        // bits in a quarter
  static constexpr uint32_t MASK = (1u << BITS) - 1u;
  static_assert(K == 4 || K == 8, "direct kernel: k = 4 or 8");
  static_assert(QBITS * 4 == W * 32, "four quarters fill the record");
  static_assert(W == 1 || W == 2 || W == 4, "record of 1, 2 or 4 words");
};

template <int W>
struct DTile {
  uint32_t k[W];   // key record of token 16 (col / 4) + 4 grp + col % 4
  uint32_t v[W];   // value record of token 16 grp + 4 (col % 4) + col / 4
  u32x4 nk;        // key norms of tokens 16 grp + 8 (col / 8) + 0..7
  u32x4 nv;        // value norms of the same tokens
};

template <int K, int BITS>
struct DirectLds {
  // at least 16 bytes per thread, so that every thread stores its table load
  static constexpr int TABLE = (1 << BITS) * K * 2 > ATT_THREADS * 16 ? (1 << BITS) * K * 2
                                                                       : ATT_THREADS * 16;
  static constexpr int QOFF = 2 * TABLE;                       // query operand rows
  static constexpr int MOFF = QOFF + 16 * Q_PITCH * 2;         // wave partials
  static constexpr int TOTAL = MOFF + ATT_WAVES * MAX_G * MERGE_PITCH * 4;
};

// The four quarters of a record, each in the low bits of a word.
template <int K, int BITS, int W>
__device__ inline void quarters(const uint32_t (&w)[W], uint32_t (&q)[4]) {
  constexpr int QBITS = DirectCfg<K, BITS>::QBITS;
  if constexpr (W == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = w[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = j * QBITS;
      q[j] = (w[pos >> 5] >> (pos & 31)) & ((1u << QBITS) - 1u);
    }
  }
}

// 4 x 4 transpose across the four 16-lane rows: on return, register c of the
// lane in row r holds what register r of the same column's lane in row c held.
__device__ inline void transpose_rows(uint32_t (&x)[4]) {
  auto s02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  x[0] = s01[0];
  x[1] = s01[1];
  x[2] = s23[0];
  x[3] = s23[1];
}

// 4 x 4 transpose within each quad of lanes: on return, register j of quad
// lane q holds what register q of quad lane j held.
__device__ inline void transpose_quads(uint32_t (&x)[4], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2;
  // exchange across lane bit 0 / register bit 0
#pragma unroll
  for (int p = 0; p < 4; p += 2) {
    const uint32_t send = b0 ? x[p] : x[p + 1];
    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    if (b0) x[p] = got; else x[p + 1] = got;
  }
  // exchange across lane bit 1 / register bit 1
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t send = b1 ? x[p] : x[p + 2];
    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    if (b1) x[p] = got; else x[p + 2] = got;
  }
}

__device__ inline uint32_t rot8u(uint32_t x) {   // value of lane (l +- 8) within its 16-lane row
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, true);
}

// Reductions over the four 16-lane rows of the wave (lanes l, l + 16, l + 32,
// l + 48), on permlane swaps: no LDS round trip.
__device__ inline float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ inline float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ inline float half_at(const u32x4& v, int i) {   // binary16 number i of 8
  const uint32_t w = v[i >> 1];
  return f16_bits_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

template <int K, int BITS>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void attend_direct_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kc,
    const uint16_t* __restrict__ kn, const uint32_t* __restrict__ vc,
    const uint16_t* __restrict__ vn, int Hq, int Hkv, int64_t T, int64_t Tld, int Mq,
    int64_t chunk, int S,
    float scale, const _Float16* __restrict__ pih_g, const _Float16* __restrict__ pil_g,
    const _Float16* __restrict__ kh_g, const _Float16* __restrict__ vh_g, int N,
    float* __restrict__ ws, const float* __restrict__ pi32t, uint16_t* __restrict__ out,
    AppendIn app) {
  using C = DirectCfg<K, BITS>;
  using L = DirectLds<K, BITS>;
  constexpr int W = C::W;
  const int G = Hq / Hkv;
  const int sw = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int half = col >> 3;   // which 8 tokens of the row's 16 the lane's softmax takes

  // static layout, so that table offsets fold into the LDS instructions
  __shared__ __align__(16) unsigned char smem[L::TOTAL];
  _Float16* sK = reinterpret_cast<_Float16*>(smem);                 // [N][K]
  _Float16* sV = reinterpret_cast<_Float16*>(smem + L::TABLE);      // [N][K]
  _Float16* sQ = reinterpret_cast<_Float16*>(smem + L::QOFF);       // [16][Q_PITCH]
  float* sMerge = reinterpret_cast<float*>(smem + L::MOFF);         // [wave][h][pitch]

  const int64_t t0 = (int64_t)sw * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
  const uint32_t ntok = (uint32_t)(t1 - t0);
  const int64_t rec0 = ((int64_t)b * Hkv + g) * Tld + t0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(kc + rec0 * W), (short)0, (int)(ntok * W * 4), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(vc + rec0 * W), (short)0, (int)(ntok * W * 4), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kn + rec0), (short)0, (int)(ntok * 2), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vn + rec0), (short)0, (int)(ntok * 2), BUF_DWORD3);

  // Every tile load is unconditional: a tile past the split's end reads
  // nothing (out of the buffer range) and yields zeros.
  const uint32_t tok_k = 16 * (col >> 2) + 4 * grp + (col & 3);
  const uint32_t tok_v = 16 * grp + 4 * (col & 3) + (col >> 2);
  const uint32_t tok_n = 16 * grp + 8 * half;
  auto load = [&](DTile<W>& t, uint32_t rel) __attribute__((always_inline)) {
    if constexpr (W == 4) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rk, (rel + tok_k) * 16, 0, 0);
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rv, (rel + tok_v) * 16, 0, 0);
      t.k[0] = a.x; t.k[1] = a.y; t.k[2] = a.z; t.k[3] = a.w;
      t.v[0] = c.x; t.v[1] = c.y; t.v[2] = c.z; t.v[3] = c.w;
    } else if constexpr (W == 2) {
      const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rk, (rel + tok_k) * 8, 0, 0);
      const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(rv, (rel + tok_v) * 8, 0, 0);
      t.k[0] = a.x; t.k[1] = a.y;
      t.v[0] = c.x; t.v[1] = c.y;
    } else {
      t.k[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, (rel + tok_k) * 4, 0, 0);
      t.v[0] = __builtin_amdgcn_raw_buffer_load_b32(rv, (rel + tok_v) * 4, 0, 0);
    }
    t.nk = __builtin_amdgcn_raw_buffer_load_b128(rkn, (rel + tok_n) * 2, 0, 0);
    t.nv = __builtin_amdgcn_raw_buffer_load_b128(rvn, (rel + tok_n) * 2, 0, 0);
    // one group per tile, in the same order everywhere: the load counter
    // waits are static, so a reordered group would make every wait in the
    // loop drain later tiles too
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue loads first (tables, query and rotation fragments), then
  //      the first tiles, so the tile loads fly while the prologue computes
  const int tbytes = N * K * 2;
  const __amdgpu_buffer_rsrc_t rkt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(kh_g), (short)0, tbytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rvt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(vh_g), (short)0, tbytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q + ((int64_t)b * Hq + (int64_t)g * G) * D), (short)0, G * D * 2,
      BUF_DWORD3);
  const u32x4 kt4 = __builtin_amdgcn_raw_buffer_load_b128(rkt, threadIdx.x * 16, 0, 0);
  const u32x4 vt4 = __builtin_amdgcn_raw_buffer_load_b128(rvt, threadIdx.x * 16, 0, 0);
  // rotation on v_mfma_f32_16x16x32_f16: wave w forms rotated coordinates
  // 16 w .. 16 w + 15 of every head, qrot[h][n] = sum_k q[h][k] Pi[n][k], with
  // Pi = hi + 2^-11 lo (both binary16): A = query rows (heads), B = Pi rows
  half8 qa[2], ph[2], pl[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    qa[s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                                          rq, (col * D + 32 * s + 8 * grp) * 2, 0, 0));
    ph[s] = *reinterpret_cast<const half8*>(pih_g + (16 * wave + col) * D + 32 * s + 8 * grp);
    pl[s] = *reinterpret_cast<const half8*>(pil_g + (16 * wave + col) * D + 32 * s + 8 * grp);
  }
  __builtin_amdgcn_sched_barrier(0);

  constexpr int DEPTH = 4;
  constexpr uint32_t WSTEP = ATT_WAVES * TILE;
  uint32_t rel = (uint32_t)wave * TILE;
  DTile<W> rr[DEPTH];
  // masks: tiles from mstart on (relative to the split) reach past its end or
  // past T - Mq, where the queries of a head see different token counts;
  // lim_lane = the last token (relative) this lane's query sees, clamped
  const int64_t vis = T - Mq + 1 - t0 < (int64_t)ntok ? T - Mq + 1 - t0 : (int64_t)ntok;
  const uint32_t mstart = vis < 0 ? 0u : (uint32_t)vis;
  const int64_t ll = T - Mq + (col % MAX_G) % Mq - t0;
  const int lim_lane = ll < -1 ? -1 : (ll > (int64_t)ntok ? (int)ntok : (int)ll);
  // a workgroup holding appended tokens encodes them first (below), so its
  // tile loads wait until then
  const int64_t ap0 = T - app.M > t0 ? T - app.M : t0;
  const bool appends = app.M > 0 && ap0 < t1;
  if (!appends) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load(rr[d], rel + d * WSTEP);
  }

  // tables (zeros past the end: out-of-range loads)
  *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sK) + threadIdx.x * 16) = kt4;
  *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sV) + threadIdx.x * 16) = vt4;
  {
    floatx4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      ah = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[s], ph[s], ah, 0, 0, 0);
      al = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[s], pl[s], al, 0, 0, 0);
    }
    // lane (col, grp) holds heads 4 grp + r, coordinate 16 wave + col; row h
    // = binary16 part of head h, row 8 + h = the rest (log2 units)
    if (grp < 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = fmaf(al[r], 0x1p-11f, ah[r]) * (scale * 1.4426950408889634f);
        const _Float16 h = (_Float16)a;
        sQ[(4 * grp + r) * Q_PITCH + 16 * wave + col] = h;
        sQ[(8 + 4 * grp + r) * Q_PITCH + 16 * wave + col] = (_Float16)(a - (float)h);
      }
    }
  }
  __syncthreads();
  if (appends) {
    // tokens ap0 .. t1 - 1, key and value together on all four waves, from the
    // binary16 tables now in LDS; the merge area is free until the end
    append_pairs<K, BITS>(app, (int64_t)b * Hkv + g, T, Tld, ap0, t1, sK, sV, N,
                          reinterpret_cast<double*>(sMerge), wave, lane);
    __threadfence_block();   // the new records are stored before any wave reads them
    __syncthreads();
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load(rr[d], rel + d * WSTEP);
  }
  // B operands of the scores, K-step s2: coordinates 16 grp + 8 s2 + 0..7
  half8 qb[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    qb[s2] = *reinterpret_cast<const half8*>(sQ + col * Q_PITCH + 16 * grp + 8 * s2);

  float m_run = NEG_BIG, l_run = 0.f;
  floatx4 oacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const DTile<W>& t, uint32_t tr) __attribute__((always_inline)) {
    uint32_t kq[4], vq[4];
    quarters<K, BITS, W>(t.k, kq);
    quarters<K, BITS, W>(t.v, vq);
    transpose_rows(kq);        // register s: quarter grp of row col's token in sub-tile s
    transpose_quads(vq, lane);   // register j: quarter col % 4 of token 16 grp + 4 j + col / 4
    // ---- scores: raw[4 s + r] = D[4 grp + r][col] of sub-tile s = token 16 grp + 4 s + r
    float raw[16];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w = kq[s];
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        half8 a;
        if constexpr (K == 4) {
          const uint32_t i0 = (w >> (2 * s2 * BITS)) & C::MASK;
          const uint32_t i1 = (w >> ((2 * s2 + 1) * BITS)) & C::MASK;
          const half4 c0 = *reinterpret_cast<const half4*>(sK + i0 * 4);
          const half4 c1 = *reinterpret_cast<const half4*>(sK + i1 * 4);
          a = half8{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        } else {
          const uint32_t i0 = (w >> (s2 * BITS)) & C::MASK;
          a = *reinterpret_cast<const half8*>(sK + i0 * 8);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[s2], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) raw[4 * s + r] = acc[r];
    }
    // hi + lo columns, then this lane's 8 tokens 16 grp + 8 half + i
    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // the lane's own sub-tile value plus the partner lane's part of it
      const float own = half ? raw[8 + i] : raw[i], give = half ? raw[i] : raw[8 + i];
      const uint32_t nw = t.nk[i >> 1];
      const _Float16 nu = __builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (nw >> 16) : (nw & 0xFFFFu)));
      sc[i] = __builtin_fmaf(own + rot8(give), (float)nu, 0.f);
    }
    if (tr + (uint32_t)TILE > mstart) {
      // past the split's end, or past this query's causal limit (several
      // queries per head: query m of Mq sees tokens up to T - Mq + m)
      const int valid = (int)(ntok - tr);
      const int lq = lim_lane - (int)tr + 1;
      const int vq = lq < valid ? lq : valid;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((int)tok_n + i >= vq) sc[i] = NEG_BIG;
    }
    // ---- online softmax over the row's 16 tokens x 4 rows (lane pair col,
    //      col + 8 shares head col % 8)
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = rows_max(fmaxf(mx, rot8(mx)));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oacc[mt] *= alpha;
    }
    m_run = m_new;
    float ps = 0.f;
    half8 own;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[i] - m_new);
      const float p1 = __builtin_amdgcn_exp2f(sc[i + 1] - m_new);
      ps += p0 + p1;
      // P' = p nu_v: p rounded to binary16, times the binary16 norm pair
      typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
      const uint32_t nw = t.nv[i >> 1];
      const half2_t nv2 = {__builtin_bit_cast(_Float16, (uint16_t)(nw & 0xFFFFu)),
                           __builtin_bit_cast(_Float16, (uint16_t)(nw >> 16))};
      const half2_t pp = {(_Float16)p0, (_Float16)p1};
      const half2_t w = pp * nv2;
      own[i] = w[0];
      own[i + 1] = w[1];
    }
    l_run += rows_sum(ps + rot8(ps));
    // K-step 0 takes this lane's weights, K-step 1 those of lane col + 8
    half8 pb[2];
    pb[0] = own;
    {
      const u32x4 ow = __builtin_bit_cast(u32x4, own);
      const u32x4 ot = {rot8u(ow.x), rot8u(ow.y), rot8u(ow.z), rot8u(ow.w)};
      pb[1] = __builtin_bit_cast(half8, ot);
    }
    // ---- values, K-step ks: transpose reads j = 2 ks, 2 ks + 1; slot (grp,
    //      e) is token 16 grp + 8 ks + e
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t wa = vq[2 * ks], wb = vq[2 * ks + 1];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const _Float16 *pa, *pbp;
        if constexpr (K == 4) {
          pa = sV + ((wa >> (mt * BITS)) & C::MASK) * 4;
          pbp = sV + ((wb >> (mt * BITS)) & C::MASK) * 4;
        } else {
          pa = sV + ((wa >> ((mt >> 1) * BITS)) & C::MASK) * 8 + 4 * (mt & 1);
          pbp = sV + ((wb >> ((mt >> 1) * BITS)) & C::MASK) * 8 + 4 * (mt & 1);
        }
        const half4 ha = read_tr(pa), hb = read_tr(pbp);
        const half8 a = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[ks], oacc[mt], 0, 0, 0);
      }
    }
  };

  if (rel < ntok) {
    for (;;) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (rel < ntok) process(rr[d], rel);
        load(rr[d], rel + DEPTH * WSTEP);
        rel += WSTEP;
      }
      if (rel >= ntok) break;
    }
  }

  // ---- merge the four waves' partials (lanes col < G hold head col,
  //      coordinates 16 grp + 4 mt + r), write one partial per head
  if (col < G) {
    float* mine = sMerge + (wave * MAX_G + col) * MERGE_PITCH;
    if (grp == 0) {
      mine[0] = m_run;
      mine[1] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[2 + 16 * grp + 4 * mt + r] = oacc[mt][r];
  }
  __syncthreads();
  finish_heads(sMerge, G, Hq, b, g, S, sw, ws, pi32t, out);
}

template <int K, int BITS>
size_t attend_lds_bytes(int N) {
  return AttLds<K, BITS>::total(N);
}

template <int K, int BITS>
hipError_t launch_v(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                    const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                    const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, int64_t Tld, int Mq,
                    float scale, void* workspace, uint16_t* out, hipStream_t s,
                    const AppendIn& app) {
  float* ws = static_cast<float*>(workspace);
  hipError_t e;
  // kernel A' over binary16 tables kt, vt of Nt entries of KD coordinates
  auto direct = [&](auto kern, const _Float16* kt, const _Float16* vt, int Nt) {
    const SplitPlan p = plan_splits(B, Hkv, T, SPLIT_TARGET_DIRECT);
    hipLaunchKernelGGL(kern, dim3((unsigned)p.S, Hkv, B), dim3(ATT_THREADS), 0, s, q, kc, kn, vc, vn,
                       Hq, Hkv, T, Tld, Mq, p.chunk, p.S, scale, ck->t.pi16hi, ck->t.pi16lo, kt, vt,
                       Nt, ws, ck->t.pi32t, out, app);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.S == 1) return err;
    hipLaunchKernelGGL(attend_merge_kernel, dim3(Hq * B), dim3(256), 0, s, ws, p.S, ck->t.pi32t, out);
    return hipGetLastError();
  };
  if constexpr (K == 4 || K == 8) {
    if (ck->half_exact && cv->half_exact && T % 8 == 0 && Tld % 8 == 0)
      return direct(attend_direct_kernel<K, BITS>, ck->t.cb16hi, cv->t.cb16hi, ck->N);
  }
  if constexpr (K == 2 && BITS == 4) {
    // k = 2, N = 16: a record's bytes index codeword pairs, so it is read as a
    // k = 4, N = 256 record over the pair tables (the appended tokens are then
    // searched over pairs: the nearest pair is the pair of nearest codewords)
    if (ck->t.pair16 && cv->t.pair16 && T % 8 == 0 && Tld % 8 == 0)
      return direct(attend_direct_kernel<4, 8>, ck->t.pair16, cv->t.pair16, 256);
  }
  const bool fuse = app.M > 0 && ck->half_exact && cv->half_exact;
  if (app.M > 0 && !fuse) {   // appended tokens first, by their own launch
    OutRows rows;
    rows.inner = app.M;
    rows.stride = Tld;
    rows.pos = T - app.M;
    const int64_t n = (int64_t)B * Hkv * app.M;
    if (ck == cv) {
      e = launch_append(ck, app.k_new, app.v_new, n, 2 * n, app.kc, app.kn, app.vc, app.vn, rows, s);
    } else {
      e = launch_append(ck, app.k_new, nullptr, n, n, app.kc, app.kn, nullptr, nullptr, rows, s);
      if (e == hipSuccess)
        e = launch_append(cv, app.v_new, nullptr, n, n, app.vc, app.vn, nullptr, nullptr, rows, s);
    }
    if (e != hipSuccess) return e;
  }
  const SplitPlan p = plan_splits(B, Hkv, T, SPLIT_TARGET);
  const size_t shm = attend_lds_bytes<K, BITS>(ck->N);
  auto kern = attend_split_kernel<K, BITS>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.S, Hkv, B), dim3(ATT_THREADS), shm, s, q, kc, kn, vc, vn, Hq,
                     Hkv, T, Tld, Mq, p.chunk, p.S, scale, ck->t.pi32, ck->t.cb16hi, ck->t.cb16lo,
                     cv->t.cb16hi, cv->t.cb16lo, ck->N, ws, ck->t.pi32t, out,
                     fuse ? app : AppendIn());
  e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(Hq * B), dim3(256), 0, s, ws, p.S, ck->t.pi32t, out);
  return hipGetLastError();
}

}  // namespace

bool attend_supported(const fq_codebook* cb) {
#define FQ_ATS(KK, BB) \
  if (cb->k == KK && cb->bits == BB)                                            \
    return attend_lds_bytes<KK, BB>(cb->N) + MAX_G * D * 4 <= 160 * 1024;   /* + static */
  FQ_VARIANTS(FQ_ATS)
#undef FQ_ATS
  return false;
}

size_t attend_workspace_bytes(const fq_codebook* /*cb_k*/, int B, int Hq, int Hkv, int64_t T) {
  // room for either kernel's partials
  const SplitPlan p = plan_splits(B, Hkv, T, SPLIT_TARGET), pd = plan_splits(B, Hkv, T, SPLIT_TARGET_DIRECT);
  const int S = p.S > pd.S ? p.S : pd.S;
  return ((size_t)B * Hq * S * PART * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_attend(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                         const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                         const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, int64_t Tld,
                         int Mq, float scale, void* ws, uint16_t* out, hipStream_t s,
                         const AppendIn& app) {
#define FQ_ATT(KK, BB)                                                                           \
  if (ck->k == KK && ck->bits == BB)                                                             \
    return launch_v<KK, BB>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, Tld, Mq, scale, ws, out, s, \
                            app);
  FQ_VARIANTS(FQ_ATT)
#undef FQ_ATT
  return hipErrorInvalidValue;
}

}  // namespace fq
