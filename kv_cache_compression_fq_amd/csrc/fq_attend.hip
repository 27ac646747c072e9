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

// About 1024 workgroups (4096 waves) over the device; each wave gets at least
// one tile.  The four waves of a workgroup take interleaved tiles of its split.
SplitPlan plan_splits(int B, int Hkv, int64_t T) {
  constexpr int64_t STEP = (int64_t)ATT_WAVES * TILE;
  const int64_t pairs = (int64_t)B * Hkv;
  int64_t S = (1024 + pairs - 1) / pairs;
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
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
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

template <int K, int BITS>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void attend_split_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kc,
    const uint16_t* __restrict__ kn, const uint32_t* __restrict__ vc,
    const uint16_t* __restrict__ vn, int Hq, int Hkv, int64_t T, int64_t chunk, int S,
    float scale, const float* __restrict__ pi32, const _Float16* __restrict__ kh_g,
    const _Float16* __restrict__ kl_g, const _Float16* __restrict__ vh_g,
    const _Float16* __restrict__ vl_g, int N, float* __restrict__ ws) {
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
    const int64_t rec0 = stream * T + (left <= 0 ? 0 : tb);
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
      const int valid = (int)(t1 - tb);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * sub + 4 * grp + r >= valid) sc[sub][r] = NEG_BIG;
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
      const int valid = (int)(t1 - tb);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * sub + 4 * grp + r >= valid) sc[sub][r] = NEG_BIG;
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
    auto run = [&](int64_t t) __attribute__((always_inline)) {
      if constexpr (AS::EXPAND) {
        if (t1 - t >= TILE)
          process(t, std::false_type());
        else
          process(t, std::true_type());
      } else {
        if (t1 - t >= TILE)
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
    float* dst = ws + (((int64_t)b * Hq + (int64_t)g * G + h) * S + sw) * PART;
    if (c == 0) {
      dst[0] = M;
      dst[1] = Ls;
    }
    dst[2 + c] = o;
  }
}

// One workgroup per (batch, query head): log-sum-exp merge of the S split
// partials, then out = Pi^T o_rot in binary16.
__global__ __launch_bounds__(256) void attend_merge_kernel(const float* __restrict__ ws, int S,
                                                           int Hq, const float* __restrict__ pi32,
                                                           uint16_t* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* src = ws + ((int64_t)b * Hq + h) * S * PART;
  __shared__ float sRed[256];
  __shared__ float sO[4][D];
  __shared__ float sL[4];
  float M = NEG_BIG;
  for (int s = tid; s < S; s += 256) M = fmaxf(M, src[(int64_t)s * PART]);
  sRed[tid] = M;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) sRed[tid] = fmaxf(sRed[tid], sRed[tid + w]);
    __syncthreads();
  }
  M = sRed[0];
  const int c = tid & 63, part = tid >> 6;
  float o = 0.f, Ls = 0.f;
  for (int s = part; s < S; s += 4) {
    const float* p = src + (int64_t)s * PART;
    const float wt = __builtin_amdgcn_exp2f(p[0] - M);   // partials are in log2 units
    Ls = fmaf(wt, p[1], Ls);
    o = fmaf(wt, p[2 + c], o);
  }
  sO[part][c] = o;
  if (c == 0) sL[part] = Ls;
  __syncthreads();
  if (tid < D) {
    const float Lt = sL[0] + sL[1] + sL[2] + sL[3];
    sRed[tid] = (sO[0][tid] + sO[1][tid] + sO[2][tid] + sO[3][tid]) / Lt;
  }
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int j = 0; j < D; ++j) a = fmaf(pi32[j * D + tid], sRed[j], a);
    out[((int64_t)b * Hq + h) * D + tid] = f32_to_f16_rne(a);
  }
}

template <int K, int BITS>
size_t attend_lds_bytes(int N) {
  return AttLds<K, BITS>::total(N);
}

template <int K, int BITS>
hipError_t launch_v(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                    const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                    const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, float scale,
                    float* ws, uint16_t* out, hipStream_t s) {
  const SplitPlan p = plan_splits(B, Hkv, T);
  const size_t shm = attend_lds_bytes<K, BITS>(ck->N);
  auto kern = attend_split_kernel<K, BITS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.S, Hkv, B), dim3(ATT_THREADS), shm, s, q, kc, kn, vc, vn, Hq,
                     Hkv, T, p.chunk, p.S, scale, ck->t.pi32, ck->t.cb16hi, ck->t.cb16lo,
                     cv->t.cb16hi, cv->t.cb16lo, ck->N, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(Hq, B), dim3(256), 0, s, ws, p.S, Hq, ck->t.pi32,
                     out);
  return hipGetLastError();
}

}  // namespace

bool attend_supported(const fq_codebook* cb) {
#define FQ_ATS(KK, BB) \
  if (cb->k == KK && cb->bits == BB) return attend_lds_bytes<KK, BB>(cb->N) <= 160 * 1024;
  FQ_VARIANTS(FQ_ATS)
#undef FQ_ATS
  return false;
}

size_t attend_workspace_bytes(const fq_codebook* /*cb_k*/, int B, int Hq, int Hkv, int64_t T) {
  const SplitPlan p = plan_splits(B, Hkv, T);
  return ((size_t)B * Hq * p.S * PART * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_attend(const fq_codebook* ck, const fq_codebook* cv, const uint16_t* q,
                         const uint32_t* kc, const uint16_t* kn, const uint32_t* vc,
                         const uint16_t* vn, int B, int Hq, int Hkv, int64_t T, float scale,
                         void* ws, uint16_t* out, hipStream_t s) {
  float* w = static_cast<float*>(ws);
#define FQ_ATT(KK, BB)                                                                           \
  if (ck->k == KK && ck->bits == BB)                                                             \
    return launch_v<KK, BB>(ck, cv, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale, w, out, s);
  FQ_VARIANTS(FQ_ATT)
#undef FQ_ATT
  return hipErrorInvalidValue;
}

}  // namespace fq
