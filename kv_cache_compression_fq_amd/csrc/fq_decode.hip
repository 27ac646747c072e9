// FibQuant decode (FibQuant technical summary, section 2.3): fetch the
// codewords of a fixed-address record (section 1), concatenate the blocks,
// apply Pi^T and scale by the stored norm.  Random access: output row i may
// decode any record rows[i].
//
// Layout of the work (one persistent wave per SIMD slot):
//  * A wave decodes chunks of 64 vectors.  Lane v loads record v of the chunk
//    (and its norm) with unconditional buffer loads; the loads of the next two
//    chunks are in flight while the current one is decoded.
//  * Staging: each lane unpacks its own record (field widths are compile-time,
//    so every shift is static) into a table of 16-bit indices in LDS; for
//    k = 3 it writes the vector's 64 binary16 coordinates there instead.
//  * Per tile of 16 vectors, v_mfma_f32_16x16x32_f16 forms Y^T = Pi^T Z_hat^T:
//    A = Pi^T, rounded to binary16, in registers for the whole kernel;
//    B = Z_hat^T, gathered from the LDS codebook (binary16) by index, or read
//    from the staged coordinates (k = 3).  Both
//    operands carry binary16 rounding (relative 2^-12 per entry); over the
//    64-term sums that is ~3e-5 nu rms and ~2e-4 nu worst case, inside the
//    1e-3 nu decode tolerance before the output's own rounding.  Accumulation
//    is float32.
//  * Each lane ends up with 4 consecutive outputs of one vector; they are
//    scaled by the norm, converted, transposed through LDS and written as
//    16-byte buffer stores (out-of-range rows fall outside the descriptor).
//  * Loads and stores share one wait counter on this architecture, so every
//    load and store is unconditional and the loop is arranged so that the only
//    wait inside it covers the prefetched loads, never the stores behind them.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int TILE = 16;           // vectors per MFMA tile
constexpr int CHUNK = 64;          // vectors per wave iteration (one lane per record)
constexpr int OUT_PITCH = D + 8;   // LDS row (elements) of the transpose buffer

// k = 3: a record is expanded once, when staged, into its 64 binary16
// coordinates (row pitch ZR_PITCH elements), so the product reads one 16-byte
// piece per operand instead of gathering eight coordinates one by one; the
// LDS table then holds each codeword padded to four entries (8 bytes).
constexpr int ZR_PITCH = D + 8;
template <int K>
constexpr bool expand_rows() { return K == 3; }
template <int K>
constexpr int table_k() { return expand_rows<K>() ? 4 : K; }

template <int K, int BITS>
constexpr size_t stage_bytes() {
  return expand_rows<K>() ? (size_t)CHUNK * ZR_PITCH * 2 : (size_t)CHUNK * Shape<K, BITS>::IDX_PITCH * 2;
}

template <int K, int BITS, typename TY>
constexpr size_t wave_lds() {
  return stage_bytes<K, BITS>() + CHUNK * 4 + TILE * OUT_PITCH * sizeof(TY);
}

// Record fields -> the vector's 64 binary16 coordinates in LDS row `row`
// (k = 3: 21 blocks of three and a last block of one).  Codeword i sits at
// tab[4 i .. 4 i + 2]; output word w holds coordinates 2 w and 2 w + 1, each
// taken with one byte permute from the codeword registers that hold them.
template <int K, int BITS, int W>
__device__ inline void expand_record(const uint32_t (&w)[W], const _Float16* tab, _Float16* row) {
  constexpr int NB = Shape<K, BITS>::NB;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  uint32_t c[NB][2];   // c[j][0] = coordinates 0, 1 of block j; c[j][1] = coordinate 2
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int pos = j * BITS, wi = pos >> 5, o = pos & 31;
    uint32_t v = w[wi] >> o;
    if (o + BITS > 32) v |= w[wi + 1] << (32 - o);
    const uint2 cw = *reinterpret_cast<const uint2*>(tab + (v & MASK) * 4);
    c[j][0] = cw.x;
    c[j][1] = cw.y;
  }
  u32x4* out = reinterpret_cast<u32x4*>(row);
#pragma unroll
  for (int q = 0; q < D / 8; ++q) {
    uint32_t wd[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c0 = 8 * q + 2 * h, c1 = c0 + 1;   // coordinates of this word
      const int j0 = c0 / K, t0 = c0 % K, j1 = c1 / K, t1 = c1 % K;
      const uint32_t a = c[j0][t0 >> 1], b = c[j1][t1 >> 1];
      const uint32_t alo = (t0 & 1) ? 2u : 0u, blo = (t1 & 1) ? 2u : 0u;
      // bytes 0-3 select from a, 4-7 from b
      wd[h] = __builtin_amdgcn_perm(b, a, alo | (alo + 1) << 8 | (4 + blo) << 16 | (5 + blo) << 24);
    }
    out[q] = u32x4{wd[0], wd[1], wd[2], wd[3]};
  }
}

template <int W>
struct ChunkRegs {
  uint32_t w[W];
  uint32_t nu_bits;  // raw binary16 norm, converted only when staged
};

// Record v of a chunk into lane v's registers.  Non-gathered: a descriptor over
// the chunk's own records, so lanes past the end read 0 (hardware range check).
template <int W>
__device__ inline void load_chunk(ChunkRegs<W>& t, int64_t chunk, int lane, const uint32_t* codes,
                                  const uint16_t* norms, int64_t n) {
  const int64_t base = chunk * CHUNK;
  const int64_t left = n - base;
  const int cnt = left <= 0 ? 0 : (left < CHUNK ? (int)left : CHUNK);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(codes + base * W), (short)0, cnt * W * 4, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(norms + base), (short)0, cnt * 2, BUF_DWORD3);
  load_record<W>(t.w, rc, (uint32_t)(lane * W * 4));
  t.nu_bits = __builtin_amdgcn_raw_buffer_load_b16(rn, lane * 2, 0, 0);
}

// Gathered records rows[r]: one descriptor over the whole code array (at most
// 2 GiB, checked on the host); an invalid address reads 0 and decodes to 0.
template <int W>
__device__ inline void load_chunk_gather(ChunkRegs<W>& t, int64_t chunk, int lane,
                                         const uint32_t* codes, const uint16_t* norms,
                                         const int64_t* rows, int64_t n_records, int64_t n) {
  const int64_t r = chunk * CHUNK + lane;
  const int64_t rr = r < n ? r : n - 1;
  const int64_t rec = rows[rr];
  const bool ok = r < n && rec >= 0 && rec < n_records;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(codes), (short)0, (int)(n_records * W * 4), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(norms), (short)0, (int)(n_records * 2), BUF_DWORD3);
  const uint32_t off = ok ? (uint32_t)(rec * W) * 4u : 0x80000000u;
  const uint32_t offn = ok ? (uint32_t)rec * 2u : 0x80000000u;
  load_record<W>(t.w, rc, off);
  t.nu_bits = __builtin_amdgcn_raw_buffer_load_b16(rn, offn, 0, 0);
}

// Packed records (fq_pack_records): record r at bits [r R, r R + R) of one
// word stream, R = F + 16 with F = NB BITS field bits, then the binary16 norm.
template <int K, int BITS>
struct PackedShape {
  static constexpr int F = Shape<K, BITS>::NB * BITS;   // field bits
  static constexpr int R = F + 16;                      // record bits
  static constexpr int NWR = (R + 31 + 31) / 32;        // stream words one record can touch
};

// Re-align a record from the stream words wd (the first holding its bit sh)
// into the word-aligned layout: fields in t.w (bits past F zero), norm in t.nu_bits.
template <int K, int BITS, int W>
__device__ inline void realign(const uint32_t (&wd)[PackedShape<K, BITS>::NWR + 1], uint32_t sh,
                               ChunkRegs<W>& t) {
  using P = PackedShape<K, BITS>;
  constexpr int NS = (P::F + 15) / 32 + 1;   // record-string words holding fields and norm
  uint32_t rs[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) rs[i] = __builtin_amdgcn_alignbit(wd[i + 1], wd[i], sh);
#pragma unroll
  for (int i = 0; i < W; ++i) t.w[i] = rs[i];
  constexpr int TOP = P::F - 32 * (W - 1);   // field bits in the last word
  if constexpr (TOP < 32) t.w[W - 1] &= (1u << TOP) - 1u;
  constexpr int NW0 = P::F >> 5, NSH = P::F & 31;
  if constexpr (NSH <= 16)
    t.nu_bits = (rs[NW0] >> NSH) & 0xFFFFu;
  else
    t.nu_bits = __builtin_amdgcn_alignbit(rs[NW0 + 1], rs[NW0], NSH) & 0xFFFFu;
}

// Record `chunk * CHUNK + lane` of a packed stream of n records.
template <int K, int BITS, int W>
__device__ inline void load_chunk_packed(ChunkRegs<W>& t, int64_t chunk, int lane,
                                         const uint32_t* packed, int64_t n) {
  using P = PackedShape<K, BITS>;
  const int64_t base = chunk * CHUNK;
  const int64_t left = n - base;
  const int cnt = left <= 0 ? 0 : (left < CHUNK ? (int)left : CHUNK);
  const int64_t bit0 = base * P::R;
  const int64_t word0 = bit0 >> 5;
  const int64_t words_total = (n * P::R + 31) >> 5;
  // the chunk's words: those of its cnt records (none past the stream's end)
  const int64_t span = cnt == 0 ? 0 : (((bit0 & 31) + (int64_t)cnt * P::R + 31) >> 5);
  const int64_t have = words_total - word0 < span ? words_total - word0 : span;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed + word0), (short)0, (int)(have > 0 ? have * 4 : 0), BUF_DWORD3);
  const uint32_t bit = (uint32_t)(bit0 & 31) + (uint32_t)lane * P::R;
  uint32_t wd[P::NWR + 1];
#pragma unroll
  for (int i = 0; i < P::NWR; ++i)
    wd[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, ((bit >> 5) + i) * 4, 0, 0);
  wd[P::NWR] = 0u;
  realign<K, BITS, W>(wd, bit & 31, t);
}

// Packed record rows[r] (at most 2^31 - 1 bytes of stream, checked on the
// host); an invalid address reads 0 and decodes to 0.
template <int K, int BITS, int W>
__device__ inline void load_chunk_packed_gather(ChunkRegs<W>& t, int64_t chunk, int lane,
                                                const uint32_t* packed, const int64_t* rows,
                                                int64_t n_records, int64_t n) {
  using P = PackedShape<K, BITS>;
  const int64_t r = chunk * CHUNK + lane;
  const int64_t rr = r < n ? r : n - 1;
  const int64_t rec = rows[rr];
  const bool ok = r < n && rec >= 0 && rec < n_records;
  const int64_t words_total = (n_records * P::R + 31) >> 5;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed), (short)0, (int)(words_total * 4), BUF_DWORD3);
  const int64_t bit = ok ? rec * P::R : 0;
  const uint32_t w0 = ok ? (uint32_t)(bit >> 5) : 0x20000000u;   // past the range: reads 0
  uint32_t wd[P::NWR + 1];
#pragma unroll
  for (int i = 0; i < P::NWR; ++i)
    wd[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, (w0 + i) * 4, 0, 0);
  wd[P::NWR] = 0u;
  realign<K, BITS, W>(wd, (uint32_t)(bit & 31), t);
}

// Coordinates [c0, c0 + 8) of z_hat (binary16) for one staged vector.
template <int K>
__device__ inline half8 gather8(const uint16_t* idx, const _Float16* cbh, int c0) {
  if constexpr (K == 8) {
    const uint32_t i0 = idx[c0 >> 3];
    return *reinterpret_cast<const half8*>(cbh + i0 * 8);
  } else if constexpr (K == 4) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(idx + (c0 >> 2));
    const uint32_t i0 = pair & 0xFFFFu, i1 = pair >> 16;
    const uint2 h0 = *reinterpret_cast<const uint2*>(cbh + i0 * 4);
    const uint2 h1 = *reinterpret_cast<const uint2*>(cbh + i1 * 4);
    const u32x4 hv = {h0.x, h0.y, h1.x, h1.y};
    return __builtin_bit_cast(half8, hv);
  } else if constexpr (K == 2) {
    const uint2 q = *reinterpret_cast<const uint2*>(idx + (c0 >> 1));
    const uint32_t i0 = q.x & 0xFFFFu, i1 = q.x >> 16, i2 = q.y & 0xFFFFu, i3 = q.y >> 16;
    const uint32_t* h = reinterpret_cast<const uint32_t*>(cbh);
    const u32x4 hv = {h[i0], h[i1], h[i2], h[i3]};
    return __builtin_bit_cast(half8, hv);
  } else {   // 8 coordinates of one codeword (k = 3 is expanded at staging instead)
    static_assert(K % 8 == 0 && K >= 16, "gather8: k = 2, 4, 8 or a multiple of 8");
    const uint32_t i0 = idx[c0 / K];
    return *reinterpret_cast<const half8*>(cbh + i0 * K + c0 % K);
  }
}

template <int K, int BITS, typename TY, bool GATHER, bool PACKED>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ norms,
    const int64_t* __restrict__ rows, int64_t n_records, int64_t n, TY* __restrict__ y,
    int64_t ld, const _Float16* __restrict__ pifrag, const _Float16* __restrict__ cbh_g,
    int N) {
  using Sh = Shape<K, BITS>;
  constexpr int W = Sh::W;
  // large blocks: the table (N k binary16) stays in global memory (L2-resident)
  constexpr bool GTAB = large_block(K);
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* sCbh = reinterpret_cast<_Float16*>(smem);
  constexpr int TK = table_k<K>();
  const size_t cb_bytes = GTAB ? 0 : ((size_t)N * TK * sizeof(_Float16) + 15) / 16 * 16;
  // the wave index is uniform: keep it (and the buffer descriptors derived from
  // it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  unsigned char* wbase = smem + cb_bytes + (size_t)wave * wave_lds<K, BITS, TY>();
  uint16_t* sIdx = reinterpret_cast<uint16_t*>(wbase);   // [CHUNK][IDX_PITCH] (or k = 3: rows)
  _Float16* sZr = reinterpret_cast<_Float16*>(wbase);    // k = 3: [CHUNK][ZR_PITCH]
  float* sNu = reinterpret_cast<float*>(wbase + stage_bytes<K, BITS>());   // [CHUNK]
  TY* sOut = reinterpret_cast<TY*>(wbase + stage_bytes<K, BITS>() + CHUNK * 4);

  if constexpr (expand_rows<K>()) {
    for (int i = threadIdx.x; i < N; i += DEC_THREADS) {
      const _Float16 z = (_Float16)0.f;
      const half4 h = {cbh_g[i * K], cbh_g[i * K + 1], cbh_g[i * K + 2], z};
      *reinterpret_cast<half4*>(sCbh + i * 4) = h;
    }
  } else if constexpr (!GTAB) {
    for (int e = threadIdx.x; e < N * K; e += DEC_THREADS) sCbh[e] = cbh_g[e];
  }
  // A operands: Pi^T as 16 x 32 fragments, [mt][s] = Pi[32 s + 8 grp + e][16 mt + col]
  half8 pa[4][2];
  const int col = lane & 15, grp = lane >> 4;
  const half8* frag = reinterpret_cast<const half8*>(pifrag);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) pa[mt][s] = frag[(s * 4 + mt) * 64 + lane];
  // consume the fragments here so their loads are waited for once, before the
  // loop, not at their first use inside it (where the wait would also cover
  // the stores of the previous iteration)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) asm volatile("" ::"v"(pa[mt][s]));
  __syncthreads();

  const int64_t n_chunks = (n + CHUNK - 1) / CHUNK;
  const int64_t stride = (int64_t)gridDim.x * DEC_WAVES;
  int64_t chunk = (int64_t)blockIdx.x * DEC_WAVES + wave;
  if (chunk >= n_chunks) return;

  ChunkRegs<W> ra, rb;
  // a chunk index past the end gives an empty descriptor: its loads read 0
  auto load = [&](ChunkRegs<W>& t, int64_t c) {
    c = c < n_chunks ? c : n_chunks;
    if constexpr (PACKED && GATHER)
      load_chunk_packed_gather<K, BITS, W>(t, c, lane, codes, rows, n_records, n);
    else if constexpr (PACKED)
      load_chunk_packed<K, BITS, W>(t, c, lane, codes, n);
    else if constexpr (GATHER)
      load_chunk_gather<W>(t, c, lane, codes, norms, rows, n_records, n);
    else
      load_chunk<W>(t, c, lane, codes, norms, n);
  };
  auto stage = [&](const ChunkRegs<W>& t) {
    if constexpr (expand_rows<K>())
      expand_record<K, BITS, W>(t.w, sCbh, sZr + lane * ZR_PITCH);
    else
      unpack_record<K, BITS, W>(t.w, sIdx + lane * Sh::IDX_PITCH);
    sNu[lane] = f16_bits_to_f32((uint16_t)t.nu_bits);
  };
  auto decode_chunk = [&](int64_t base) {
    // global-table gathers of the whole chunk are issued together, ahead of use
    half8 zg[CHUNK / TILE][2];
    if constexpr (GTAB) {
#pragma unroll
      for (int m = 0; m < CHUNK / TILE; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          zg[m][s] = gather8<K>(sIdx + (TILE * m + col) * Sh::IDX_PITCH, cbh_g, 32 * s + 8 * grp);
    }
#pragma unroll
    for (int m = 0; m < CHUNK / TILE; ++m) {
      const uint16_t* vidx = sIdx + (TILE * m + col) * Sh::IDX_PITCH;
      floatx4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        half8 zh;
        if constexpr (GTAB)
          zh = zg[m][s];
        else if constexpr (expand_rows<K>())
          zh = *reinterpret_cast<const half8*>(sZr + (TILE * m + col) * ZR_PITCH + 32 * s + 8 * grp);
        else
          zh = gather8<K>(vidx, sCbh, 32 * s + 8 * grp);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[mt][s], zh, acc[mt], 0, 0, 0);
      }
      // lane holds coordinates 16 mt + 4 grp + r (r = 0..3) of vector col
      const float nu = sNu[TILE * m + col];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        TY o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (TY)(acc[mt][r] * nu);
        if constexpr (sizeof(TY) == 2) {
          uint2 pk;
          __builtin_memcpy(&pk, o, 8);
          *reinterpret_cast<uint2*>(sOut + col * OUT_PITCH + 16 * mt + 4 * grp) = pk;
        } else {
          uint4 pk;
          __builtin_memcpy(&pk, o, 16);
          *reinterpret_cast<uint4*>(sOut + col * OUT_PITCH + 16 * mt + 4 * grp) = pk;
        }
      }
      wave_lds_sync();
      constexpr int PER = 16 / sizeof(TY);          // elements per 16-byte piece
      constexpr int PIECES = D / PER;               // pieces per row
      const int64_t row0 = base + TILE * m;
      const int64_t rows_left = n - row0;
      const int valid_rows = rows_left < TILE ? (int)(rows_left > 0 ? rows_left : 0) : TILE;
      const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
          y + row0 * ld, (short)0, (int)(valid_rows * ld * (int64_t)sizeof(TY)), BUF_DWORD3);
#pragma unroll
      for (int u = 0; u < TILE * PIECES / 64; ++u) {
        const int slot = lane + 64 * u;
        const int v = slot / PIECES, q = slot - v * PIECES;
        const uint4 val = *reinterpret_cast<const uint4*>(sOut + v * OUT_PITCH + q * PER);
        const u32x4 vv = {val.x, val.y, val.z, val.w};
        // non-temporal: the output streams past the caches (measured 10-25 %
        // faster than default-policy stores; at system scope, nt sc1, another
        // 1-3 % on 2^24 vectors and up to 10 % on a 1.18 M-vector cache)
        __builtin_amdgcn_raw_buffer_store_b128(vv, ry, (int)((v * ld + q * PER) * sizeof(TY)), 0,
                                               CPOL_NT_SC1);
      }
      wave_lds_sync();
    }
  };

  load(ra, chunk);
  stage(ra);
  wave_lds_sync();
  load(rb, chunk + stride);
  // Unrolled by two so each register set keeps a fixed name.  In each half the
  // loads of chunk c + 2 stride are issued before chunk c's stores, and the
  // other set (loaded one half earlier) is waited for after those stores on a
  // straight path, so the wait covers only loads.
  for (;;) {
    load(ra, chunk + 2 * stride);
    decode_chunk(chunk * CHUNK);
    chunk += stride;
    if (chunk >= n_chunks) break;
    stage(rb);
    wave_lds_sync();
    load(rb, chunk + 2 * stride);
    decode_chunk(chunk * CHUNK);
    chunk += stride;
    if (chunk >= n_chunks) break;
    stage(ra);
    wave_lds_sync();
  }
}

template <int K, int BITS, typename TY, bool GATHER, bool PACKED>
hipError_t launch_k(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, TY* y, int64_t ld,
                    hipStream_t s) {
  const size_t cb_bytes = large_block(K) ? 0 : ((size_t)cb->N * table_k<K>() * sizeof(_Float16) + 15) / 16 * 16;
  const size_t shm = cb_bytes + DEC_WAVES * wave_lds<K, BITS, TY>();
  auto kern = decode_kernel<K, BITS, TY, GATHER, PACKED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  // persistent grid: as many workgroups as fit at once (queried on first use;
  // one (k, bits) pair fixes the LDS need)
  static DeviceCache cap_cache;   // resident workgroups per device
  const int64_t cap = cap_cache.get(reinterpret_cast<const void*>(kern), DEC_THREADS, shm);
  if (cap <= 0) return hipErrorInvalidConfiguration;
  const int64_t n_chunks = (n + CHUNK - 1) / CHUNK;
  int64_t blocks = (n_chunks + DEC_WAVES - 1) / DEC_WAVES;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(DEC_THREADS), shm, s, codes, norms, rows,
                     n_records, n, y, ld, cb->t.pifrag, cb->t.cb16hi, cb->N);
  return hipGetLastError();
}

template <typename TY, bool GATHER, bool PACKED>
hipError_t dispatch(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, TY* y, int64_t ld,
                    hipStream_t s) {
#define FQ_DEC(KK, BB)                                                                     \
  if (cb->k == KK && cb->bits == BB)                                                       \
    return launch_k<KK, BB, TY, GATHER, PACKED>(cb, codes, norms, rows, n_records, n, y, ld, s);
  FQ_VARIANTS(FQ_DEC)
  FQ_VARIANTS_LARGE(FQ_DEC)
#undef FQ_DEC
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                         const int64_t* rows, int64_t n_records, int64_t n, void* y, fq_dtype yt,
                         int64_t ld, hipStream_t s, bool packed) {
  if (yt == FQ_F16) {
    _Float16* yy = static_cast<_Float16*>(y);
    if (packed)
      return rows ? dispatch<_Float16, true, true>(cb, codes, norms, rows, n_records, n, yy, ld, s)
                  : dispatch<_Float16, false, true>(cb, codes, norms, rows, n_records, n, yy, ld, s);
    return rows ? dispatch<_Float16, true, false>(cb, codes, norms, rows, n_records, n, yy, ld, s)
                : dispatch<_Float16, false, false>(cb, codes, norms, rows, n_records, n, yy, ld, s);
  }
  float* yy = static_cast<float*>(y);
  if (packed)
    return rows ? dispatch<float, true, true>(cb, codes, norms, rows, n_records, n, yy, ld, s)
                : dispatch<float, false, true>(cb, codes, norms, rows, n_records, n, yy, ld, s);
  return rows ? dispatch<float, true, false>(cb, codes, norms, rows, n_records, n, yy, ld, s)
              : dispatch<float, false, false>(cb, codes, norms, rows, n_records, n, yy, ld, s);
}

// ---------------------------------------------------------------- packing
namespace {

// Bits [lo, lo + 32) of record r's bit string: its F field bits (from the
// word-aligned record, bits past F ignored), then the 16 norm bits, then zeros.
template <int K, int BITS>
__device__ inline uint32_t record_string_bits(const uint32_t* rec, uint32_t norm, int lo) {
  using P = PackedShape<K, BITS>;
  constexpr int W = Shape<K, BITS>::W;
  auto sword = [&](int j) -> uint32_t {
    uint32_t v = 0;
    if (j < W) {
      const int top = P::F - 32 * j;   // field bits in word j
      v = top >= 32 ? rec[j] : (top > 0 ? rec[j] & ((1u << top) - 1u) : 0u);
    }
    constexpr int NW0 = P::F >> 5, NSH = P::F & 31;
    if (j == NW0) v |= norm << NSH;
    if (NSH > 16 && j == NW0 + 1) v |= norm >> (32 - NSH);
    return v;
  };
  const int i = lo >> 5;
  return __builtin_amdgcn_alignbit(sword(i + 1), sword(i), (uint32_t)(lo & 31));
}

// One thread per word of the stream: the bits of the (at most two) records
// that fall in it.
template <int K, int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint32_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ norms, int64_t n,
                                                   uint32_t* __restrict__ packed, int64_t words) {
  using P = PackedShape<K, BITS>;
  constexpr int W = Shape<K, BITS>::W;
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= words) return;
  const int64_t b0 = 32 * w, b1 = b0 + 32;
  const int64_t r_last = (b1 - 1) / P::R < n - 1 ? (b1 - 1) / P::R : n - 1;
  uint32_t out = 0;
  for (int64_t r = b0 / P::R; r <= r_last; ++r) {
    const int64_t rs = r * P::R;
    const int64_t lo = (b0 > rs ? b0 : rs) - rs;                         // record bits [lo, hi)
    const int64_t hi = (b1 < rs + P::R ? b1 : rs + P::R) - rs;
    const int len = (int)(hi - lo);
    const uint32_t v = record_string_bits<K, BITS>(codes + r * W, norms[r], (int)lo);
    const uint32_t m = len >= 32 ? ~0u : ((1u << len) - 1u);
    out |= (v & m) << (int)((b0 > rs ? b0 : rs) - b0);
  }
  packed[w] = out;
}

}  // namespace

int packed_record_bits(const fq_codebook* cb) { return cb->nb * cb->bits + 16; }

hipError_t launch_pack(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                       int64_t n, uint32_t* packed, hipStream_t s) {
  const int64_t words = (n * packed_record_bits(cb) + 31) / 32;
  const int64_t blocks = (words + 255) / 256;
#define FQ_PACK(KK, BB)                                                                      \
  if (cb->k == KK && cb->bits == BB) {                                                       \
    hipLaunchKernelGGL((pack_kernel<KK, BB>), dim3((unsigned)blocks), dim3(256), 0, s, codes, \
                       norms, n, packed, words);                                             \
    return hipGetLastError();                                                                \
  }
  FQ_VARIANTS(FQ_PACK)
  FQ_VARIANTS_LARGE(FQ_PACK)
#undef FQ_PACK
  return hipErrorInvalidValue;
}

}  // namespace fq
