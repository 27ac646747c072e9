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
//    so every shift is static) into a table of 16-bit indices in LDS.
//  * Per tile of 16 vectors, v_mfma_f32_16x16x32_f16 forms Y^T = Pi^T Z_hat^T:
//    A = Pi^T, rounded to binary16, in registers for the whole kernel;
//    B = Z_hat^T, gathered from the LDS codebook (binary16) by index.  Both
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

template <int K, int BITS, typename TY>
constexpr size_t wave_lds() {
  return CHUNK * Shape<K, BITS>::IDX_PITCH * 2 + CHUNK * 4 + TILE * OUT_PITCH * sizeof(TY);
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
  } else if constexpr (K % 8 == 0 && K >= 16) {   // 8 coordinates of one codeword
    const uint32_t i0 = idx[c0 / K];
    return *reinterpret_cast<const half8*>(cbh + i0 * K + c0 % K);
  } else {  // K = 3: one coordinate at a time; the last block may be partial
    half8 hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const int j = c / K, t = c - j * K;
      hi[e] = cbh[idx[j] * K + t];
    }
    return hi;
  }
}

template <int K, int BITS, typename TY, bool GATHER>
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
  const size_t cb_bytes = GTAB ? 0 : ((size_t)N * K * sizeof(_Float16) + 15) / 16 * 16;
  // the wave index is uniform: keep it (and the buffer descriptors derived from
  // it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  unsigned char* wbase = smem + cb_bytes + (size_t)wave * wave_lds<K, BITS, TY>();
  uint16_t* sIdx = reinterpret_cast<uint16_t*>(wbase);                       // [CHUNK][IDX_PITCH]
  float* sNu = reinterpret_cast<float*>(wbase + CHUNK * Sh::IDX_PITCH * 2);  // [CHUNK]
  TY* sOut = reinterpret_cast<TY*>(wbase + CHUNK * Sh::IDX_PITCH * 2 + CHUNK * 4);

  if constexpr (!GTAB)
    for (int e = threadIdx.x; e < N * K; e += DEC_THREADS) sCbh[e] = cbh_g[e];
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
    if constexpr (GATHER)
      load_chunk_gather<W>(t, c, lane, codes, norms, rows, n_records, n);
    else
      load_chunk<W>(t, c, lane, codes, norms, n);
  };
  auto stage = [&](const ChunkRegs<W>& t) {
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
        const half8 zh = GTAB ? zg[m][s] : gather8<K>(vidx, sCbh, 32 * s + 8 * grp);
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
        // faster than default-policy stores)
        __builtin_amdgcn_raw_buffer_store_b128(vv, ry, (int)((v * ld + q * PER) * sizeof(TY)), 0,
                                               CPOL_NT);
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

template <int K, int BITS, typename TY, bool GATHER>
hipError_t launch_k(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, TY* y, int64_t ld,
                    hipStream_t s) {
  const size_t cb_bytes = large_block(K) ? 0 : ((size_t)cb->N * K * sizeof(_Float16) + 15) / 16 * 16;
  const size_t shm = cb_bytes + DEC_WAVES * wave_lds<K, BITS, TY>();
  auto kern = decode_kernel<K, BITS, TY, GATHER>;
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

template <typename TY, bool GATHER>
hipError_t dispatch(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, TY* y, int64_t ld,
                    hipStream_t s) {
#define FQ_DEC(KK, BB)                                                                     \
  if (cb->k == KK && cb->bits == BB)                                                       \
    return launch_k<KK, BB, TY, GATHER>(cb, codes, norms, rows, n_records, n, y, ld, s);
  FQ_VARIANTS(FQ_DEC)
  FQ_VARIANTS_LARGE(FQ_DEC)
#undef FQ_DEC
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                         const int64_t* rows, int64_t n_records, int64_t n, void* y, fq_dtype yt,
                         int64_t ld, hipStream_t s) {
  if (yt == FQ_F16) {
    _Float16* yy = static_cast<_Float16*>(y);
    return rows ? dispatch<_Float16, true>(cb, codes, norms, rows, n_records, n, yy, ld, s)
                : dispatch<_Float16, false>(cb, codes, norms, rows, n_records, n, yy, ld, s);
  }
  float* yy = static_cast<float*>(y);
  return rows ? dispatch<float, true>(cb, codes, norms, rows, n_records, n, yy, ld, s)
              : dispatch<float, false>(cb, codes, norms, rows, n_records, n, yy, ld, s);
}

}  // namespace fq
