// FibQuant encode (FibQuant technical summary, section 2.3): norm, shared
// rotation, per-block nearest codeword, fixed-rate packing (section 1).
//
// One wave encodes a chunk of 16 vectors at a time:
//
//  1. norm: nu = |x|_2 from a pairwise float32 sum of squares (of the input
//     scaled by a power of two) and the hardware square root, within
//     3.3e-7 relative of the exact norm; the stored norm is that value
//     rounded to binary16, the rounding of the exact norm except within that
//     distance of a rounding midpoint.
//  2. rotation on the matrix cores: Pi = Pi_hi + 2^-11 Pi_lo (both binary16),
//     y = Pi_hi x + 2^-11 Pi_lo x with v_mfma_f32_16x16x16_f16 (binary16 input
//     is exact; float32 input is scaled by a power of two and split the same
//     way), z~ = y / nu in float32, staged in LDS.
//  3. block search: every (vector, block) column looks for
//     argmin_n t(n) = |c_n|^2 - 2 <z~, c_n> (the distance without |z|^2) over
//     the exact candidate list of its grid cell (k = 2, 3, and 4 with N >= 64;
//     see fq_grid.cpp) or over the whole codebook, in float32, keeping the
//     best and second-best value.
//  4. certification: with D = t + |z|^2, the computed t of every codeword is
//     within gv (sqrt D + 3|z|)^2 of its exact value at z~ (a chain of k
//     float32 fused multiply-adds, each rounded once), and z~ is within ez of
//     the exact z per coordinate, which moves a difference t(n) - t(m) by at
//     most 2 ez sqrt(k) (sqrt D_n + sqrt D_m).  Both bounds grow more slowly
//     than the gap as D_n grows, so when the second-best gap exceeds their sum
//     for the runner-up, the float32 winner is the exact argmin for the exact
//     z and the result is final.
//  5. otherwise (near ties, non-finite data, blocks outside the candidate
//     grid) the block is redone exactly by 16 lanes: z's block in float64 from
//     x and the float64 Pi, then sum_t (z_t - c_t)^2 in float64 over the
//     candidates of that block's cell (all N codewords where the cell has no
//     list), ties to the lowest index.
//  For k = 3 the one-coordinate last block is searched on its coordinate
//  computed exactly in float64 (the codewords' first coordinates are packed
//  too closely for the float32 certificate to settle most of those blocks).
//  6. the chunk's indices are packed LSB-first into fixed-size records and
//     written with coalesced word stores, norms beside them.
//
// ez covers the binary16 split of Pi (and of x), the float32 accumulation
// (each 16-product group summed from zero on the matrix cores, taken as at
// most one rounding of 2^-23 relative per accumulated term, then the groups
// added in float32) and the final scaling; it is computed on the host from the
// actual split residuals.
#include "fq_common.h"
#include "fq_encode_x.h"
#include "fq_internal.h"

namespace fq {
namespace {

using namespace encx;

// waves per workgroup: 8, so that the rotation fragments and the codebook
// table (staged once per workgroup) are shared by more waves and two
// workgroups fit a compute unit: 16 waves per CU, 4 per SIMD (with 4 waves
// per workgroup the LDS allowed 3 workgroups, 3 waves per SIMD, and the
// encodes ran about 11 % slower).  The 4096-entry table (64 KB) leaves room
// for one workgroup per compute unit only, so that one gets 12 waves (3 per
// SIMD; 23 % faster than 8 on the 2^24-vector stress set; 16 waves with the
// table split into binary16 codewords and float32 norms gained under 2 %).
template <int BITS>
constexpr int enc_waves() { return BITS == 12 ? 12 : 8; }
constexpr float SLACK = 1e-5f;  // covers |D~ - D| inside the square roots of the bound

// Values of other lanes of the same 16-lane row through DPP: row_ror:8
// (0x128), row_ror:4 (0x124), quad_perm [2,3,0,1] (0x4E) and [1,0,3,2]
// (0xB1).  Each step combines a lane with a partner, so after the four steps
// every lane of the row holds the reduction over all 16.
template <int CTRL>
__device__ inline int row_dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline double row_dpp(double v) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = row_dpp_i<CTRL>(p.x);
  p.y = row_dpp_i<CTRL>(p.y);
  return __builtin_bit_cast(double, p);
}
__device__ inline double row16_sum(double v) {
  v += row_dpp<0x128>(v);
  v += row_dpp<0x124>(v);
  v += row_dpp<0x4E>(v);
  v += row_dpp<0xB1>(v);
  return v;
}

// 1 / sqrt(a) in float64 for a > 0 (infinity for 0, NaN for NaN): the hardware
// estimate refined by two Newton steps y <- y + y (1 - a y^2) / 2, each of
// which squares the relative error, so the result is within a few units in
// the last place.
__device__ inline double rsqrt_f64(double a) {
  double y = __builtin_amdgcn_rsq(a);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-a * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// Fields of BITS bits that can overlap one 32-bit word of a record.
template <int BITS>
constexpr int pack_fields() { return 31 / BITS + 2; }

template <int K, int BITS>
struct EncShape {
  static constexpr int NB = (D + K - 1) / K;
  static constexpr int LAST = D - (NB - 1) * K;
  static constexpr int S = ((K + 1) + 3) / 4 * 4;   // search-table stride (floats)
  static constexpr int W = (NB * BITS + 31) / 32;
  // u16 per staged index row: the NB indices, then zeros for the packer
  static constexpr int IP = (NB + pack_fields<BITS>()) / 2 * 2;
  static constexpr int NCOL = EV * NB;              // columns per chunk
  static constexpr bool EXACT_LAST = LAST < K;      // one-coordinate last block
  static constexpr size_t WAVE_BYTES =
      ((size_t)EV * ZP * 4 + (EXACT_LAST ? EV * 8 : 0) + (size_t)EV * IP * 2 + (size_t)NCOL * 2 +
       15) / 16 * 16;
  // workgroup-shared bytes after the search table: the last row of Pi (float64)
  static constexpr size_t SHARED_EXTRA = EXACT_LAST ? D * 8 : 0;
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
  const uint16_t* grid;    // candidate records of the block grid (k = 2, 3, 4)
  const uint16_t* grid1;   // candidate records of the one-coordinate last block
  uint32_t grid_bytes, grid1_bytes;
  int G, G1;               // cells per dimension
  float gscale, g1scale;   // cells per unit length
  OutRows rows;            // record of each encoded row
  // rows n1 .. n - 1: a second input and its outputs (same codebook);
  // n1 = n when there is none
  const void* x2;
  uint32_t* codes2;
  uint16_t* norms2;
  int64_t n1;
};

__host__ __device__ inline size_t enc_table_bytes(int N, int S) {   // N rows + sentinel
  return ((size_t)(N + 1) * S * 4 + 15) / 16 * 16;
}

// Word w of a record from the staged indices of one vector (4-byte aligned
// row of uint16, zero past the NB indices for pack_fields - 1 entries): byte
// permutes for 8-bit fields, nibble merges for 4-bit fields, otherwise the
// overlapping fields gathered into 64 bits and shifted into place.
template <int BITS, int NB>
__device__ inline uint32_t pack_word(const uint16_t* idx, int w) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(idx);
  if constexpr (BITS == 8 && NB % 4 == 0) {
    const uint32_t d0 = p[2 * w], d1 = p[2 * w + 1];   // (i0 | i1 << 16), (i2 | i3 << 16)
    return __builtin_amdgcn_perm(d1, d0, 0x06040200u);
  } else if constexpr (BITS == 4 && NB % 8 == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t d = p[4 * w + q];
      v |= ((d & 0xFu) | ((d >> 12) & 0xF0u)) << (8 * q);
    }
    return v;
  } else {
    constexpr int F = pack_fields<BITS>();
    const int j0 = (32 * w) / BITS;
    const int sh = 32 * w - j0 * BITS;   // 0 <= sh < BITS
    uint64_t acc = 0;
#pragma unroll
    for (int u = 0; u < F; ++u) acc |= (uint64_t)idx[j0 + u] << (u * BITS);
    return (uint32_t)(acc >> sh);
  }
}

// A column (one block of one vector) ready for the search: its coordinates,
// squared norm, and for the grid whether it lies inside plus its cell record.
template <int K, int RW>
struct ColPrep {
  float z[K];
  float zz;
  bool inside;
  uint32_t rec[RW];
};

// Candidate records are read through a buffer resource (32-bit offsets; the
// grid of a codebook is at most a few MB).
template <int K, int RW, bool GRID>
__device__ inline void prepare_column(ColPrep<K, RW>& cp, const float* zrow, bool live,
                                      __amdgpu_buffer_rsrc_t grid, int G, float gscale) {
  float zz = 0.f;
#pragma unroll
  for (int t = 0; t < K; ++t) {
    cp.z[t] = live ? zrow[t] : 0.f;
    zz = fmaf(cp.z[t], cp.z[t], zz);
  }
  cp.zz = zz;
  cp.inside = live;
  if constexpr (GRID) {
    uint32_t cell = 0, mul = 1;
#pragma unroll
    for (int t = 0; t < K; ++t) {
      const float u = grid_pos(cp.z[t], gscale);
      cp.inside = cp.inside && grid_pos_inside(u, G);
      cell += (uint32_t)(int)u * mul;   // used only when every coordinate is inside
      mul *= (uint32_t)G;
    }
    const uint32_t off = (cp.inside ? cell : 0u) * (4u * RW);
#pragma unroll
    for (int h = 0; h < RW / 4; ++h) {
      const u32x4 r0 = __builtin_amdgcn_raw_buffer_load_b128(grid, off + 16 * h, 0, 0);
      cp.rec[4 * h] = r0.x;
      cp.rec[4 * h + 1] = r0.y;
      cp.rec[4 * h + 2] = r0.z;
      cp.rec[4 * h + 3] = r0.w;
    }
  }
}

// Best and second-best t(n) = |c_n|^2 - 2 <z, c_n> over the cell's list (grid)
// or the whole codebook (scan; NC > 0: a compile-time trip count of NC = N
// entries, as every artifact holds N = 2^bits codewords), and the gap test.
// The search table read through the constant address space: the table is
// never written while a kernel runs, so uniform reads become scalar loads
// whose values feed the vector instructions straight from scalar registers.
typedef const float __attribute__((address_space(4)))* ConstFloatPtr;

template <int K, int S, int RW, bool GRID, int NC>
__device__ inline void search_column(const ColPrep<K, RW>& cp, const float* sEnc, ConstFloatPtr gEnc,
                                     int N, float gv, float ez, int& i1out, bool& certain) {
  float m1 = INFINITY, m2 = INFINITY;
  int i1 = 0;
  bool listed = true;   // the search covered every possible nearest codeword
  // list slots past the count hold the sentinel row N (zero codeword with an
  // infinite norm), so a full block needs no per-slot test
  auto visit = [&](const float (&er)[K + 1], int i) {
    float t = er[K];
#pragma unroll
    for (int tt = 0; tt < K; ++tt) t = fmaf(er[tt], cp.z[tt], t);
    const bool p = t < m1;
    m2 = __builtin_amdgcn_fmed3f(m1, m2, t);
    m1 = p ? t : m1;
    i1 = p ? i : i1;
  };
  auto row = [&](uint32_t i, float (&er)[K + 1]) {
#pragma unroll
    for (int tt = 0; tt <= K; ++tt) er[tt] = sEnc[i * S + tt];
  };
  if constexpr (GRID) {
    // the cell's exact candidate list (count first, then increasing indices),
    // two entries per step so that two table reads are in flight together
    const uint32_t c0 = cp.rec[0] & 0xFFFFu;
    const int cnt = (cp.inside && c0 != GRID_OVERFLOW) ? (int)c0 : 0;
    listed = cnt > 0;
    auto idx_of = [&](int e) -> uint32_t {
      const uint32_t w = cp.rec[e >> 1];
      // low half by a byte permute, which keeps the row address one shift-add
      return (e & 1) ? (w >> 16) : __builtin_amdgcn_perm(0u, w, 0x0c0c0100u);
    };
#pragma unroll
    for (int e0 = 1; e0 < 2 * RW; e0 += 2) {
      if (__builtin_amdgcn_ballot_w64(e0 <= cnt) == 0) break;
      const uint32_t ia = idx_of(e0);
      float ea[K + 1], eb[K + 1];
      row(ia, ea);
      if (e0 + 1 < 2 * RW) {
        const uint32_t ib = idx_of(e0 + 1);
        row(ib, eb);
        visit(ea, (int)ia);
        visit(eb, (int)ib);
      } else {
        visit(ea, (int)ia);
      }
    }
  } else if constexpr (NC > 0 && NC * (K + 1) <= 32) {
    // a table of at most 32 floats: fully unrolled, its rows (the same for
    // every lane) in scalar registers across the chunk's columns
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      float er[K + 1];
#pragma unroll
      for (int tt = 0; tt <= K; ++tt) er[tt] = gEnc[i * S + tt];
      visit(er, i);
    }
  } else if constexpr (NC > 0) {
    // the whole codebook with the trip count known at compile time, unrolled
    // by four (fully unrolled, the compiler would keep every row live across
    // the columns and spill); every lane reads the same row, so the rows come
    // through scalar loads instead of LDS
#pragma unroll 4
    for (int i = 0; i < NC; ++i) {
      float er[K + 1];
#pragma unroll
      for (int tt = 0; tt <= K; ++tt) er[tt] = gEnc[i * S + tt];
      visit(er, i);
    }
  } else {
#pragma unroll 4
    for (int i = 0; i < N; ++i) {
      float er[K + 1];
      row((uint32_t)i, er);
      visit(er, i);
    }
  }
  // gap test of the header, with the runner-up's terms doubled for both
  // (m1 <= m2) and (r + 3|z|)^2 <= 2 r^2 + 18 |z|^2
  constexpr float KSQ = K == 2 ? 1.41421356f : (K == 3 ? 1.73205081f : (K == 4 ? 2.f : 2.82842712f));
  const float d2 = fmaxf(m2 + cp.zz, 0.f) + SLACK;
  // hardware square root (within 1 ulp), nudged up to stay an upper bound
  const float rt = __builtin_amdgcn_sqrtf(d2);
  const float thr = fmaf(4.f * gv, d2, fmaf(36.f * gv, cp.zz, fmaf(4.0004f * ez * KSQ, rt, 1e-12f)));
  // a single listed candidate is the nearest codeword everywhere in the cell
  certain = listed && m1 < INFINITY && (m2 == INFINITY || (m2 - m1) > thr);
  i1out = i1;
}

template <int K, int BITS, typename TX, bool GRID>
__global__ __launch_bounds__(enc_waves<BITS>() * 64) __attribute__((amdgpu_waves_per_eu(4))) void encode_kernel(EncArgs a) {
  using Sh = EncShape<K, BITS>;
  constexpr int NB = Sh::NB, S = Sh::S, IP = Sh::IP;
  constexpr int NBF = (Sh::LAST == K) ? NB : NB - 1;   // full blocks per vector
  constexpr int NCF = EV * NBF;                         // full-block columns per chunk
  constexpr int CPLF = (NCF + 63) / 64;
  constexpr int QB = (CPLF + 1) / 2;
  constexpr int RW = grid_record_entries(K) / 2;        // record words
  extern __shared__ __align__(16) unsigned char smem[];
  const int N = a.N;
  _Float16* sRot = reinterpret_cast<_Float16*>(smem);
  float* sEnc = reinterpret_cast<float*>(smem + ROT_BYTES);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  double* sPiL = reinterpret_cast<double*>(smem + ROT_BYTES + enc_table_bytes(N, S));
  unsigned char* wb = smem + ROT_BYTES + enc_table_bytes(N, S) + Sh::SHARED_EXTRA +
                      wave * Sh::WAVE_BYTES;
  float* sZ = reinterpret_cast<float*>(wb);
  double* sZL = reinterpret_cast<double*>(wb + EV * ZP * 4);             // k = 3: exact z_63
  uint16_t* sIdx = reinterpret_cast<uint16_t*>(wb + EV * ZP * 4 + (Sh::EXACT_LAST ? EV * 8 : 0));
  uint16_t* sFb = sIdx + EV * IP;

  // the staged index rows' zero tails (never written afterwards)
  for (int i = lane; i < EV * (IP - NB); i += 64) sIdx[(i / (IP - NB)) * IP + NB + i % (IP - NB)] = 0;
  for (int i = threadIdx.x; i < ROT_BYTES / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(sRot)[i] = reinterpret_cast<const u32x4*>(a.rotfrag)[i];
  for (int i = threadIdx.x; i < (N + 1) * S / 4; i += blockDim.x)
    reinterpret_cast<floatx4*>(sEnc)[i] = reinterpret_cast<const floatx4*>(a.enc)[i];
  if constexpr (Sh::EXACT_LAST)
    for (int i = threadIdx.x; i < D; i += blockDim.x) sPiL[i] = a.pi64[(D - 1) * D + i];
  __syncthreads();

  const TX* __restrict__ x = static_cast<const TX*>(a.x);
  const __amdgpu_buffer_rsrc_t grid_rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.grid), (short)0, (int)a.grid_bytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t grid1_rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.grid1), (short)0, (int)a.grid1_bytes, BUF_DWORD3);
  const int64_t nchunks = (a.n + EV - 1) / EV;
  constexpr int WAVES = enc_waves<BITS>();
  const int64_t tw = (int64_t)gridDim.x * WAVES;
  const int j = lane & 15, g = lane >> 4;

  // the lane's row of a chunk (rows past the end repeat the last one)
  // row r of the input: rows >= a.n1 come from the second input (keys and
  // values of one decode step in one launch)
  auto xrow = [&](int64_t r) {
    return r < a.n1 ? x + r * a.ld : static_cast<const TX*>(a.x2) + (r - a.n1) * a.ld;
  };
  auto row_of = [&](int64_t chunk) {
    const int64_t base = chunk * EV;
    const int64_t last = a.n - 1 - base;
    return xrow(base + (j < last ? j : last));
  };
  int64_t ch = (int64_t)blockIdx.x * WAVES + wave;
  XRaw<TX> xraw;
  // the 4096-entry table's candidate grid (8 MB) does not fit in L2 beside
  // the input stream: non-temporal input loads leave its lines there (18 %
  // less fetch traffic at the same speed; the smaller grids fit anyway and
  // ran 3-6 % slower with them)
  constexpr bool NT_IN = BITS == 12;
  if (ch < nchunks) load_raw<TX, NT_IN>(row_of(ch), g, xraw);
  for (; ch < nchunks; ch += tw) {
    const int64_t base = ch * EV;
    const int nv = (int)((a.n - base) < EV ? (a.n - base) : EV);

    // ---- 1. norm (float32) and the binary16 fragments; next chunk's x in flight
    XFrag<TX> xf;
    finish_x<TX>(xraw, xf);
    if constexpr (Sh::EXACT_LAST) {
      // k = 3: the first coordinates of the codewords lie too close together
      // for the float32 certificate on the one-coordinate last block, so its
      // coordinate z_63 = <Pi row 63, x> / |x| is taken exactly in float64
      double ss = 0.0, dt = 0.0;
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        double xv[4];
        if constexpr (sizeof(TX) == 2) {
          const half4 h = __builtin_bit_cast(half4, xraw.q[kq]);
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = (double)(float)h[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = (double)xraw.q[kq][e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ss = fma(xv[e], xv[e], ss);
          dt = fma(sPiL[16 * kq + 4 * g + e], xv[e], dt);
        }
      }
      ss += shfl_xor_f64(ss, 16);
      ss += shfl_xor_f64(ss, 32);
      dt += shfl_xor_f64(dt, 16);
      dt += shfl_xor_f64(dt, 32);
      if (g == 0) sZL[j] = dt * rsqrt_f64(ss);   // a zero vector gives NaN
    }
    if (ch + tw < nchunks) load_raw<TX, NT_IN>(row_of(ch + tw), g, xraw);
    // norm within 3.3e-7 relative (pairwise sum, hardware square root): its
    // binary16 rounding differs from that of the exact norm only within that
    // distance of a rounding midpoint
    const float nus = __builtin_amdgcn_sqrtf(xf.ss);     // norm of the scaled vector
    const uint16_t nbits = f32_to_f16_rne(nus * xf.escale);
    // a zero vector gets NaN coordinates (0 * inf): its blocks go to the exact
    // path, which returns index 0 for them
    const float inv = __builtin_amdgcn_rcpf(nus);

    // ---- 2. rotation: lane holds z~[vector j][16 ot + 4 g + r]
    rotate_to_lds<TX>(xf, sRot, inv, sZ, lane);
    wave_lds_sync();

    // ---- 3-4. search + certification.  Full blocks first, in batches of QB
    //      columns per lane: gather the blocks and issue their candidate
    //      record loads, then search; the one-coordinate last block (k = 3)
    //      gets a pass of its own.  Column ids: full c < NCF is (c / NBF,
    //      c % NBF); c = NCF + v is vector v's last block.
    int nfb = 0;
    auto record = [&](int c, bool live, int v, int b, int i1, bool certain) {
      if (live) sIdx[v * IP + b] = (uint16_t)i1;
      const bool fb = live && !certain;
      const uint64_t m = __builtin_amdgcn_ballot_w64(fb);
      if (fb) {
        const int pos = nfb + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        sFb[pos] = (uint16_t)c;
      }
      nfb += __builtin_popcountll(m);
    };
#pragma unroll
    for (int qb = 0; qb < CPLF; qb += QB) {
      ColPrep<K, RW> cp[QB];
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int c = lane + 64 * (qb + q);
        const int v = c / NBF, b = c - v * NBF;
        const bool live = c < NCF && v < nv;
        prepare_column<K, RW, GRID>(cp[q], sZ + v * ZP + K * b, live, grid_rc, a.G, a.gscale);
      }
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int c = lane + 64 * (qb + q);
        const int v = c / NBF, b = c - v * NBF;
        const bool live = c < NCF && v < nv;
        int i1;
        bool certain;
        search_column<K, S, RW, GRID, (BITS <= 4 ? (1 << BITS) : 0)>(
            cp[q], sEnc, (ConstFloatPtr)a.enc, N, a.gv, a.ez, i1, certain);
        record(c, live, v, b, i1, certain);
      }
    }
    if constexpr (Sh::EXACT_LAST) {
      // the last block of vector `lane`: its cell's candidates compared in
      // float64 on the exact coordinate, increasing indices with a strict
      // comparison (ties to the lowest index); exact, so no gap test
      const bool live = lane < nv;
      const int v = lane < EV ? lane : 0;
      const double z0 = sZL[v];
      const float u = grid_pos((float)z0, a.g1scale);
      const bool inside = live && grid_pos_inside(u, a.G1);
      const uint32_t off = (inside ? (uint32_t)(int)u : 0u) * (4u * RW);
      uint32_t rec[RW];
#pragma unroll
      for (int h = 0; h < RW / 4; ++h) {
        const u32x4 r0 = __builtin_amdgcn_raw_buffer_load_b128(grid1_rc, off + 16 * h, 0, 0);
        rec[4 * h] = r0.x;
        rec[4 * h + 1] = r0.y;
        rec[4 * h + 2] = r0.z;
        rec[4 * h + 3] = r0.w;
      }
      const uint32_t c0 = rec[0] & 0xFFFFu;
      const int cnt = (inside && c0 != GRID_OVERFLOW) ? (int)c0 : 0;
      double best = INFINITY;
      int bi = 0;
      auto consider = [&](int e, uint32_t i, float c) {
        const double df = z0 + 0.5 * (double)c;   // c_0 = -e_0 / 2, exact
        const double dd = df * df;
        if (e <= cnt && dd < best) {
          best = dd;
          bi = (int)i;
        }
      };
#pragma unroll
      for (int e0 = 1; e0 < 2 * RW; e0 += 2) {   // two table reads in flight per step
        if (__builtin_amdgcn_ballot_w64(e0 <= cnt) == 0) break;
        const uint32_t ia = rec[e0 >> 1] >> 16;   // odd entries: high halves
        const float ca = sEnc[ia * S];
        if (e0 + 1 < 2 * RW) {
          const uint32_t ib = rec[(e0 + 1) >> 1] & 0xFFFFu;
          const float cb = sEnc[ib * S];
          consider(e0, ia, ca);
          consider(e0 + 1, ib, cb);
        } else {
          consider(e0, ia, ca);
        }
      }
      record(NCF + v, live, v, NB - 1, bi, cnt > 0);
    }
    wave_lds_sync();

    // ---- 5. exact float64 redo of uncertified columns: four at a time, one
    //      per 16-lane group (lane i of a group holds coordinates 4i .. 4i + 3).
    //      Binary16 input is staged in LDS (the z rows are free now), so the
    //      only global reads are the rows of Pi and the cell's record.
    _Float16* sXh = reinterpret_cast<_Float16*>(sZ);   // [EV][64]
    if constexpr (sizeof(TX) == 2) {
      if (nfb > 0) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
          *reinterpret_cast<half4*>(sXh + j * D + 16 * kq + 4 * g) = xf.hi[kq];
        wave_lds_sync();
      }
    }
    for (int e0 = 0; e0 < nfb; e0 += 4) {
      const int l16 = lane & 15;
      const bool ok = e0 + g < nfb;
      const int c = sFb[ok ? e0 + g : e0];
      const bool last = c >= NCF;
      const int v = last ? c - NCF : c / NBF, b = last ? NB - 1 : c - (c / NBF) * NBF;
      const int rj = last ? Sh::LAST : K;
      double pr[K][4];
#pragma unroll
      for (int t = 0; t < K; ++t)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          pr[t][qq] = t < rj ? a.pi64[(K * b + t < D ? K * b + t : D - 1) * D + 4 * l16 + qq] : 0.0;
      double xq[4];
      if constexpr (sizeof(TX) == 2) {
        const half4 h = *reinterpret_cast<const half4*>(sXh + v * D + 4 * l16);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) xq[qq] = (double)(float)h[qq];
      } else {
        const TX* xr = xrow(base + v) + 4 * l16;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) xq[qq] = (double)xr[qq];
      }
      double ssd = 0.0;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ssd = fma(xq[qq], xq[qq], ssd);
      const double inv = rsqrt_f64(row16_sum(ssd));   // 1 / |x|
      double zd[K];
#pragma unroll
      for (int t = 0; t < K; ++t) {
        double sum = 0.0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) sum = fma(pr[t][qq], xq[qq], sum);
        zd[t] = row16_sum(sum) * inv;
      }
      double best = INFINITY;
      int bi = 0;
      auto consider = [&](int i) {
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
      };
      // the exact block lies in its own grid cell, whose list holds every
      // codeword that can be nearest there: each lane takes every 16th one;
      // outside the grid (or for an over-full cell) scan the whole codebook
      int cnt = 0;
      uint32_t mine = 0, mine2 = 0;   // this lane's list entries (read with the count)
      if constexpr (GRID) {
        const int dims = last ? 1 : K;
        bool inside = true;
        int cell = 0, mul = 1;
        const int G = last ? a.G1 : a.G;
        const float sc = last ? a.g1scale : a.gscale;
#pragma unroll
        for (int t = 0; t < K; ++t)
          if (t < dims) {
            const float u = grid_pos((float)zd[t], sc);
            const bool in = grid_pos_inside(u, G);
            inside = inside && in;
            cell += (in ? (int)u : 0) * mul;   // stays inside the table
            mul *= G;
          }
        const uint16_t* rec = (last ? a.grid1 : a.grid) + (size_t)cell * (2 * RW);
        const uint32_t c0 = rec[0];
        mine = rec[1 + (l16 < 2 * RW - 1 ? l16 : 2 * RW - 2)];
        if constexpr (2 * RW - 1 > 16) mine2 = rec[1 + (l16 + 16 < 2 * RW - 1 ? l16 + 16 : 2 * RW - 2)];
        cnt = (inside && c0 != GRID_OVERFLOW) ? (int)c0 : 0;
      }
      if (cnt > 0) {   // a list holds at most 2 RW - 1 <= 31 entries
        if (l16 < cnt) consider((int)mine);
        if constexpr (2 * RW - 1 > 16)
          if (l16 + 16 < cnt) consider((int)mine2);
      } else {
        for (int i = l16; i < N; i += 16) consider(i);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {   // the lowest index among the smallest distances
        const double ob = m == 0 ? row_dpp<0x128>(best) : m == 1 ? row_dpp<0x124>(best)
                        : m == 2 ? row_dpp<0x4E>(best) : row_dpp<0xB1>(best);
        const int oi = m == 0 ? row_dpp_i<0x128>(bi) : m == 1 ? row_dpp_i<0x124>(bi)
                     : m == 2 ? row_dpp_i<0x4E>(bi) : row_dpp_i<0xB1>(bi);
        if (ob < best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      if (ok && l16 == 0) sIdx[v * IP + b] = (uint16_t)bi;
    }
    wave_lds_sync();

    // ---- 6. pack + store (contiguous records, or appended to caches)
    if (a.rows.inner == 0) {
      uint32_t* __restrict__ out = a.codes + base * Sh::W;
#pragma unroll
      for (int it = 0; it < (EV * Sh::W + 63) / 64; ++it) {   // the same words of every chunk
        const int t = lane + 64 * it;
        const int v = t / Sh::W, w = t - v * Sh::W;
        if (t < nv * Sh::W) out[t] = pack_word<BITS, NB>(sIdx + v * IP, w);
      }
      if (g == 0 && j < nv) a.norms[base + j] = nbits;
    } else {
      auto rec_of = [&](int64_t r) {
        if (r >= a.n1) r -= a.n1;
        return (r / a.rows.inner) * a.rows.stride + a.rows.pos + r % a.rows.inner;
      };
      for (int t = lane; t < nv * Sh::W; t += 64) {
        const int v = t / Sh::W, w = t - v * Sh::W;
        uint32_t* codes = base + v < a.n1 ? a.codes : a.codes2;
        codes[rec_of(base + v) * Sh::W + w] = pack_word<BITS, NB>(sIdx + v * IP, w);
      }
      if (g == 0 && j < nv) (base + j < a.n1 ? a.norms : a.norms2)[rec_of(base + j)] = nbits;
    }
    wave_lds_sync();
  }
}

template <int K, int BITS, typename TX>
hipError_t launch_k(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                    uint16_t* norms, hipStream_t s, OutRows rows, SecondInput second) {
  using Sh = EncShape<K, BITS>;
  constexpr int WAVES = enc_waves<BITS>();
  const size_t shm =
      ROT_BYTES + enc_table_bytes(cb->N, Sh::S) + Sh::SHARED_EXTRA + WAVES * Sh::WAVE_BYTES;
  // candidate lists for k = 2, 3 and for k = 4 with N >= 64 (see the codebook
  // load); full scans otherwise
  constexpr bool GRID = (K == 2 || K == 3 || (K == 4 && BITS >= 6));
  auto kern = encode_kernel<K, BITS, TX, GRID>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  // resident workgroups per device, computed on first use (the dynamic LDS
  // size depends only on the variant, like the kernel)
  static DeviceCache cap_cache;
  const int64_t cap = cap_cache.get(reinterpret_cast<const void*>(kern), WAVES * 64, shm);
  const int64_t chunks = (n + (second.x ? second.n : 0) + EV - 1) / EV;
  int64_t blocks = (chunks + WAVES - 1) / WAVES;
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
  a.grid = cb->t.grid;
  a.grid1 = cb->t.grid1 ? cb->t.grid1 : cb->t.grid;
  a.grid_bytes = (uint32_t)(cb->grid_host.size() * sizeof(uint16_t));
  a.grid1_bytes = (uint32_t)((cb->t.grid1 ? cb->grid1_host : cb->grid_host).size() * sizeof(uint16_t));
  a.G = cb->grid_G;
  a.G1 = cb->grid1_G > 0 ? cb->grid1_G : 1;
  a.gscale = grid_scale(cb->grid_G);
  a.g1scale = grid_scale(a.G1);
  a.rows = rows;
  a.n1 = n;
  a.x2 = nullptr;
  a.codes2 = nullptr;
  a.norms2 = nullptr;
  if (second.x && rows.inner == 0) return hipErrorInvalidValue;   // needs a record map
  if (second.x) {   // the second input's rows follow the first's
    a.n1 = n;
    a.n = n + second.n;
    a.x2 = second.x;
    a.codes2 = second.codes;
    a.norms2 = second.norms;
  }
  if (GRID && (cb->t.grid == nullptr || cb->grid_G <= 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WAVES * 64), shm, s, a);
  return hipGetLastError();
}

template <typename TX>
hipError_t dispatch(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                    uint16_t* norms, hipStream_t s, OutRows rows, SecondInput second) {
#define FQ_ENC_CASE(KK, BB) \
  if (cb->k == KK && cb->bits == BB)                                                        \
    return launch_k<KK, BB, TX>(cb, x, n, ld, codes, norms, s, rows, second);
  FQ_VARIANTS(FQ_ENC_CASE)
#undef FQ_ENC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n, int64_t ld,
                         uint32_t* codes, uint16_t* norms, hipStream_t s, OutRows rows,
                         SecondInput second) {
  if (xt == FQ_F16)
    return dispatch<_Float16>(cb, static_cast<const _Float16*>(x), n, ld, codes, norms, s, rows,
                              second);
  return dispatch<float>(cb, static_cast<const float*>(x), n, ld, codes, norms, s, rows, second);
}

}  // namespace fq
