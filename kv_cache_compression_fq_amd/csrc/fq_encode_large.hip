// FibQuant encode on the matrix cores (FibQuant technical summary, sections
// 2.2 and 2.3): large blocks, k = 32 and k = 64 (one or two blocks per vector)
// with N = 4096 codewords, and k = 64 with N = 16384 (a 14-bit index: with the
// 16-bit norm a 30-bit record, the most compressed point of the rate sweep of
// section 4.2), and k = 8 with N = 256 (one bit per coordinate; at the end of
// the file).
//
// The nearest-codeword search is a dense contraction here: every block is
// compared with all N codewords of k coordinates, N k multiply-adds per
// block, and the table (N k binary16 values, 256 KB to 2 MB) is larger than
// LDS.  So the search runs on the matrix cores:
//
//  * One workgroup of 8 waves streams the codebook through LDS in stages of
//    256 codewords with their -|c|^2 / 2 (double-buffered, each stage loaded
//    once per workgroup and shared by its 8 waves).  A wave holds 64 block
//    columns (64 vectors at k = 64, 32 vectors at k = 32) as binary16 B
//    operands, split z~ = z_hi + z_lo (both binary16, the lo part unscaled
//    so it accumulates into the same sum), and for every tile of 16 codewords
//    forms
//    s(n) = <c_n, z~> - |c_n|^2 / 2 with v_mfma_f32_16x16x32_f16, the
//    accumulator starting at -|c_n|^2 / 2 (float32 from the host).  The
//    nearest codeword maximises s.
//  * Each lane keeps, for its 4 accumulator rows ("slots": the codewords
//    16 t + 4 (lane / 16) + r of every tile t), the best and second-best key,
//    where a key is the float32 score with its low TB mantissa bits replaced
//    by the tile number t (TB = log2(N / 16): 8 bits for 4096 codewords, 10
//    for 16384), compared as a signed integer (the scores' order for scores
//    >= 0).  The 16 slots of a column are merged at the end.
//  * Certification.  The computed score of every codeword is within
//    E = EA |z~| + EB of its exact value at z~ (binary16 split of z~: 2^-22
//    relative plus 2^-25 absolute per coordinate; float32 accumulation of
//    2k + 2 terms, taken as one rounding of 2^-23 per term relative to the
//    sum of their magnitudes; the rounded |c|^2 / 2), z~ is within ez of the
//    exact z per coordinate, which moves a score difference by at most
//    2 ez sqrt(k) max|c|, and a key is within 2^(TB-23) of its score
//    relative (so two keys' order is their scores' within 2^(TB-22)).
//    A codeword whose key is more than M below the best key cannot be the
//    exact nearest.  When the best key exceeds M, only the best slot is
//    within M and no slot's second key is, the float32 winner is final.
//  * Otherwise the block goes to the wave's list (its row, its candidates:
//    the slot leaders within M, and the slots whose second key is within M)
//    and its record keeps the float32 winner for now.  After the last pass
//    the workgroup settles its lists exactly in float64, shared out over its
//    waves: z's block from x and the float64 Pi, then the candidates and every
//    codeword of each such slot (all N codewords for non-finite scores or
//    more than 8 candidates); ties go to the lowest index; the exact index
//    replaces the field.  A list that could overflow during a pass is
//    settled at the start of the pass instead.
//  * Records (one 32-bit word: one or two 12-bit fields, or one 14-bit field)
//    and norms are written with coalesced stores.
#include "fq_common.h"
#include "fq_encode_x.h"
#include "fq_internal.h"

namespace fq {
namespace {

using namespace encx;

constexpr int LW = 8;        // waves per workgroup
constexpr int CG = 4;        // column groups of 16 per wave pass
constexpr int TCW = 256;     // codewords per LDS stage
// Uncertain blocks listed per wave: row (2 words), block | count << 8 |
// all-codewords flag << 16, hidden-slot mask, up to 8 candidate indices
// (u16; more set the all-codewords flag).  A pass adds at most 64 entries,
// so the list is settled early when fewer than 64 places are left.
constexpr int FL_MAX = 84;
constexpr int FL_WORDS = 8;
constexpr int FL_CAND = 8;

// LB = log2 N: 12 (k = 32, 64) or 14 (k = 64)
template <int K, int LB>
struct LShape {
  static constexpr int LN = 1 << LB;               // codewords
  static constexpr int NSTAGE = LN / TCW;          // LDS stages per sweep
  static constexpr int TB = LB - 4;                // bits of a tile number (16 codewords a tile)
  static constexpr int NB = D / K;                 // blocks per vector (k divides d)
  static constexpr int KC = K / 32;                // 32-coordinate steps per block
  static constexpr int VPW = 16 * CG / NB;         // vectors per wave pass
  static constexpr int BATCHES = VPW / EV;         // rotation batches of 16 vectors per pass
  static constexpr int STAGE_BYTES = TCW * K * 2;  // one stage of codebook fragments
  static constexpr int LOADS = STAGE_BYTES / (16 * LW * 64);   // 16-byte loads per thread
  static constexpr size_t WAVE_BYTES = (size_t)EV * ZP * 4 + 2 * 64 * 8 + FL_MAX * FL_WORDS * 4;
  static constexpr size_t HN_BYTES = 2 * TCW * 4;    // -|c|^2 / 2 of the two stages
  static constexpr size_t LDS = 2 * (size_t)STAGE_BYTES + HN_BYTES + ROT_BYTES + LW * WAVE_BYTES + LW * 4;
};

struct LArgs {
  const void* x;
  int64_t n, ld;
  uint32_t* codes;
  uint16_t* norms;
  const _Float16* rotfrag;  // Pi hi / lo as 16x16x16 A fragments
  const _Float16* lfrag;    // codebook as 16x16x32 A fragments [tile][kc][lane][8]
  const float* hn;          // -|c_n|^2 / 2, float32
  const _Float16* cbh;      // [N][k] codebook, binary16 (exact)
  const float* enc;         // [N + 1][S] search table (-2 c, |c|^2): c = -enc / 2 exactly
  int S;
  const double* pi64t;       // Pi^T, float64
  float EA, EB, ZT;         // certification constants (see the header)
};

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f64(v, m);
  return v;
}

// Keys compare as signed integers: the order of the float scores for scores
// >= 0 (the only ones a certified or listed winner can have, see the margin
// test), below every non-negative score otherwise.  The low TB bits hold the
// tile number.  Either form is one VALU instruction: a byte permute for
// TB = 8; otherwise v_and_or_b32 with the mask held in a vector register (the
// tile number is a scalar, and the instruction takes one scalar operand and
// no literal).
template <int TB>
__device__ inline int make_key(float score, uint32_t tile, uint32_t vmask) {
  if constexpr (TB == 8)
    return (int)__builtin_amdgcn_perm(__float_as_uint(score), tile, 0x07060500u);
  else
    return (int)((__float_as_uint(score) & vmask) | tile);
}
template <int TB>
__device__ inline uint32_t key_tile(int key) { return (uint32_t)key & ((1u << TB) - 1u); }
__device__ inline float key_value(int key) { return __int_as_float(key); }

// The exact nearest codeword of one listed block (the whole wave): z's block
// in float64 from x and Pi (lane t < k holds z_t), then float64 distances to
// the listed candidates, to every codeword 16 t + s of each hidden slot s,
// or to all N codewords (binary16 table `cbt`, exact); ties to the lowest index.
template <int K, typename TX, int NCW>
__device__ int settle_block(const LArgs& a, const TX* x, const _Float16* cbt, const uint32_t* ent,
                            double* sX, double* sZd, int lane) {
  const int64_t row = (int64_t)((uint64_t)ent[0] | ((uint64_t)ent[1] << 32));
  const uint32_t info = ent[2], hm = ent[3];
  const int b = (int)(info & 0xFFu), nc = (int)((info >> 8) & 0xFFu);
  const bool full = (info >> 16) & 1u;
  const uint16_t* ce = reinterpret_cast<const uint16_t*>(ent + 4);
  // every load first (the block is latency-bound): x, column b K + t of Pi^T
  // (row b K + t of Pi, one coalesced line per i) and the candidates' rows
  const double xv = (double)(float)x[row * a.ld + lane];
  const double* pt = a.pi64t + b * K + (lane < K ? lane : 0);
  constexpr int PH = D / 2;   // Pi^T lines per batch of loads
  double pv[PH];
#pragma unroll
  for (int i = 0; i < PH; ++i) pv[i] = pt[(size_t)i * D];
  float cv[FL_CAND];
#pragma unroll
  for (int e = 0; e < FL_CAND; ++e)
    cv[e] = (!full && e < nc && lane < K) ? (float)cbt[(size_t)ce[e] * K + lane] : 0.f;
  const double nu = sqrt(wave_sum_f64(xv * xv));
  sX[lane] = xv;
  wave_lds_sync();
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < PH; ++i) acc = fma(pv[i], sX[i], acc);
#pragma unroll
  for (int i = 0; i < PH; ++i) pv[i] = pt[(size_t)(PH + i) * D];
#pragma unroll
  for (int i = 0; i < PH; ++i) acc = fma(pv[i], sX[PH + i], acc);
  const double zd = lane < K ? acc / nu : 0.0;   // a zero vector gives NaN: index 0
  sZd[lane] = zd;
  wave_lds_sync();
  double best = INFINITY;
  int bi = 0;
  auto dist = [&](int cn) {   // this lane's codeword, all k coordinates (binary16, exact)
    const half8* cr = reinterpret_cast<const half8*>(cbt + (size_t)cn * K);
    half8 hv[K / 8];
#pragma unroll
    for (int q = 0; q < K / 8; ++q) hv[q] = cr[q];
    double dd = 0.0;
#pragma unroll
    for (int q = 0; q < K / 8; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double df = sZd[8 * q + e] - (double)(float)hv[q][e];
        dd = fma(df, df, dd);
      }
    return dd;
  };
  if (!full) {
#pragma unroll
    for (int e = 0; e < FL_CAND; ++e) {
      if (e < nc) {
        const int cn = ce[e];
        const double df = lane < K ? zd - (double)cv[e] : 0.0;
        const double dd = wave_sum_f64(df * df);
        if (dd < best || (dd == best && cn < bi)) {
          best = dd;
          bi = cn;
        }
      }
    }
    uint32_t h = hm;
    while (h) {
      const int slot = __builtin_ctz(h);
      h &= h - 1;
#pragma unroll 1
      for (int m = 0; m < (NCW / 16 + 63) / 64; ++m) {
        if (lane + 64 * m >= NCW / 16) continue;
        const int cn = 16 * (lane + 64 * m) + slot;
        const double dd = dist(cn);
        if (dd < best || (dd == best && cn < bi)) {
          best = dd;
          bi = cn;
        }
      }
    }
  } else {
#pragma unroll 1
    for (int cn = lane; cn < NCW; cn += 64) {
      const double dd = dist(cn);
      if (dd < best) {
        best = dd;
        bi = cn;
      }
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
  wave_lds_sync();
  return bi;
}

template <int K, int LB, typename TX>
__global__ __launch_bounds__(LW * 64) void encode_large_kernel(LArgs a) {
  using Sh = LShape<K, LB>;
  constexpr int NB = Sh::NB, KC = Sh::KC, LN = Sh::LN, NSTAGE = Sh::NSTAGE, TB = Sh::TB;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sStage = smem;                                           // 2 stages
  float* sHn = reinterpret_cast<float*>(smem + 2 * Sh::STAGE_BYTES);      // [2][TCW]
  _Float16* sRot = reinterpret_cast<_Float16*>(smem + 2 * Sh::STAGE_BYTES + Sh::HN_BYTES);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  unsigned char* wb = smem + 2 * Sh::STAGE_BYTES + Sh::HN_BYTES + ROT_BYTES + wave * Sh::WAVE_BYTES;
  float* sZ = reinterpret_cast<float*>(wb);                               // [EV][ZP]
  double* sX = reinterpret_cast<double*>(wb + EV * ZP * 4);              // exact path: x
  double* sZd = sX + 64;                                                  // exact path: z block
  uint32_t* sList = reinterpret_cast<uint32_t*>(sZd + 64);                // uncertain blocks
  int* sCount = reinterpret_cast<int*>(smem + 2 * Sh::STAGE_BYTES + Sh::HN_BYTES + ROT_BYTES +
                                       LW * Sh::WAVE_BYTES);              // list lengths
  int nfl = 0;
  const int j = lane & 15, grp = lane >> 4;

  for (int i = threadIdx.x; i < ROT_BYTES / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(sRot)[i] = reinterpret_cast<const u32x4*>(a.rotfrag)[i];
  for (int i = threadIdx.x; i < TCW / 4; i += blockDim.x)
    reinterpret_cast<floatx4*>(sHn)[i] = reinterpret_cast<const floatx4*>(a.hn)[i];
  const u32x4* gfrag = reinterpret_cast<const u32x4*>(a.lfrag);
  const u32x4* ghn = reinterpret_cast<const u32x4*>(a.hn);
  constexpr int STAGE_Q = Sh::STAGE_BYTES / 16;   // 16-byte pieces per stage
#pragma unroll
  for (int u = 0; u < Sh::LOADS; ++u)
    reinterpret_cast<u32x4*>(sStage)[threadIdx.x + LW * 64 * u] = gfrag[threadIdx.x + LW * 64 * u];
  __syncthreads();

  const TX* __restrict__ x = static_cast<const TX*>(a.x);
  const int64_t n = a.n;
  const int64_t wg_vecs = (int64_t)LW * Sh::VPW;
  const int64_t passes = (n + wg_vecs - 1) / wg_vecs;
  int sbuf = 0;

  // the lane's x row of batch h of pass gp (rows past the end repeat the last one)
  auto xrow = [&](int64_t gp, int h) {
    const int64_t row0 = gp * wg_vecs + (int64_t)wave * Sh::VPW + EV * h;
    const int64_t last = n - 1 - row0;
    return x + (last < 0 ? n - 1 : row0 + (j < last ? j : last)) * a.ld;
  };
  // x of the next batch is always in flight: batch h + 1 while batch h is
  // rotated, the next pass's batch 0 during the last codebook stage
  XRaw<TX> xnext;
  if (blockIdx.x < passes) load_raw<TX>(xrow(blockIdx.x, 0), grp, xnext);

  // settle one listed block and replace its field of the record
  auto settle_fix = [&](const uint32_t* ent) {
    const int bi = settle_block<K, TX, LN>(a, x, a.cbh, ent, sX, sZd, lane);
    if (lane == 0) {
      const int64_t row = (int64_t)((uint64_t)ent[0] | ((uint64_t)ent[1] << 32));
      const int sh = LB * (int)(ent[2] & 0xFFu);
      uint32_t* rp = a.codes + row;
      atomicAnd(rp, ~(((uint32_t)LN - 1u) << sh));
      atomicOr(rp, (uint32_t)bi << sh);
    }
  };

  for (int64_t gp = blockIdx.x; gp < passes; gp += gridDim.x) {
    const int64_t vbase = gp * wg_vecs + (int64_t)wave * Sh::VPW;
    if (nfl > FL_MAX - 16 * CG) {   // room for this pass's blocks: settle the list now
      __builtin_amdgcn_s_waitcnt(0);   // this wave's record stores have completed
      for (int e = 0; e < nfl; ++e) settle_fix(sList + e * FL_WORDS);
      nfl = 0;
    }

    // ---- norm, rotation and B operands of the wave's 64 columns.  Column
    //      group c = h NB + b holds block b of batch h (vectors 16 h .. + 15).
    half8 bh[CG][KC], bl[CG][KC];
    float zz[CG];
#pragma unroll
    for (int h = 0; h < Sh::BATCHES; ++h) {
      const int64_t row0 = vbase + EV * h;
      const int64_t last = n - 1 - row0;
      const XRaw<TX> xraw = xnext;
      if (h + 1 < Sh::BATCHES) load_raw<TX>(xrow(gp, h + 1), grp, xnext);
      XFrag<TX> xf;
      finish_x<TX>(xraw, xf);
      const float nus = __builtin_amdgcn_sqrtf(xf.ss);
      if (grp == 0 && j <= last) a.norms[row0 + j] = f32_to_f16_rne(nus * xf.escale);
      rotate_to_lds<TX>(xf, sRot, __builtin_amdgcn_rcpf(nus), sZ, lane);
      wave_lds_sync();
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c = h * NB + b;
        float ss = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const float* zr = sZ + j * ZP + b * K + 32 * kc + 8 * grp;
          const floatx4 z0 = *reinterpret_cast<const floatx4*>(zr);
          const floatx4 z1 = *reinterpret_cast<const floatx4*>(zr + 4);
          const float zv[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const _Float16 hi = (_Float16)zv[e];
            bh[c][kc][e] = hi;
            bl[c][kc][e] = (_Float16)(zv[e] - (float)hi);
            ss = fmaf(zv[e], zv[e], ss);
          }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        zz[c] = ss;
      }
      wave_lds_sync();
    }

    // ---- the codebook sweep
    int m1[CG][4], m2[CG][4];
    uint32_t vmask = ~((1u << TB) - 1u);   // in a vector register: see make_key
    asm volatile("" : "+v"(vmask));
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) m1[c][r] = m2[c][r] = INT32_MIN;
    for (int s = 0; s < NSTAGE; ++s) {
      // next stage (cyclic: the last one fetches stage 0 of the next pass)
      // straight into the other LDS buffer (free since the last barrier):
      // lane l of a wave writes 16 bytes at the wave's base + 16 l
      const int sn = s + 1 < NSTAGE ? s + 1 : 0;
      if (s == NSTAGE - 1 && gp + gridDim.x < passes) load_raw<TX>(xrow(gp + gridDim.x, 0), grp, xnext);
#pragma unroll
      for (int u = 0; u < Sh::LOADS; ++u) {
        const int piece = LW * 64 * u + 64 * wave;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(gfrag + sn * STAGE_Q + piece + lane),
            (__attribute__((address_space(3))) void*)(sStage + (sbuf ^ 1) * Sh::STAGE_BYTES + 16 * piece),
            16, 0, 0);
      }
      if (wave == 0)   // the stage's -|c|^2 / 2: 64 lanes x 16 bytes
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(ghn + sn * (TCW / 4) + lane),
            (__attribute__((address_space(3))) void*)(sHn + (sbuf ^ 1) * TCW), 16, 0, 0);
      static_assert(TCW / 4 == 64, "one 16-byte piece per lane");
      const unsigned char* st = sStage + sbuf * Sh::STAGE_BYTES;
      const float* hs = sHn + sbuf * TCW;
      // scores of codeword tile i (16 codewords) for the wave's 64 columns
      auto scores = [&](int i, floatx4 (&acc)[CG]) {
        half8 av[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          av[kc] = *reinterpret_cast<const half8*>(st + ((i * KC + kc) * 64 + lane) * 16);
        const floatx4 c0 = *reinterpret_cast<const floatx4*>(hs + 16 * i + 4 * grp);
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[c] = c0;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
          for (int c = 0; c < CG; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[kc], bh[c][kc], acc[c], 0, 0, 0);
#pragma unroll
          for (int c = 0; c < CG; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[kc], bl[c][kc], acc[c], 0, 0, 0);
        }
      };
      auto track = [&](const floatx4 (&acc)[CG], int i) {
        const uint32_t t = (uint32_t)(16 * s + i);
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = make_key<TB>(acc[c][r], t, vmask);
            // median of the three (the canonical form of v_med3_i32)
            m2[c][r] = max(min(m1[c][r], m2[c][r]), min(max(m1[c][r], m2[c][r]), key));
            m1[c][r] = max(m1[c][r], key);
          }
      };
      // software pipeline: the key updates of tile i - 1 run in the shadow of
      // tile i's matrix-core work (one MFMA, then VALU work, in turn)
      constexpr int NM = 2 * KC * CG;        // MFMAs per tile
      constexpr int NV = 3 * 4 * CG;         // VALU operations per tile
      floatx4 accA[CG], accB[CG];
      scores(0, accA);
#pragma unroll
      for (int i = 1; i < TCW / 16; ++i) {
        if (i & 1) {
          scores(i, accB);
          track(accA, i - 1);
        } else {
          scores(i, accA);
          track(accB, i - 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, KC + 1, 0);   // this tile's LDS reads
#pragma unroll
        for (int u = 0; u < NM; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, NV / NM, 0);
        }
      }
      track(accB, TCW / 16 - 1);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the stage has landed in LDS
      __syncthreads();
      sbuf ^= 1;
    }

    // ---- merge the slots, certify, settle the rest exactly
    int res[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      int b1 = m1[c][0], b2 = m2[c][0];
      int r1 = 0;
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        const int o1 = m1[c][r], o2 = m2[c][r];
        b2 = max(max(b2, o2), min(b1, o1));
        const bool tk = o1 > b1;
        b1 = tk ? o1 : b1;
        r1 = tk ? r : r1;
      }
      int n1 = 16 * (int)key_tile<TB>(b1) + 4 * grp + r1;
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        const int o1 = __shfl_xor(b1, m, 64), o2 = __shfl_xor(b2, m, 64);
        const int on = __shfl_xor(n1, m, 64);
        b2 = max(max(b2, o2), min(b1, o1));
        const bool tk = o1 > b1 || (o1 == b1 && on < n1);
        b1 = tk ? o1 : b1;
        n1 = tk ? on : n1;
      }
      const float bv = key_value(b1);
      const float zn = __builtin_amdgcn_sqrtf(zz[c]);
      const float E = fmaf(a.EA, zn, a.EB);
      constexpr float KEYREL = (float)(1u << TB) * 0x1p-22f;   // two keys' rounding, relative
      const float M = fmaf(2.f, E, fmaf(KEYREL, fabsf(bv), a.ZT)) * 1.0001f + 1e-12f;
      const float lim = bv - M;
      int ncand = 0;
      bool hidden = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ncand += key_value(m1[c][r]) >= lim ? 1 : 0;
        hidden = hidden || key_value(m2[c][r]) >= lim;
      }
      ncand += __shfl_xor(ncand, 16, 64);
      ncand += __shfl_xor(ncand, 32, 64);
      int hid = hidden ? 1 : 0;
      hid |= __shfl_xor(hid, 16, 64);
      hid |= __shfl_xor(hid, 32, 64);
      // a winner at or below the margin may compete with negative scores,
      // whose keys do not order like the scores: settle those exactly
      const bool finite = __builtin_isfinite(bv) && __builtin_isfinite(zz[c]) &&
                          __builtin_isfinite(lim) && lim > 0.f;
      const bool certain = finite && hid == 0 && ncand == 1;
      const bool full = !finite || hid != 0;
      res[c] = n1;

      // uncertain blocks: their candidates go to the wave's list and are
      // settled after the last pass (no workgroup waits on them); the
      // record gets the float32 winner meanwhile
      uint64_t need = __builtin_amdgcn_ballot_w64(lane < 16 && !certain);
      while (need) {
        const int jj = __builtin_ctzll(need);
        need &= need - 1;
        const int b = NB == 1 ? 0 : (c % NB);
        const int vec = NB == 1 ? 16 * c + jj : 16 * (c / NB) + jj;
        const int64_t row = vbase + vec;
        if (row >= n) continue;
        const bool col_full = __builtin_amdgcn_readlane((int)full, jj) != 0;
        const float col_lim = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(lim), jj));
        uint32_t* ent = sList + nfl * FL_WORDS;
        uint16_t* ce = reinterpret_cast<uint16_t*>(ent + 4);
        int nc = 0;
        uint32_t hm = 0;
        if (!col_full) {
#pragma unroll
          for (int lg = 0; lg < 4; ++lg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = __builtin_amdgcn_readlane(m1[c][r], 16 * lg + jj);
              const int key2 = __builtin_amdgcn_readlane(m2[c][r], 16 * lg + jj);
              if (key_value(key) >= col_lim) {
                if (lane == 0 && nc < FL_CAND) ce[nc] = (uint16_t)(16 * (int)key_tile<TB>(key) + 4 * lg + r);
                ++nc;
              }
              if (key_value(key2) >= col_lim) hm |= 1u << (4 * lg + r);
            }
        }
        if (lane == 0) {
          ent[0] = (uint32_t)row;
          ent[1] = (uint32_t)(row >> 32);
          ent[2] = (uint32_t)b | ((uint32_t)(nc < FL_CAND ? nc : FL_CAND) << 8) |
                   ((col_full || nc > FL_CAND ? 1u : 0u) << 16);
          ent[3] = hm;
        }
        wave_lds_sync();
        ++nfl;
      }
    }

    // ---- records: lane l writes vector l of the wave (k = 64) or, for
    //      l < 32, vector l with fields from groups 2 (l / 16) and + 1 (k = 32)
    if constexpr (NB == 1) {
      const int row_in = lane;
      const int v0 = res[0], v1 = res[1], v2 = res[2], v3 = res[3];
      const int vv = grp == 0 ? v0 : (grp == 1 ? v1 : (grp == 2 ? v2 : v3));
      if (vbase + row_in < n) a.codes[vbase + row_in] = (uint32_t)vv;
    } else {
      const int h = grp & 1;
      const uint32_t f0 = (uint32_t)(h == 0 ? res[0] : res[2]);
      const uint32_t f1 = (uint32_t)(h == 0 ? res[1] : res[3]);
      if (lane < 32 && vbase + lane < n) a.codes[vbase + lane] = f0 | (f1 << LB);
    }
  }

  // ---- the workgroup's uncertain blocks, settled exactly and shared out
  //      over its waves; each replaces its field of a record stored above
  //      (every wave's stores have completed before the barrier)
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) sCount[wave] = nfl;
  __syncthreads();
  int tot = 0;
  for (int w = 0; w < LW; ++w) tot += sCount[w];
  for (int g = wave; g < tot; g += LW) {
    int w = 0, e = g;
    while (e >= sCount[w]) e -= sCount[w++];
    const uint32_t* ent = reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const unsigned char*>(sList) + (ptrdiff_t)(w - wave) * (ptrdiff_t)Sh::WAVE_BYTES) +
        e * FL_WORDS;
    settle_fix(ent);
  }
}

void set_bounds(LArgs& a, const fq_codebook* cb, int k, size_t xsize);

template <int K, int LB, typename TX>
hipError_t launch_large_k(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld,
                          uint32_t* codes, uint16_t* norms, hipStream_t s) {
  using Sh = LShape<K, LB>;
  if (cb->N != Sh::LN || cb->t.lfrag == nullptr || cb->t.hnorm == nullptr) return hipErrorInvalidValue;
  auto kern = encode_large_kernel<K, LB, TX>;
  const size_t shm = Sh::LDS;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  static DeviceCache cap_cache;   // resident workgroups per device
  const int64_t cap = cap_cache.get(reinterpret_cast<const void*>(kern), LW * 64, shm);
  if (cap <= 0) return hipErrorInvalidConfiguration;
  const int64_t wg_vecs = (int64_t)LW * Sh::VPW;
  int64_t blocks = (n + wg_vecs - 1) / wg_vecs;
  if (blocks > cap) blocks = cap;
  LArgs a;
  a.x = x;
  a.n = n;
  a.ld = ld;
  a.codes = codes;
  a.norms = norms;
  a.rotfrag = cb->t.encfrag;
  a.lfrag = cb->t.lfrag;
  a.hn = cb->t.hnorm;
  a.cbh = cb->t.cb16hi;
  a.enc = cb->t.enc;
  a.S = cb->enc_stride;
  a.pi64t = cb->t.pi64t;
  set_bounds(a, cb, K, sizeof(TX));
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(LW * 64), shm, s, a);
  return hipGetLastError();
}

// ---- k = 8, N = 256 (one bit per coordinate) ---------------------------------
//
// The same search with the whole codebook (4 KB of binary16) resident in LDS:
// a block of 8 coordinates is one column, and v_mfma_f32_16x16x16_f16
// contracts [z_hi | z_lo] (16 values) against [c | c], so one instruction
// scores 16 codewords against 16 columns with both halves of the split.  A
// wave rotates 16 vectors and then takes their 128 columns in two sub-passes
// of 4 blocks (4 column groups), each a sweep over the 16 tiles with the same
// keys, slot tracking, certificate and exact settle of listed blocks; a
// sub-pass stores one record word (4 byte-wide fields) per vector.  The
// accumulator starts at K0 - |c|^2 / 2 (K0 = r + r^2 / 2, r the smallest
// codeword norm): K0 cancels in every comparison and makes the best score of
// any block of norm <= 1 non-negative, so blocks near the origin need no
// full scan.
constexpr int EW = 4;          // waves per workgroup
constexpr int E8CG = 4;        // blocks (column groups) per sub-pass
constexpr int E8N = 256;
constexpr int E8NT = E8N / 16; // tiles
constexpr size_t E8_WAVE_BYTES = (size_t)EV * ZP * 4 + 2 * 64 * 8 + FL_MAX * FL_WORDS * 4;
constexpr size_t E8_TAB = (size_t)E8N * 8 * 2 + E8N * 4;   // codebook + -|c|^2 / 2
constexpr size_t E8_LDS = E8_TAB + ROT_BYTES + EW * E8_WAVE_BYTES + EW * 4;

template <typename TX>
// (at least 3 waves per SIMD: at most 168 registers, no AGPR copies of the scores)
__global__ __launch_bounds__(EW * 64, 3) void encode_k8_kernel(LArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const _Float16* sCb = reinterpret_cast<const _Float16*>(smem);        // [N][8]
  float* sHn = reinterpret_cast<float*>(smem + E8N * 16);                // [N]
  _Float16* sRot = reinterpret_cast<_Float16*>(smem + E8_TAB);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  unsigned char* wb = smem + E8_TAB + ROT_BYTES + wave * E8_WAVE_BYTES;
  float* sZ = reinterpret_cast<float*>(wb);                               // [EV][ZP]
  double* sX = reinterpret_cast<double*>(wb + EV * ZP * 4);              // exact path: x
  double* sZd = sX + 64;                                                  // exact path: z block
  uint32_t* sList = reinterpret_cast<uint32_t*>(sZd + 64);                // uncertain blocks
  int* sCount = reinterpret_cast<int*>(smem + E8_TAB + ROT_BYTES + EW * E8_WAVE_BYTES);
  int nfl = 0;
  const int j = lane & 15, grp = lane >> 4;

  for (int i = threadIdx.x; i < ROT_BYTES / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(sRot)[i] = reinterpret_cast<const u32x4*>(a.rotfrag)[i];
  for (int i = threadIdx.x; i < E8N; i += blockDim.x)
    reinterpret_cast<u32x4*>(smem)[i] = reinterpret_cast<const u32x4*>(a.cbh)[i];
  for (int i = threadIdx.x; i < E8N / 4; i += blockDim.x)
    reinterpret_cast<floatx4*>(sHn)[i] = reinterpret_cast<const floatx4*>(a.hn)[i];
  __syncthreads();

  const TX* __restrict__ x = static_cast<const TX*>(a.x);
  const int64_t n = a.n;
  const int64_t wg_vecs = (int64_t)EW * EV;
  const int64_t passes = (n + wg_vecs - 1) / wg_vecs;
  // the lane's x row of pass gp (rows past the end repeat the last one)
  auto xrow = [&](int64_t gp) {
    const int64_t row0 = gp * wg_vecs + (int64_t)wave * EV;
    const int64_t last = n - 1 - row0;
    return x + (last < 0 ? n - 1 : row0 + (j < last ? j : last)) * a.ld;
  };
  XRaw<TX> xnext;
  if (blockIdx.x < passes) load_raw<TX>(xrow(blockIdx.x), grp, xnext);

  // settle one listed block and replace its byte of the record
  auto settle_fix = [&](const uint32_t* ent) {
    const int bi = settle_block<8, TX, E8N>(a, x, sCb, ent, sX, sZd, lane);
    if (lane == 0) {
      const int64_t row = (int64_t)((uint64_t)ent[0] | ((uint64_t)ent[1] << 32));
      const int b = (int)(ent[2] & 0xFFu);
      uint32_t* rp = a.codes + 2 * row + (b >> 2);
      const int sh = 8 * (b & 3);
      atomicAnd(rp, ~(0xFFu << sh));
      atomicOr(rp, (uint32_t)bi << sh);
    }
  };

  for (int64_t gp = blockIdx.x; gp < passes; gp += gridDim.x) {
    const int64_t vbase = gp * wg_vecs + (int64_t)wave * EV;
    const int64_t last = n - 1 - vbase;
    {   // norm and rotation of the wave's 16 vectors; the next pass's x in flight
      const XRaw<TX> xraw = xnext;
      if (gp + gridDim.x < passes) load_raw<TX>(xrow(gp + gridDim.x), grp, xnext);
      XFrag<TX> xf;
      finish_x<TX>(xraw, xf);
      const float nus = __builtin_amdgcn_sqrtf(xf.ss);
      if (grp == 0 && j <= last) a.norms[vbase + j] = f32_to_f16_rne(nus * xf.escale);
      rotate_to_lds<TX>(xf, sRot, __builtin_amdgcn_rcpf(nus), sZ, lane);
      wave_lds_sync();
    }

#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      if (nfl > FL_MAX - 16 * E8CG) {   // room for this sub-pass's blocks
        __builtin_amdgcn_s_waitcnt(0);   // this wave's record stores have completed
        for (int e = 0; e < nfl; ++e) settle_fix(sList + e * FL_WORDS);
        nfl = 0;
      }
      // B operands: lanes of groups 0, 1 hold z_hi of coordinates 0-3, 4-7 of
      // block 4 half + c, groups 2, 3 the lo parts of the same coordinates
      half4 bz[E8CG];
      float zz[E8CG];
#pragma unroll
      for (int c = 0; c < E8CG; ++c) {
        const floatx4 z4 = *reinterpret_cast<const floatx4*>(sZ + j * ZP + 8 * (E8CG * half + c) + 4 * (grp & 1));
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 hi = (_Float16)z4[e];
          const _Float16 lo = (_Float16)(z4[e] - (float)hi);
          bz[c][e] = grp < 2 ? hi : lo;
          ss = fmaf(z4[e], z4[e], ss);
        }
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        zz[c] = __uint_as_float(q[0]) + __uint_as_float(q[1]);   // coordinates 0-3 and 4-7
      }
      wave_lds_sync();

      int m1[E8CG][4], m2[E8CG][4];
#pragma unroll
      for (int c = 0; c < E8CG; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) m1[c][r] = m2[c][r] = INT32_MIN;
      // tile operands, read one tile ahead
      const _Float16* ap = sCb + j * 8 + 4 * (grp & 1);
      const float* hp = sHn + 4 * grp;
      half4 avn = *reinterpret_cast<const half4*>(ap);
      floatx4 c0n = *reinterpret_cast<const floatx4*>(hp);
      auto scores = [&](int i, floatx4 (&acc)[E8CG]) {
        const half4 av = avn;
        const floatx4 c0 = c0n;
        const int in = i + 1 < E8NT ? i + 1 : i;
        avn = *reinterpret_cast<const half4*>(ap + 128 * in);
        c0n = *reinterpret_cast<const floatx4*>(hp + 16 * in);
#pragma unroll
        for (int c = 0; c < E8CG; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bz[c], c0, 0, 0, 0);
      };
      auto track = [&](const floatx4 (&acc)[E8CG], int i) {
#pragma unroll
        for (int c = 0; c < E8CG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = (int)__builtin_amdgcn_perm(__float_as_uint(acc[c][r]), (uint32_t)i, 0x07060500u);
            m2[c][r] = max(min(m1[c][r], m2[c][r]), min(max(m1[c][r], m2[c][r]), key));
            m1[c][r] = max(m1[c][r], key);
          }
      };
      // a loop (not unrolled): the running keys are carried tile to tile, so
      // only two tiles' scores are live at a time
      floatx4 accA[E8CG], accB[E8CG];
      scores(0, accA);
#pragma unroll 1
      for (int i = 1; i < E8NT - 1; i += 2) {
        scores(i, accB);
        track(accA, i - 1);
        scores(i + 1, accA);
        track(accB, i);
      }
      scores(E8NT - 1, accB);
      track(accA, E8NT - 2);
      track(accB, E8NT - 1);

      // merge the slots (in the lane, then over the four 16-lane rows on
      // permlane swaps), certify (as for the large blocks); all four column
      // groups first, so their latencies overlap, then the listing
      int res[E8CG];
      float lims[E8CG];
      bool fulls[E8CG];
      uint64_t unc[E8CG];
#pragma unroll
      for (int c = 0; c < E8CG; ++c) {
        int b1 = m1[c][0], b2 = m2[c][0];
        int r1 = 0;
#pragma unroll
        for (int r = 1; r < 4; ++r) {
          const int o1 = m1[c][r], o2 = m2[c][r];
          b2 = max(max(b2, o2), min(b1, o1));
          const bool tk = o1 > b1;
          b1 = tk ? o1 : b1;
          r1 = tk ? r : r1;
        }
        int n1 = 16 * (int)key_tile<8>(b1) + 4 * grp + r1;
        // a swap hands each lane its partner's triple beside its own (in
        // either order); the merge is symmetric, so both lanes agree
        auto merge = [&](auto q1, auto q2, auto qn) {
          const int u1 = (int)q1[0], v1 = (int)q1[1], u2 = (int)q2[0], v2 = (int)q2[1];
          const int un = (int)qn[0], vn = (int)qn[1];
          b2 = max(max(u2, v2), min(u1, v1));
          const bool tk = v1 > u1 || (v1 == u1 && vn < un);
          b1 = tk ? v1 : u1;
          n1 = tk ? vn : un;
        };
        merge(__builtin_amdgcn_permlane16_swap((uint32_t)b1, (uint32_t)b1, false, false),
              __builtin_amdgcn_permlane16_swap((uint32_t)b2, (uint32_t)b2, false, false),
              __builtin_amdgcn_permlane16_swap((uint32_t)n1, (uint32_t)n1, false, false));
        merge(__builtin_amdgcn_permlane32_swap((uint32_t)b1, (uint32_t)b1, false, false),
              __builtin_amdgcn_permlane32_swap((uint32_t)b2, (uint32_t)b2, false, false),
              __builtin_amdgcn_permlane32_swap((uint32_t)n1, (uint32_t)n1, false, false));
        const float bv = key_value(b1);
        const float zn = __builtin_amdgcn_sqrtf(zz[c]);
        const float E = fmaf(a.EA, zn, a.EB);
        const float M = fmaf(2.f, E, fmaf(0x1p-14f, fabsf(bv), a.ZT)) * 1.0001f + 1e-12f;
        const float lim = bv - M;
        // candidates (slot leaders within the margin) in the low byte, hidden
        // slots (second keys within it) above
        uint32_t cnt = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cnt += (key_value(m1[c][r]) >= lim ? 1u : 0u) + (key_value(m2[c][r]) >= lim ? 0x100u : 0u);
        const auto c16 = __builtin_amdgcn_permlane16_swap(cnt, cnt, false, false);
        cnt = c16[0] + c16[1];
        const auto c32 = __builtin_amdgcn_permlane32_swap(cnt, cnt, false, false);
        cnt = c32[0] + c32[1];
        const bool finite = __builtin_isfinite(bv) && __builtin_isfinite(zz[c]) &&
                            __builtin_isfinite(lim) && lim > 0.f;
        const bool hid = (cnt >> 8) != 0;
        const bool certain = finite && !hid && (cnt & 0xFFu) == 1;
        res[c] = n1;
        lims[c] = lim;
        fulls[c] = !finite || hid;
        unc[c] = __builtin_amdgcn_ballot_w64(lane < 16 && !certain);
      }
#pragma unroll
      for (int c = 0; c < E8CG; ++c) {
        uint64_t need = unc[c];
        while (need) {
          const int jj = __builtin_ctzll(need);
          need &= need - 1;
          const int64_t row = vbase + jj;
          if (row >= n) continue;
          const bool col_full = __builtin_amdgcn_readlane((int)fulls[c], jj) != 0;
          const float col_lim = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(lims[c]), jj));
          uint32_t* ent = sList + nfl * FL_WORDS;
          uint16_t* ce = reinterpret_cast<uint16_t*>(ent + 4);
          int nc = 0;
          uint32_t hm = 0;
          if (!col_full) {
#pragma unroll
            for (int lg = 0; lg < 4; ++lg)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key = __builtin_amdgcn_readlane(m1[c][r], 16 * lg + jj);
                const int key2 = __builtin_amdgcn_readlane(m2[c][r], 16 * lg + jj);
                if (key_value(key) >= col_lim) {
                  if (lane == 0 && nc < FL_CAND) ce[nc] = (uint16_t)(16 * (int)key_tile<8>(key) + 4 * lg + r);
                  ++nc;
                }
                if (key_value(key2) >= col_lim) hm |= 1u << (4 * lg + r);
              }
          }
          if (lane == 0) {
            ent[0] = (uint32_t)row;
            ent[1] = (uint32_t)(row >> 32);
            ent[2] = (uint32_t)(E8CG * half + c) | ((uint32_t)(nc < FL_CAND ? nc : FL_CAND) << 8) |
                     ((col_full || nc > FL_CAND ? 1u : 0u) << 16);
            ent[3] = hm;
          }
          wave_lds_sync();
          ++nfl;
        }
      }
      // word `half` of the record of vector j
      if (grp == 0 && j <= last)
        a.codes[2 * (vbase + j) + half] = (uint32_t)res[0] | ((uint32_t)res[1] << 8) |
                                          ((uint32_t)res[2] << 16) | ((uint32_t)res[3] << 24);
    }
  }

  // the workgroup's uncertain blocks, settled exactly and shared out over its waves
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) sCount[wave] = nfl;
  __syncthreads();
  int tot = 0;
  for (int w = 0; w < EW; ++w) tot += sCount[w];
  for (int g = wave; g < tot; g += EW) {
    int w = 0, e = g;
    while (e >= sCount[w]) e -= sCount[w++];
    const uint32_t* ent = reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const unsigned char*>(sList) + (ptrdiff_t)(w - wave) * (ptrdiff_t)E8_WAVE_BYTES) +
        e * FL_WORDS;
    settle_fix(ent);
  }
}

// certification constants for block length k (bounds in the header), from
// the largest codeword norm
void set_bounds(LArgs& a, const fq_codebook* cb, int k, size_t xsize) {
  const double cm = cb->cmax, kk = k;
  const double acc = (2.0 * kk + 2.0) * 0x1p-23;
  a.EA = (float)(cm * (0x1p-22 + acc * 1.001) * 1.01);
  a.EB = (float)((0x1p-25 * sqrt(kk) * cm + (acc + 0x1p-24) * (cm * cm * 0.5 + cb->hshift)) * 1.01);
  const double ez = xsize == 2 ? cb->enc_ez16 : cb->enc_ez32;
  a.ZT = (float)(2.0 * ez * sqrt(kk) * cm * 1.01);
}

template <typename TX>
hipError_t launch_k8(const fq_codebook* cb, const TX* x, int64_t n, int64_t ld, uint32_t* codes,
                     uint16_t* norms, hipStream_t s) {
  if (cb->k != 8 || cb->N != E8N || cb->W != 2 || !cb->half_exact || cb->t.hnorm == nullptr)
    return hipErrorInvalidValue;
  auto kern = encode_k8_kernel<TX>;
  const size_t shm = E8_LDS;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  static DeviceCache cap_cache;   // resident workgroups per device
  const int64_t cap = cap_cache.get(reinterpret_cast<const void*>(kern), EW * 64, shm);
  if (cap <= 0) return hipErrorInvalidConfiguration;
  const int64_t wg_vecs = (int64_t)EW * EV;
  int64_t blocks = (n + wg_vecs - 1) / wg_vecs;
  if (blocks > cap) blocks = cap;
  LArgs a;
  a.x = x;
  a.n = n;
  a.ld = ld;
  a.codes = codes;
  a.norms = norms;
  a.rotfrag = cb->t.encfrag;
  a.lfrag = nullptr;
  a.hn = cb->t.hnorm;
  a.cbh = cb->t.cb16hi;
  a.enc = cb->t.enc;
  a.S = cb->enc_stride;
  a.pi64t = cb->t.pi64t;
  set_bounds(a, cb, 8, sizeof(TX));
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(EW * 64), shm, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_large(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n,
                               int64_t ld, uint32_t* codes, uint16_t* norms, hipStream_t s) {
  if (xt == FQ_F16) {
    const _Float16* xx = static_cast<const _Float16*>(x);
    if (cb->k == 32 && cb->bits == 12) return launch_large_k<32, 12, _Float16>(cb, xx, n, ld, codes, norms, s);
    if (cb->k == 64 && cb->bits == 12) return launch_large_k<64, 12, _Float16>(cb, xx, n, ld, codes, norms, s);
    if (cb->k == 64 && cb->bits == 14) return launch_large_k<64, 14, _Float16>(cb, xx, n, ld, codes, norms, s);
  } else {
    const float* xx = static_cast<const float*>(x);
    if (cb->k == 32 && cb->bits == 12) return launch_large_k<32, 12, float>(cb, xx, n, ld, codes, norms, s);
    if (cb->k == 64 && cb->bits == 12) return launch_large_k<64, 12, float>(cb, xx, n, ld, codes, norms, s);
    if (cb->k == 64 && cb->bits == 14) return launch_large_k<64, 14, float>(cb, xx, n, ld, codes, norms, s);
  }
  return hipErrorInvalidValue;
}

bool encode_k8_applies(const fq_codebook* cb) {
  return cb->k == 8 && cb->N == E8N && cb->W == 2 && cb->half_exact && cb->t.hnorm != nullptr;
}

hipError_t launch_encode_k8(const fq_codebook* cb, const void* x, fq_dtype xt, int64_t n,
                            int64_t ld, uint32_t* codes, uint16_t* norms, hipStream_t s) {
  if (xt == FQ_F16) return launch_k8<_Float16>(cb, static_cast<const _Float16*>(x), n, ld, codes, norms, s);
  return launch_k8<float>(cb, static_cast<const float*>(x), n, ld, codes, norms, s);
}

}  // namespace fq
