// C ABI of the FibQuant codec: artifact parsing, device tables, argument checks.
//
// The artifact holds the shared rotation and the shared codebook (FibQuant
// technical summary, sections 2.1-2.3).  Everything here runs on the host;
// kernels live in fq_encode.hip, fq_decode.hip and fq_attend.hip.
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>

#include "fq_internal.h"

// Attention scratch of fq_attend_decode_static: split-K partials for callers
// that cannot allocate.  One copy per device, held until the process ends.
// Host code never uses this name as an address: the device address of each
// device's copy is looked up once (scratch_address) and kept per device.
static __device__ __align__(256) unsigned char scratch[FQ_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each device, looked up at set-up (the first
// codebook load on that device, with the device current); null if the lookup
// failed.
constexpr int SCRATCH_DEVICES = fq::DeviceCache::MAX_DEVICES;
std::mutex scratch_mu;
void* scratch_dev[SCRATCH_DEVICES] = {};
bool scratch_done[SCRATCH_DEVICES] = {};

// Must run with `device` current.
void scratch_setup(int device) {
  if (device < 0 || device >= SCRATCH_DEVICES) return;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_done[device]) return;
  scratch_done[device] = true;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr)
    scratch_dev[device] = p;
  else
    (void)hipGetLastError();
}

void* scratch_address(int device) {
  if (device < 0 || device >= SCRATCH_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  return scratch_dev[device];
}

void fill_info(const fq::ArtifactHeader& h, fq_info* o) {
  o->d = h.d;
  o->k = h.k;
  o->N = h.N;
  o->nb = h.nb;
  o->idx_bits = h.bits;
  o->record_words = h.W;
  o->last_block = h.last;
  o->packed_bits = (int32_t)(h.nb * h.bits + 16);
  o->rate_nominal = (double)h.bits / h.k;
  o->rate_actual = (double)h.nb * h.bits / h.d;
  o->distortion = h.d_test;
  o->artifact_hash = 0;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Keys and values attended together: the same (k, N) variant and the same
// rotation.  The kernels score and accumulate in one rotated domain and rotate
// the output back once, which is exact only when both caches were coded with
// the one shared rotation (FibQuant technical summary, sections 1 and 2.3).
bool same_variant(const fq_codebook* a, const fq_codebook* b) {
  return a->k == b->k && a->N == b->N && a->pi_digest == b->pi_digest;
}

}  // namespace

extern "C" {

const char* fq_status_string(fq_status s) {
  switch (s) {
    case FQ_OK: return "ok";
    case FQ_ERR_INVALID_ARG: return "invalid argument";
    case FQ_ERR_BAD_ARTIFACT: return "bad codebook artifact";
    case FQ_ERR_UNSUPPORTED: return "unsupported codebook or shape";
    case FQ_ERR_NO_MEMORY: return "device allocation failed";
    case FQ_ERR_DEVICE: return "HIP device error";
    case FQ_ERR_SCRATCH: return "shape needs more than the library's static attention scratch";
  }
  return "unknown status";
}

fq_status fq_artifact_check(const void* artifact, size_t nbytes, fq_info* out) {
  fq::ArtifactHeader h;
  fq_status st = fq::parse_artifact(artifact, nbytes, &h, nullptr, nullptr);
  if ((st == FQ_OK || st == FQ_ERR_UNSUPPORTED) && out) {
    fill_info(h, out);
    uint64_t hh;
    memcpy(&hh, static_cast<const unsigned char*>(artifact) + nbytes - 8, 8);
    out->artifact_hash = hh;
  }
  return st;
}

fq_status fq_codebook_load(const void* artifact, size_t nbytes, int device, fq_codebook** out) {
  if (!out) return FQ_ERR_INVALID_ARG;
  *out = nullptr;
  fq::ArtifactHeader h;
  const unsigned char *pi_p = nullptr, *cw_p = nullptr;
  fq_status st = fq::parse_artifact(artifact, nbytes, &h, &pi_p, &cw_p);
  if (st != FQ_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return FQ_ERR_DEVICE;
  if (device < 0 || device >= ndev) return FQ_ERR_INVALID_ARG;

  fq_codebook* cb = new (std::nothrow) fq_codebook();
  if (!cb) return FQ_ERR_NO_MEMORY;
  cb->device = device;
  cb->d = h.d;
  cb->k = h.k;
  cb->N = h.N;
  cb->nb = h.nb;
  cb->bits = h.bits;
  cb->W = h.W;
  cb->last = h.last;
  cb->enc_stride = ((h.k + 1) + 3) / 4 * 4;
  cb->rate_nominal = (double)h.bits / h.k;
  cb->rate_actual = (double)h.nb * h.bits / h.d;
  cb->distortion = h.d_test;
  memcpy(&cb->hash, static_cast<const unsigned char*>(artifact) + nbytes - 8, 8);
  const int d = cb->d, k = cb->k, N = cb->N, S = cb->enc_stride;
  cb->pi.resize((size_t)d * d);
  cb->c.resize((size_t)N * k);
  memcpy(cb->pi.data(), pi_p, 8ull * d * d);
  cb->pi_digest = fq::fnv1a64(pi_p, 8ull * d * d);
  memcpy(cb->c.data(), cw_p, 4ull * N * k);

  // host-side tables
  // search table: N rows (-2c, |c|^2) and a sentinel row N (zero codeword,
  // infinite norm) that padded candidate slots point at
  std::vector<float> pi32((size_t)d * d), enc((size_t)(N + 1) * S, 0.f);
  enc[(size_t)N * S + k] = INFINITY;
  std::vector<_Float16> pih((size_t)d * d), pil((size_t)d * d), cbh((size_t)N * k),
      cbl((size_t)N * k);
  double rho_pi = 0.0;   // largest |Pi - hi - 2^-11 lo|
  for (size_t i = 0; i < pi32.size(); ++i) {
    pi32[i] = (float)cb->pi[i];
    pih[i] = (_Float16)cb->pi[i];
    pil[i] = (_Float16)((cb->pi[i] - (double)pih[i]) * 2048.0);
    rho_pi = fmax(rho_pi, fabs(cb->pi[i] - (double)pih[i] - (double)pil[i] / 2048.0));
  }
  cb->half_exact = true;
  cb->cmax = 0.0;
  // The matrix-core searches keep -|c|^2 / 2 per codeword in float32.  At
  // k = 8 a constant K0 = r + r^2 / 2 (r the smallest codeword norm) is added
  // to every score: it cancels in every comparison, and it lifts the score of
  // the smallest codeword, and so the best score, above zero for any block of
  // norm <= 1, which the certificate needs (its integer keys order only
  // non-negative scores); the bounds charge its rounding.
  const bool k8mma = k == 8 && N == 256;
  std::vector<float> hnorm(fq::large_block(k) || k8mma ? N : 0);
  cb->hshift = 0.0;
  if (k8mma) {
    double rmin = INFINITY;
    for (int n = 0; n < N; ++n) {
      double cc = 0;
      for (int t = 0; t < k; ++t) cc += cb->c[(size_t)n * k + t] * cb->c[(size_t)n * k + t];
      rmin = fmin(rmin, sqrt(cc));
    }
    cb->hshift = rmin + 0.5 * rmin * rmin;
  }
  for (int n = 0; n < N; ++n) {
    double cc = 0;
    for (int t = 0; t < k; ++t) {
      const double v = cb->c[(size_t)n * k + t];
      enc[(size_t)n * S + t] = (float)(-2.0 * v);
      cc += v * v;
      cbh[(size_t)n * k + t] = (_Float16)v;
      if ((double)cbh[(size_t)n * k + t] != v) cb->half_exact = false;
      cbl[(size_t)n * k + t] = (_Float16)((v - (double)cbh[(size_t)n * k + t]) * 2048.0);
    }
    enc[(size_t)n * S + k] = (float)cc;
    cb->cmax = fmax(cb->cmax, sqrt(cc));
    if (!hnorm.empty()) hnorm[n] = (float)(cb->hshift - 0.5 * cc);
  }
  // k >= 32: the codebook as A fragments of v_mfma_f32_16x16x32_f16 (binary16;
  // the large-block kernels need a table on the binary16 grid)
  std::vector<_Float16> lfrag;
  if (fq::large_block(k)) {
    if (!cb->half_exact || k % 32 != 0 || N % 16 != 0) {
      delete cb;
      return FQ_ERR_UNSUPPORTED;
    }
    const int kcs = k / 32;
    lfrag.resize((size_t)N * k);
    for (int tile = 0; tile < N / 16; ++tile)
      for (int kc = 0; kc < kcs; ++kc)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e)
            lfrag[(((size_t)tile * kcs + kc) * 64 + lane) * 8 + e] =
                cbh[(size_t)(16 * tile + lane % 16) * k + 32 * kc + 8 * (lane / 16) + e];
  }
  // k = 2, N = 16 on the binary16 grid: the table of codeword pairs (byte j of
  // a record holds the fields of blocks 2 j and 2 j + 1, LSB first, so it is
  // the index of the pair (c_i0, c_i1) in this table)
  std::vector<_Float16> pair16;
  if (k == 2 && N == 16 && cb->half_exact) {
    pair16.resize(256 * 4);
    for (int i1 = 0; i1 < 16; ++i1)
      for (int i0 = 0; i0 < 16; ++i0)
        for (int t = 0; t < 2; ++t) {
          pair16[(size_t)(i0 + 16 * i1) * 4 + t] = cbh[(size_t)i0 * 2 + t];
          pair16[(size_t)(i0 + 16 * i1) * 4 + 2 + t] = cbh[(size_t)i1 * 2 + t];
        }
  }
  // Encode rotation error bound per coordinate of a unit vector.  Each output
  // is a float32 sum of four 16-product groups of the hi part (each
  // accumulated from zero, at most 15 roundings), then one fused multiply-add
  // with the lo part and one product: at most 20 roundings of 2^-23 relative
  // to sum_j |Pi_ij x_j| <= |x|.  The lo part (Pi_lo x, and Pi_hi x_lo for
  // float32 input, with |Pi_lo| < 1 and |x_lo|_1 <= 8 |x|) is one chained
  // accumulation of at most 128 terms of size sum <= 16 |x| in all, each
  // rounding at most 2^-24 of the running sum, weighted 2^-11: below
  // 128 * 16 * 2^-35 |x| = 2^-24 |x|.  Plus the binary16 split of Pi
  // (|x|_1 <= 8 |x|) and the float32 reciprocal of the norm; for float32 input
  // the split of x adds 2^-23.
  {
    const double acc = 20.0 * 0x1p-23 * (1.0 + 0x1p-10) * (1.0 + 0x1p-11) + 0x1p-24;
    // scaling: norm within 3.3e-7 relative, reciprocal 1 ulp, final fma and product
    const double scal = 3.3e-7 + 3.0 * 0x1p-24;
    cb->enc_ez16 = (float)((acc + 8.0 * rho_pi + scal) * 1.01);
    cb->enc_ez32 = (float)((acc + 8.0 * rho_pi + scal + 0x1p-23 + 0x1p-24) * 1.01);
  }
  // Pi as B fragments of v_mfma_f32_16x16x32_f16 for Y = Z Pi: fragment
  // [part][s][nt][lane][e] = part(Pi)[32 s + 8 (lane / 16) + e][16 nt + lane % 16],
  // part 0 = hi, part 1 = lo; one 16-byte load per lane per (part, s, nt).
  std::vector<_Float16> frag(2 * 2 * 4 * 64 * 8);
  for (int part = 0; part < 2; ++part)
    for (int s2 = 0; s2 < 2; ++s2)
      for (int nt = 0; nt < 4; ++nt)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const size_t src = (size_t)(32 * s2 + 8 * (lane / 16) + e) * d + 16 * nt + lane % 16;
            frag[(((size_t)(part * 2 + s2) * 4 + nt) * 64 + lane) * 8 + e] =
                part == 0 ? pih[src] : pil[src];
          }
  // Pi as A fragments of v_mfma_f32_16x16x16_f16 for z = Pi x (encode):
  // [part][ot][kq][lane][e] = part(Pi)[16 ot + lane % 16][16 kq + 4 (lane / 16) + e].
  std::vector<_Float16> efrag(2 * 4 * 4 * 64 * 4);
  for (int part = 0; part < 2; ++part)
    for (int ot = 0; ot < 4; ++ot)
      for (int kq = 0; kq < 4; ++kq)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 4; ++e) {
            const size_t src = (size_t)(16 * ot + lane % 16) * d + 16 * kq + 4 * (lane / 16) + e;
            efrag[(((size_t)(part * 4 + ot) * 4 + kq) * 64 + lane) * 4 + e] =
                part == 0 ? pih[src] : pil[src];
          }

  // candidate grids for the block search (k = 2, 3, and 4 with N >= 64)
  fq::GridTable grid, grid1;
  cb->grid_G = 0;
  cb->grid1_G = 0;
  {
    int G = 0, G1 = 0;
    if (fq::grid_plan(k, N, cb->last, &G, &G1)) {
      fq::build_grid(cb->c.data(), N, k, k, G, fq::GRID_R, fq::grid_record_entries(k), (uint16_t)N,
                     &grid);
      cb->grid_G = G;
      if (G1 > 0) {
        fq::build_grid(cb->c.data(), N, k, 1, G1, fq::GRID_R, fq::grid_record_entries(k),
                       (uint16_t)N, &grid1);
        cb->grid1_G = G1;
      }
    }
  }

  // one device allocation, 256-byte aligned sub-buffers
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t o_pi64 = take(8ull * d * d), o_pi32 = take(4ull * d * d),
               o_enc = take(4ull * (N + 1) * S), o_cbh = take(2ull * N * k),
               o_cbl = take(2ull * N * k), o_frag = take(2ull * frag.size()),
               o_efrag = take(2ull * efrag.size()),
               o_grid = take(2ull * grid.rec.size() + 64), o_grid1 = take(2ull * grid1.rec.size() + 64),
               o_pih = take(2ull * d * d), o_pil = take(2ull * d * d), o_pit = take(4ull * d * d),
               o_lfrag = take(2ull * lfrag.size()), o_hn = take(4ull * hnorm.size()),
               o_pi64t = take(8ull * d * d), o_pair = take(2ull * pair16.size());
  cb->dev_bytes = off;
  {
    DeviceGuard g(device);
    if (g.err != hipSuccess) {
      delete cb;
      return FQ_ERR_DEVICE;
    }
    scratch_setup(device);
    if (hipMalloc(&cb->dev_block, off) != hipSuccess) {
      (void)hipGetLastError();
      delete cb;
      return FQ_ERR_NO_MEMORY;
    }
    char* base = static_cast<char*>(cb->dev_block);
    cb->t.pi64 = reinterpret_cast<double*>(base + o_pi64);
    cb->t.pi64t = reinterpret_cast<double*>(base + o_pi64t);
    cb->t.pi32 = reinterpret_cast<float*>(base + o_pi32);
    cb->t.enc = reinterpret_cast<float*>(base + o_enc);
    cb->t.cb16hi = reinterpret_cast<_Float16*>(base + o_cbh);
    cb->t.cb16lo = reinterpret_cast<_Float16*>(base + o_cbl);
    cb->t.pifrag = reinterpret_cast<_Float16*>(base + o_frag);
    cb->t.encfrag = reinterpret_cast<_Float16*>(base + o_efrag);
    cb->t.pi16hi = reinterpret_cast<_Float16*>(base + o_pih);
    cb->t.pi16lo = reinterpret_cast<_Float16*>(base + o_pil);
    cb->t.pi32t = reinterpret_cast<float*>(base + o_pit);
    cb->t.grid = grid.rec.empty() ? nullptr : reinterpret_cast<uint16_t*>(base + o_grid);
    cb->t.grid1 = grid1.rec.empty() ? nullptr : reinterpret_cast<uint16_t*>(base + o_grid1);
    cb->t.lfrag = lfrag.empty() ? nullptr : reinterpret_cast<_Float16*>(base + o_lfrag);
    cb->t.hnorm = hnorm.empty() ? nullptr : reinterpret_cast<float*>(base + o_hn);
    cb->t.pair16 = pair16.empty() ? nullptr : reinterpret_cast<_Float16*>(base + o_pair);
    std::vector<char> staging(off, 0);
    memcpy(staging.data() + o_pi64, cb->pi.data(), 8ull * d * d);
    memcpy(staging.data() + o_pi32, pi32.data(), 4ull * d * d);
    memcpy(staging.data() + o_enc, enc.data(), 4ull * (N + 1) * S);
    memcpy(staging.data() + o_cbh, cbh.data(), 2ull * N * k);
    memcpy(staging.data() + o_cbl, cbl.data(), 2ull * N * k);
    memcpy(staging.data() + o_frag, frag.data(), 2ull * frag.size());
    memcpy(staging.data() + o_efrag, efrag.data(), 2ull * efrag.size());
    memcpy(staging.data() + o_pih, pih.data(), 2ull * d * d);
    memcpy(staging.data() + o_pil, pil.data(), 2ull * d * d);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        reinterpret_cast<float*>(staging.data() + o_pit)[(size_t)j * d + i] = pi32[(size_t)i * d + j];
        reinterpret_cast<double*>(staging.data() + o_pi64t)[(size_t)j * d + i] = cb->pi[(size_t)i * d + j];
      }
    if (!lfrag.empty()) memcpy(staging.data() + o_lfrag, lfrag.data(), 2ull * lfrag.size());
    if (!hnorm.empty()) memcpy(staging.data() + o_hn, hnorm.data(), 4ull * hnorm.size());
    if (!pair16.empty()) memcpy(staging.data() + o_pair, pair16.data(), 2ull * pair16.size());
    if (!grid.rec.empty()) memcpy(staging.data() + o_grid, grid.rec.data(), 2ull * grid.rec.size());
    if (!grid1.rec.empty())
      memcpy(staging.data() + o_grid1, grid1.rec.data(), 2ull * grid1.rec.size());
    cb->grid_host = std::move(grid.rec);
    cb->grid1_host = std::move(grid1.rec);
    if (hipMemcpy(cb->dev_block, staging.data(), off, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(cb->dev_block);
      delete cb;
      return FQ_ERR_DEVICE;
    }
  }
  *out = cb;
  return FQ_OK;
}

fq_status fq_codebook_info(const fq_codebook* cb, fq_info* out) {
  if (!cb || !out) return FQ_ERR_INVALID_ARG;
  out->d = cb->d;
  out->k = cb->k;
  out->N = cb->N;
  out->nb = cb->nb;
  out->idx_bits = cb->bits;
  out->record_words = cb->W;
  out->last_block = cb->last;
  out->packed_bits = fq::packed_record_bits(cb);
  out->rate_nominal = cb->rate_nominal;
  out->rate_actual = cb->rate_actual;
  out->distortion = cb->distortion;
  out->artifact_hash = cb->hash;
  return FQ_OK;
}

fq_status fq_search_cost(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                         int64_t x_ld, double* entries_per_vector, double* full_scan_share) {
  if (!cb || !x || n < 1 || x_ld < fq::D || !entries_per_vector) return FQ_ERR_INVALID_ARG;
  if (x_dtype != FQ_F16 && x_dtype != FQ_F32) return FQ_ERR_INVALID_ARG;
  const int k = cb->k, N = cb->N, nb = cb->nb, last = cb->last;
  const bool grid = cb->grid_G > 0 && !cb->grid_host.empty();
  const int re = fq::grid_record_entries(k);
  const float sc = grid ? fq::grid_scale(cb->grid_G) : 0.f;
  const float sc1 = cb->grid1_G > 0 ? fq::grid_scale(cb->grid1_G) : 0.f;
  double entries = 0.0, scans = 0.0;
  double xv[fq::D], z[fq::D];
  for (int64_t r = 0; r < n; ++r) {
    double ss = 0.0;
    for (int i = 0; i < fq::D; ++i) {
      if (x_dtype == FQ_F16) {
        _Float16 h;
        memcpy(&h, static_cast<const unsigned char*>(x) + 2 * (r * x_ld + i), 2);
        xv[i] = (double)h;
      } else {
        float f;
        memcpy(&f, static_cast<const unsigned char*>(x) + 4 * (r * x_ld + i), 4);
        xv[i] = (double)f;
      }
      ss += xv[i] * xv[i];
    }
    const double nu = sqrt(ss);
    for (int i = 0; i < fq::D; ++i) {
      double t = 0.0;
      for (int j = 0; j < fq::D; ++j) t += cb->pi[(size_t)i * fq::D + j] * xv[j];
      z[i] = nu > 0.0 ? t / nu : NAN;
    }
    for (int j = 0; j < nb; ++j) {
      const bool part = j == nb - 1 && last < k;
      const int dims = part ? 1 : k;
      int cnt = 0;
      if (grid && (!part || cb->grid1_G > 0)) {
        const int G = part ? cb->grid1_G : cb->grid_G;
        bool inside = true;
        int cell = 0, mul = 1;
        for (int t = 0; t < dims; ++t) {
          const float u = fq::grid_pos((float)z[j * k + t], part ? sc1 : sc);
          const bool in = fq::grid_pos_inside(u, G);
          inside = inside && in;
          if (in) cell += (int)u * mul;
          mul *= G;
        }
        const uint16_t c0 = (part ? cb->grid1_host : cb->grid_host)[(size_t)cell * re];
        if (inside && c0 != fq::GRID_OVERFLOW) cnt = c0;
      }
      entries += cnt > 0 ? cnt : N;
      scans += cnt > 0 ? 0.0 : 1.0;
    }
  }
  *entries_per_vector = entries / (double)n;
  if (full_scan_share) *full_scan_share = scans / ((double)n * nb);
  return FQ_OK;
}

void fq_codebook_free(fq_codebook* cb) {
  if (!cb) return;
  {
    DeviceGuard g(cb->device);
    if (cb->dev_block) (void)hipFree(cb->dev_block);
  }
  delete cb;
}

fq_status fq_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                    int64_t x_ld, uint32_t* codes, uint16_t* norms, void* stream) {
  if (!cb || n < 0) return FQ_ERR_INVALID_ARG;
  if (x_dtype != FQ_F16 && x_dtype != FQ_F32) return FQ_ERR_INVALID_ARG;
  if (n == 0) return FQ_OK;
  const int esz = x_dtype == FQ_F16 ? 2 : 4;
  if (!x || !codes || !norms || x_ld < fq::D || (x_ld * esz) % 16 != 0 || !aligned(x, 16) ||
      !aligned(codes, 4) || !aligned(norms, 2))
    return FQ_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 40)) return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fq::large_block(cb->k)        ? fq::launch_encode_large(cb, x, x_dtype, n, x_ld, codes, norms, st)
                 : fq::encode_k8_applies(cb) ? fq::launch_encode_k8(cb, x, x_dtype, n, x_ld, codes, norms, st)
                                             : fq::launch_encode(cb, x, x_dtype, n, x_ld, codes, norms, st);
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

fq_status fq_decode(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                    const int64_t* rows, int64_t n_records, int64_t n, void* y, fq_dtype y_dtype,
                    int64_t y_ld, void* stream) {
  if (!cb || n < 0) return FQ_ERR_INVALID_ARG;
  if (y_dtype != FQ_F16 && y_dtype != FQ_F32) return FQ_ERR_INVALID_ARG;
  if (n == 0) return FQ_OK;
  const int esz = y_dtype == FQ_F16 ? 2 : 4;
  if (!codes || !norms || !y || y_ld < fq::D || (y_ld * esz) % 16 != 0 || !aligned(y, 16) ||
      !aligned(codes, 4) || !aligned(norms, 2))
    return FQ_ERR_INVALID_ARG;
  if (rows && (!aligned(rows, 8) || n_records < 0)) return FQ_ERR_INVALID_ARG;
  if (y_ld > (int64_t(1) << 22)) return FQ_ERR_UNSUPPORTED;  // 32-bit offsets per 16-row tile
  // gathered records are addressed with 32-bit buffer offsets
  if (rows && n_records * cb->W * 4 > (int64_t(1) << 31) - 1) return FQ_ERR_UNSUPPORTED;
  if (n > (int64_t(1) << 40)) return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_decode(cb, codes, norms, rows, rows ? n_records : n, n, y, y_dtype,
                                   y_ld, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

fq_status fq_pack_records(const fq_codebook* cb, const uint32_t* codes, const uint16_t* norms,
                          int64_t n, uint32_t* packed, void* stream) {
  if (!cb || n < 0) return FQ_ERR_INVALID_ARG;
  if (n == 0) return FQ_OK;
  if (!codes || !norms || !packed || !aligned(codes, 4) || !aligned(norms, 2) ||
      !aligned(packed, 4))
    return FQ_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 40)) return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_pack(cb, codes, norms, n, packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

fq_status fq_decode_packed(const fq_codebook* cb, const uint32_t* packed, const int64_t* rows,
                           int64_t n_records, int64_t n, void* y, fq_dtype y_dtype, int64_t y_ld,
                           void* stream) {
  if (!cb || n < 0) return FQ_ERR_INVALID_ARG;
  if (y_dtype != FQ_F16 && y_dtype != FQ_F32) return FQ_ERR_INVALID_ARG;
  if (n == 0) return FQ_OK;
  const int esz = y_dtype == FQ_F16 ? 2 : 4;
  if (!packed || !y || y_ld < fq::D || (y_ld * esz) % 16 != 0 || !aligned(y, 16) ||
      !aligned(packed, 4))
    return FQ_ERR_INVALID_ARG;
  if (rows && (!aligned(rows, 8) || n_records < 0)) return FQ_ERR_INVALID_ARG;
  if (y_ld > (int64_t(1) << 22)) return FQ_ERR_UNSUPPORTED;
  // gathered records are addressed with 32-bit buffer offsets over the whole stream
  if (rows && (n_records * fq::packed_record_bits(cb) + 31) / 32 * 4 > (int64_t(1) << 31) - 1)
    return FQ_ERR_UNSUPPORTED;
  if (n > (int64_t(1) << 40)) return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_decode(cb, packed, nullptr, rows, rows ? n_records : n, n, y, y_dtype,
                                   y_ld, static_cast<hipStream_t>(stream), true);
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

static fq_status check_attend_shape(const fq_codebook* ck, int B, int Hq, int Hkv, int64_t T) {
  if (!ck || B < 1 || Hq < 1 || Hkv < 1 || T < 1) return FQ_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FQ_ERR_INVALID_ARG;
  if (Hq / Hkv > 8) return FQ_ERR_UNSUPPORTED;
  if (!fq::attend_supported(ck)) return FQ_ERR_UNSUPPORTED;
  if (T > (int64_t(1) << 31) || (int64_t)B * Hkv > (1 << 20)) return FQ_ERR_UNSUPPORTED;
  return FQ_OK;
}

fq_status fq_attend_workspace_size(const fq_codebook* cb_k, int B, int Hq, int Hkv, int64_t T,
                                   size_t* bytes) {
  if (!bytes) return FQ_ERR_INVALID_ARG;
  fq_status st = check_attend_shape(cb_k, B, Hq, Hkv, T);
  if (st != FQ_OK) return st;
  *bytes = fq::attend_workspace_bytes(cb_k, B, Hq, Hkv, T);
  return FQ_OK;
}

// Arguments shared by fq_attend_decode and fq_attend_decode_static.
static fq_status check_attend_args(const fq_codebook* cb_k, const fq_codebook* cb_v,
                                   const uint16_t* q, const uint32_t* k_codes,
                                   const uint16_t* k_norms, const uint32_t* v_codes,
                                   const uint16_t* v_norms, int B, int Hq, int Hkv, int64_t T,
                                   float scale, const uint16_t* out) {
  fq_status st = check_attend_shape(cb_k, B, Hq, Hkv, T);
  if (st != FQ_OK) return st;
  if (!cb_v || cb_v->device != cb_k->device) return FQ_ERR_INVALID_ARG;
  if (!same_variant(cb_k, cb_v)) return FQ_ERR_UNSUPPORTED;
  if (!q || !k_codes || !k_norms || !v_codes || !v_norms || !out) return FQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_norms, 16) || !aligned(v_norms, 16))
    return FQ_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FQ_ERR_INVALID_ARG;
  return FQ_OK;
}

fq_status fq_attend_decode(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                           const uint32_t* k_codes, const uint16_t* k_norms,
                           const uint32_t* v_codes, const uint16_t* v_norms, int B, int Hq,
                           int Hkv, int64_t T, float scale, void* workspace,
                           size_t workspace_bytes, uint16_t* out, void* stream) {
  fq_status st = check_attend_args(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv,
                                   T, scale, out);
  if (st != FQ_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return FQ_ERR_INVALID_ARG;
  if (workspace_bytes < fq::attend_workspace_bytes(cb_k, B, Hq, Hkv, T))
    return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb_k->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_attend(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv,
                                   T, T, 1, scale, workspace, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

fq_status fq_attend_decode_static(const fq_codebook* cb_k, const fq_codebook* cb_v,
                                  const uint16_t* q, const uint32_t* k_codes,
                                  const uint16_t* k_norms, const uint32_t* v_codes,
                                  const uint16_t* v_norms, int B, int Hq, int Hkv, int64_t T,
                                  float scale, uint16_t* out, void* stream) {
  fq_status st = check_attend_args(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv,
                                   T, scale, out);
  if (st != FQ_OK) return st;
  if (fq::attend_workspace_bytes(cb_k, B, Hq, Hkv, T) > FQ_STATIC_SCRATCH_BYTES)
    return FQ_ERR_SCRATCH;
  void* ws = scratch_address(cb_k->device);   // set up when cb_k was loaded
  if (!ws) return FQ_ERR_DEVICE;
  DeviceGuard g(cb_k->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_attend(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv,
                                   T, T, 1, scale, ws, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

// appends of up to this many vectors per cache take the float64 append kernel
constexpr int64_t APPEND_DIRECT_MAX = 8192;

static fq_status check_queries(const fq_codebook* cb_k, const fq_codebook* cb_v, int B, int Hq,
                               int Hkv, int64_t T, int64_t T_ld, int M) {
  if (M < 1 || M > fq::MAX_QUERIES || T < M || T_ld < T) return FQ_ERR_INVALID_ARG;
  if (Hq < 1 || (int64_t)Hq * M > (1 << 20)) return FQ_ERR_INVALID_ARG;
  fq_status st = check_attend_shape(cb_k, B, Hq * M, Hkv, T);
  if (st != FQ_OK) return st;
  if (!cb_v || cb_v->device != cb_k->device) return FQ_ERR_INVALID_ARG;
  if (!same_variant(cb_k, cb_v)) return FQ_ERR_UNSUPPORTED;
  if (T_ld > (int64_t(1) << 31)) return FQ_ERR_UNSUPPORTED;
  return FQ_OK;
}

fq_status fq_attend_queries(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                            const uint32_t* k_codes, const uint16_t* k_norms,
                            const uint32_t* v_codes, const uint16_t* v_norms, int B, int Hq,
                            int Hkv, int64_t T, int64_t T_ld, int M, float scale, void* workspace,
                            size_t workspace_bytes, uint16_t* out, void* stream) {
  fq_status st = check_queries(cb_k, cb_v, B, Hq, Hkv, T, T_ld, M);
  if (st != FQ_OK) return st;
  if (!q || !k_codes || !k_norms || !v_codes || !v_norms || !workspace || !out)
    return FQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_norms, 16) || !aligned(v_norms, 16) || !aligned(workspace, 256))
    return FQ_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FQ_ERR_INVALID_ARG;
  if (workspace_bytes < fq::attend_workspace_bytes(cb_k, B, Hq * M, Hkv, T))
    return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb_k->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipError_t e = fq::launch_attend(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq * M,
                                   Hkv, T, T_ld, M, scale, workspace, out,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

fq_status fq_decode_step(const fq_codebook* cb_k, const fq_codebook* cb_v, const uint16_t* q,
                         const uint16_t* k_new, const uint16_t* v_new, uint32_t* k_codes,
                         uint16_t* k_norms, uint32_t* v_codes, uint16_t* v_norms, int B, int Hq,
                         int Hkv, int64_t T_ld, int64_t pos, int M, float scale, void* workspace,
                         size_t workspace_bytes, uint16_t* out, void* stream) {
  if (pos < 0 || M < 1 || pos > T_ld - M) return FQ_ERR_INVALID_ARG;
  const int64_t T = pos + M;
  fq_status st = check_queries(cb_k, cb_v, B, Hq, Hkv, T, T_ld, M);
  if (st != FQ_OK) return st;
  if (!q || !k_new || !v_new || !k_codes || !k_norms || !v_codes || !v_norms || !workspace || !out)
    return FQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_norms, 16) ||
      !aligned(v_norms, 16) || !aligned(workspace, 256))
    return FQ_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FQ_ERR_INVALID_ARG;
  if (workspace_bytes < fq::attend_workspace_bytes(cb_k, B, Hq * M, Hkv, T))
    return FQ_ERR_INVALID_ARG;
  DeviceGuard g(cb_k->device);
  if (g.err != hipSuccess) return FQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the M new tokens of stream (b, h) are rows (b Hkv + h) M + m: record
  // (b Hkv + h) T_ld + pos + m of the caches
  fq::OutRows rows;
  rows.inner = M;
  rows.stride = T_ld;
  rows.pos = pos;
  const int64_t n = (int64_t)B * Hkv * M;
  if (n <= APPEND_DIRECT_MAX) {
    // a few vectors: encoded from the float64 definition, inside the
    // attention kernel where it can (see launch_attend)
    fq::AppendIn app;
    app.k_new = k_new;
    app.v_new = v_new;
    app.M = M;
    app.pi64t = cb_k->t.pi64t;
    app.kc = k_codes;
    app.kn = k_norms;
    app.vc = v_codes;
    app.vn = v_norms;
    hipError_t e = fq::launch_attend(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq * M,
                                     Hkv, T, T_ld, M, scale, workspace, out, s, app);
    return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
  }
  hipError_t e;
  if (cb_v == cb_k) {   // one launch encodes the keys and then the values
    fq::SecondInput vals;
    vals.x = v_new;
    vals.n = n;
    vals.codes = v_codes;
    vals.norms = v_norms;
    e = fq::launch_encode(cb_k, k_new, FQ_F16, n, fq::D, k_codes, k_norms, s, rows, vals);
  } else {
    e = fq::launch_encode(cb_k, k_new, FQ_F16, n, fq::D, k_codes, k_norms, s, rows);
    if (e == hipSuccess) e = fq::launch_encode(cb_v, v_new, FQ_F16, n, fq::D, v_codes, v_norms, s, rows);
  }
  if (e == hipSuccess)
    e = fq::launch_attend(cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, B, Hq * M, Hkv, T,
                          T_ld, M, scale, workspace, out, s);
  return e == hipSuccess ? FQ_OK : FQ_ERR_DEVICE;
}

}  // extern "C"
