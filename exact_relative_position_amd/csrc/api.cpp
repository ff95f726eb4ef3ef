// api.cpp -- the C ABI: argument validation, workspace planning and the
// launch sequence of the forward and backward passes.
//
// Forward (pipeline section of "Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels", nanless.github.io digest):
//   map tables (bucket unfold) -> relation projection of the reachable window ->
//   fused tiled forward.
// Backward (backward section of the same page):
//   the padded row terms (LSE, D, the key pass's seeds) ->
//   query-parallel pass -> key-parallel pass ->
//   dZ . table into dQ / dK -> dZ^T . Q / K into the table gradients ->
//   fold of copied bucket columns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "geometry.hpp"
#include "relpos_attn.h"
#include "buckets.hpp"

namespace relpos {
hipError_t launch_fwd(int dtype, const AttnArgs& a, hipStream_t st);
hipError_t launch_rowterm(int dtype, const RowTermArgs& a, hipStream_t st);
hipError_t launch_bwd_f32(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st);
hipError_t launch_bwd_f16(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st);
hipError_t launch_bwd_bf16(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st);
hipError_t launch_phi_rows(const PhiArgs& p, int32_t* rows, hipStream_t st);
hipError_t launch_phi_fold(const PhiArgs& p, int32_t* fold, int32_t* ub, int32_t* ue, int R,
                           hipStream_t st);
hipError_t launch_bias_unfold(int dtype, const BiasArgs& a, hipStream_t st);
hipError_t launch_proj(int dtype, const ProjArgs& a, hipStream_t st);
hipError_t launch_rows(int dtype, const RowsArgs& a, hipStream_t st);
hipError_t launch_tab_unfold(int dtype, const TabUnfoldArgs& a, hipStream_t st);
hipError_t launch_cols(int dtype, const ColsArgs& a, int Ho, hipStream_t st);
hipError_t launch_cols1(int dtype, const ColsArgs& a, int Ho, hipStream_t st);
hipError_t launch_xsplit(const SplitArgs& a, hipStream_t st);
hipError_t launch_fold(const FoldArgs& a, hipStream_t st);
}  // namespace relpos

using namespace relpos;

namespace {

thread_local std::string g_err;

relpos_status fail(relpos_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr int64_t kMaxN = 1 << 20;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int elem_size(int dtype) { return dtype == RELPOS_F32 ? 4 : 2; }

// Resolved description of one call.
struct Plan {
  int dtype = 0, esz = 0;
  int B = 0, H = 0, N = 0;
  int Np = 0;      // N rounded up to the 64-token tile
  Geo geo{};
  PhiArgs phi{};
  int R = 0;       // rows of the caller's tables
  int Runf = 0;    // rows of the unfolded truncated map
  bool bucketed = false;  // T5 or log buckets: unfolded, gradients folded back
  bool has_aq = false, has_ak = false, has_b = false;
  bool keypad = false;
  int drop_t = 0;      // dropout threshold t (p = t / 256), 0 = off
  int64_t aq_hs = 0, ak_hs = 0, b_hs = 0;
  int nblk = 0;        // 128-row blocks per (b, h)
  int ncol_q = 0, ncol_k = 0;
  int zr = 0;          // query rows per chunk of the query-side projection
  int nchunk = 1;      // chunks of queries (1: the whole sequence at once)
  bool inblock = false;  // forward: query-side relation computed in the block
  size_t zq_elems = 0; // query-side projection buffer (Z^Q, dZ^Q), elements
  size_t zk_elems = 0; // key-side projection buffer (Z^K, dZ^K), elements
  int rtiles = 0, Rpad = 0;
  int split_q = 1, split_k = 1, split_b = 1;
  int ho_aq = 1, ho_ak = 1, ho_b = 1;
};

// Least n in [lo, hi] with pred(n), for a predicate that is false then true
// over the range and true at hi.
template <typename P>
int first_true(int lo, int hi, P pred) {
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (pred(mid)) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Unfolded thresholds of a map.  Truncated: its own thresholds.  Bucketed:
// the first offsets on each side beyond which the row no longer changes,
// clipped to the offsets that exist at this length, +-(N - 1), so that the
// unfolded tables and the contraction grow with N and not with max_distance
// (bucket rows no offset reaches get no unfolded row and a zero gradient).
relpos_status unfold_range(const relpos_phi& p, int64_t N, int64_t& R, int64_t& lo, int64_t& hi) {
  switch (p.kind) {
    case RELPOS_PHI_TRUNCATED:
      if (p.lo > p.hi) return fail(RELPOS_ERR_INVALID_ARG, "truncated map needs lo <= hi");
      if (p.lo < -(1 << 29) || p.hi > (1 << 29))
        return fail(RELPOS_ERR_INVALID_ARG, "truncation thresholds out of range");
      R = (int64_t)p.hi - p.lo + 1;
      lo = p.lo;
      hi = p.hi;
      return RELPOS_OK;
    case RELPOS_PHI_IDENTITY:
      R = 2 * N - 1;
      lo = -(N - 1);
      hi = N - 1;
      return RELPOS_OK;
    case RELPOS_PHI_BUCKET_T5: {
      if (p.num_buckets < 2 || p.num_buckets > 4096)
        return fail(RELPOS_ERR_INVALID_ARG, "T5 num_buckets must be in [2, 4096]");
      if (p.bidirectional && (p.num_buckets & 1))
        return fail(RELPOS_ERR_INVALID_ARG, "bidirectional T5 needs an even num_buckets");
      const int nb = p.bidirectional ? p.num_buckets / 2 : p.num_buckets;
      const int me = p.max_exact > 0 ? p.max_exact : nb / 2;
      if (me < 1 || me >= nb)
        return fail(RELPOS_ERR_INVALID_ARG, "T5 max_exact must be in [1, buckets per side)");
      if (p.max_distance <= me || p.max_distance > (1 << 24))
        return fail(RELPOS_ERR_INVALID_ARG, "T5 max_distance must exceed max_exact");
      // the bucket of -n is non-decreasing in n and reaches nb - 1 by
      // n = max_distance: the first such n by bisection
      const int nsat = first_true(0, p.max_distance, [&](int n) {
        return t5_bucket_dev(-n, p.num_buckets, p.max_exact, p.max_distance, p.bidirectional) ==
               nb - 1;
      });
      R = p.num_buckets;
      lo = std::max<int64_t>(-nsat, -(N - 1));
      hi = std::min<int64_t>(p.bidirectional ? nsat : 0, N - 1);
      return RELPOS_OK;
    }
    case RELPOS_PHI_BUCKET_LOG: {
      const int k = p.num_buckets, m = p.max_distance;
      if (k < 4 || k > 4096 || (k & 1))
        return fail(RELPOS_ERR_INVALID_ARG, "log-bucket num_buckets must be even, in [4, 4096]");
      if (m < k / 2 + 2 || m > (1 << 24))
        return fail(RELPOS_ERR_INVALID_ARG, "log-bucket max_distance must be in [k/2 + 2, 2^24]");
      // the row is monotone in o and reaches 2k - 1 by o = m - 1 and 0 by
      // o = -m: the first offsets of the two constant runs, by bisection
      const int nhi = first_true(0, m - 1, [&](int n) { return log_bucket_dev(n, k, m) == 2 * k - 1; });
      const int nlo = first_true(0, m, [&](int n) { return log_bucket_dev(-n, k, m) == 0; });
      R = 2 * k;
      lo = std::max<int64_t>(-nlo, -(N - 1));
      hi = std::min<int64_t>(nhi, N - 1);
      return RELPOS_OK;
    }
    default:
      return fail(RELPOS_ERR_INVALID_ARG, "unknown phi kind");
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

relpos_status make_plan(const relpos_problem* prob, const relpos_phi* phi,
                        const relpos_mask* mask, int terms, Plan& pl) {
  if (!prob || !phi || !mask) return fail(RELPOS_ERR_INVALID_ARG, "null descriptor");
  if (prob->dtype < RELPOS_F32 || prob->dtype > RELPOS_BF16)
    return fail(RELPOS_ERR_INVALID_ARG, "unknown dtype");
  if (prob->B < 0 || prob->H < 0 || prob->N < 0)
    return fail(RELPOS_ERR_INVALID_ARG, "negative size");
  if (prob->d != kHeadDim) return fail(RELPOS_ERR_UNSUPPORTED, "only head dim 64 is implemented");
  if (prob->N > kMaxN) return fail(RELPOS_ERR_UNSUPPORTED, "N above 1048576");
  if (prob->B > 65535 || prob->H > 65535) return fail(RELPOS_ERR_UNSUPPORTED, "B or H too large");
  if (!(prob->tau > 0.f) || !std::isfinite(prob->tau))
    return fail(RELPOS_ERR_INVALID_ARG, "tau must be finite and > 0");
  if (mask->flags & ~(RELPOS_MASK_CAUSAL | RELPOS_MASK_KEY_PADDING))
    return fail(RELPOS_ERR_INVALID_ARG, "unknown mask bits");
  if ((mask->flags & RELPOS_MASK_KEY_PADDING) && !mask->key_len)
    return fail(RELPOS_ERR_INVALID_ARG, "key padding needs key_len");
  if (terms & ~(RELPOS_TERM_AQ | RELPOS_TERM_AK | RELPOS_TERM_B))
    return fail(RELPOS_ERR_INVALID_ARG, "unknown term bits");
  if (!(prob->dropout_p >= 0.f) || !(prob->dropout_p < 1.f))
    return fail(RELPOS_ERR_INVALID_ARG, "dropout_p must be in [0, 1)");
  pl.drop_t = (int)std::nearbyint(prob->dropout_p * 256.f);
  if (pl.drop_t > 255)
    return fail(RELPOS_ERR_INVALID_ARG, "dropout_p rounds to 1 (t = 256 of 256)");
  if (pl.drop_t == 0 && prob->dropout_p > 0.f)
    return fail(RELPOS_ERR_INVALID_ARG,
                "dropout_p rounds to 0 (below 1/512): it would silently turn dropout off");
  if (pl.drop_t > 0 && elem_size(prob->dtype) != 2)
    return fail(RELPOS_ERR_UNSUPPORTED, "dropout is implemented for fp16 and bf16 inputs");
  pl.dtype = prob->dtype;
  pl.esz = elem_size(prob->dtype);
  pl.B = (int)prob->B;
  pl.H = (int)prob->H;
  pl.N = (int)prob->N;
  pl.Np = (pl.N + 63) / 64 * 64;
  pl.has_aq = terms & RELPOS_TERM_AQ;
  pl.has_ak = terms & RELPOS_TERM_AK;
  pl.has_b = terms & RELPOS_TERM_B;
  pl.keypad = mask->flags & RELPOS_MASK_KEY_PADDING;
  pl.bucketed = phi->kind == RELPOS_PHI_BUCKET_T5 || phi->kind == RELPOS_PHI_BUCKET_LOG;
  const int64_t Nn = pl.N > 0 ? pl.N : 1;
  int64_t R, lo, hi;
  relpos_status s = unfold_range(*phi, Nn, R, lo, hi);
  if (s != RELPOS_OK) return s;
  pl.R = (int)R;
  pl.Runf = (int)(hi - lo + 1);
  pl.geo.N = pl.N;
  pl.geo.lo = (int)lo;
  pl.geo.hi = (int)hi;
  pl.geo.R = pl.Runf;
  pl.geo.W = (int)std::min<int64_t>(pl.Runf, (int64_t)pl.N + kGroup - 1);
  pl.geo.causal = (mask->flags & RELPOS_MASK_CAUSAL) ? 1 : 0;
  if (pl.geo.W < 1) pl.geo.W = 1;
  // rows of dZ^Q shifted (band runs on whole lines) for wide bands, where
  // most tiles of a row are band tiles
  pl.geo.dsm = wide_band(pl.geo) ? 31 : 0;
  pl.geo.Wp = z_pitch(pl.geo.W, pl.geo.dsm != 0);
  pl.phi.kind = phi->kind;
  pl.phi.N = pl.N;
  pl.phi.lo_unf = (int)lo;
  pl.phi.hi_unf = (int)hi;
  pl.phi.num_buckets = phi->num_buckets;
  pl.phi.max_exact = phi->max_exact;
  pl.phi.max_distance = phi->max_distance;
  pl.phi.bidirectional = phi->bidirectional ? 1 : 0;
  pl.phi.lo = phi->lo;
  pl.phi.hi = phi->hi;
  pl.aq_hs = prob->aq_head_stride;
  pl.ak_hs = prob->ak_head_stride;
  pl.b_hs = prob->b_head_stride;
  if (pl.aq_hs < 0 || pl.ak_hs < 0 || pl.b_hs < 0)
    return fail(RELPOS_ERR_INVALID_ARG, "negative table head stride");
  if ((pl.has_aq && (pl.aq_hs * pl.esz) % 16) || (pl.has_ak && (pl.ak_hs * pl.esz) % 16))
    return fail(RELPOS_ERR_INVALID_ARG, "table head stride must be a multiple of 16 bytes");
  if ((size_t)pl.B * pl.H * pl.N * (size_t)pl.geo.Wp > (size_t)1 << 40)
    return fail(RELPOS_ERR_UNSUPPORTED, "projection window too large");
  pl.ho_aq = pl.aq_hs == 0 ? 1 : pl.H;
  pl.ho_ak = pl.ak_hs == 0 ? 1 : pl.H;
  pl.ho_b = pl.b_hs == 0 ? 1 : pl.H;
  pl.nblk = (pl.N + kBlockRows - 1) / kBlockRows;
  if (prob->zchunk < 0 || prob->zchunk % kBlockRows)
    return fail(RELPOS_ERR_INVALID_ARG, "zchunk must be a non-negative multiple of 128");
  pl.zr = pl.N;
  if (prob->zchunk > 0 && prob->zchunk < pl.N) {
    pl.zr = (int)prob->zchunk;
    pl.nchunk = (pl.N + pl.zr - 1) / pl.zr;
    if (pl.has_ak)
      return fail(RELPOS_ERR_UNSUPPORTED,
                  "a chunked projection covers the query-side terms only (aK must be absent)");
  }
  // how the forward gets the query-side relation (length-bucket table: the
  // in-block path for sequences no longer than the relation window, where a
  // stored window is as large as a dense bias; the stored projection beyond)
  if (prob->relation < RELPOS_REL_AUTO || prob->relation > RELPOS_REL_INBLOCK)
    return fail(RELPOS_ERR_INVALID_ARG, "unknown relation mode");
  {
    // (with zchunk the in-block forward needs no chunks: it holds no Z^Q at
    // all; the backward still projects one chunk of queries at a time)
    const bool can = pl.esz == 2 && !pl.has_ak;
    if (prob->relation == RELPOS_REL_INBLOCK && pl.has_aq && !can)
      return fail(RELPOS_ERR_UNSUPPORTED,
                  "the in-block relation needs fp16 or bf16 inputs and no aK");
    const bool shortn = pl.geo.W >= pl.N;
    pl.inblock = pl.has_aq && can &&
                 (prob->relation == RELPOS_REL_INBLOCK ||
                  (prob->relation == RELPOS_REL_AUTO && shortn));
  }
  pl.geo.zr = pl.zr;
  pl.geo.z0 = 0;
  pl.zq_elems = (size_t)pl.B * pl.H * pl.zr * pl.geo.Wp;
  pl.zk_elems = (size_t)pl.B * pl.H * pl.N * pl.geo.Wp;
  // column tiles of the projection (max over groups)
  for (int grp = 0; grp < pl.nblk; ++grp) {
    int cb, ce;
    cols_q(pl.geo, grp, cb, ce);
    pl.ncol_q = std::max(pl.ncol_q, (ce - cb + 63) / 64);
    cols_k(pl.geo, grp, cb, ce);
    pl.ncol_k = std::max(pl.ncol_k, (ce - cb + 63) / 64);
    if (!grouped(pl.geo)) break;
  }
  pl.Rpad = (pl.Runf + 63) / 64 * 64;  // 64-row tiles of the column contraction
  pl.rtiles = pl.Rpad / 32;
  auto splits = [&](int ho, bool shared) {
    const int64_t rows = (int64_t)(shared ? pl.B * pl.H : pl.B) * pl.N;
    const int64_t tiles = (int64_t)(pl.Rpad / 64) * ho;
    int64_t want = (4096 + tiles - 1) / std::max<int64_t>(1, tiles);
    int64_t cap = std::max<int64_t>(1, rows / 512);
    return (int)std::max<int64_t>(1, std::min(want, cap));
  };
  pl.split_q = splits(pl.ho_aq, pl.aq_hs == 0);
  pl.split_k = splits(pl.ho_ak, pl.ak_hs == 0);
  pl.split_b = splits(pl.ho_b, pl.b_hs == 0);
  return RELPOS_OK;
}

relpos_status check_tensor(const Plan& pl, const relpos_problem* prob, int role, const void* ptr,
                           const char* name) {
  if (!ptr) return fail(RELPOS_ERR_INVALID_ARG, std::string("null pointer: ") + name);
  if (!aligned16(ptr)) return fail(RELPOS_ERR_INVALID_ARG, std::string("misaligned: ") + name);
  for (int t = 0; t < 3; ++t) {
    const int64_t s = prob->strides[role][t];
    if (s < 0 || (s * pl.esz) % 16)
      return fail(RELPOS_ERR_INVALID_ARG,
                  std::string("stride must be a non-negative multiple of 16 bytes: ") + name);
  }
  if (prob->strides[role][2] < kHeadDim && pl.N > 1)
    return fail(RELPOS_ERR_INVALID_ARG, std::string("row stride smaller than d: ") + name);
  // a 64-row tile is addressed with 32-bit byte offsets
  if (prob->strides[role][2] > (int64_t(1) << 24))
    return fail(RELPOS_ERR_UNSUPPORTED, std::string("row stride above 2^24 elements: ") + name);
  return RELPOS_OK;
}

Str str_of(const relpos_problem* prob, int role) {
  return Str{prob->strides[role][0], prob->strides[role][1], prob->strides[role][2]};
}

// Workspace carving ---------------------------------------------------------
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += align256(bytes);
    return p;
  }
};

struct WsFwd {
  int32_t* fold = nullptr;
  float* bunf = nullptr;
  float* zq = nullptr;
  float* zk = nullptr;
};

struct WsBwd {
  int32_t* fold = nullptr;
  int32_t* ub = nullptr;
  int32_t* ue = nullptr;
  float* bunf = nullptr;
  float* zq = nullptr;
  float* zk = nullptr;
  float* L2 = nullptr;  // [B*H][Np]
  float* D = nullptr;   // [B*H][Np]
  float* kseed = nullptr;  // [4][B*H][Np]
  // [ho][Runf + 32][64] unfolded tables: fp32, or for 16-bit inputs a bf16
  // high part followed by a bf16 low part (fp16) in the same bytes
  float* tunf_q = nullptr;
  float* tunf_k = nullptr;
  // fp16 Q / K split into two bf16 parts, [B*H][N][64] each (column contraction)
  void* xq_h = nullptr;
  void* xq_l = nullptr;
  void* xk_h = nullptr;
  void* xk_l = nullptr;
  float* dq_part = nullptr;
  float* dk_part = nullptr;
  float* dzq = nullptr;
  float* dzk = nullptr;
  float* part_q = nullptr;
  float* part_qb = nullptr;
  float* part_k = nullptr;
  float* dk_acc = nullptr;
  float* dv_acc = nullptr;
};

bool need_bunf(const Plan& pl) { return pl.has_b && !pl.has_aq; }

size_t carve_fwd(const Plan& pl, bool zsave_given, void* base, WsFwd& w) {
  Carve c(base);
  if (pl.bucketed) w.fold = c.take<int32_t>(sizeof(int32_t) * pl.Runf);
  if (need_bunf(pl)) w.bunf = c.take<float>(sizeof(float) * pl.Runf * pl.ho_b);
  if (!zsave_given && !pl.inblock) {
    if (pl.has_aq) w.zq = c.take<float>(sizeof(float) * pl.zq_elems);
    if (pl.has_ak) w.zk = c.take<float>(sizeof(float) * pl.zk_elems);
  }
  return c.off;
}

size_t carve_bwd(const Plan& pl, bool zsave_given, void* base, WsBwd& w) {
  Carve c(base);
  const size_t bhn = (size_t)pl.B * pl.H * pl.N;
  if (pl.bucketed) {
    w.fold = c.take<int32_t>(sizeof(int32_t) * pl.Runf);
    w.ub = c.take<int32_t>(sizeof(int32_t) * pl.R);
    w.ue = c.take<int32_t>(sizeof(int32_t) * pl.R);
  }
  if (need_bunf(pl)) w.bunf = c.take<float>(sizeof(float) * pl.Runf * pl.ho_b);
  if (!zsave_given) {
    if (pl.has_aq) w.zq = c.take<float>(sizeof(float) * pl.zq_elems);
    if (pl.has_ak) w.zk = c.take<float>(sizeof(float) * pl.zk_elems);
  }
  const size_t bhnp = (size_t)pl.B * pl.H * pl.Np;
  w.L2 = c.take<float>(sizeof(float) * bhnp);
  w.D = c.take<float>(sizeof(float) * bhnp);
  w.kseed = c.take<float>(sizeof(float) * 4 * bhnp);
  const size_t tu = (size_t)(pl.Runf + 32) * kHeadDim;
  if (pl.has_aq) w.tunf_q = c.take<float>(sizeof(float) * pl.ho_aq * tu);
  if (pl.has_ak) w.tunf_k = c.take<float>(sizeof(float) * pl.ho_ak * tu);
  if (pl.dtype == 1) {
    const size_t xb = sizeof(uint16_t) * bhn * kHeadDim;
    if (pl.has_aq) {
      w.xq_h = c.take<uint16_t>(xb);
      w.xq_l = c.take<uint16_t>(xb);
    }
    if (pl.has_ak) {
      w.xk_h = c.take<uint16_t>(xb);
      w.xk_l = c.take<uint16_t>(xb);
    }
  }
  if (pl.has_aq) w.dq_part = c.take<float>(sizeof(float) * bhn * kHeadDim);
  if (pl.has_ak) w.dk_part = c.take<float>(sizeof(float) * bhn * kHeadDim);
  if (pl.has_aq || pl.has_b) w.dzq = c.take<float>(sizeof(float) * pl.zq_elems);
  if (pl.has_ak) w.dzk = c.take<float>(sizeof(float) * pl.zk_elems);
  if (pl.nchunk > 1) {
    // dK, dV summed over the chunks (fp32)
    w.dk_acc = c.take<float>(sizeof(float) * bhn * kHeadDim);
    w.dv_acc = c.take<float>(sizeof(float) * bhn * kHeadDim);
  }
  if (pl.has_aq)
    w.part_q = c.take<float>(sizeof(float) * pl.split_q * pl.ho_aq * pl.Rpad * kHeadDim);
  if (pl.has_b) w.part_qb = c.take<float>(sizeof(float) * pl.split_b * pl.ho_b * pl.Rpad);
  if (pl.has_ak)
    w.part_k = c.take<float>(sizeof(float) * pl.split_k * pl.ho_ak * pl.Rpad * kHeadDim);
  return c.off;
}

size_t zsave_bytes(const Plan& pl) {
  if (pl.nchunk > 1) return 0;  // a chunked projection is never kept
  if (pl.inblock) return 0;     // nor is there one with the in-block relation
  size_t n = 0;
  if (pl.has_aq) n += align256(sizeof(float) * pl.zq_elems);
  if (pl.has_ak) n += align256(sizeof(float) * pl.zk_elems);
  return n;
}

relpos_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return RELPOS_OK;
  return fail(RELPOS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int terms_of(const void* aQ, const void* aK, const void* b) {
  return (aQ ? RELPOS_TERM_AQ : 0) | (aK ? RELPOS_TERM_AK : 0) | (b ? RELPOS_TERM_B : 0);
}

// Map tables needed by both passes: bucket fold table (+ ranges), unfolded bias.
// Column contraction: 16-bit problems stream their dZ rows through the
// 64-row tiled kernel (grouped windows shift the loaded columns per group);
// fp32 inputs use the general kernel.
hipError_t cols(const Plan& pl, const ColsArgs& c, int Ho, hipStream_t st) {
  if (pl.esz == 2) return launch_cols1(pl.dtype, c, Ho, st);
  return launch_cols(pl.dtype, c, Ho, st);
}

relpos_status prepare_tables(const Plan& pl, const void* b, int32_t* fold, int32_t* ub,
                             int32_t* ue, float* bunf, hipStream_t st) {
  if (pl.bucketed) {
    relpos_status s = hip_check(launch_phi_fold(pl.phi, fold, ub, ue, pl.R, st), "phi fold");
    if (s != RELPOS_OK) return s;
  }
  if (bunf) {
    BiasArgs ba{b, pl.b_hs, pl.bucketed ? fold : nullptr, bunf, pl.ho_b, pl.Runf};
    relpos_status s = hip_check(launch_bias_unfold(pl.dtype, ba, st), "bias unfold");
    if (s != RELPOS_OK) return s;
  }
  return RELPOS_OK;
}

// Z^Q (query groups [g0, g0 + ngroups), into the query-side buffer laid out
// by geo) and Z^K (every key group).
relpos_status project(const Plan& pl, const relpos_problem* prob, const void* Q, const void* K,
                      const void* aQ, const void* aK, const void* b, const int32_t* fold,
                      float* zq, float* zk, hipStream_t st, const Geo& geo, int g0,
                      int ngroups) {
  if (pl.has_aq) {
    ProjArgs pa{};
    pa.x = Q;
    pa.sx = str_of(prob, RELPOS_T_Q);
    pa.tab = aQ;
    pa.tab_hs = pl.aq_hs;
    pa.bias = pl.has_b ? b : nullptr;
    pa.bias_hs = pl.b_hs;
    pa.fold = pl.bucketed ? fold : nullptr;
    pa.z = zq;
    pa.B = pl.B;
    pa.H = pl.H;
    pa.geo = geo;
    pa.key_side = 0;
    pa.ncol_tiles = pl.ncol_q;
    pa.ngroups = ngroups;
    pa.g0 = g0;
    relpos_status s = hip_check(launch_proj(pl.dtype, pa, st), "projection Q");
    if (s != RELPOS_OK) return s;
  }
  if (pl.has_ak) {
    ProjArgs pa{};
    pa.x = K;
    pa.sx = str_of(prob, RELPOS_T_K);
    pa.tab = aK;
    pa.tab_hs = pl.ak_hs;
    pa.bias = nullptr;
    pa.fold = pl.bucketed ? fold : nullptr;
    pa.z = zk;
    pa.B = pl.B;
    pa.H = pl.H;
    pa.geo = pl.geo;
    pa.key_side = 1;
    pa.ncol_tiles = pl.ncol_k;
    pa.ngroups = pl.nblk;
    relpos_status s = hip_check(launch_proj(pl.dtype, pa, st), "projection K");
    if (s != RELPOS_OK) return s;
  }
  return RELPOS_OK;
}

// Compute units of the current device, queried once per device.  The cache
// is the library's only shared state: each entry is written with the same
// value by whichever thread queries it first, through an atomic store.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Causal 16-bit launches whose blocks all fit on the device at once (two
// per CU) split each block's tiles between two wave groups: the longest
// block then bounds the pass, and splitting halves it.  With more blocks the
// longest-first order already balances the CUs.
int split_blocks(const Plan& pl, int64_t blocks) {
  return pl.geo.causal && pl.esz == 2 && blocks <= 2 * (int64_t)device_cus();
}

AttnArgs attn_args(const Plan& pl, const relpos_problem* prob, const relpos_mask* mask,
                   const void* Q, const void* K, const void* V) {
  AttnArgs a{};
  a.q = Q;
  a.k = K;
  a.v = V;
  a.key_len = mask->key_len;
  a.sq = str_of(prob, RELPOS_T_Q);
  a.sk = str_of(prob, RELPOS_T_K);
  a.sv = str_of(prob, RELPOS_T_V);
  a.so = str_of(prob, RELPOS_T_O);
  a.sdo = str_of(prob, RELPOS_T_DO);
  a.sdq = str_of(prob, RELPOS_T_DQ);
  a.sdk = str_of(prob, RELPOS_T_DK);
  a.sdv = str_of(prob, RELPOS_T_DV);
  a.B = pl.B;
  a.H = pl.H;
  a.geo = pl.geo;
  a.tau = prob->tau;
  a.scale2 = prob->tau * 1.4426950408889634f;
  a.flags = (pl.has_aq ? F_ZQ : 0) | (pl.has_ak ? F_ZK : 0) | (need_bunf(pl) ? F_B : 0) |
            (pl.keypad ? F_KEYPAD : 0) | ((pl.has_aq || pl.has_b) ? F_ZQ_NEEDED : 0);
  if (pl.drop_t > 0) {
    a.flags |= F_DROP;
    a.seed_lo = (uint32_t)(prob->dropout_seed & 0xFFFFFFFFu);
    a.seed_hi = (uint32_t)(prob->dropout_seed >> 32);
    a.drop_off = prob->dropout_offset;
    a.drop_t = (uint32_t)pl.drop_t;
    a.drop_scale = 256.f / (float)(256 - pl.drop_t);
  }
  a.bunf_hs = pl.b_hs == 0 ? 0 : pl.Runf;
  a.nblk = pl.nblk;
  a.Np = pl.Np;
  a.qb0 = 0;
  a.nqb = pl.nblk;
  a.qt0 = 0;
  a.qt1 = (pl.N + 63) / 64;  // every 64-row query tile
  a.kacc = 0;
  a.split = split_blocks(pl, (int64_t)pl.B * pl.H * pl.nblk);
  return a;
}

relpos_status check_tables(const Plan& pl, const void* aQ, const void* aK, const void* b) {
  if (aQ && !aligned16(aQ)) return fail(RELPOS_ERR_INVALID_ARG, "misaligned: aQ");
  if (aK && !aligned16(aK)) return fail(RELPOS_ERR_INVALID_ARG, "misaligned: aK");
  (void)pl;
  (void)b;
  return RELPOS_OK;
}

// Allocation-free forward: the scratch the forward needs (fold table,
// unfolded bias, the projections when no zsave buffer is given) lives in one
// file-scope device array instead of a caller workspace.  Each device that
// runs the library holds its own copy until the process ends; its address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to kernels.  Calls on one
// device share the array, so calls that overlap on one device race.
constexpr size_t kScratchBytes = RELPOS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

relpos_status scratch_address(void** out) {
  int dev = 0;
  relpos_status s = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (s != RELPOS_OK) return s;
  if (dev < 0 || dev >= kMaxDevices) return fail(RELPOS_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    s = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
    if (s != RELPOS_OK) return s;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RELPOS_OK;
}

// The forward: validation of every argument, then the stages asked for.
// With use_scratch the workspace is the library's static scratch (its
// address is looked up only once everything else has been validated).
relpos_status fwd_run(const relpos_problem* prob, const relpos_phi* phi, const relpos_mask* mask,
                      const void* Q, const void* K, const void* V, const void* aQ,
                      const void* aK, const void* b, void* O, float* lse, void* zsave,
                      void* workspace, size_t workspace_bytes, void* stream, int32_t stages,
                      bool use_scratch) {
  g_err.clear();
  if (stages & ~RELPOS_FWD_ALL) return fail(RELPOS_ERR_INVALID_ARG, "unknown forward stage bits");
  Plan pl;
  relpos_status s = make_plan(prob, phi, mask, terms_of(aQ, aK, b), pl);
  if (s != RELPOS_OK) return s;
  if (pl.B * pl.H * pl.N == 0) return RELPOS_OK;
  if ((s = check_tensor(pl, prob, RELPOS_T_Q, Q, "Q")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_K, K, "K")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_V, V, "V")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_O, O, "O")) != RELPOS_OK) return s;
  if ((s = check_tables(pl, aQ, aK, b)) != RELPOS_OK) return s;
  if (!lse || !aligned16(lse)) return fail(RELPOS_ERR_INVALID_ARG, "lse null or misaligned");
  if (zsave && !aligned16(zsave)) return fail(RELPOS_ERR_INVALID_ARG, "misaligned: zsave");
  if (zsave && pl.nchunk > 1)
    return fail(RELPOS_ERR_INVALID_ARG, "zsave must be NULL when the projection is chunked");
  if (zsave && pl.inblock)
    return fail(RELPOS_ERR_INVALID_ARG,
                "zsave must be NULL with the in-block relation (relpos_attn_zsave_size is 0)");
  WsFwd w;
  const size_t need = carve_fwd(pl, zsave != nullptr, nullptr, w);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(RELPOS_ERR_WORKSPACE,
                  "this forward needs " + std::to_string(need) +
                      " bytes of scratch, above the allocation-free limit of " +
                      std::to_string(kScratchBytes) +
                      " (pass a zsave buffer to hold the projections, or call relpos_attn_fwd)");
    if ((s = scratch_address(&workspace)) != RELPOS_OK) return s;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(RELPOS_ERR_WORKSPACE, "workspace smaller than relpos_attn_workspace_size()");
  if (workspace && !aligned16(workspace))
    return fail(RELPOS_ERR_INVALID_ARG, "misaligned: workspace");
  carve_fwd(pl, zsave != nullptr, workspace, w);
  if (zsave) {
    Carve c(zsave);
    if (pl.has_aq) w.zq = c.take<float>(sizeof(float) * pl.zq_elems);
    if (pl.has_ak) w.zk = c.take<float>(sizeof(float) * pl.zk_elems);
  }
  hipStream_t st = (hipStream_t)stream;
  // (in the block, the attention launch reads the map tables itself, so
  // they are built with it, in the same call, and there is nothing to
  // project)
  if ((stages & RELPOS_FWD_PROJECT) && !pl.inblock) {
    if ((s = prepare_tables(pl, b, w.fold, nullptr, nullptr, w.bunf, st)) != RELPOS_OK) return s;
    if (pl.nchunk == 1 &&
        (s = project(pl, prob, Q, K, aQ, aK, b, w.fold, w.zq, w.zk, st, pl.geo, 0, pl.nblk)) !=
            RELPOS_OK)
      return s;
  }
  if (!(stages & RELPOS_FWD_ATTEND)) return RELPOS_OK;
  if (pl.inblock &&
      (s = prepare_tables(pl, b, w.fold, nullptr, nullptr, w.bunf, st)) != RELPOS_OK)
    return s;
  AttnArgs a = attn_args(pl, prob, mask, Q, K, V);
  a.o_out = O;
  a.lse = lse;
  a.zq = w.zq;
  a.zk = w.zk;
  a.bunf = w.bunf;
  if (pl.inblock) {
    a.flags |= F_ZIB;
    a.tabq = aQ;
    a.tabq_hs = pl.aq_hs;
    a.tabb = b;
    a.tabb_hs = pl.b_hs;
    a.fold = pl.bucketed ? w.fold : nullptr;
    a.split = 0;  // one wave group per block
  }
  if (pl.nchunk == 1 || pl.inblock) return hip_check(launch_fwd(pl.dtype, a, st), "forward");
  // chunked projection: Z^Q of one chunk of queries, then their attention
  for (int c = 0; c < pl.nchunk; ++c) {
    Geo gc = pl.geo;
    gc.z0 = c * pl.zr;
    const int nb = (std::min(pl.zr, pl.N - gc.z0) + kBlockRows - 1) / kBlockRows;
    if ((s = project(pl, prob, Q, K, aQ, aK, b, w.fold, w.zq, w.zk, st, gc, gc.z0 / kBlockRows,
                     nb)) != RELPOS_OK)
      return s;
    a.geo = gc;
    a.qb0 = gc.z0 / kBlockRows;
    a.nqb = nb;
    a.split = split_blocks(pl, (int64_t)pl.B * pl.H * nb);
    if ((s = hip_check(launch_fwd(pl.dtype, a, st), "forward")) != RELPOS_OK) return s;
  }
  return RELPOS_OK;
}

// Backward with a chunked projection (the query-side terms only).  The map
// tables come with BWD_PREPARE; the passes (both bits) run, per chunk of zr
// queries in order: Z^Q of the chunk, the chunk's row terms, the query pass
// over its query blocks, the key pass over its query tiles (dK, dV summed in
// fp32 over the chunks, the last chunk writing the outputs), then the
// chunk's share of the contraction (dQ rows; daQ, db summed over the chunks).
relpos_status bwd_chunks(const Plan& pl, const relpos_problem* prob, int32_t stages,
                         const void* Q, const void* K, const void* aQ, const void* b,
                         const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                         void* dV, float* daQ, float* db, const WsBwd& w, AttnArgs a,
                         hipStream_t st) {
  (void)K;
  (void)dK;
  (void)dV;
  relpos_status s;
  if (stages & RELPOS_BWD_PREPARE) {
    if ((s = prepare_tables(pl, b, w.fold, w.ub, w.ue, w.bunf, st)) != RELPOS_OK) return s;
  }
  if (!(stages & RELPOS_BWD_QUERY_PASS)) return RELPOS_OK;
  const int64_t tu_hs = (int64_t)(pl.Runf + 32) * kHeadDim;
  void* tunf_lo = nullptr;
  if (pl.has_aq) {
    tunf_lo = pl.dtype == 1 ? (void*)((uint16_t*)w.tunf_q + (size_t)pl.ho_aq * tu_hs) : nullptr;
    TabUnfoldArgs t{aQ, pl.aq_hs, pl.bucketed ? w.fold : nullptr, w.tunf_q, tunf_lo, pl.ho_aq,
                    pl.Runf};
    if ((s = hip_check(launch_tab_unfold(pl.dtype, t, st), "table unfold aQ")) != RELPOS_OK)
      return s;
    if (pl.dtype == 1) {
      SplitArgs x{Q, str_of(prob, RELPOS_T_Q), w.xq_h, w.xq_l, pl.B, pl.H, pl.N};
      if ((s = hip_check(launch_xsplit(x, st), "split Q")) != RELPOS_OK) return s;
    }
  }
  const float dseed_scale = pl.drop_t > 0 ? (float)(256 - pl.drop_t) / 256.f : 1.f;
  const int32_t* ub = pl.bucketed ? w.ub : nullptr;
  const int32_t* ue = pl.bucketed ? w.ue : nullptr;
  const bool joint_b = pl.has_aq && pl.has_b && pl.ho_aq == pl.ho_b && pl.split_q == pl.split_b;
  a.dk_acc = w.dk_acc;
  a.dv_acc = w.dv_acc;
  for (int c = 0; c < pl.nchunk; ++c) {
    Geo gc = pl.geo;
    gc.z0 = c * pl.zr;
    const int rows = std::min(pl.zr, pl.N - gc.z0);
    const int nb = (rows + kBlockRows - 1) / kBlockRows;
    const int rb0 = gc.z0 / kBlockRows;
    if (pl.has_aq &&
        (s = project(pl, prob, Q, K, aQ, nullptr, b, w.fold, w.zq, nullptr, st, gc, rb0, nb)) !=
            RELPOS_OK)
      return s;
    RowTermArgs r{O,    dO,   str_of(prob, RELPOS_T_O), str_of(prob, RELPOS_T_DO), lse,
                  w.L2, w.D,  w.kseed, dseed_scale, w.zq, gc,
                  prob->tau * 1.4426950408889634f, pl.B, pl.H, pl.N, pl.Np,
                  gc.z0, std::min(gc.z0 + pl.zr, pl.Np)};
    if ((s = hip_check(launch_rowterm(pl.dtype, r, st), "backward (row terms)")) != RELPOS_OK)
      return s;
    a.geo = gc;
    a.qb0 = rb0;
    a.nqb = nb;
    a.split = split_blocks(pl, (int64_t)pl.B * pl.H * nb);
    auto launch_passes = [&](bool q, bool k) {
      return pl.dtype == 0   ? launch_bwd_f32(a, q, k, st)
             : pl.dtype == 1 ? launch_bwd_f16(a, q, k, st)
                             : launch_bwd_bf16(a, q, k, st);
    };
    if ((s = hip_check(launch_passes(true, false), "backward (query pass)")) != RELPOS_OK)
      return s;
    a.qt0 = gc.z0 / 64;
    a.qt1 = (gc.z0 + rows + 63) / 64;
    a.kacc = (c > 0 ? 1 : 0) | (c + 1 < pl.nchunk ? 2 : 0);
    a.split = split_blocks(pl, (int64_t)pl.B * pl.H * pl.nblk);
    if ((s = hip_check(launch_passes(false, true), "backward (key pass)")) != RELPOS_OK) return s;
    // this chunk's contraction: dQ rows, then its share of daQ and db
    if (pl.has_aq) {
      RowsArgs ra{w.dq_part, w.dzq, w.tunf_q, tunf_lo, pl.aq_hs == 0 ? 0 : tu_hs, dQ,
                  str_of(prob, RELPOS_T_DQ), pl.B, pl.H, gc, 0, nb, rb0};
      if ((s = hip_check(launch_rows(pl.dtype, ra, st), "contraction dQ")) != RELPOS_OK) return s;
      ColsArgs cq{};
      cq.dz = w.dzq;
      cq.x = Q;
      cq.xh = w.xq_h;
      cq.xl = w.xq_l;
      cq.sx = str_of(prob, RELPOS_T_Q);
      cq.part = w.part_q;
      cq.partb = joint_b ? w.part_qb : nullptr;
      cq.B = pl.B;
      cq.H = pl.H;
      cq.geo = gc;
      cq.key_side = 0;
      cq.shared = pl.aq_hs == 0;
      cq.splits = pl.split_q;
      cq.rtiles = pl.rtiles;
      cq.Rpad = pl.Rpad;
      cq.want_x = 1;
      if ((s = hip_check(cols(pl, cq, pl.ho_aq, st), "contraction daQ")) != RELPOS_OK) return s;
      FoldArgs f{w.part_q, joint_b ? w.part_qb : nullptr, ub, ue, daQ, joint_b ? db : nullptr,
                 pl.ho_aq, pl.R, pl.Rpad, pl.split_q, c > 0 ? 1 : 0};
      if ((s = hip_check(launch_fold(f, st), "fold daQ")) != RELPOS_OK) return s;
    }
    if (pl.has_b && !joint_b) {
      ColsArgs cb{};
      cb.dz = w.dzq;
      cb.x = Q;
      cb.sx = str_of(prob, RELPOS_T_Q);
      cb.part = nullptr;
      cb.partb = w.part_qb;
      cb.B = pl.B;
      cb.H = pl.H;
      cb.geo = gc;
      cb.key_side = 0;
      cb.shared = pl.b_hs == 0;
      cb.splits = pl.split_b;
      cb.rtiles = pl.rtiles;
      cb.Rpad = pl.Rpad;
      cb.want_x = 0;
      if ((s = hip_check(cols(pl, cb, pl.ho_b, st), "contraction db")) != RELPOS_OK) return s;
      FoldArgs f{nullptr, w.part_qb, ub, ue, nullptr, db, pl.ho_b, pl.R, pl.Rpad, pl.split_b,
                 c > 0 ? 1 : 0};
      if ((s = hip_check(launch_fold(f, st), "fold db")) != RELPOS_OK) return s;
    }
  }
  return RELPOS_OK;
}

}  // namespace

extern "C" {

const char* relpos_status_string(int32_t status) {
  switch (status) {
    case RELPOS_OK: return "RELPOS_OK";
    case RELPOS_ERR_INVALID_ARG: return "RELPOS_ERR_INVALID_ARG";
    case RELPOS_ERR_UNSUPPORTED: return "RELPOS_ERR_UNSUPPORTED";
    case RELPOS_ERR_WORKSPACE: return "RELPOS_ERR_WORKSPACE";
    case RELPOS_ERR_HIP: return "RELPOS_ERR_HIP";
    default: return "RELPOS_UNKNOWN_STATUS";
  }
}

const char* relpos_last_error(void) { return g_err.c_str(); }

relpos_status relpos_phi_info(const relpos_phi* phi, int64_t N, int64_t* R, int64_t* lo_unf,
                              int64_t* hi_unf) {
  g_err.clear();
  if (!phi || !R || !lo_unf || !hi_unf) return fail(RELPOS_ERR_INVALID_ARG, "null argument");
  if (N < 1 || N > kMaxN) return fail(RELPOS_ERR_INVALID_ARG, "N must be in [1, 1048576]");
  return unfold_range(*phi, N, *R, *lo_unf, *hi_unf);
}

relpos_status relpos_phi_rows(const relpos_phi* phi, int64_t N, int32_t* rows, int32_t* fold,
                              void* stream) {
  g_err.clear();
  if (!phi) return fail(RELPOS_ERR_INVALID_ARG, "null phi");
  if (N < 1 || N > kMaxN) return fail(RELPOS_ERR_INVALID_ARG, "N must be in [1, 1048576]");
  int64_t R, lo, hi;
  relpos_status s = unfold_range(*phi, N, R, lo, hi);
  if (s != RELPOS_OK) return s;
  PhiArgs p{};
  p.kind = phi->kind;
  p.N = (int)N;
  p.lo_unf = (int)lo;
  p.hi_unf = (int)hi;
  p.num_buckets = phi->num_buckets;
  p.max_exact = phi->max_exact;
  p.max_distance = phi->max_distance;
  p.bidirectional = phi->bidirectional ? 1 : 0;
  p.lo = phi->lo;
  p.hi = phi->hi;
  hipStream_t st = (hipStream_t)stream;
  if (rows) {
    s = hip_check(launch_phi_rows(p, rows, st), "phi rows");
    if (s != RELPOS_OK) return s;
  }
  if (fold) {
    s = hip_check(launch_phi_fold(p, fold, nullptr, nullptr, (int)R, st), "phi fold");
    if (s != RELPOS_OK) return s;
  }
  return RELPOS_OK;
}

relpos_status relpos_attn_zsave_size(const relpos_problem* prob, const relpos_phi* phi,
                                     int32_t terms, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(RELPOS_ERR_INVALID_ARG, "null bytes");
  relpos_mask m{0, nullptr};
  Plan pl;
  relpos_status s = make_plan(prob, phi, &m, terms, pl);
  if (s != RELPOS_OK) return s;
  *bytes = zsave_bytes(pl);
  return RELPOS_OK;
}

relpos_status relpos_attn_workspace_size(const relpos_problem* prob, const relpos_phi* phi,
                                         const relpos_mask* mask, int32_t terms, int32_t pass,
                                         int32_t zsave_given, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(RELPOS_ERR_INVALID_ARG, "null bytes");
  if (pass != RELPOS_PASS_FWD && pass != RELPOS_PASS_BWD)
    return fail(RELPOS_ERR_INVALID_ARG, "unknown pass");
  Plan pl;
  relpos_status s = make_plan(prob, phi, mask, terms, pl);
  if (s != RELPOS_OK) return s;
  if (pass == RELPOS_PASS_FWD) {
    WsFwd w;
    *bytes = carve_fwd(pl, zsave_given != 0, nullptr, w);
  } else {
    WsBwd w;
    *bytes = carve_bwd(pl, zsave_given != 0, nullptr, w);
  }
  return RELPOS_OK;
}

relpos_status relpos_attn_fwd_stages(const relpos_problem* prob, const relpos_phi* phi,
                                     const relpos_mask* mask, const void* Q, const void* K,
                                     const void* V, const void* aQ, const void* aK, const void* b,
                                     void* O, float* lse, void* zsave, void* workspace,
                                     size_t workspace_bytes, void* stream, int32_t stages) {
  return fwd_run(prob, phi, mask, Q, K, V, aQ, aK, b, O, lse, zsave, workspace, workspace_bytes,
                 stream, stages, false);
}

relpos_status relpos_attn_fwd(const relpos_problem* prob, const relpos_phi* phi,
                              const relpos_mask* mask, const void* Q, const void* K, const void* V,
                              const void* aQ, const void* aK, const void* b, void* O, float* lse,
                              void* zsave, void* workspace, size_t workspace_bytes, void* stream) {
  return relpos_attn_fwd_stages(prob, phi, mask, Q, K, V, aQ, aK, b, O, lse, zsave, workspace,
                                workspace_bytes, stream, RELPOS_FWD_ALL);
}

relpos_status relpos_attn_fwd_noalloc(const relpos_problem* prob, const relpos_phi* phi,
                                      const relpos_mask* mask, const void* Q, const void* K,
                                      const void* V, const void* aQ, const void* aK,
                                      const void* b, void* O, float* lse, void* zsave,
                                      void* stream) {
  return fwd_run(prob, phi, mask, Q, K, V, aQ, aK, b, O, lse, zsave, nullptr, 0, stream,
                 RELPOS_FWD_ALL, true);
}

relpos_status relpos_attn_bwd_stages(const relpos_problem* prob, const relpos_phi* phi,
                                     const relpos_mask* mask, const void* Q, const void* K,
                                     const void* V, const void* aQ, const void* aK, const void* b,
                                     const void* O, const float* lse, const void* dO,
                                     const void* zsave, void* dQ, void* dK, void* dV, float* daQ,
                                     float* daK, float* db, void* workspace,
                                     size_t workspace_bytes, void* stream, int32_t stages) {
  g_err.clear();
  if (stages & ~RELPOS_BWD_ALL) return fail(RELPOS_ERR_INVALID_ARG, "unknown backward stage bits");
  Plan pl;
  relpos_status s = make_plan(prob, phi, mask, terms_of(aQ, aK, b), pl);
  if (s != RELPOS_OK) return s;
  if ((aQ == nullptr) != (daQ == nullptr))
    return fail(RELPOS_ERR_INVALID_ARG, "daQ must be given exactly when aQ is");
  if ((aK == nullptr) != (daK == nullptr))
    return fail(RELPOS_ERR_INVALID_ARG, "daK must be given exactly when aK is");
  if ((b == nullptr) != (db == nullptr))
    return fail(RELPOS_ERR_INVALID_ARG, "db must be given exactly when b is");
  hipStream_t st = (hipStream_t)stream;
  if (pl.B * pl.H * pl.N == 0) {
    if (!(stages & RELPOS_BWD_CONTRACT)) return RELPOS_OK;
    // no token pairs: the table gradients are zero (an identity map at N = 0 has no rows)
    const int Rout = (phi->kind == RELPOS_PHI_IDENTITY && pl.N == 0) ? 0 : pl.R;
    if (daQ) {
      FoldArgs f{nullptr, nullptr, nullptr, nullptr, daQ, nullptr, pl.ho_aq, Rout, pl.Rpad, 0};
      if ((s = hip_check(launch_fold(f, st), "zero daQ")) != RELPOS_OK) return s;
    }
    if (daK) {
      FoldArgs f{nullptr, nullptr, nullptr, nullptr, daK, nullptr, pl.ho_ak, Rout, pl.Rpad, 0};
      if ((s = hip_check(launch_fold(f, st), "zero daK")) != RELPOS_OK) return s;
    }
    if (db) {
      FoldArgs f{nullptr, nullptr, nullptr, nullptr, nullptr, db, pl.ho_b, Rout, pl.Rpad, 0};
      if ((s = hip_check(launch_fold(f, st), "zero db")) != RELPOS_OK) return s;
    }
    return RELPOS_OK;
  }
  if ((s = check_tensor(pl, prob, RELPOS_T_Q, Q, "Q")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_K, K, "K")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_V, V, "V")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_O, O, "O")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_DO, dO, "dO")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_DQ, dQ, "dQ")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_DK, dK, "dK")) != RELPOS_OK) return s;
  if ((s = check_tensor(pl, prob, RELPOS_T_DV, dV, "dV")) != RELPOS_OK) return s;
  if ((s = check_tables(pl, aQ, aK, b)) != RELPOS_OK) return s;
  if (!lse) return fail(RELPOS_ERR_INVALID_ARG, "null lse");
  WsBwd w;
  const size_t need = carve_bwd(pl, zsave != nullptr, nullptr, w);
  if (!workspace || workspace_bytes < need)
    return fail(RELPOS_ERR_WORKSPACE, "workspace smaller than relpos_attn_workspace_size()");
  if (!aligned16(workspace)) return fail(RELPOS_ERR_INVALID_ARG, "misaligned: workspace");
  if (zsave && !aligned16(zsave)) return fail(RELPOS_ERR_INVALID_ARG, "misaligned: zsave");
  if (zsave && pl.nchunk > 1)
    return fail(RELPOS_ERR_INVALID_ARG, "zsave must be NULL when the projection is chunked");
  if (pl.nchunk > 1 && (stages & (RELPOS_BWD_QUERY_PASS | RELPOS_BWD_KEY_PASS)) &&
      (stages & (RELPOS_BWD_QUERY_PASS | RELPOS_BWD_KEY_PASS)) !=
          (RELPOS_BWD_QUERY_PASS | RELPOS_BWD_KEY_PASS))
    return fail(RELPOS_ERR_INVALID_ARG, "a chunked backward runs both passes together");
  if (zsave && pl.inblock)
    return fail(RELPOS_ERR_INVALID_ARG,
                "zsave must be NULL with the in-block relation (the forward keeps no projection)");
  carve_bwd(pl, zsave != nullptr, workspace, w);
  if (zsave) {
    Carve c(const_cast<void*>(zsave));
    if (pl.has_aq) w.zq = c.take<float>(sizeof(float) * pl.zq_elems);
    if (pl.has_ak) w.zk = c.take<float>(sizeof(float) * pl.zk_elems);
  }

  if (stages & RELPOS_BWD_PREPARE) {
    if ((s = prepare_tables(pl, b, w.fold, w.ub, w.ue, w.bunf, st)) != RELPOS_OK) return s;
    if (!zsave && pl.nchunk == 1) {
      if ((s = project(pl, prob, Q, K, aQ, aK, b, w.fold, w.zq, w.zk, st, pl.geo, 0, pl.nblk)) !=
        RELPOS_OK)
      return s;
    }
  }

  AttnArgs a = attn_args(pl, prob, mask, Q, K, V);
  a.o = O;
  a.lse = const_cast<float*>(lse);
  a.dO = dO;
  a.L2 = w.L2;
  a.D = w.D;
  a.kseed = w.kseed;
  a.zq = w.zq;
  a.zk = w.zk;
  a.bunf = w.bunf;
  a.dq = pl.has_aq ? (void*)w.dq_part : dQ;
  a.dk = pl.has_ak ? (void*)w.dk_part : dK;
  a.dv = dV;
  a.dzq = w.dzq;
  a.dzk = w.dzk;
  if (pl.nchunk > 1)
    return bwd_chunks(pl, prob, stages, Q, K, aQ, b, O, lse, dO, dQ, dK, dV, daQ, db, w, a, st);
  if (stages & RELPOS_BWD_PREPARE) {
    const float dseed_scale = pl.drop_t > 0 ? (float)(256 - pl.drop_t) / 256.f : 1.f;
    RowTermArgs r{O,      dO,    str_of(prob, RELPOS_T_O), str_of(prob, RELPOS_T_DO), lse,
                  w.L2,   w.D,   w.kseed, dseed_scale, w.zq, pl.geo,
                  prob->tau * 1.4426950408889634f, pl.B, pl.H, pl.N, pl.Np, 0, pl.Np};
    if ((s = hip_check(launch_rowterm(pl.dtype, r, st), "backward (row terms)")) != RELPOS_OK)
      return s;
  }
  // The query and key passes share one launch when both are asked for: a
  // pass alone may end with a partly filled last round of blocks, the two
  // together fill it.  Problems that split their blocks between two wave
  // groups (a.split: every block of a pass fits on the device at once, so
  // the longest block bounds the pass) gain nothing from that and run the
  // passes one after the other.
  const bool want_q = stages & RELPOS_BWD_QUERY_PASS, want_k = stages & RELPOS_BWD_KEY_PASS;
  auto launch_passes = [&](bool q, bool k) {
    return pl.dtype == 0   ? launch_bwd_f32(a, q, k, st)
           : pl.dtype == 1 ? launch_bwd_f16(a, q, k, st)
                           : launch_bwd_bf16(a, q, k, st);
  };
  if (want_q && want_k && a.split) {
    if ((s = hip_check(launch_passes(true, false), "backward (query pass)")) != RELPOS_OK)
      return s;
    if ((s = hip_check(launch_passes(false, true), "backward (key pass)")) != RELPOS_OK) return s;
  } else if (want_q || want_k) {
    if ((s = hip_check(launch_passes(want_q, want_k), "backward (query and key passes)")) !=
        RELPOS_OK)
      return s;
  }
  if (!(stages & RELPOS_BWD_CONTRACT)) return RELPOS_OK;

  // dQ += dZ^Q aQ, dK += dZ^K aK
  const int64_t tu_hs = (int64_t)(pl.Runf + 32) * kHeadDim;
  // low bf16 part of an fp16 table: after the high part, in the same bytes
  auto tab_lo = [&](float* t, int ho) -> void* {
    return pl.dtype == 1 ? (void*)((uint16_t*)t + (size_t)ho * tu_hs) : nullptr;
  };
  if (pl.has_aq) {
    TabUnfoldArgs t{aQ, pl.aq_hs, pl.bucketed ? w.fold : nullptr, w.tunf_q, tab_lo(w.tunf_q, pl.ho_aq),
                    pl.ho_aq, pl.Runf};
    if ((s = hip_check(launch_tab_unfold(pl.dtype, t, st), "table unfold aQ")) != RELPOS_OK)
      return s;
    RowsArgs r{w.dq_part, w.dzq, w.tunf_q, t.out_lo, pl.aq_hs == 0 ? 0 : tu_hs, dQ,
               str_of(prob, RELPOS_T_DQ), pl.B, pl.H, pl.geo, 0, pl.nblk};
    if ((s = hip_check(launch_rows(pl.dtype, r, st), "contraction dQ")) != RELPOS_OK) return s;
  }
  if (pl.has_ak) {
    TabUnfoldArgs t{aK, pl.ak_hs, pl.bucketed ? w.fold : nullptr, w.tunf_k, tab_lo(w.tunf_k, pl.ho_ak),
                    pl.ho_ak, pl.Runf};
    if ((s = hip_check(launch_tab_unfold(pl.dtype, t, st), "table unfold aK")) != RELPOS_OK)
      return s;
    RowsArgs r{w.dk_part, w.dzk, w.tunf_k, t.out_lo, pl.ak_hs == 0 ? 0 : tu_hs, dK,
               str_of(prob, RELPOS_T_DK), pl.B, pl.H, pl.geo, 1, pl.nblk};
    if ((s = hip_check(launch_rows(pl.dtype, r, st), "contraction dK")) != RELPOS_OK) return s;
  }
  // fp16 Q / K as two exact bf16 parts for the column contraction
  if (pl.dtype == 1 && pl.has_aq) {
    SplitArgs x{Q, str_of(prob, RELPOS_T_Q), w.xq_h, w.xq_l, pl.B, pl.H, pl.N};
    if ((s = hip_check(launch_xsplit(x, st), "split Q")) != RELPOS_OK) return s;
  }
  if (pl.dtype == 1 && pl.has_ak) {
    SplitArgs x{K, str_of(prob, RELPOS_T_K), w.xk_h, w.xk_l, pl.B, pl.H, pl.N};
    if ((s = hip_check(launch_xsplit(x, st), "split K")) != RELPOS_OK) return s;
  }
  // table gradients: dZ^T Q, dZ^T K, column sums of dZ^Q; then the fold
  const int32_t* ub = pl.bucketed ? w.ub : nullptr;
  const int32_t* ue = pl.bucketed ? w.ue : nullptr;
  const bool joint_b = pl.has_aq && pl.has_b && pl.ho_aq == pl.ho_b && pl.split_q == pl.split_b;
  if (pl.has_aq) {
    ColsArgs c{};
    c.dz = w.dzq;
    c.x = Q;
    c.xh = w.xq_h;
    c.xl = w.xq_l;
    c.sx = str_of(prob, RELPOS_T_Q);
    c.part = w.part_q;
    c.partb = joint_b ? w.part_qb : nullptr;
    c.B = pl.B;
    c.H = pl.H;
    c.geo = pl.geo;
    c.key_side = 0;
    c.shared = pl.aq_hs == 0;
    c.splits = pl.split_q;
    c.rtiles = pl.rtiles;
    c.Rpad = pl.Rpad;
    c.want_x = 1;
    if ((s = hip_check(cols(pl, c, pl.ho_aq, st), "contraction daQ")) != RELPOS_OK)
      return s;
    FoldArgs f{w.part_q, joint_b ? w.part_qb : nullptr, ub, ue, daQ, joint_b ? db : nullptr,
               pl.ho_aq, pl.R, pl.Rpad, pl.split_q};
    if ((s = hip_check(launch_fold(f, st), "fold daQ")) != RELPOS_OK) return s;
  }
  if (pl.has_b && !joint_b) {
    ColsArgs c{};
    c.dz = w.dzq;
    c.x = Q;
    c.sx = str_of(prob, RELPOS_T_Q);
    c.part = nullptr;
    c.partb = w.part_qb;
    c.B = pl.B;
    c.H = pl.H;
    c.geo = pl.geo;
    c.key_side = 0;
    c.shared = pl.b_hs == 0;
    c.splits = pl.split_b;
    c.rtiles = pl.rtiles;
    c.Rpad = pl.Rpad;
    c.want_x = 0;
    if ((s = hip_check(cols(pl, c, pl.ho_b, st), "contraction db")) != RELPOS_OK)
      return s;
    FoldArgs f{nullptr, w.part_qb, ub, ue, nullptr, db, pl.ho_b, pl.R, pl.Rpad, pl.split_b};
    if ((s = hip_check(launch_fold(f, st), "fold db")) != RELPOS_OK) return s;
  }
  if (pl.has_ak) {
    ColsArgs c{};
    c.dz = w.dzk;
    c.x = K;
    c.xh = w.xk_h;
    c.xl = w.xk_l;
    c.sx = str_of(prob, RELPOS_T_K);
    c.part = w.part_k;
    c.partb = nullptr;
    c.B = pl.B;
    c.H = pl.H;
    c.geo = pl.geo;
    c.key_side = 1;
    c.shared = pl.ak_hs == 0;
    c.splits = pl.split_k;
    c.rtiles = pl.rtiles;
    c.Rpad = pl.Rpad;
    c.want_x = 1;
    if ((s = hip_check(cols(pl, c, pl.ho_ak, st), "contraction daK")) != RELPOS_OK)
      return s;
    FoldArgs f{w.part_k, nullptr, ub, ue, daK, nullptr, pl.ho_ak, pl.R, pl.Rpad, pl.split_k};
    if ((s = hip_check(launch_fold(f, st), "fold daK")) != RELPOS_OK) return s;
  }
  return RELPOS_OK;
}

relpos_status relpos_attn_bwd(const relpos_problem* prob, const relpos_phi* phi,
                              const relpos_mask* mask, const void* Q, const void* K, const void* V,
                              const void* aQ, const void* aK, const void* b, const void* O,
                              const float* lse, const void* dO, const void* zsave, void* dQ,
                              void* dK, void* dV, float* daQ, float* daK, float* db,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return relpos_attn_bwd_stages(prob, phi, mask, Q, K, V, aQ, aK, b, O, lse, dO, zsave, dQ, dK,
                                dV, daQ, daK, db, workspace, workspace_bytes, stream,
                                RELPOS_BWD_ALL);
}

}  // extern "C"
