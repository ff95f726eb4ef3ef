// geometry.hpp -- offset-map geometry shared by the host dispatcher and the
// kernels: the unfolded truncated map, the reachable offset windows of the
// relation projections, and the kernel argument blocks.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest):
//  * every map is handled as a truncated map r(o) = clip(o, lo, hi) - lo
//    (section on constant tiles: bucketed maps are unfolded to this form;
//    the identity map is the truncation at +-(N-1));
//  * section on the grouped reachable range: G consecutive queries reach a
//    contiguous range of at most N + G - 1 offsets, so only that window of the
//    projection is computed; G = 128 equals the largest block, so a query
//    block lies in one group; when the table is shorter than the window a
//    single group covers everything.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define RP_HD __host__ __device__ inline
#else
#define RP_HD inline
#endif

namespace relpos {

constexpr int kGroup = 128;   // G: query/key group = largest block
constexpr int kHeadDim = 64;  // d
constexpr int kBlockRows = kGroup;  // rows owned by a workgroup (4 waves x 32)
// Window width from which a band counts as wide (see wide_band).
constexpr int kWideW = 1024;

struct Geo {
  int N;       // sequence length
  int lo, hi;  // unfolded truncated map
  int R;       // rows of the unfolded map = hi - lo + 1
  int W;       // projection window width (= R for a single group, else N + G - 1)
  int Wp;      // row stride of the Z / dZ buffers: W rounded up to 32 floats (128 B)
  int causal;  // 1 if j > i is masked
  // The query-side buffers Z^Q and dZ^Q hold the query rows [z0, z0 + zr)
  // of each (b, h), zr rows per (b, h): the whole sequence (z0 = 0, zr = N)
  // unless the projection is computed one chunk of queries at a time.  The
  // key-side buffers always hold every key row.
  int zr, z0;
  // Column shift mask of the rows of dZ^Q (see dz_shift): 31 (rows shifted)
  // or 0 (unshifted).
  int dsm;
};

RP_HD int imin(int a, int b) { return a < b ? a : b; }
RP_HD int imax(int a, int b) { return a > b ? a : b; }

// Unfolded row of offset o = j - i.
RP_HD int rrow(const Geo& g, int o) { return imin(imax(o, g.lo), g.hi) - g.lo; }

RP_HD bool grouped(const Geo& g) { return g.W < g.R; }

// Whether most key tiles of a query row are band tiles: a window of kWideW
// columns or more (the identity map), or a sequence no longer than the
// window (short sequences).  Then the lane = query kernels stage the band
// rows of Z^Q through LDS instead of gathering them per score, and the rows
// of dZ^Q are stored shifted (dz_shift); narrower bands, where only a few
// tiles per row are band tiles, gather.
RP_HD bool wide_band(const Geo& g) { return g.W >= kWideW || g.W >= g.N; }

// Float offset of query row i of (b, h) in the query-side Z / dZ buffers
// (rows outside [z0, z0 + zr) are not held).
RP_HD int64_t zq_off(const Geo& g, int64_t bh, int i) {
  return (bh * g.zr + (i - g.z0)) * (int64_t)g.Wp;
}
// Last query row the query-side buffers hold (the clamp of rows beyond N).
RP_HD int zq_last(const Geo& g) { return imin(g.N, g.z0 + g.zr) - 1; }

// Row pitch of the Z / dZ buffers for a window of w columns: w rounded up to
// 32 floats (128 bytes), plus 32 floats of slack when the rows of dZ^Q are
// shifted (see dz_shift).
RP_HD int z_pitch(int w, bool shifted) { return (w + 31) / 32 * 32 + (shifted ? 32 : 0); }
// Columns of a row below which every access, shifted, stays inside the row.
RP_HD int z_span(const Geo& g) { return g.dsm ? g.Wp - 32 : g.Wp; }

// First unfolded row stored for query group `grp` (window [ws, ws + W)).
RP_HD int win_q(const Geo& g, int grp) {
  if (!grouped(g)) return 0;
  int s = rrow(g, -(grp * kGroup + kGroup - 1));
  return imin(s, g.R - g.W);
}
// Column shift of query row i in the storage of dZ^Q: window column c of the
// row sits at storage column c + dz_shift(g, i).  The band run of row i
// against the 32 keys [jb, jb + 32) starts at window column jb - i - lo - ws
// (ws the row group's window start); adding (i + lo + ws) mod 32 turns that
// into jb minus a multiple of 32, so with jb a multiple of 32 every such run
// fills whole 128-byte lines, and the query pass writes whole lines
// (unshifted, the runs of most rows straddle two lines and their halves are
// written at different times).  Z^Q and the key-side buffers are not
// shifted: their band runs are read, and a read of two half lines costs
// less than the projection would pay to write shifted rows.
RP_HD int dz_shift(const Geo& g, int i) {
  const int ws = grouped(g) ? win_q(g, i / kGroup) : 0;
  return (i + g.lo + ws) & g.dsm;
}

// First unfolded row stored for key group `grp`.
RP_HD int win_k(const Geo& g, int grp) {
  if (!grouped(g)) return 0;
  int s = rrow(g, grp * kGroup - (g.N - 1));
  return imin(s, g.R - g.W);
}

// Window columns [cb, ce) that can hold a live entry for some query of group
// `grp` (all queries when ungrouped): offsets from -(last query) to
// N-1-(first query), and not beyond 0 when causal.
RP_HD void cols_q(const Geo& g, int grp, int& cb, int& ce) {
  int first = grouped(g) ? grp * kGroup : 0;
  int last = grouped(g) ? imin(g.N - 1, grp * kGroup + kGroup - 1) : g.N - 1;
  int omin = -last, omax = g.N - 1 - first;
  if (g.causal) omax = imin(omax, 0);
  int ws = win_q(g, grp);
  cb = imax(0, rrow(g, omin) - ws);
  ce = imin(g.W, rrow(g, omax) - ws + 1);
}
// Same for key group `grp`: offsets from (first key)-(N-1) to (last key).
RP_HD void cols_k(const Geo& g, int grp, int& cb, int& ce) {
  int first = grouped(g) ? grp * kGroup : 0;
  int last = grouped(g) ? imin(g.N - 1, grp * kGroup + kGroup - 1) : g.N - 1;
  int omin = first - (g.N - 1), omax = last;
  if (g.causal) omax = imin(omax, 0);
  int ws = win_k(g, grp);
  cb = imax(0, rrow(g, omin) - ws);
  ce = imin(g.W, rrow(g, omax) - ws + 1);
}

enum : int {
  F_ZQ = 1, F_ZK = 2, F_B = 4, F_KEYPAD = 8, F_ZQ_NEEDED = 16, F_DROP = 32,
  F_ZIB = 64  // forward: the query-side relation computed in the block (no Z^Q)
};

// Strides of a [B, H, N, d] tensor in elements.
struct Str {
  int64_t b, h, n;
};

// Map kernel (tables + projection) ------------------------------------------
struct PhiArgs {
  int kind;  // relpos_phi_kind
  int N;
  int lo_unf, hi_unf;
  int num_buckets, max_exact, max_distance, bidirectional;
  int lo, hi;  // truncated map parameters (kind 0)
};

struct ProjArgs {
  const void* x;       // Q or K
  Str sx;
  const void* tab;     // aQ or aK
  int64_t tab_hs;      // table head stride (elements)
  const void* bias;    // b folded into the projection (query side only), or null
  int64_t bias_hs;
  const int32_t* fold; // unfolded row -> table row, or null (identity)
  float* z;            // [B*H][N][W]
  int B, H;
  Geo geo;
  int key_side;        // 0: query windows, 1: key windows
  int ncol_tiles;      // 64-column tiles per group launched
  int ngroups;         // groups per (b, h) launched
  int g0;              // first group launched
};

// Attention kernels -----------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;   // forward output (backward reads it only through D)
  void* o_out;     // forward output pointer
  float* lse;      // [B*H][N]
  const void* dO;
  const float* L2; // [B*H][Np] padded log2-domain LSE (backward)
  const float* D;  // [B*H][Np] padded row terms (backward)
  const float* kseed;  // [4][B*H][Np] per-query seeds of the key pass (RowTermArgs)
  int Np;          // N rounded up to 64
  const float* zq; // [B*H][N][W] or null
  const float* zk;
  const float* bunf;  // [Hb][R] fp32 unfolded scalar bias, or null
  int64_t bunf_hs;
  // F_ZIB: the tables themselves (input dtype), their head strides in
  // elements, and the fold table of a bucketed map (or null)
  const void* tabq;
  int64_t tabq_hs;
  const void* tabb;
  int64_t tabb_hs;
  const int32_t* fold;
  const int32_t* key_len;
  void* dq;        // output (dtype) or fp32 partial when F_ZQ
  void* dk;
  void* dv;
  float* dzq;      // [B*H][N][W]
  float* dzk;
  Str sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H;
  Geo geo;
  float tau;
  float scale2;    // tau * log2(e)
  int flags;
  int nblk;        // blocks per (b, h) along the parallel dimension
  int split;       // causal launches: two wave groups per block split its tiles
  // attention dropout (F_DROP): Philox key, counter word 3, threshold t
  // (drop probability t / 256) and 1 / (1 - p)
  uint32_t seed_lo, seed_hi, drop_off, drop_t;
  float drop_scale;
  // Launch ranges: the forward and the query pass take the query blocks
  // [qb0, qb0 + nqb) of every (b, h); the key pass takes the query tiles
  // [qt0, qt1) (64 rows each).  The key pass accumulates across launches
  // when kacc is set: bit 0 adds the fp32 sums in dk_acc / dv_acc ([B*H][N][64],
  // dK carrying its tau) before writing, bit 1 writes those sums instead of
  // the outputs.
  int qb0, nqb, qt0, qt1, kacc;
  float* dk_acc;
  float* dv_acc;
};

struct RowTermArgs {     // padded backward row terms
  const void* o;
  const void* dO;
  Str so, sdo;
  const float* lse;      // [B*H][N]
  float* L2;             // [B*H][Np]  LSE * log2(e), +inf for dead and padded rows
  float* D;              // [B*H][Np]  sum_d dO O, 0 for padded rows
  // Seeds of the key pass's MFMA accumulators, [4][B*H][Np], in units of the
  // score before the tau * log2(e) scale:
  //  0 / 1: Z^Q[i, first / last row] - L2 / (tau log2 e)  (saturated tiles)
  //  2:     -L2 / (tau log2 e)                              (band tiles)
  //  3:     -D (-D (1 - p) under attention dropout)
  float* kseed;
  float dseed_scale;     // multiplies -D in seed 3 (1 - p under dropout, else 1)
  const float* zq;       // query-side Z buffer (rows of geo) or null
  Geo geo;
  float scale2;          // tau * log2(e)
  int B, H, N, Np;
  int r0, r1;            // rows [r0, r1) of each (b, h) are prepared
};

struct RowsArgs {       // dX = part + dZ . table   (per row)
  const float* part;    // [B*H][N][64] fp32
  const float* dz;      // [B*H][N][Wp] (query side: the rows of geo)
  const void* tunf;     // [Ho][Runf + 32][64] unfolded table: fp32 for fp32 inputs,
                        // else its bf16 high part
  const void* tunf_lo;  // bf16 low part (fp16 tables), or null
  int64_t tunf_hs;      // 0 (shared) or (Runf + 32) * 64
  void* out;            // dtype
  Str sout;
  int B, H;
  Geo geo;
  int key_side;
  int nblk;             // 128-row blocks per (b, h) launched
  int rb0;              // first 128-row block launched
};

struct TabUnfoldArgs {  // out[ho][u][:] = tab[ho][fold(u)][:], 32 zero rows after Runf
  const void* tab;
  int64_t tab_hs;
  const int32_t* fold;
  void* out;            // fp32 (fp32 tables) or the bf16 high part (16-bit tables)
  void* out_lo;         // bf16 low part (fp16 tables), or null
  int Ho, Runf;
};

struct SplitArgs {      // xh + xl = x exactly (fp16 x split into two bf16 parts)
  const void* x;        // [B, H, N, 64] with strides sx
  Str sx;
  void* xh;             // [B*H][N][64] bf16
  void* xl;
  int B, H, N;
};

struct ColsArgs {       // partial[s][ho][u][:] = sum_i dZ[i][u - ws] x_i[:]
  const float* dz;
  const void* x;        // X in the input type (bf16: the MFMA operand as it is)
  const void* xh;       // fp16 X split into bf16 parts, [B*H][N][64] (else null)
  const void* xl;
  Str sx;
  float* part;          // [S][Ho][Rpad][64]
  float* partb;         // [S][Ho][Rpad] or null
  int B, H;
  Geo geo;
  int key_side;
  int shared;           // 1: sum over heads too (Ho = 1)
  int splits;
  int rtiles;
  int Rpad;
  int want_x;           // 0: only the column sums (db)
};

struct FoldArgs {       // out[ho][k][:] = sum_s sum_{u in fold range of k} part[s][ho][u][:]
  const float* part;
  const float* partb;
  const int32_t* ub;    // [R] first unfolded row of table row k (or null: identity)
  const int32_t* ue;
  float* out;           // [Ho][R][64] or null
  float* outb;          // [Ho][R] or null
  int Ho, R, Rpad, splits;
  int accumulate;       // 1: out += the sums (in call order), 0: out = the sums
};

struct BiasArgs {       // bunf[h][u] = b[h][fold[u]]
  const void* b;
  int64_t b_hs;
  const int32_t* fold;
  float* bunf;
  int Hb, Runf;
};

}  // namespace relpos
