// contract.hip -- final contraction of the per-offset relation gradients.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), end of the backward section: the table
// gradients are matrix products, dZ^T times Q (or K) gives the gradient of the
// relation table, and dZ times the table gives the extra term of dQ (dK);
// copied bucket columns are summed back into their bucket in a fixed order.
// The scalar-bias gradient is read here as the column sums of dZ^Q
// (db[r] = tau * sum over all pairs with phi = r of dS, from Eq. 1 and 4).
//
// fp32 inputs run on v_mfma_f32_32x32x2_f32.  16-bit inputs run on
// v_mfma_f32_32x32x16_bf16 with every fp32 operand split into two bf16 parts
// (z = hi + lo + r, |r| <= 2^-16 |z|) and fp16 operands split exactly into two
// bf16 parts; the products hi*hi, hi*lo and lo*hi are kept (the dropped lo*lo
// is below 2^-16 of the term).  Summation orders are fixed (no atomics):
//  * rows_kernel / rows2_kernel: dX[i] = dX_part[i] + sum_c dZ[i][c] tab[fold(ws + c)],
//                  with the table unfolded first (tab_unfold_kernel)
//  * cols_kernel / cols1_kernel: part[s][h][u] = sum over the rows i of split s
//                  of dZ[i][u - ws(i)] x_i (and the column sums for db), window-aware;
//  * fold_kernel:  out[h][k] = sum over splits and over the unfolded rows u of k.
#include "device.hpp"
#include "tiles.hpp"

namespace relpos {

__device__ inline f32x16 mma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// z = hi + lo + r with |r| <= 2^-16 |z|: hi = bf16(z), lo = bf16(z - hi)
// (z - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(const float (&z)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = (__bf16)z[j];
    lo[j] = (__bf16)(z[j] - (float)hi[j]);
  }
}

// Row contraction, one block = 128 rows of one (b, h) (one group), 4 waves x
// 32 rows x 64 d, over the group's live window columns [cb, ce) in chunks of
// 32 columns aligned to 128 bytes.  Each chunk of dZ (128 rows x 32 floats)
// and the matching 32 rows of the fp32 unfolded table go straight from HBM
// into LDS with global_load_lds_dwordx4, double buffered, so the next chunk
// streams in while the MFMAs run.  Inside an LDS row of dZ the 16-byte
// chunks are XOR-permuted with (row / 2) % 8, which keeps the operand reads
// of 32 rows at one column at most two-way on a bank.  Columns of an edge
// chunk outside [cb, ce) are never written by the backward passes; they are
// read but replaced by zero before the MFMA.
constexpr int kRC = 32;  // columns per chunk

// SH: the rows are shifted query rows of dZ^Q (dz_shift with dsm = 31)
template <typename T, bool SH>
struct RowsK {
  const float* dzb;   // dZ of this (b, h), row stride Wp
  const float* tub;   // unfolded fp32 table of this head, [Runf + 32][64]
  int N, Wp, i0, ws, cb, ce, w, lane, hl, l32;
  int shb = 0;  // (SH) column shift of row i: (i + shb) & 31 (dz_shift)

  __device__ static int zswz(int r) { return (r >> 1) & 7; }

  // dZ rows [i0, i0 + 128) x columns [c0, c0 + 32) and the table rows
  // ws + c0 .. + 31 into (zb, tb), asynchronously
  __device__ __forceinline__ void issue(float* zb, float* tb, int c0) const {
    // (a block whose 128 rows all exist, a wave-uniform test, loads with no
    // per-lane condition and so without exec-mask branches)
    const bool whole = i0 + kBlockRows <= N;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 4 * w + u;  // 8 rows per instruction
      const int r = 8 * j + (lane >> 3);
      const int lc = (lane & 7) ^ zswz(r);
      float* dst = zb + 256 * j;
      if (whole) {
        const int sc = c0 + 4 * lc + (SH ? (i0 + r + shb) & 31 : 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(dzb + (int64_t)(i0 + r) * Wp + sc),
                                         (lds_void_t*)dst, 16, 0, 0);
      } else if (i0 + r < N) {
        const int sc = c0 + 4 * lc + (SH ? (i0 + r + shb) & 31 : 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(dzb + (int64_t)(i0 + r) * Wp + sc),
                                         (lds_void_t*)dst, 16, 0, 0);
      } else {
        *reinterpret_cast<Chunk*>(dst + 4 * lane) = Chunk{{0u, 0u, 0u, 0u}};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * w + u;  // 4 table rows per instruction
      const int r = 4 * j + (lane >> 4);
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(tub + (int64_t)(ws + c0 + r) * kHeadDim + 4 * (lane & 15)),
          (lds_void_t*)(tb + 256 * j), 16, 0, 0);
    }
  }
  // acc += dZ chunk (this wave's 32 rows) x table chunk
  template <bool EDGE>
  __device__ __forceinline__ void mma_chunk(const float* zb, const float* tb, int c0,
                                            f32x16 (&acc)[2]) const {
    const int r = 32 * w + l32;
    const float* zr = zb + 32 * r;
    const int sw = zswz(r);
#pragma unroll
    for (int ks = 0; ks < kRC / 2; ++ks) {
      const int c = 2 * ks + hl;
      float av = zr[4 * ((c >> 2) ^ sw) + (c & 3)];
      if (EDGE) av = (c0 + c >= cb && c0 + c < ce) ? av : 0.f;
      const float* trow = tb + c * kHeadDim + l32;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mma32(av, trow[32 * nt], acc[nt]);
    }
  }
  __device__ __forceinline__ void chunk(const float* zb, const float* tb, int c0,
                                        f32x16 (&acc)[2]) const {
    if (c0 < cb || c0 + kRC > ce)
      mma_chunk<true>(zb, tb, c0, acc);
    else
      mma_chunk<false>(zb, tb, c0, acc);
  }
};

template <typename T, bool SH>
__global__ __launch_bounds__(kThreads) void rows_kernel(RowsArgs a) {
  __shared__ __align__(16) float sZ0[128 * kRC], sZ1[128 * kRC];
  __shared__ __align__(16) float sT0[kRC * kHeadDim], sT1[kRC * kHeadDim];
  const Geo g = a.geo;
  const int N = g.N;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk, rb = a.rb0 + lid - bh * a.nblk;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int tid = threadIdx.x;
  RowsK<T, SH> k;
  k.w = wave_id();
  k.lane = tid & 63;
  k.hl = k.lane >> 5;
  k.l32 = k.lane & 31;
  k.N = N;
  k.Wp = g.Wp;
  k.i0 = rb * kBlockRows;
  if (a.key_side) {
    cols_k(g, rb, k.cb, k.ce);
    k.ws = win_k(g, rb);
  } else {
    cols_q(g, rb, k.cb, k.ce);
    k.ws = win_q(g, rb);
    k.shb = g.lo + k.ws;  // (dz_shift)
  }
  // rows addressed by token (key side: every key; query side: the held rows)
  k.dzb = a.key_side ? a.dz + (int64_t)bh * N * g.Wp : a.dz + zq_off(g, bh, 0);
  k.tub = (const float*)a.tunf + hh * a.tunf_hs;
  const int w = k.w, hl = k.hl, l32 = k.l32;

  f32x16 acc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = k.i0 + 32 * w + res_row(hl, e);
      acc[nt][e] = i < N ? a.part[((int64_t)bh * N + i) * kHeadDim + 32 * nt + l32] : 0.f;
    }

  // chunks c0 = cb0, cb0 + 32, ... (cb0 = cb rounded down to 32); chunk n
  // sits in buffer n & 1
  const int cb0 = k.cb & ~(kRC - 1);
  const int nch = k.ce > k.cb ? (k.ce - cb0 + kRC - 1) / kRC : 0;
  if (nch > 0) k.issue(sZ0, sT0, cb0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int n = 0; n < nch; n += 2) {
    const int c0 = cb0 + n * kRC;
    const bool more1 = n + 1 < nch;
    if (more1) k.issue(sZ1, sT1, c0 + kRC);
    k.chunk(sZ0, sT0, c0, acc);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (!more1) break;
    if (n + 2 < nch) k.issue(sZ0, sT0, c0 + 2 * kRC);
    k.chunk(sZ1, sT1, c0 + kRC, acc);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  T* ob = (T*)a.out + bb * a.sout.b + hh * a.sout.h;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = k.i0 + 32 * w + res_row(hl, e);
      if (i < N) ob[(int64_t)i * a.sout.n + 32 * nt + l32] = MT<T>::from_f(acc[nt][e]);
    }
}

// Row contraction for 16-bit inputs: the blocks, chunks and dZ loads of
// rows_kernel; the table chunk (32 unfolded rows, bf16 high and, for fp16
// tables, low part) goes into LDS in the swizzled 16-bit tile layout and is
// read as the MFMA B operand with transpose reads; each lane splits its 8 dZ
// values of a k-step into bf16 parts.
template <typename T, bool SH>
struct Rows2K {
  using BF = MT<__bf16>;
  static constexpr bool kLo = std::is_same<T, _Float16>::value;  // table has a low part
  const float* dzb;   // dZ of this (b, h), row stride Wp
  const __bf16* thb;  // unfolded table of this head, high part, [Runf + 32][64]
  const __bf16* tlb;  // low part (fp16 tables)
  int N, Wp, i0, ws, cb, ce, w, lane, hl, l32;
  int shb = 0;  // (SH) column shift of row i: (i + shb) & 31 (dz_shift)
  TrReader<__bf16> tr;

  __device__ __forceinline__ void issue(float* zb, char* th, char* tl, int c0) const {
    const bool whole = i0 + kBlockRows <= N;  // (as in RowsK::issue)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 4 * w + u;  // 8 rows per instruction
      const int r = 8 * j + (lane >> 3);
      const int lc = (lane & 7) ^ RowsK<T, SH>::zswz(r);
      float* dst = zb + 256 * j;
      if (whole) {
        const int sc = c0 + 4 * lc + (SH ? (i0 + r + shb) & 31 : 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(dzb + (int64_t)(i0 + r) * Wp + sc),
                                         (lds_void_t*)dst, 16, 0, 0);
      } else if (i0 + r < N) {
        const int sc = c0 + 4 * lc + (SH ? (i0 + r + shb) & 31 : 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(dzb + (int64_t)(i0 + r) * Wp + sc),
                                         (lds_void_t*)dst, 16, 0, 0);
      } else {
        *reinterpret_cast<Chunk*>(dst + 4 * lane) = Chunk{{0u, 0u, 0u, 0u}};
      }
    }
    // table rows ws + c0 + r, r = 8 w + lane / 8: slot lane % 8 of the row
    // holds its chunk (lane % 8) ^ swz(r)
    const int r = 8 * w + (lane >> 3);
    const int cg = (lane & 7) ^ swz<__bf16>(r);
    const int64_t off = (int64_t)(ws + c0 + r) * kHeadDim + 8 * cg;
    __builtin_amdgcn_global_load_lds((glb_void_t*)(thb + off), (lds_void_t*)(th + 1024 * w), 16,
                                     0, 0);
    if (kLo)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(tlb + off), (lds_void_t*)(tl + 1024 * w),
                                       16, 0, 0);
  }
  // acc += dZ chunk (this wave's 32 rows) x table chunk
  template <bool EDGE>
  __device__ __forceinline__ void mma_chunk(const float* zb, const char* th, const char* tl,
                                            int c0, f32x16 (&acc)[2]) const {
    const int r = 32 * w + l32;
    const float* zr = zb + 32 * r;
    const int sw = RowsK<T, SH>::zswz(r);
#pragma unroll
    for (int ks = 0; ks < kRC / 16; ++ks) {
      const int c = 16 * ks + 8 * hl;  // first of the lane's 8 columns
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(zr + 4 * ((c >> 2) ^ sw));
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(zr + 4 * (((c >> 2) + 1) ^ sw));
      float z[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      if (EDGE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = (c0 + c + j >= cb && c0 + c + j < ce) ? z[j] : 0.f;
      }
      bf16x8 ah, al;
      split_bf16(z, ah, al);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bf16x8 bh = tr.read(th, nt, ks);
        acc[nt] = BF::mma(ah, bh, acc[nt]);
        acc[nt] = BF::mma(al, bh, acc[nt]);
        if (kLo) acc[nt] = BF::mma(ah, tr.read(tl, nt, ks), acc[nt]);
      }
    }
  }
  __device__ __forceinline__ void chunk(const float* zb, const char* th, const char* tl, int c0,
                                        f32x16 (&acc)[2]) const {
    if (c0 < cb || c0 + kRC > ce)
      mma_chunk<true>(zb, th, tl, c0, acc);
    else
      mma_chunk<false>(zb, th, tl, c0, acc);
  }
};

template <typename T, bool SH>
__global__ __launch_bounds__(kThreads) void rows2_kernel(RowsArgs a) {
  static_assert(sizeof(T) == 2, "16-bit inputs");
  constexpr int TT = kRC * kHeadDim * 2;  // bytes of one table part chunk
  constexpr int TL = Rows2K<T, SH>::kLo ? TT : 16;
  __shared__ __align__(16) float sZ0[128 * kRC], sZ1[128 * kRC];
  __shared__ __align__(16) char sH0[TT], sH1[TT], sL0[TL], sL1[TL];
  const Geo g = a.geo;
  const int N = g.N;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk, rb = a.rb0 + lid - bh * a.nblk;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int tid = threadIdx.x;
  Rows2K<T, SH> k;
  k.w = wave_id();
  k.lane = tid & 63;
  k.hl = k.lane >> 5;
  k.l32 = k.lane & 31;
  k.N = N;
  k.Wp = g.Wp;
  k.i0 = rb * kBlockRows;
  if (a.key_side) {
    cols_k(g, rb, k.cb, k.ce);
    k.ws = win_k(g, rb);
  } else {
    cols_q(g, rb, k.cb, k.ce);
    k.ws = win_q(g, rb);
    k.shb = g.lo + k.ws;  // (dz_shift)
  }
  k.dzb = a.key_side ? a.dz + (int64_t)bh * N * g.Wp : a.dz + zq_off(g, bh, 0);
  k.thb = (const __bf16*)a.tunf + hh * a.tunf_hs;
  k.tlb = a.tunf_lo ? (const __bf16*)a.tunf_lo + hh * a.tunf_hs : nullptr;
  k.tr.init(k.lane);
  const int w = k.w, hl = k.hl, l32 = k.l32;

  f32x16 acc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = k.i0 + 32 * w + res_row(hl, e);
      acc[nt][e] = i < N ? a.part[((int64_t)bh * N + i) * kHeadDim + 32 * nt + l32] : 0.f;
    }

  const int cb0 = k.cb & ~(kRC - 1);
  const int nch = k.ce > k.cb ? (k.ce - cb0 + kRC - 1) / kRC : 0;
  if (nch > 0) k.issue(sZ0, sH0, sL0, cb0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int n = 0; n < nch; n += 2) {
    const int c0 = cb0 + n * kRC;
    const bool more1 = n + 1 < nch;
    if (more1) k.issue(sZ1, sH1, sL1, c0 + kRC);
    k.chunk(sZ0, sH0, sL0, c0, acc);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (!more1) break;
    if (n + 2 < nch) k.issue(sZ0, sH0, sL0, c0 + 2 * kRC);
    k.chunk(sZ1, sH1, sL1, c0 + kRC, acc);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  T* ob = (T*)a.out + bb * a.sout.b + hh * a.sout.h;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = k.i0 + 32 * w + res_row(hl, e);
      if (i < N) ob[(int64_t)i * a.sout.n + 32 * nt + l32] = MT<T>::from_f(acc[nt][e]);
    }
}

// Column contraction for a single-group window (every row's window starts
// at unfolded row 0, so column u of every dZ row is unfolded row u).
// Block (ut, s, ho): unfolded rows u in [64 ut, 64 ut + 64), all 64 d, over
// the rows of split s, in chunks of 64 rows.  Each chunk of dZ (64 rows x 64
// floats) and of X (64 rows x 64 elements) goes straight into LDS with
// global_load_lds_dwordx4, double buffered.  Wave w owns the output tile
// u in 64 ut + 32 (w & 1) + [0, 32), d in 32 (w >> 1) + [0, 32); waves with
// w >> 1 == 0 also sum the columns (db).  Columns outside the live window
// [cb, ce) hold no gradient and are read as zero.
constexpr int kCU = 64;  // unfolded rows per block

// Position in the flattened row range: row i of segment seg (b, or b*H + h
// for a table shared by all heads).
struct RowPos {
  int seg, i;
};
__device__ __forceinline__ bool before(RowPos a, RowPos b) {
  return a.seg < b.seg || (a.seg == b.seg && a.i < b.i);
}

template <typename T, bool SH>
struct ColsK {
  const float* dz;
  const __bf16* x;   // X operand (bf16 inputs: X itself; fp16: its high part)
  const __bf16* xl;  // low part of a split fp16 X, or null
  Str sx;            // strides of x (a split X is [B*H][N][64])
  Geo g;
  int N, Wp, H, ho, u0, w, lane, hl, l32, key_side;
  int rlo, rhi;  // rows of each segment taken: every key, or the held query rows
  bool shared, grp_on;
  RowPos end;  // end of this split's row range
  int cb0, ce0, ws0;  // the single window (ungrouped)
  DLoader<__bf16> ldx;

  // live window of group grp: columns [cb, ce) hold entries, column c is
  // unfolded row ws + c
  __device__ __forceinline__ void window(int grp, int& cb, int& ce, int& ws) const {
    if (!grp_on) {
      cb = cb0;
      ce = ce0;
      ws = ws0;
    } else if (key_side) {
      cols_k(g, grp, cb, ce);
      ws = win_k(g, grp);
    } else {
      cols_q(g, grp, cb, ce);
      ws = win_q(g, grp);
    }
  }
  __device__ __forceinline__ int group_of(RowPos p) const { return grp_on ? p.i / kGroup : 0; }
  // end of the run of rows that shares p's segment and window
  __device__ __forceinline__ RowPos run_end(RowPos p) const {
    RowPos e = grp_on ? RowPos{p.seg, imin(rhi, (p.i / kGroup + 1) * kGroup)} : RowPos{p.seg, rhi};
    if (e.i >= rhi) e = RowPos{p.seg + 1, rlo};
    return before(end, e) ? end : e;
  }
  // first row at or after p (end if none) whose window's live columns meet
  // this block's unfolded rows [u0, u0 + kCU); whole runs are skipped
  __device__ __forceinline__ RowPos next_live(RowPos p) const {
    while (before(p, end)) {
      int cb, ce, ws;
      window(group_of(p), cb, ce, ws);
      if (ws + ce > u0 && ws + cb < u0 + kCU) return p;
      p = run_end(p);
    }
    return end;
  }
  // rows of the chunk starting at p: up to 64, inside one run
  __device__ __forceinline__ int chunk_rows(RowPos p) const {
    const RowPos e = run_end(p);
    const int n = e.seg == p.seg ? e.i - p.i : rhi - p.i;
    return n < 64 ? n : 64;
  }
  __device__ __forceinline__ RowPos advance(RowPos p, int n) const {
    p.i += n;
    if (p.i >= rhi) p = RowPos{p.seg + 1, rlo};
    return p;
  }

  // rows [p.i, p.i + nrow) of segment p.seg into zb (and, when WANT_X, the
  // X rows into the 16-bit tiles xh, xl), asynchronously: zb[r][uo] holds
  // dZ[i + r][u0 + uo - ws] (zero outside the stored row)
  template <bool WANT_X>
  __device__ __forceinline__ void issue(float* zb, char* xh, char* xlo, RowPos p,
                                        int nrow) const {
    const int seg = p.seg, i = p.i;
    const int b_ = shared ? seg / H : seg;
    const int h_ = shared ? seg % H : ho;
    const float* dzs =
        key_side ? dz + (int64_t)(b_ * H + h_) * N * Wp : dz + zq_off(g, b_ * H + h_, 0);
    int cb, ce, ws;
    window(group_of(p), cb, ce, ws);
    const int colb = u0 - ws;  // window column of the block's first unfolded row
    // rows of dZ^Q may be stored shifted (dz_shift); columns below z_span
    // stay inside the row after the shift
    const int shb = i + g.lo + ws;
    const int span = SH ? z_span(g) : Wp;
    if ((colb & 3) == 0) {
      // (every lane's row and columns inside the stored rows, a wave-uniform
      // test: loads with no per-lane condition, without exec-mask branches)
      const bool whole = nrow >= 16 * w + 16 && colb >= 0 && colb + 64 <= span;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 4 * w + u;  // 4 rows of 64 floats per instruction
        const int r = 4 * j + (lane >> 4);
        const int col = colb + 4 * (lane & 15);
        float* dst = zb + 256 * j;
        if (whole) {
          const int sc = col + (SH ? (r + shb) & 31 : 0);
          __builtin_amdgcn_global_load_lds((glb_void_t*)(dzs + (int64_t)(i + r) * Wp + sc),
                                           (lds_void_t*)dst, 16, 0, 0);
        } else if (r < nrow && col >= 0 && col < span) {
          const int sc = col + (SH ? (r + shb) & 31 : 0);
          __builtin_amdgcn_global_load_lds((glb_void_t*)(dzs + (int64_t)(i + r) * Wp + sc),
                                           (lds_void_t*)dst, 16, 0, 0);
        } else {
          *reinterpret_cast<Chunk*>(dst + 4 * lane) = Chunk{{0u, 0u, 0u, 0u}};
        }
      }
    } else {
      // window not 16-byte aligned with the block: one row of 64 floats per
      // instruction
      const int col = colb + lane;
#pragma unroll 4
      for (int u = 0; u < 16; ++u) {
        const int r = 16 * w + u;
        float* dst = zb + kCU * r;
        if (r < nrow && col >= 0 && col < span) {
          __builtin_amdgcn_global_load_lds(
              (glb_void_t*)(dzs + (int64_t)(i + r) * Wp + col + (SH ? (r + shb) & 31 : 0)),
              (lds_void_t*)dst, 4, 0, 0);
        } else {
          dst[lane] = 0.f;
        }
      }
    }
    if constexpr (WANT_X) {
      if (xl) {
        const int64_t row0 = ((int64_t)(b_ * H + h_) * N + i) * kHeadDim;
        ldx.load(xh, x + row0, nrow, lane);
        ldx.load(xlo, xl + row0, nrow, lane);
      } else {
        ldx.load(xh, x + b_ * sx.b + h_ * sx.h + (int64_t)i * sx.n, nrow, lane);
      }
    }
  }
  // whether unfolded row u0 + uo is a live column of the chunk at p
  __device__ __forceinline__ bool live(RowPos p, int uo) const {
    int cb, ce, ws;
    window(group_of(p), cb, ce, ws);
    const int c = u0 + uo - ws;
    return c >= cb && c < ce;
  }
};

// One 64-row chunk: acc (this wave's 32 u x 32 d tile) += dZ^T X on
// v_mfma_f32_32x32x16_bf16, dZ split into two bf16 parts by each lane (its
// 8 rows of a k-step at its column), X read from the 16-bit tile with
// transpose reads; csum += the column's live values.  Without X only the
// sums run.
template <typename T, bool WANT_X>
struct ColsMma {
  using BF = MT<__bf16>;
  static constexpr bool kLo = std::is_same<T, _Float16>::value;  // X split in two parts
  __device__ static __forceinline__ void run(const float* zb, const char* xh, const char* xlo,
                                             const TrReader<__bf16>& tr, int uo, int dh, int hl,
                                             bool uvalid, bool sums, f32x16& acc, float& csum) {
    if constexpr (WANT_X) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          z[j] = zb[(16 * ks + 8 * hl + j) * kCU + uo];
          z[j] = uvalid ? z[j] : 0.f;
        }
        if (sums) {
#pragma unroll
          for (int j = 0; j < 8; ++j) csum += z[j];
        }
        bf16x8 ah, al;
        split_bf16(z, ah, al);
        const bf16x8 bh = tr.read(xh, dh, ks);
        acc = BF::mma(ah, bh, acc);
        acc = BF::mma(al, bh, acc);
        if (kLo) acc = BF::mma(ah, tr.read(xlo, dh, ks), acc);
      }
    } else {
#pragma unroll 8
      for (int r = hl; r < 64; r += 2) {
        const float av = zb[r * kCU + uo];
        csum += uvalid ? av : 0.f;
      }
    }
  }
};

template <typename T, bool WANT_X, bool SH>
__global__ __launch_bounds__(kThreads) void cols1_kernel(ColsArgs a) {
  static_assert(sizeof(T) == 2, "16-bit inputs");
  constexpr int XB = WANT_X ? DTile<__bf16>::BYTES : 16;
  constexpr int XL = (WANT_X && std::is_same<T, _Float16>::value) ? DTile<__bf16>::BYTES : 16;
  __shared__ __align__(16) float sZ0[64 * kCU], sZ1[64 * kCU];
  __shared__ __align__(16) char sX0[XB], sX1[XB], sL0[XL], sL1[XL];
  const Geo g = a.geo;
  const int N = g.N;
  const int nblk = gridDim.x * gridDim.y * gridDim.z;
  const int lid = xcd_remap(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), nblk);
  const int ut = lid % gridDim.x, sp = (lid / gridDim.x) % gridDim.y;
  const int ho = lid / (gridDim.x * gridDim.y);
  ColsK<T, SH> k;
  k.w = wave_id();
  k.lane = threadIdx.x & 63;
  k.hl = k.lane >> 5;
  k.l32 = k.lane & 31;
  k.g = g;
  k.N = N;
  k.Wp = g.Wp;
  k.H = a.H;
  k.ho = ho;
  k.u0 = kCU * ut;
  k.key_side = a.key_side;
  k.shared = a.shared;
  k.dz = a.dz;
  k.xl = (const __bf16*)a.xl;
  k.x = a.xl ? (const __bf16*)a.xh : (const __bf16*)a.x;
  k.sx = a.sx;
  if (WANT_X) k.ldx.init(a.xl ? kHeadDim : a.sx.n, k.w, k.lane);
  TrReader<__bf16> tr;
  tr.init(k.lane);
  const int w = k.w, hl = k.hl, l32 = k.l32;
  const int uo = 32 * (w & 1) + l32;  // this lane's unfolded row inside the block
  const int u = k.u0 + uo;
  const bool sums = w < 2;
  const int dh = w >> 1;  // d half of this wave's tile
  const int d = 32 * dh + l32;

  // this split's range of the flattened rows (segment-major, rows [rlo, rhi)
  // of each segment)
  k.rlo = a.key_side ? 0 : g.z0;
  k.rhi = a.key_side ? N : zq_last(g) + 1;
  const int nr = k.rhi - k.rlo;
  const int nseg = a.shared ? a.B * a.H : a.B;
  const int64_t nrows = (int64_t)nseg * nr;
  const int64_t per = (nrows + a.splits - 1) / a.splits;
  const int64_t f0 = (int64_t)sp * per;
  const int64_t f1 = f0 + per < nrows ? f0 + per : nrows;
  k.end = RowPos{(int)(f1 / nr), k.rlo + (int)(f1 % nr)};
  k.grp_on = grouped(g);
  if (a.key_side) cols_k(g, 0, k.cb0, k.ce0); else cols_q(g, 0, k.cb0, k.ce0);
  k.ws0 = 0;

  f32x16 acc = zero16();
  float csum = 0.f;
  // live chunk n (rows [p.i, p.i + nrow) of segment p.seg) sits in buffer n & 1
  RowPos p = k.next_live(RowPos{(int)(f0 / nr), k.rlo + (int)(f0 % nr)});
  int nrow = before(p, k.end) ? k.chunk_rows(p) : 0;
  if (nrow > 0) k.template issue<WANT_X>(sZ0, sX0, sL0, p, nrow);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  while (before(p, k.end)) {
    RowPos pn = k.next_live(k.advance(p, nrow));
    int nrow1 = before(pn, k.end) ? k.chunk_rows(pn) : 0;
    if (nrow1 > 0) k.template issue<WANT_X>(sZ1, sX1, sL1, pn, nrow1);
    ColsMma<T, WANT_X>::run(sZ0, sX0, sL0, tr, uo, dh, hl, k.live(p, uo), sums, acc, csum);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    p = pn;
    nrow = nrow1;
    if (!before(p, k.end)) break;
    pn = k.next_live(k.advance(p, nrow));
    nrow1 = before(pn, k.end) ? k.chunk_rows(pn) : 0;
    if (nrow1 > 0) k.template issue<WANT_X>(sZ0, sX0, sL0, pn, nrow1);
    ColsMma<T, WANT_X>::run(sZ1, sX1, sL1, tr, uo, dh, hl, k.live(p, uo), sums, acc, csum);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    p = pn;
    nrow = nrow1;
  }

  if (WANT_X) {
    float* outp = a.part + (((int64_t)sp * gridDim.z + ho) * a.Rpad + k.u0) * 64;
#pragma unroll
    for (int e = 0; e < 16; ++e) outp[(32 * (w & 1) + res_row(hl, e)) * 64 + d] = acc[e];
  }
  if (a.partb && sums) {
    csum = sum_xor32(csum);
    if (hl == 0) a.partb[((int64_t)sp * gridDim.z + ho) * a.Rpad + u] = csum;
  }
}

// fp16 X split exactly into two bf16 parts (hi + lo = x): an fp16 value has
// 11 significant bits, bf16 keeps 8, and the remainder needs at most 3, all
// inside bf16's exponent range.  xh, xl are [B*H][N][64].
__global__ __launch_bounds__(kThreads) void xsplit_kernel(SplitArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // 8 elements each
  const int64_t n = (int64_t)a.B * a.H * a.N * (kHeadDim / 8);
  if (idx >= n) return;
  const int part = (int)(idx % (kHeadDim / 8));
  const int64_t row = idx / (kHeadDim / 8);
  const int i = (int)(row % a.N);
  const int bh = (int)(row / a.N);
  const int b = bh / a.H, h = bh - b * a.H;
  const f16x8 v = *reinterpret_cast<const f16x8*>((const _Float16*)a.x + b * a.sx.b + h * a.sx.h +
                                                  (int64_t)i * a.sx.n + 8 * part);
  bf16x8 hi, lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float f = (float)v[j];
    hi[j] = (__bf16)f;
    lo[j] = (__bf16)(f - (float)hi[j]);
  }
  *reinterpret_cast<bf16x8*>((__bf16*)a.xh + row * kHeadDim + 8 * part) = hi;
  *reinterpret_cast<bf16x8*>((__bf16*)a.xl + row * kHeadDim + 8 * part) = lo;
}

// Unfolded copy of a vector table: out[ho][u][:] = tab[ho][fold(u)][:] for
// u < Runf, zero for the 32 padding rows after it.  fp32 tables are copied as
// they are; 16-bit tables become bf16 (fp16 ones split exactly into a high
// and a low bf16 part, as in xsplit_kernel).
template <typename T>
__global__ __launch_bounds__(kThreads) void tab_unfold_kernel(TabUnfoldArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int rows = a.Runf + 32;
  const int64_t n = (int64_t)a.Ho * rows * kHeadDim;
  if (idx >= n) return;
  const int d = (int)(idx % kHeadDim);
  const int64_t hu = idx / kHeadDim;
  const int u = (int)(hu % rows), ho = (int)(hu / rows);
  float v = 0.f;
  if (u < a.Runf) {
    const int r = a.fold ? a.fold[u] : u;
    v = MT<T>::to_f(((const T*)a.tab)[ho * a.tab_hs + (int64_t)r * kHeadDim + d]);
  }
  if constexpr (sizeof(T) == 4) {
    ((float*)a.out)[idx] = v;
  } else {
    const __bf16 hi = (__bf16)v;
    ((__bf16*)a.out)[idx] = hi;
    if (a.out_lo) ((__bf16*)a.out_lo)[idx] = (__bf16)(v - (float)hi);
  }
}

// Block (rt, s, ho): unfolded rows u in [32 rt, 32 rt + 32), all 64 d, over
// the rows of split s.  The 4 waves take interleaved pairs of rows (one MFMA
// k-step each) and are summed in LDS in wave order.
template <typename T>
__global__ __launch_bounds__(kThreads) void cols_kernel(ColsArgs a) {
  __shared__ float sAcc[4][32 * 64];
  __shared__ float sSum[4][32];
  const Geo g = a.geo;
  const int N = g.N;
  // the row tiles of one (split, head) are consecutive logical blocks, which
  // xcd_remap keeps on one XCD: they read the same dZ rows and X rows, so
  // those lines are fetched into that XCD's L2 once
  const int nblk = gridDim.x * gridDim.y * gridDim.z;
  const int lid = xcd_remap(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), nblk);
  const int rt = lid % gridDim.x, sp = (lid / gridDim.x) % gridDim.y, ho = lid / (gridDim.x * gridDim.y);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int u = 32 * rt + l32;  // unfolded row of this lane (operand A row)
  // rows [rlo, rlo + nr) of each segment: every key, or the held query rows
  const int rlo = a.key_side ? 0 : g.z0;
  const int nr = (a.key_side ? N : zq_last(g) + 1) - rlo;
  const int nseg = a.shared ? a.B * a.H : a.B;
  const int64_t nrows = (int64_t)nseg * nr;
  const int64_t per = (nrows + a.splits - 1) / a.splits;
  const int64_t f0 = (int64_t)sp * per;
  const int64_t f1 = f0 + per < nrows ? f0 + per : nrows;

  f32x16 acc[2];
  acc[0] = zero16();
  acc[1] = zero16();
  float csum = 0.f;

  int64_t f = f0;
  while (f < f1) {
    const int seg = (int)(f / nr);
    const int i_start = rlo + (int)(f - (int64_t)seg * nr);
    const int grp = grouped(g) ? i_start / kGroup : 0;
    const int i_gend = grouped(g) ? imin(rlo + nr, (grp + 1) * kGroup) : rlo + nr;
    const int64_t fend0 = (int64_t)seg * nr + (i_gend - rlo);
    const int64_t fend = fend0 < f1 ? fend0 : f1;
    int cb, ce, ws;
    if (a.key_side) {
      cols_k(g, grp, cb, ce);
      ws = win_k(g, grp);
    } else {
      cols_q(g, grp, cb, ce);
      ws = win_q(g, grp);
    }
    // skip the chunk when its live columns miss this block's rows
    if (ws + ce > 32 * rt && ws + cb < 32 * rt + 32) {
      const int b_ = a.shared ? seg / a.H : seg;
      const int h_ = a.shared ? seg % a.H : ho;
      const int bh = b_ * a.H + h_;
      const float* dzb = a.key_side ? a.dz + (int64_t)bh * N * g.Wp : a.dz + zq_off(g, bh, 0);
      const T* xb = (const T*)a.x + b_ * a.sx.b + h_ * a.sx.h;
      const int col = u - ws;
      const bool colv = col >= cb && col < ce;
      const int i_end = rlo + (int)(fend - (int64_t)seg * nr);
      // each wave takes 16 consecutive rows (8 MFMA k-steps) per round, loads first
      for (int ib = i_start + 16 * w; ib < i_end; ib += 64) {
        float av[8], bv[8][2];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int i = ib + 2 * s2 + hl;
          const bool rv = i < i_end;
          const int sc = col + (a.key_side ? 0 : ((i + g.lo + ws) & g.dsm));  // (dz_shift)
          av[s2] = (rv && colv) ? dzb[(int64_t)i * g.Wp + sc] : 0.f;
          const T* xr = xb + (int64_t)i * a.sx.n;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            bv[s2][nt] = (rv && a.want_x) ? MT<T>::to_f(xr[32 * nt + l32]) : 0.f;
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          csum += av[s2];
          if (a.want_x) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[nt] = mma32(av[s2], bv[s2][nt], acc[nt]);
          }
        }
      }
    }
    f = fend;
  }

  csum += __shfl_xor(csum, 32);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) sAcc[w][res_row(hl, e) * 64 + 32 * nt + l32] = acc[nt][e];
  if (hl == 0) sSum[w][l32] = csum;
  __syncthreads();
  float* outp = a.part + (((int64_t)sp * gridDim.z + ho) * a.Rpad + 32 * rt) * 64;
  for (int idx = tid; idx < 32 * 64; idx += kThreads) {
    const float v = ((sAcc[0][idx] + sAcc[1][idx]) + sAcc[2][idx]) + sAcc[3][idx];
    if (a.want_x) outp[idx] = v;
  }
  if (a.partb && tid < 32) {
    const float v = ((sSum[0][tid] + sSum[1][tid]) + sSum[2][tid]) + sSum[3][tid];
    a.partb[((int64_t)sp * gridDim.z + ho) * a.Rpad + 32 * rt + tid] = v;
  }
}

// s += the `splits` values at p, p + stride, ... in that order.  BATCH: the
// loads of 8 splits are issued together before their adds (many splits);
// otherwise one at a time (few splits: a smaller kernel, for launches of
// many short blocks).
template <bool BATCH>
__device__ __forceinline__ float sum_splits(float s, const float* p, int64_t stride, int splits) {
  if constexpr (!BATCH) {
    for (int sp = 0; sp < splits; ++sp) s += p[sp * stride];
    return s;
  }
  for (int sp = 0; sp < splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = sp + j < splits ? p[(sp + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (sp + j < splits) s += v[j];
  }
  return s;
}

// out[ho][k][d] = sum_{u in [ub[k], ue[k])} sum_s part[s][ho][u][d], u ascending
// (added to out when accumulate is set: one call per chunk of rows, in order).
// Block (k4, ho): table rows k = 4 k4 .. 4 k4 + 3 of head ho, one thread per
// (row, d); lane d = 0 also sums the bias column.  Fixed order: u ascending,
// then the splits.
template <bool BATCH>
__global__ __launch_bounds__(256) void fold_kernel(FoldArgs a) {
  const int d = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ho = blockIdx.y;
  if (k >= a.R) return;
  const int b = a.ub ? a.ub[k] : k;
  const int e = a.ub ? a.ue[k] : k + 1;
  const int64_t sstride = (int64_t)a.Ho * a.Rpad;  // rows between splits
  if (a.out) {
    const float* p = a.part + ((int64_t)ho * a.Rpad) * 64 + d;
    float s = 0.f;
    for (int u = b; u < e; ++u)
      s = sum_splits<BATCH>(s, p + (int64_t)u * 64, sstride * 64, a.splits);
    float* o = a.out + ((int64_t)ho * a.R + k) * 64 + d;
    *o = a.accumulate ? *o + s : s;
  }
  if (a.outb && d == 0) {
    const float* p = a.partb + (int64_t)ho * a.Rpad;
    float s = 0.f;
    for (int u = b; u < e; ++u) s = sum_splits<BATCH>(s, p + u, sstride, a.splits);
    float* o = a.outb + (int64_t)ho * a.R + k;
    *o = a.accumulate ? *o + s : s;
  }
}

template <typename T, bool SPLIT>
static void launch_rows_t(const RowsArgs& a, int total, bool sh, hipStream_t st) {
  if constexpr (SPLIT) {
    if (sh) hipLaunchKernelGGL((rows2_kernel<T, true>), dim3(total), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((rows2_kernel<T, false>), dim3(total), dim3(kThreads), 0, st, a);
  } else {
    if (sh) hipLaunchKernelGGL((rows_kernel<T, true>), dim3(total), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((rows_kernel<T, false>), dim3(total), dim3(kThreads), 0, st, a);
  }
}

hipError_t launch_rows(int dtype, const RowsArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nblk;
  if (total <= 0) return hipSuccess;
  const bool sh = !a.key_side && a.geo.dsm;  // shifted rows of dZ^Q
  switch (dtype) {
    case 0: launch_rows_t<float, false>(a, total, sh, st); break;
    case 1: launch_rows_t<_Float16, true>(a, total, sh, st); break;
    default: launch_rows_t<__bf16, true>(a, total, sh, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_xsplit(const SplitArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.H * a.N * (kHeadDim / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(xsplit_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tab_unfold(int dtype, const TabUnfoldArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.Ho * (a.Runf + 32) * kHeadDim;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  switch (dtype) {
    case 0: hipLaunchKernelGGL(tab_unfold_kernel<float>, grid, dim3(kThreads), 0, st, a); break;
    case 1: hipLaunchKernelGGL(tab_unfold_kernel<_Float16>, grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(tab_unfold_kernel<__bf16>, grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <typename T, bool SH>
static void launch_cols1_t(const ColsArgs& a, dim3 grid, hipStream_t st) {
  if (a.want_x) hipLaunchKernelGGL((cols1_kernel<T, true, SH>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((cols1_kernel<T, false, SH>), grid, dim3(kThreads), 0, st, a);
}

hipError_t launch_cols1(int dtype, const ColsArgs& a, int Ho, hipStream_t st) {
  dim3 grid((a.Rpad + kCU - 1) / kCU, a.splits, Ho);
  const bool sh = !a.key_side && a.geo.dsm;  // shifted rows of dZ^Q
  if (dtype == 1) {
    if (sh) launch_cols1_t<_Float16, true>(a, grid, st);
    else launch_cols1_t<_Float16, false>(a, grid, st);
  } else {
    if (sh) launch_cols1_t<__bf16, true>(a, grid, st);
    else launch_cols1_t<__bf16, false>(a, grid, st);
  }
  return hipGetLastError();
}

hipError_t launch_cols(int dtype, const ColsArgs& a, int Ho, hipStream_t st) {
  dim3 grid(a.rtiles, a.splits, Ho);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(cols_kernel<float>, grid, dim3(kThreads), 0, st, a); break;
    case 1: hipLaunchKernelGGL(cols_kernel<_Float16>, grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(cols_kernel<__bf16>, grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t st) {
  if (a.Ho <= 0 || a.R <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.R + 3) / 4), (unsigned)a.Ho);
  if (a.splits > 4)
    hipLaunchKernelGGL(fold_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(fold_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace relpos
