// tiles.hpp -- staging of 64 x 64 operand tiles from HBM into LDS.
//
// A tile is 64 rows (tokens) x 64 columns (head dim) of the input dtype.
// It is kept in LDS row-major ("RM", rows padded to PITCH elements) and, for
// 16-bit types, also transposed ("TR", [column][row]) when an MFMA needs the
// token index as its contraction index: the contraction index must be
// contiguous inside a lane's fragment.  fp32 fragments hold one element, so
// fp32 tiles are only stored row-major and the transposed view reads them
// with swapped indices.
//
// Two thread->chunk maps are used for the HBM loads (a chunk is 16 bytes):
//  * row map: 8 lanes cover one row (coalesced), used for RM-only tiles;
//  * col map: 64 consecutive lanes cover 64 rows at one column chunk, which
//    makes the 2-byte transposed LDS writes hit 32 distinct banks.
#pragma once
#include <type_traits>

#include "device.hpp"

namespace relpos {

constexpr int kTile = 64;        // inner-loop tile
constexpr int kThreads = 256;

template <typename T>
struct TileCfg {
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr int PITCH = kHalf ? 72 : 65;      // elements per LDS row
  static constexpr int ELEMS = 64 * PITCH;
  static constexpr int CH = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int NCH = 64 * 64 / CH / kThreads;  // chunks per thread
};

struct alignas(16) Chunk {
  uint32_t w[4];
};

template <typename T, bool COLMAP>
__device__ inline void chunk_pos(int c, int& row, int& col) {
  constexpr int CH = TileCfg<T>::CH;
  if (COLMAP) {
    row = c & 63;
    col = (c >> 6) * CH;
  } else {
    row = c / (64 / CH);
    col = (c % (64 / CH)) * CH;
  }
}

// Load rows [row0, row0 + 64) of a [*, 64] matrix (row stride sn elements);
// rows >= nrows read as zero.
template <typename T, bool COLMAP>
__device__ inline void tile_load(Chunk (&r)[TileCfg<T>::NCH], const T* base, int64_t sn, int row0,
                                 int nrows, int tid) {
#pragma unroll
  for (int u = 0; u < TileCfg<T>::NCH; ++u) {
    int row, col;
    chunk_pos<T, COLMAP>(tid + kThreads * u, row, col);
    if (row0 + row < nrows) {
      r[u] = *reinterpret_cast<const Chunk*>(base + (int64_t)(row0 + row) * sn + col);
    } else {
      r[u] = Chunk{{0u, 0u, 0u, 0u}};
    }
  }
}

// Per-thread view of the 64-row tiles of one [N, 64] matrix: the chunk
// offsets inside a tile are computed once; a tile load is one scalar row
// offset plus NCH vector loads (bounds checks only on a partial last tile).
template <typename T, bool COLMAP>
struct TileReader {
  const T* base;
  int64_t sn;
  int off[TileCfg<T>::NCH];
  int row[TileCfg<T>::NCH];
  __device__ inline void init(const T* b, int64_t sn_, int tid) {
    base = b;
    sn = sn_;
#pragma unroll
    for (int u = 0; u < TileCfg<T>::NCH; ++u) {
      int r, c;
      chunk_pos<T, COLMAP>(tid + kThreads * u, r, c);
      row[u] = r;
      off[u] = r * (int)sn_ + c;
    }
  }
  __device__ inline void load(Chunk (&r)[TileCfg<T>::NCH], int row0, int nrows) const {
    const T* p = base + (int64_t)row0 * sn;
    if (row0 + 64 <= nrows) {
#pragma unroll
      for (int u = 0; u < TileCfg<T>::NCH; ++u) r[u] = *reinterpret_cast<const Chunk*>(p + off[u]);
    } else {
#pragma unroll
      for (int u = 0; u < TileCfg<T>::NCH; ++u)
        r[u] = (row0 + row[u] < nrows) ? *reinterpret_cast<const Chunk*>(p + off[u])
                                       : Chunk{{0u, 0u, 0u, 0u}};
    }
  }
};

template <typename T, bool COLMAP>
__device__ inline void tile_store_rm(T* lds, const Chunk (&r)[TileCfg<T>::NCH], int tid) {
  constexpr int P = TileCfg<T>::PITCH;
#pragma unroll
  for (int u = 0; u < TileCfg<T>::NCH; ++u) {
    int row, col;
    chunk_pos<T, COLMAP>(tid + kThreads * u, row, col);
    if constexpr (TileCfg<T>::kHalf) {
      *reinterpret_cast<Chunk*>(lds + row * P + col) = r[u];
    } else {
      const float* f = reinterpret_cast<const float*>(&r[u]);
#pragma unroll
      for (int t = 0; t < 4; ++t) lds[row * P + col + t] = f[t];
    }
  }
}

// 16-bit only: write the transposed tile lds[col][row] from col-map chunks.
template <typename T>
__device__ inline void tile_store_tr(T* lds, const Chunk (&r)[TileCfg<T>::NCH], int tid) {
  constexpr int P = TileCfg<T>::PITCH;
  static_assert(TileCfg<T>::kHalf, "transposed tiles are for 16-bit types");
#pragma unroll
  for (int u = 0; u < TileCfg<T>::NCH; ++u) {
    int row, col;
    chunk_pos<T, true>(tid + kThreads * u, row, col);
    const T* e = reinterpret_cast<const T*>(&r[u]);
#pragma unroll
    for (int t = 0; t < 8; ++t) lds[(col + t) * P + row] = e[t];
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS tiles.  A tile of 64 rows x 64 elements is written into LDS by
// global_load_lds_dwordx4: each lane's 16 bytes land at lds_base + 16 * lane,
// so the LDS position is set by which lane loads which chunk.  Rows are
// stored unpadded (ROWB bytes); inside a row the 16-byte chunks are permuted
// by an XOR with swz(row).  The MFMA operand reads are ds_read_b128 of one
// chunk column over 16 rows at a time, either 16 consecutive rows or the
// sigma-permuted set {0-3, 8-11, 4-7, 12-15}; the transpose reads (below)
// take two adjacent chunks of 4 consecutive rows per 16 lanes.  With
// 128-byte rows (16-bit types) the swizzle below keeps both kinds of read
// free of bank conflicts whether the LDS serves 128 bytes a cycle (8 lanes of
// a 16-byte read, 16 lanes of an 8-byte read) or 256.
// Rows beyond the valid count are zero-filled with ordinary LDS stores.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <typename T>
struct DTile {
  static constexpr int ROWB = 64 * (int)sizeof(T);  // bytes per row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  static constexpr int BYTES = 64 * ROWB;
  static constexpr int PER_WAVE = 64 * CPR / 64 / 4;  // 64-lane loads per wave per tile
};

// Chunk permutation of row r.  16-bit, with r3..r0 the low row bits: chunk
// bits 2..1 = (r1 r0) ^ r3 and bit 0 = r2 ^ r3.  Bits 2..1 take 4 distinct
// values on every 4 aligned rows (so the chunk pairs {2m, 2m+1} of a
// transpose read's 4 rows are disjoint), bit 2 differs between rows 4k and
// 4k+2 and between 4k+1 and 4k+3 (its 4-chunk spans at 256 bytes), and the
// map is a bijection on rows 0-7, 8-15, {0-3, 8-11}, {4-7, 12-15}, the even
// rows of 16 and the odd rows of 16 (the 16-byte operand reads).
template <typename T>
__device__ __forceinline__ int swz(int r) {
  if constexpr (sizeof(T) == 2) {
    return (((r & 3) ^ ((r >> 3) & 1)) << 1) | (((r >> 2) ^ (r >> 3)) & 1);
  } else {
    return (r + ((r >> 3) << 2)) & (DTile<T>::CPR - 1);
  }
}

// Byte offset of element (r, c) inside a direct tile.
template <typename T>
__device__ __forceinline__ int dt_off(int r, int c) {
  constexpr int EPC = DTile<T>::EPC;
  return r * DTile<T>::ROWB + (((c / EPC) ^ swz<T>(r)) << 4) + (c % EPC) * (int)sizeof(T);
}

// Per-lane plan of the direct loads of one 64 x 64 tile.
template <typename T>
struct DLoader {
  static constexpr int PW = DTile<T>::PER_WAVE;
  int off[PW];   // element offset of the lane's chunk, relative to the tile's first row
  int row[PW];
  int blk0;      // first 64-slot block of this wave
  __device__ __forceinline__ void init(int64_t sn, int w, int lane) {
    blk0 = w * PW;
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int p = (blk0 + u) * 64 + lane;
      const int r = p / DTile<T>::CPR, cs = p % DTile<T>::CPR;
      const int cg = cs ^ swz<T>(r);
      row[u] = r;
      off[u] = r * (int)sn + cg * DTile<T>::EPC;
    }
  }
  // Load rows [0, nvalid) of the tile starting at src; zero the others.
  // A whole tile (the common case, a wave-uniform test) issues its loads
  // with no per-lane condition, so they need no exec-mask branches.
  __device__ __forceinline__ void load(char* lds, const T* src, int nvalid, int lane) const {
    if (nvalid >= 64) {
#pragma unroll
      for (int u = 0; u < PW; ++u)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(src + off[u]),
                                         (lds_void_t*)(lds + (blk0 + u) * 1024), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      char* dst = lds + (blk0 + u) * 1024;
      if (row[u] < nvalid) {
        __builtin_amdgcn_global_load_lds((glb_void_t*)(src + off[u]), (lds_void_t*)dst, 16, 0, 0);
      } else {
        *reinterpret_cast<Chunk*>(dst + lane * 16) = Chunk{{0u, 0u, 0u, 0u}};
      }
    }
  }
};

// Fragment (row, columns [col, col + E)) of a direct tile.
template <typename T>
__device__ __forceinline__ typename MT<T>::frag dfrag(const char* lds, int row, int col) {
  return *reinterpret_cast<const typename MT<T>::frag*>(lds + dt_off<T>(row, col));
}
// Fragment of the transposed view of a direct tile (fp32 only: one element).
__device__ __forceinline__ float dfrag_t32(const char* lds, int row, int col) {
  return *reinterpret_cast<const float*>(lds + dt_off<float>(col, row));
}

// Transposed MFMA operand read straight from a row-major 16-bit direct tile
// with ds_read_b64_tr_b16 (gfx950).  That instruction works on groups of 16
// lanes: input lane i of a group supplies 4 consecutive elements x_i[0..3]
// from its address, and output lane m receives x_{m/4 + 4j}[m % 4] for
// j = 0..3.  If input lane i reads tile row R + i/4 at columns C + 4 (i % 4)
// .. + 3, output lane m therefore holds column C + m of rows R .. R + 3.
// Two such reads (rows +0..3 and +4..7) give the 8 k-values of a 32x32x16
// operand fragment: lane l holds tile column 32 dt + (l % 32) (the MFMA free
// index) and tile rows 16 c + 8 (l / 32) + 0..7 (its k-values of k-step c).
template <typename T>
struct TrReader {
  static_assert(sizeof(T) == 2, "transpose reads are for 16-bit tiles");
  using frag = typename MT<T>::frag;
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  int o[2][2];  // byte offset of read r for column block dt, k-step 0
  // base: byte offset added to every read (a tile placed inside a larger buffer)
  __device__ __forceinline__ void init(int lane, int base = 0) {
    const int i = lane & 15, grp = lane >> 4, h = lane >> 5;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        o[r][dt] =
            base + dt_off<T>(8 * h + 4 * r + (i >> 2), 32 * dt + 16 * (grp & 1) + 4 * (i & 3));
  }
  // operand for column block dt and k-step c (tile rows 16 c .. 16 c + 15)
  __device__ __forceinline__ frag read(const char* lds, int dt, int c) const {
    const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4*)(lds + o[0][dt] + c * 16 * DTile<T>::ROWB));
    const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4*)(lds + o[1][dt] + c * 16 * DTile<T>::ROWB));
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(frag, v);
  }
};

// One 4-byte value per lane, written to lds + 4 * lane (when valid, else 0).
__device__ __forceinline__ void dword_direct(char* lds, const float* src, bool valid, int lane) {
  if (valid) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 4, 0, 0);
  } else {
    reinterpret_cast<float*>(lds)[lane] = 0.f;
  }
}

// Fragment of row `row`, columns [col, col + E) of an RM tile.
template <typename T>
__device__ inline typename MT<T>::frag frag_rm(const T* lds, int row, int col) {
  if constexpr (TileCfg<T>::kHalf) {
    return *reinterpret_cast<const typename MT<T>::frag*>(lds + row * TileCfg<T>::PITCH + col);
  } else {
    return lds[row * TileCfg<T>::PITCH + col];
  }
}
// Fragment of the transposed view: element (row, col..col+E) of X^T where X
// is the staged tile (TR layout for 16-bit, RM read with swapped indices for fp32).
template <typename T>
__device__ inline typename MT<T>::frag frag_t(const T* lds, int row, int col) {
  if constexpr (TileCfg<T>::kHalf) {
    return *reinterpret_cast<const typename MT<T>::frag*>(lds + row * TileCfg<T>::PITCH + col);
  } else {
    return lds[col * TileCfg<T>::PITCH + row];
  }
}

// Fragment straight from HBM: row pointer p, columns [col, col + E).
template <typename T>
__device__ inline typename MT<T>::frag frag_g(const T* p, int col) {
  if constexpr (TileCfg<T>::kHalf) {
    return *reinterpret_cast<const typename MT<T>::frag*>(p + col);
  } else {
    return p[col];
  }
}

// The 16 per-row values of a 32-row subtile in result-element order
// (element e <- v[kappa(h, e)]), read from an fp32 LDS vector.
template <typename T>
__device__ inline void lds_rows16(const float* v, int h, float (&out)[16]) {
  if constexpr (TileCfg<T>::kHalf) {
    const f32x4* a = reinterpret_cast<const f32x4*>(v + 8 * h);
    const f32x4* b = reinterpret_cast<const f32x4*>(v + 16 + 8 * h);
    f32x4 x0 = a[0], x1 = a[1], y0 = b[0], y1 = b[1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      out[t] = x0[t];
      out[4 + t] = x1[t];
      out[8 + t] = y0[t];
      out[12 + t] = y1[t];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = v[kappa<T>(h, e)];
  }
}

// Store 4 consecutive outputs (fp32 values) as dtype T.
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  if constexpr (TileCfg<T>::kHalf) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 x;
    x[0] = MT<T>::from_f(a);
    x[1] = MT<T>::from_f(b);
    x[2] = MT<T>::from_f(c);
    x[3] = MT<T>::from_f(d);
    *reinterpret_cast<v4*>(p) = x;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
}

}  // namespace relpos
