// Grouped (per-expert segment) bf16 MFMA GEMM tiles for gfx950 with pluggable
// operand loaders: plain bf16 rows (optionally gathered through the routing
// permutation), 4-bit stacks decoded on the fly (NF4, NF4 with double-quantised
// absmax, MXFP4) in either orientation, and a rank-r LoRA K-extension that feeds
// the same accumulator before the epilogue.
//
// Two tile shapes.  The small one (BM x BN <= 128 x 128, 256 threads = 4 wave64s laid
// out WM x WN) serves the skinny bf16 products: LoRA-A projections and the LoRA
// weight gradients.  The large one (256 x 256, 512 threads) serves the four 4-bit
// GEMMs of the layer.  Both stage operands in LDS as [rows][64 (+8 pad)] bf16, k
// contiguous, so MFMA fragment reads are 16-byte ds_read_b128 per lane.
#pragma once
#include "common.hpp"

namespace e4b {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS tile row (144 bytes)
constexpr int NTHREADS = 256;

// ---------------------------------------------------------------- tile lookup
// Workgroup `slot` of the grid's M dimension -> (expert, first sorted row, rows)
// over the expert segments described by off[0..E].  Returns false past the end.
struct TileM {
  int e, row0, rows;
};

__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ off, int E, int BMt, int slot,
                                          TileM &t) {
  __shared__ int s_e, s_row0, s_rows;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) s_e = -1;
    int base = 0;
    for (int c = 0; c < E; c += 64) {
      const int ee = c + lane;
      const int cnt = ee < E ? off[ee + 1] - off[ee] : 0;
      const int nt = (cnt + BMt - 1) / BMt;
      int incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      const int excl = incl - nt;
      if (nt > 0 && slot >= base + excl && slot < base + incl) {
        const int mt = slot - base - excl;
        s_e = ee;
        s_row0 = off[ee] + mt * BMt;
        s_rows = min(BMt, cnt - mt * BMt);
      }
      base += __shfl(incl, 63);
      if (base > slot) break;
    }
  }
  __syncthreads();
  t.e = s_e;
  t.row0 = s_row0;
  t.rows = s_rows;
  return t.e >= 0;
}

// ---------------------------------------------------------------- LDS tiles
template <int R>
struct LdsTile {
  uint16_t v[R][LDS_STRIDE];
};

__device__ __forceinline__ void st_lds16(uint16_t *p, u32x4 v) { *(u32x4 *)p = v; }

// ---------------------------------------------------------------- A loader
// Rows of a row-major bf16 matrix (k contiguous).  Tile row i <-> sorted row
// row0 + i; with a gather, the source row is gather[row0 + i] / gdiv.
template <int BR>
struct RowLoader {
  static constexpr int VECS = BR / 32;                 // 16-byte vectors per thread
  static constexpr int TPR = NTHREADS / BR;            // threads per row
  u32x4 buf[VECS];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld, int rows,
                                        int64_t src_row_of_first, const int32_t *__restrict__ gather,
                                        int gdiv, int k0, int kbound) {
    const int i = threadIdx.x / TPR, part = threadIdx.x % TPR;
    const int kk = k0 + part * VECS * 8;
    bool ok = i < rows;
    int64_t src = 0;
    if (ok) src = gather ? (int64_t)(gather[src_row_of_first + i] / gdiv) : src_row_of_first + i;
    const uint16_t *p = base + src * ld + kk;
#pragma unroll
    for (int v = 0; v < VECS; ++v) {
      if (ok && kk + v * 8 < kbound)
        buf[v] = *(const u32x4 *)(p + v * 8);
      else
        buf[v] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int i = threadIdx.x / TPR, part = threadIdx.x % TPR;
#pragma unroll
    for (int v = 0; v < VECS; ++v) st_lds16(&t.v[i][part * VECS * 8 + v * 8], buf[v]);
  }
};

// ---------------------------------------------------------------- B row mapping
// Tile row lr of the B operand -> output column (weight row) index.
// Plain: n0 + lr.  SwiGLU: rows interleave 32 gate rows and 32 up rows so that a
// wave's two 32-column MFMA tiles hold gate and up of the same h column.
struct RowMap {
  int n0, I;
  bool swiglu;
  // Returns a row past every bound when the tile row falls beyond the last h column.
  __device__ __forceinline__ int operator()(int lr) const {
    if (!swiglu) return n0 + lr;
    const int blk = lr >> 5, o = lr & 31;
    const int hcol = n0 + (blk >> 1) * 32 + o;
    return hcol < I ? ((blk & 1) ? I : 0) + hcol : 0x7fffffff;
  }
};

// ---------------------------------------------------------------- dense B, NK
// B tile rows n (mapped) of a per-expert bf16 matrix [N, ld] (k contiguous).
template <int BR>
struct DenseNKLoader {
  static constexpr int VECS = BR / 32;
  static constexpr int TPR = NTHREADS / BR;
  u32x4 buf[VECS];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld,
                                        const RowMap &map, int N, int k0, int kbound) {
    const int i = threadIdx.x / TPR, part = threadIdx.x % TPR;
    const int n = map(i);
    const int kk = k0 + part * VECS * 8;
    const uint16_t *p = base + (int64_t)n * ld + kk;
#pragma unroll
    for (int v = 0; v < VECS; ++v) {
      if (n < N && kk + v * 8 < kbound)
        buf[v] = *(const u32x4 *)(p + v * 8);
      else
        buf[v] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int i = threadIdx.x / TPR, part = threadIdx.x % TPR;
#pragma unroll
    for (int v = 0; v < VECS; ++v) st_lds16(&t.v[i][part * VECS * 8 + v * 8], buf[v]);
  }
};

// ---------------------------------------------------------------- K-major loader
// Tile rows a (BR of them) x 64 k where the source is row-major [k][a] (a
// contiguous): source row of k is row0 + k (or gather[row0 + k] / gdiv).  Thread
// -> 4 k rows x (BR/16) a columns, transposed into LDS.  Used by the segmented
// weight-gradient GEMMs whose reduction runs over routed rows.
template <int BR>
struct KMajorLoader {
  static constexpr int AW = BR / 16;  // a columns per thread: 8 (BR=128) or 4 (BR=64)
  static constexpr int NW = AW / 2;   // 32-bit words per source row
  uint32_t w[4][NW];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld, int a0,
                                        int Na, int row0, int krows, const int32_t *__restrict__ gather,
                                        int gdiv, int k0) {
    const int kb = threadIdx.x >> 4, ab = threadIdx.x & 15;
    const int a = a0 + ab * AW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + kb * 4 + i;
      const bool ok = kk < krows && a < Na;
      int64_t src = 0;
      if (ok) src = gather ? (int64_t)(gather[row0 + kk] / gdiv) : (int64_t)(row0 + kk);
      const uint32_t *p = (const uint32_t *)(base + src * ld + a);
#pragma unroll
      for (int j = 0; j < NW; ++j) w[i][j] = ok ? p[j] : 0u;
    }
  }
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int kb = threadIdx.x >> 4, ab = threadIdx.x & 15;
#pragma unroll
    for (int c = 0; c < AW; ++c) {
      const int sh = (c & 1) * 16, wi = c >> 1;
      const uint32_t v0 = (w[0][wi] >> sh) & 0xffffu, v1 = (w[1][wi] >> sh) & 0xffffu;
      const uint32_t v2 = (w[2][wi] >> sh) & 0xffffu, v3 = (w[3][wi] >> sh) & 0xffffu;
      u32x2 pk{v0 | (v1 << 16), v2 | (v3 << 16)};
      *(u32x2 *)&t.v[ab * AW + c][kb * 4] = pk;
    }
  }
};

// ---------------------------------------------------------------- MFMA core
template <int BM, int BN, int WM, int WN>
struct Mma {
  static constexpr int TM = BM / (WM * 32);
  static constexpr int TN = BN / (WN * 32);
  f32x16 acc[TM][TN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }
  __device__ __forceinline__ void step(const LdsTile<BM> &A, const LdsTile<BN> &B, int ksteps) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 31, kg = (lane >> 5) * 8;
    for (int ks = 0; ks < ksteps; ++ks) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *(const bf16x8 *)&A.v[(wm * TM + i) * 32 + r][ks * 16 + kg];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *(const bf16x8 *)&B.v[(wn * TN + j) * 32 + r][ks * 16 + kg];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // Visit every accumulator element with its tile-local (row, col).
  template <class F>
  __device__ __forceinline__ void for_each(F &&f) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = (wm * TM + i) * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int col = (wn * TN + j) * 32 + (lane & 31);
          f(row, col, acc[i][j][v]);
        }
  }
};

}  // namespace e4b

// =====================================================================================
// Large-tile variant: 256 x 256 output per workgroup, 512 threads = 8 wave64s laid out
// 2 (M) x 4 (N), each wave owning 128 x 64 as 4 x 2 tiles of 32x32x16 MFMAs.  A and the
// decoded B operand are double-buffered in LDS (2 x 2 x 36 KB), so each K slab of 64
// needs one barrier: while the MFMAs consume slab s, the next slab's global loads are
// in flight and are then decoded and written into the other buffer.
// =====================================================================================
namespace e4b {

constexpr int L_BM = 256, L_BN = 256, L_THREADS = 512;

struct LTile {
  uint16_t v[L_BM][LDS_STRIDE];
};

// A: 256 rows x 64 k, row-major source (optionally gathered).  Thread -> rows
// tid/8 + 64*i (i < 4), 16-byte chunk tid%8: each load instruction of a wave covers 8
// full 128-byte row segments.
struct LRowLoader {
  u32x4 buf[4];
  int64_t src[4];
  bool ok[4];
  __device__ __forceinline__ void init(int rows, int64_t row0, const int32_t *__restrict__ gather,
                                       int gdiv, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (threadIdx.x >> 3) + 64 * i;
      ok[i] = r < rows;
      int64_t s = 0;
      if (ok[i]) s = gather ? (int64_t)(gather[row0 + r] / gdiv) : row0 + r;
      src[i] = s * ld + (threadIdx.x & 7) * 8;
    }
  }
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int k0, int kbound) {
    const int kk = k0 + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      buf[i] = (ok[i] && kk < kbound) ? *(const u32x4 *)(base + src[i] + k0) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void store(LTile &t) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st_lds16(&t.v[(threadIdx.x >> 3) + 64 * i][(threadIdx.x & 7) * 8], buf[i]);
  }
};

// B from a 4-bit stack stored [N, K] (K contiguous): thread -> (tile row tid/2, 32-k half).
struct LQuantNK {
  u32x4 codes;
  float scale;
  int64_t elem;  // flat element index of this thread's first element at k0 = 0
  bool ok;
  __device__ __forceinline__ void init(const QStack &q, int e, const RowMap &map, int Nrows) {
    const int n = map(threadIdx.x >> 1);
    ok = n < Nrows;
    elem = ((int64_t)e * q.N + (ok ? n : 0)) * q.K + (threadIdx.x & 1) * 32;
  }
  __device__ __forceinline__ void fetch(const QStack &q, int k0, const DecodeTables &tb) {
    if (ok) {
      const int64_t el = elem + k0;
      codes = *(const u32x4 *)(q.codes + el / 2);
      scale = q.fmt == FMT_MXFP4 ? e8m0_to_f32(((const uint8_t *)q.scale)[el >> 5])
                                 : nf4_block_absmax(q, el >> 6, tb);
    } else {
      codes = u32x4{0, 0, 0, 0};
      scale = 0.0f;
    }
  }
  __device__ __forceinline__ void store(LTile &t, int fmt, const DecodeTables &tb) {
    uint16_t *dst = &t.v[threadIdx.x >> 1][(threadIdx.x & 1) * 32];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      st_lds16(dst + w * 8, fmt == FMT_MXFP4 ? mxfp4_word_to_bf16(codes[w], scale)
                                             : nf4_word_to_bf16(codes[w], scale, tb));
  }
};

// B from a 4-bit stack reduced over its STORED row axis: tile rows = 256 output columns
// (stored columns n0..n0+255), k = 64 stored rows.  Thread -> 2 stored rows x 16 stored
// columns (one 8-byte code load and one block scale per row), decoded, then each
// column's two k values are packed into one dword and written transposed.
struct LQuantKN {
  u32x2 w[2];
  float scale[2];
  int64_t elem;  // flat element index of (stored row 2*kb, column n) at k0 = 0
  bool ok;
  __device__ __forceinline__ void init(const QStack &q, int e, int n0, int Nout) {
    const int kb = threadIdx.x >> 4, nb = threadIdx.x & 15;
    const int n = n0 + nb * 16;
    ok = n < Nout;
    elem = ((int64_t)e * q.N + kb * 2) * q.K + (ok ? n : 0);
  }
  __device__ __forceinline__ void fetch(const QStack &q, int k0, const DecodeTables &tb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (ok) {
        const int64_t el = elem + (int64_t)(k0 + i) * q.K;
        w[i] = *(const u32x2 *)(q.codes + el / 2);
        scale[i] = q.fmt == FMT_MXFP4 ? e8m0_to_f32(((const uint8_t *)q.scale)[el >> 5])
                                      : nf4_block_absmax(q, el >> 6, tb);
      } else {
        w[i] = u32x2{0, 0};
        scale[i] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(LTile &t, int fmt, const DecodeTables &tb) {
    const int kb = threadIdx.x >> 4, nb = threadIdx.x & 15;
    u32x4 d[2][2];  // [row][word]: 8 bf16 of columns word*8 .. +8
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        d[i][h] = fmt == FMT_MXFP4 ? mxfp4_word_to_bf16(w[i][h], scale[i])
                                   : nf4_word_to_bf16(w[i][h], scale[i], tb);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t pk = __builtin_amdgcn_perm(d[1][c >> 3][(c & 7) >> 1], d[0][c >> 3][(c & 7) >> 1], sel);
      *(uint32_t *)&t.v[nb * 16 + c][kb * 2] = pk;
    }
  }
};

// Dense bf16 B rows (LoRA K-extension): tile row lr = tid/2 -> weight row map(lr),
// 32-element half tid%2, zero past kbound.
struct LDenseNK {
  u32x4 buf[4];
  const uint16_t *row;
  bool ok;
  __device__ __forceinline__ void init(const uint16_t *__restrict__ base, int64_t ld, const RowMap &map,
                                       int Nrows) {
    const int n = map(threadIdx.x >> 1);
    ok = n < Nrows;
    row = base + (int64_t)(ok ? n : 0) * ld + (threadIdx.x & 1) * 32;
  }
  __device__ __forceinline__ void fetch(int k0, int kbound) {
    const int kk = k0 + (threadIdx.x & 1) * 32;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      buf[v] = (ok && kk + 8 * v < kbound) ? *(const u32x4 *)(row + k0 + 8 * v) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void store(LTile &t) {
    uint16_t *dst = &t.v[threadIdx.x >> 1][(threadIdx.x & 1) * 32];
#pragma unroll
    for (int v = 0; v < 4; ++v) st_lds16(dst + 8 * v, buf[v]);
  }
};

// MFMA core of the large tile: wave (wm, wn) owns rows wm*128.., cols wn*64..
struct LMma {
  f32x16 acc[4][2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }
  __device__ __forceinline__ void step(const LTile &A, const LTile &B, int ksteps) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int r = lane & 31, kg = (lane >> 5) * 8;
    for (int ks = 0; ks < ksteps; ++ks) {
      bf16x8 a[4], b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8 *)&B.v[wn * 64 + j * 32 + r][ks * 16 + kg];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8 *)&A.v[wm * 128 + i * 32 + r][ks * 16 + kg];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // tile-local (row, col) of accumulator element (i, j, v) for this lane
  __device__ __forceinline__ static int row_of(int i, int v) {
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 2;
    return wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
  }
  __device__ __forceinline__ static int col_of(int j) {
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 3;
    return wn * 64 + j * 32 + (lane & 31);
  }
};

}  // namespace e4b
