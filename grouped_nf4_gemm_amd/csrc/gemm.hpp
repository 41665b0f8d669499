// Grouped (per-expert segment) bf16 MFMA GEMM tiles for gfx950 with pluggable
// operand loaders: plain bf16 rows (optionally gathered through the routing
// permutation), 4-bit stacks decoded on the fly (NF4, NF4 with double-quantised
// absmax, MXFP4) in either orientation, and a rank-r LoRA K-extension that feeds
// the same accumulator before the epilogue.
//
// Tile: BM x BN output, K slabs of 64, 256 threads = 4 wave64s laid out WM x WN,
// each wave owning (BM/WM) x (BN/WN) as 32x32 v_mfma_f32_32x32x16_bf16 tiles.
// Both operands are staged in LDS as [rows][64 (+8 pad)] bf16, k contiguous, so
// the MFMA fragment reads are 16-byte ds_read_b128 per lane.  Global loads of the
// next slab are issued before the MFMAs of the current one (register prefetch).
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
  __device__ __forceinline__ int operator()(int lr) const {
    if (!swiglu) return n0 + lr;
    const int blk = lr >> 5, o = lr & 31;
    return ((blk & 1) ? I : 0) + n0 + (blk >> 1) * 32 + o;
  }
};

// ---------------------------------------------------------------- quant B, NK
// B tile of 128 weight rows x 64 k from a 4-bit stack stored [N, K] (K contiguous).
// Thread -> (row, 32-element half); one 16-byte code load, one block scale.
struct QuantNKLoader {
  u32x4 codes;
  float scale;
  __device__ __forceinline__ void fetch(const QStack &q, int e, const RowMap &map, int N, int k0) {
    const int lr = threadIdx.x >> 1, part = threadIdx.x & 1;
    const int n = map(lr);
    if (n < N) {
      const int64_t row = (int64_t)e * q.N + n;
      const int64_t elem = row * q.K + k0 + part * 32;
      codes = *(const u32x4 *)(q.codes + elem / 2);
      if (q.fmt == FMT_MXFP4)
        scale = e8m0_to_f32(((const uint8_t *)q.scale)[elem >> 5]);
      else
        scale = nf4_block_absmax(q, elem >> 6);
    } else {
      codes = u32x4{0, 0, 0, 0};
      scale = 0.0f;
    }
  }
  __device__ __forceinline__ void store(LdsTile<128> &t, int fmt, const float *cb) {
    const int lr = threadIdx.x >> 1, part = threadIdx.x & 1;
    uint16_t *dst = &t.v[lr][part * 32];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4 v = fmt == FMT_MXFP4 ? mxfp4_word_to_bf16(codes[w], scale)
                                 : nf4_word_to_bf16(codes[w], scale, cb);
      st_lds16(dst + w * 8, v);
    }
  }
};

// ---------------------------------------------------------------- quant B, KN
// B tile for a reduction over the STORED row axis of a 4-bit stack [Ns, Ks]:
// tile rows = 128 output columns (stored column index n0 + lr), tile k = 64 stored
// rows k0..k0+63.  Thread -> 4 stored rows x 8 stored columns (one code word per
// row), decoded then transposed into LDS as 8 rows x 4 k (8-byte writes).
struct QuantKNLoader {
  uint32_t w[4];
  float scale[4];
  __device__ __forceinline__ void fetch(const QStack &q, int e, int n0, int Nout, int k0) {
    const int kb = threadIdx.x >> 4, nb = threadIdx.x & 15;
    const int n = n0 + nb * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = k0 + kb * 4 + i;
      if (n < Nout) {
        const int64_t elem = ((int64_t)e * q.N + kr) * q.K + n;
        w[i] = *(const uint32_t *)(q.codes + elem / 2);
        if (q.fmt == FMT_MXFP4)
          scale[i] = e8m0_to_f32(((const uint8_t *)q.scale)[elem >> 5]);
        else
          scale[i] = nf4_block_absmax(q, elem >> 6);
      } else {
        w[i] = 0;
        scale[i] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(LdsTile<128> &t, int fmt, const float *cb) {
    const int kb = threadIdx.x >> 4, nb = threadIdx.x & 15;
    u32x4 d[4];  // d[i] = 8 bf16 of stored row i, columns nb*8 .. +8
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = fmt == FMT_MXFP4 ? mxfp4_word_to_bf16(w[i], scale[i]) : nf4_word_to_bf16(w[i], scale[i], cb);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int sh = (c & 1) * 16, wi = c >> 1;
      const uint32_t v0 = (d[0][wi] >> sh) & 0xffffu, v1 = (d[1][wi] >> sh) & 0xffffu;
      const uint32_t v2 = (d[2][wi] >> sh) & 0xffffu, v3 = (d[3][wi] >> sh) & 0xffffu;
      u32x2 pk{v0 | (v1 << 16), v2 | (v3 << 16)};
      *(u32x2 *)&t.v[nb * 8 + c][kb * 4] = pk;
    }
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
