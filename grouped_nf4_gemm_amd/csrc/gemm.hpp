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
                                          TileM &t, int *sh /* 3 ints of LDS */) {
  int &s_e = sh[0], &s_row0 = sh[1], &s_rows = sh[2];
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
  // the same for every lane: kept in scalar registers (buffer resources built from them
  // must be wave-uniform)
  t.e = __builtin_amdgcn_readfirstlane(s_e);
  t.row0 = __builtin_amdgcn_readfirstlane(s_row0);
  t.rows = __builtin_amdgcn_readfirstlane(s_rows);
  return t.e >= 0;
}

// The same lookup done by each wave on its own, with no LDS and no barrier; the result is
// wave-uniform (scalar registers).
__device__ __forceinline__ bool find_tile_wave(const int32_t *__restrict__ off, int E, int BMt, int slot, TileM &t) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c = 0; c < E; c += 64) {
    const int ee = c + lane;
    const int o0 = ee < E ? off[ee] : 0;
    const int cnt = ee < E ? off[ee + 1] - o0 : 0;
    const int nt = (cnt + BMt - 1) / BMt;
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int excl = incl - nt;
    const uint64_t hit = __ballot(nt > 0 && slot >= base + excl && slot < base + incl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int e = __builtin_amdgcn_readfirstlane(__shfl(ee, src));
      const int mt = slot - base - __builtin_amdgcn_readfirstlane(__shfl(excl, src));
      const int n = __builtin_amdgcn_readfirstlane(__shfl(cnt, src));
      t.e = e;
      t.row0 = __builtin_amdgcn_readfirstlane(__shfl(o0, src)) + mt * BMt;  // no second load
      t.rows = min(BMt, n - mt * BMt);
      return true;
    }
    base += __shfl(incl, 63);
    if (base > slot) break;
  }
  return false;
}

// ---------------------------------------------------------------- LDS tiles
template <int R>
struct LdsTile {
  uint16_t v[R][LDS_STRIDE];
};

__device__ __forceinline__ void st_lds16(uint16_t *p, u32x4 v) { *(u32x4 *)p = v; }

// ---------------------------------------------------------------- A loader
// Rows of a row-major bf16 matrix (k contiguous).  Tile row i <-> sorted row
// row0 + i; with a gather, the source row is gather[row0 + i] / gdiv.  Eight consecutive
// lanes read the 128 bytes of one row's slab (one cache line per eight lanes); pass v takes
// tile rows 32 v .. 32 v + 31.  The source rows are resolved once per tile (init).  Each row
// is read once per launch: non-temporal loads.
template <int BR>
struct RowLoader {
  static constexpr int VECS = BR / 32;  // passes (16-byte vectors per thread)
  u32x4 buf[VECS];
  int64_t src[VECS];  // element offset of the pass's source row, or -1
  __device__ __forceinline__ void init(int64_t ld, int rows, int64_t row0, const int32_t *__restrict__ gather,
                                       int gdiv) {
    const int r = threadIdx.x >> 3;
#pragma unroll
    for (int v = 0; v < VECS; ++v) {
      const int i = v * 32 + r;
      src[v] = i < rows ? (gather ? (int64_t)(gather[row0 + i] / gdiv) : row0 + i) * ld : -1;
    }
  }
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int k0, int kbound) {
    const int kk = k0 + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int v = 0; v < VECS; ++v)
      buf[v] = (src[v] >= 0 && kk < kbound) ? __builtin_nontemporal_load((const u32x4 *)(base + src[v] + kk)) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int r = threadIdx.x >> 3, c = threadIdx.x & 7;
#pragma unroll
    for (int v = 0; v < VECS; ++v) st_lds16(&t.v[v * 32 + r][c * 8], buf[v]);
  }
};

// ---------------------------------------------------------------- B row mapping
// Tile row lr of the B operand -> output column (weight row) index.
// Plain: n0 + lr.  Gate/up: tile rows alternate 32 gate rows and 32 up rows so that a
// wave's two 32-column MFMA tiles hold gate and up of the same h column.
struct RowMap {
  int n0, I;
  bool swiglu;
  bool interleaved;  // gate/up rows interleaved (2c, 2c + 1) instead of halves
  // Returns a row past every bound when the tile row falls beyond the last h column.
  __device__ __forceinline__ int operator()(int lr) const {
    if (!swiglu) return n0 + lr;
    const int blk = lr >> 5, o = lr & 31;
    const int hcol = n0 + (blk >> 1) * 32 + o;
    return hcol < I ? gate_up_row(hcol, blk & 1, interleaved, I) : 0x7fffffff;
  }
};

// ---------------------------------------------------------------- dense B, NK
// B tile rows n (mapped) of a per-expert bf16 matrix [N, ld] (k contiguous), read like
// RowLoader: eight lanes per row, pass v takes tile rows 32 v .. 32 v + 31.
template <int BR>
struct DenseNKLoader {
  static constexpr int VECS = BR / 32;
  u32x4 buf[VECS];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld,
                                        const RowMap &map, int N, int k0, int kbound) {
    const int r = threadIdx.x >> 3, kk = k0 + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int v = 0; v < VECS; ++v) {
      const int n = map(v * 32 + r);
      buf[v] = (n < N && kk < kbound) ? *(const u32x4 *)(base + (int64_t)n * ld + kk) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int r = threadIdx.x >> 3, c = threadIdx.x & 7;
#pragma unroll
    for (int v = 0; v < VECS; ++v) st_lds16(&t.v[v * 32 + r][c * 8], buf[v]);
  }
};

// ---------------------------------------------------------------- K-major loader
// Tile rows a (BR of them) x 64 k where the source is row-major [k][a] (a
// contiguous): source row of k is row0 + k (or gather[row0 + k] / gdiv).  Thread
// -> 4 k rows x (BR/16) a columns, transposed into LDS.  Row lengths and column offsets
// are multiples of 8 elements (LoRA ranks are), so each row piece is one vector load.  Used by the segmented
// weight-gradient GEMMs whose reduction runs over routed rows.
template <int BR>
struct KMajorLoader {
  static constexpr int AW = BR / 16;  // a columns per thread: 8 (BR=128) or 4 (BR=64)
  static constexpr int NW = AW / 2;   // 32-bit words per source row
  uint32_t w[4][NW];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld, int a0,
                                        int Na, int row0, int krows, const int32_t *__restrict__ gather,
                                        int gdiv, int k0) {
    const int kb = threadIdx.x & 15, ab = threadIdx.x >> 4;
    const int a = a0 + ab * AW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + kb * 4 + i;
      const bool ok = kk < krows && a < Na;
      int64_t src = 0;
      if (ok) src = gather ? (int64_t)(gather[row0 + kk] / gdiv) : (int64_t)(row0 + kk);
      // one 16-byte (or 8-byte) load per source row: a and ld are multiples of 8 elements
      const uint16_t *p = base + src * ld + a;
      if constexpr (NW == 4) {
        const u32x4 v = ok ? *(const u32x4 *)p : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) w[i][j] = v[j];
      } else {
        const u32x2 v = ok ? *(const u32x2 *)p : u32x2{0, 0};
#pragma unroll
        for (int j = 0; j < NW; ++j) w[i][j] = v[j];
      }
    }
  }
  // lanes 16j .. 16j+15 share a column group and cover the 64 k of a tile row: each
  // 16-lane LDS pass writes 128 contiguous bytes of one row (no bank conflicts)
  __device__ __forceinline__ void store(LdsTile<BR> &t) {
    const int kb = threadIdx.x & 15, ab = threadIdx.x >> 4;
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
// Large-tile building blocks: 256 x 256 outputs per workgroup, accumulated by eight waves
// (two per SIMD) of 128 x 64 each as 4 x 2 tiles of 32x32x16 MFMAs.  K runs in slabs of
// 64: A rows arrive by direct-to-LDS buffer loads, the 4-bit B operand by buffer loads into
// registers two slabs ahead, decoded and written into LDS a slab before it is used (the
// kernels that assemble these are in kernels.hip).  Buffer loads keep a wave-uniform
// 64-bit base in SGPRs and a 32-bit per-lane offset (the slab step goes in the scalar
// offset), and rows past the end of a segment read as zero through the buffer's range check.
// =====================================================================================
namespace e4b {

// Wave w (< 8) of the accumulating waves owns rows (w >> 2) * 128 .. +127 and columns
// (w & 3) * 64 .. +63 of the tile.
constexpr int L_BM = 256, L_BN = 256, L_THREADS = 512;
constexpr uint32_t OOB = 0x80000000u;  // per-lane offset that reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
// Packed weight codes are read exactly once per launch in the decode kernels: load them with
// the non-temporal cache policy so they do not evict the activations and scales that are reused.
constexpr int CODE_LOAD_CPOL = 2;
__device__ __forceinline__ u32x4 bload128_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CODE_LOAD_CPOL));
}
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint16_t v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void bstore32(__amdgpu_buffer_rsrc_t r, float v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, 0, 0);
}
// Lane pairs: lanes 2m and 2m+1 trade a dword (DPP quad_perm [1,0,3,2]; every lane of the
// wave is active here, so no lane keeps an old value).
__device__ __forceinline__ uint32_t lane_swap1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
// Two bf16 outputs per 4-byte store.  In the MFMA accumulator layout a lane holds one
// column; lanes 2m and 2m+1 hold columns c and c+1 of the same rows.  x0 and x1 are this
// lane's values of rows r and r+1, rounded to bf16 as one dword (row r low); after the swap
// one byte permute gives the even lane row r at columns (c, c+1) and the odd lane row r+1
// at columns (c-1, c).  The permute is its own inverse on the pairs (unpair_bf16_f32).
__device__ __forceinline__ uint32_t pair_perm(uint32_t mine, bool odd) {
  // v_perm_b32 bytes 0-3 select from the second operand, 4-7 from the first
  return __builtin_amdgcn_perm(lane_swap1(mine), mine, odd ? 0x03020706u : 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_bf16(float x0, float x1, bool odd) {
  return pair_perm(pack_bf16x2(x0, x1), odd);
}
// The tile epilogues' outputs (h, G, O, dG, dXp) are each larger than the last-level cache
// and are read back only by later kernels: their stores carry the non-temporal hint (cache
// policy bit 1, `nt`), which measured 1-2% faster on the GEMMs that write them.
constexpr int EPI_STORE_CPOL = 2;
__device__ __forceinline__ void bstore32u(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, 0, EPI_STORE_CPOL);
}
// The same pairing for fp32 outputs: two columns per 8-byte store.
__device__ __forceinline__ void bstore_pair_f32(__amdgpu_buffer_rsrc_t r, float x0, float x1, bool odd,
                                                uint32_t voff) {
  const float send = odd ? x0 : x1;
  const float recv = __uint_as_float(lane_swap1(__float_as_uint(send)));
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 d = {(int)__float_as_uint(odd ? recv : x0), (int)__float_as_uint(odd ? x1 : recv)};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)voff, 0, EPI_STORE_CPOL);
}
// The inverse for loads: the even lane loaded row r and the odd lane row r+1, each as the
// dword of columns (c, c+1) of its pair; gives this lane's column at rows r and r+1 as fp32.
__device__ __forceinline__ void unpair_bf16_f32(uint32_t d, bool odd, float &f0, float &f1) {
  const uint32_t x = pair_perm(d, odd);  // rows r (low) and r+1 (high) of this lane's column
  f0 = __uint_as_float(x << 16);
  f1 = __uint_as_float(x & 0xffff0000u);
}

// Buffer over rows row0 .. row0 + rows - 1 of a row-major matrix with ld elements of esize
// bytes per row: per-lane offsets past the last row read zero / are not written.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *base, int64_t row0, int rows, int64_t ld,
                                                            int esize) {
  return make_rsrc((const char *)base + row0 * ld * esize, (uint32_t)(rows * ld * esize));
}

// Operand tiles of 64-wide slabs: rows of 64 bf16 (128 bytes, no padding) whose eight
// 16-byte chunks sit at chunk ^ ((row >> 1) & 7).  LDS serves 16 lanes of a 16-byte access
// per pass, over 64 banks: the 16 rows one fragment read touches then hit 16 distinct
// groups of 4 banks (row parity picks the bank half, the swizzle the group), and the DMA
// writes (lane t -> bytes 16t of a 1 KB block) stay conflict-free as well.
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
struct ATile {
  uint16_t v[L_BM * BK];
};
__device__ __forceinline__ int aswz(int row, int chunk) { return row * BK + (swz_chunk(row, chunk) << 3); }
struct LTile {  // [256 n][64 k] bf16, k contiguous, chunks swizzled as the A tile
  uint16_t v[L_BN][BK];
};
__device__ __forceinline__ int bswz(int row, int chunk) { return swz_chunk(row, chunk) << 3; }
// [64 k][256 n] bf16, n contiguous, no padding.  Row k keeps its 16-byte chunk c (8 columns)
// at c ^ f(k & 3) ^ ((c >> 3) & 3), f = {0, 5, 10, 15}.  All three access patterns then touch
// distinct banks, whether a pass serves 128 or 256 bytes (checked by enumeration):
//  - transposing fragment reads: a pass covers rows 4m .. 4m+3 and an aligned pair (16
//    lanes) or quad (32 lanes) of chunks; bits 1-2 and bits 2-3 of f differ between the four
//    rows, and the (c >> 3) & 3 term is the same for the whole pass;
//  - 4-bit decode stores (LQuantKN): lane l of a wave writes chunk 8 (l & 3) + part of row
//    l >> 2, so a pass covers 2 or 4 rows x the four 64-column blocks;
//  - 8-bit decode stores (LQuantKN8): 8 lanes write chunks 4p + part (p = 0..7) of one row.
// f is linear in the bits of k, so rows 4 apart share it (fixed offsets between k-steps).
struct LTileKN {
  uint16_t v[BK][L_BN];
};
__device__ __forceinline__ int knswz(int k, int col) {
  const int c = col >> 3;
  const int f = ((k & 1) ? 5 : 0) ^ ((k & 2) ? 10 : 0);
  return ((c ^ f ^ ((c >> 3) & 3)) << 3) | (col & 7);
}
// [64 k][256 n] bf16 without padding, for B tiles that direct-to-LDS loads fill from a
// bf16 copy of a stack stored [K rows][N]: row k keeps its 16-byte chunk c at c ^ ((k & 3)
// << 2).  A 32-lane pass of the transposing fragment read covers 4 rows x 4 chunks, which
// the swizzle spreads over 16 distinct groups of 4 banks; the loads write whole 1 KB blocks.
struct LTileKD {
  uint16_t v[BK][L_BN];
};
__device__ __forceinline__ int kdswz(int k, int col) {
  return (((col >> 3) ^ ((k & 3) << 2)) << 3) | (col & 7);
}
// one LDS buffer holds any of the B tile layouts
union BBuf {
  LTile nk;
  LTileKN kn;
  LTileKD kd;
};

// A: 256 rows x 64 k of a row-major bf16 matrix (optionally gathered rows) loaded
// straight into LDS by NW waves.  Loading wave v (0 .. NW-1), instruction i fills the 1 KB
// block of rows 8*(NI*v+i) .. +7: lane l reads row 8*(NI*v+i) + l/8, the logical chunk that
// lands at physical chunk l%8.
template <int NW>
struct LDirectAN {
  static constexpr int NI = 32 / NW;  // 1 KB blocks per loading wave
  uint32_t voff[NI];
  __device__ __forceinline__ void init(int v, int rows, int64_t row0, const int32_t *__restrict__ gather,
                                       int gdiv, int64_t ld) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (v * NI + i) * 8 + (l >> 3);
      const int lc = swz_chunk(r, l & 7);  // the swizzle is its own inverse
      if (r < rows) {
        const int64_t s = gather ? (int64_t)(gather[row0 + r] / gdiv) : row0 + r;
        voff[i] = (uint32_t)((s * ld + lc * 8) * 2);
      } else {
        voff[i] = OOB;
      }
    }
  }
  // soff: byte offset of the slab's first column (OOB: the slab reads as zero)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, ATile &t, uint32_t soff, int v) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void *)&t.v[(v * NI + i) * 8 * BK], 16, voff[i], soff, 0, 0);
  }
};
// Direct-to-LDS loads of a [256][64] bf16 tile in the A (or NK B) layout from a dense
// row-major matrix: tile row r <- matrix row src(r) (negative: zero), columns [k0, k0 + 64)
// of which those at or past kbound read as zero.  NW loading waves (v: this wave).
template <int NW>
struct LDirectRows {
  static constexpr int NI = 32 / NW;
  uint32_t voff[NI];
  template <class Src>
  __device__ __forceinline__ void init(int v, Src src, int64_t ld, int k0, int kbound) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (v * NI + i) * 8 + (l >> 3);
      const int lc = swz_chunk(r, l & 7);  // the swizzle is its own inverse
      const int64_t row = src(r);
      voff[i] = (row >= 0 && k0 + lc * 8 < kbound) ? (uint32_t)((row * ld + k0 + lc * 8) * 2) : OOB;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint16_t *tile, int v) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void *)&tile[(v * NI + i) * 8 * BK], 16, voff[i], 0, 0, 0);
  }
};
// All eight waves of a 512-thread workgroup load.
struct LDirectA : LDirectAN<8> {
  __device__ __forceinline__ void init(int rows, int64_t row0, const int32_t *__restrict__ gather, int gdiv,
                                       int64_t ld) {
    LDirectAN<8>::init(threadIdx.x >> 6, rows, row0, gather, gdiv, ld);
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, ATile &t, uint32_t soff) {
    LDirectAN<8>::issue(r, t, soff, threadIdx.x >> 6);
  }
};

// B rows of a bf16 copy of a stack stored [N, K] (K contiguous) straight into an [n][k] tile,
// with the A tile's block mapping; tile row lr holds weight row map(lr).  Rows past Nrows
// read as zero.
struct LDirectBNK {
  uint32_t voff[4];
  __device__ __forceinline__ void init(const RowMap &map, int Nrows, int64_t K) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (w * 4 + i) * 8 + (l >> 3);
      const int n = map(r);
      voff[i] = n < Nrows ? (uint32_t)(((int64_t)n * K + swz_chunk(r, l & 7) * 8) * 2) : OOB;
    }
  }
  // soff: byte offset of the slab's first column (OOB: the slab reads as zero)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, LTile &t, uint32_t soff) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void *)&t.v[(w * 4 + i) * 8][0], 16, voff[i], soff, 0, 0);
  }
};
// B of a bf16 copy of a stack stored [Krows, Ncols] reduced over its stored rows, into a
// [64 k][256 n] tile (LTileKD): wave w, load i fills stored rows 2 (4w + i) and +1 of the
// slab; lane l reads row 2 (4w + i) + l / 32, the chunk that lands at physical chunk l % 32.
// Columns past Ncols read as zero.
struct LDirectBKN {
  uint32_t voff[4];
  __device__ __forceinline__ void init(int n0, int Ncols) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = (w * 4 + i) * 2 + (l >> 5);
      const int col = n0 + (((l & 31) ^ ((k & 3) << 2)) << 3);
      voff[i] = col < Ncols ? (uint32_t)(((int64_t)k * Ncols + col) * 2) : OOB;
    }
  }
  // soff: byte offset of the slab's first stored row (OOB: the slab reads as zero)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, LTileKD &t, uint32_t soff) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void *)&t.v[(w * 4 + i) * 2][0], 16, voff[i], soff, 0, 0);
  }
};

// Register-staged A rows for the LoRA extension (rows of ld elements, zero past kbound),
// written into the same swizzled layout.
struct LRegA {
  u32x4 buf[4];
  __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int64_t ld, int rows, int64_t row0,
                                       int k0, int kbound) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (w * 4 + i) * 8 + (l >> 3);
      const int kk = k0 + swz_chunk(r, l & 7) * 8;
      buf[i] = (r < rows && kk < kbound) ? *(const u32x4 *)(base + (row0 + r) * ld + kk) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(ATile &t) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) st_lds16(&t.v[(w * 4 + i) * 8 * BK + l * 8], buf[i]);
  }
};

// Block scale of one code group from its raw fetched value.
template <int FMT>
__device__ __forceinline__ float group_scale(uint32_t raw, float s2, const DecodeTables &tb) {
  if constexpr (FMT == FMT_NF4) return __uint_as_float(raw);
  else if constexpr (FMT == FMT_NF4_DQ) return tb.tab8[raw] * s2;
  else return e8m0_to_f32(raw);
}
// Per-slab decode state: the block scale, and for the NF4 formats the byte planes of the
// sixteen scaled values (the 4-bit codes are then decoded with byte permutes, no LDS reads).
template <int FMT>
struct GroupDecoder {
  float sc;
  uint32_t pl[8];
  __device__ __forceinline__ void prepare(uint32_t raw, float s2, const DecodeTables &tb) {
    sc = group_scale<FMT>(raw, s2, tb);
    if constexpr (FMT != FMT_MXFP4) nf4_planes(sc, tb.cb, pl);
  }
  __device__ __forceinline__ u32x4 operator()(uint32_t w) const {
    if constexpr (FMT == FMT_MXFP4) return mxfp4_word_to_bf16(w, sc);
    else return nf4_decode_planes(w, pl);
  }
};
// Raw scale fetch of one group: NF4 fp32 absmax, NF4_DQ 8-bit code (+ its second-level
// scale, through buffer rs2), MXFP4 E8M0 byte.  `dead` = OOB turns the loads into zero reads.
template <int FMT>
__device__ __forceinline__ void fetch_scale(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rs2, uint32_t voff,
                                            uint32_t soff, int64_t blk, uint32_t dead, uint32_t &raw,
                                            float &s2) {
  if constexpr (FMT == FMT_NF4) {
    raw = bload32(rs, voff, soff | dead);
  } else {
    raw = bload8(rs, voff, soff | dead);
    if constexpr (FMT == FMT_NF4_DQ) s2 = __uint_as_float(bload32(rs2, (uint32_t)(blk >> 8) * 4, dead));
  }
}

// B from a 4-bit stack reduced over its STORED row axis: LDS tile [64 k][256 n], k =
// stored rows k0..k0+63, n = stored columns n0..n0+255.  Thread p -> stored row p / 4 and the
// 64 stored columns n0 + 64 (p % 4) ..: two 16-byte code loads (32 contiguous bytes), one
// block scale for the NF4 formats (the 64 columns are one block) or two for MXFP4 (blocks
// of 32), decoded and written as eight 16-byte row pieces; the MFMA fragments are read with
// the transposing LDS load.  VTS: tile pieces per producer thread.
template <int FMT>
struct LQuantKN {
  static constexpr int VTS = 1, PARTS = 8;
  static constexpr int LOADS = FMT == FMT_NF4_DQ ? 4 : 3;  // two code loads, the scale (+ second level)
  u32x4 w0, w1;
  uint32_t sraw;
  float s2;
  GroupDecoder<FMT> dec;
  float sa, sb;                       // MXFP4: the scales of the two blocks of 32
  uint32_t cvoff, svoff, crow, srow;  // offsets at k0 = 0 of this thread's stored row; per-row steps
  int64_t blk0, blkrow;
  __device__ __forceinline__ void init(const QStack &q, int e, int n0, int Nout, int vt) {
    const int kb = vt >> 2, nb = vt & 3;
    const int n = n0 + nb * 64;
    crow = (uint32_t)(q.K / 2);
    blkrow = q.K / 64;
    srow = FMT == FMT_NF4 ? (uint32_t)(blkrow * 4) : FMT == FMT_NF4_DQ ? (uint32_t)blkrow : (uint32_t)(q.K / 32);
    if (n < Nout) {
      const int64_t el = ((int64_t)e * q.N + kb) * q.K + n;
      cvoff = (uint32_t)(el / 2);
      blk0 = el >> 6;
      svoff = FMT == FMT_NF4 ? (uint32_t)(blk0 * 4) : FMT == FMT_NF4_DQ ? (uint32_t)blk0 : (uint32_t)(el >> 5);
    } else {
      cvoff = svoff = OOB;
      blk0 = 0;
    }
  }
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                        __amdgpu_buffer_rsrc_t rs2, int k0, uint32_t dead) {
    w0 = bload128(rc, cvoff, ((uint32_t)k0 * crow) | dead);
    w1 = bload128(rc, cvoff + 16, ((uint32_t)k0 * crow) | dead);
    if constexpr (FMT == FMT_MXFP4) {  // the two E8M0 bytes of the 64 columns (2-byte aligned)
      sraw = bload16(rs, svoff, ((uint32_t)k0 * srow) | dead);
    } else {
      fetch_scale<FMT>(rs, rs2, svoff, (uint32_t)k0 * srow, blk0 + (int64_t)k0 * blkrow, dead, sraw, s2);
    }
  }
  template <class TB>
  __device__ __forceinline__ void prepare(const TB &tb) {
    if constexpr (FMT == FMT_MXFP4) {
      sa = e8m0_to_f32(sraw & 0xffu);
      sb = e8m0_to_f32((sraw >> 8) & 0xffu);
    } else {
      dec.prepare(sraw, s2, tb);
    }
  }
  __device__ __forceinline__ void store(LTileKN &t, int part, int vt) const {
    const int kb = vt >> 2, nb = vt & 3;
    const uint32_t w = part < 4 ? w0[part] : w1[part - 4];
    u32x4 v;
    if constexpr (FMT == FMT_MXFP4) v = mxfp4_word_to_bf16(w, part < 4 ? sa : sb);
    else v = dec(w);
    st_lds16(&t.v[kb][knswz(kb, nb * 64 + part * 8)], v);
  }
};

// B from a 4-bit stack stored [N, K] for the producer waves: thread p (0..255) -> tile row p
// (weight row map(p)) and the whole 64-k slab: two 16-byte code loads (32 contiguous bytes),
// one block scale (NF4 formats: the slab is one block of 64) or two (MXFP4: blocks of 32),
// decoded into the eight 16-byte pieces of the tile row.
template <int FMT>
struct LQuantRow {
  u32x4 c0, c1;
  uint32_t sraw;
  float s2;
  uint32_t cvoff, svoff;  // byte offsets at k0 = 0
  int64_t blk0;
  __device__ __forceinline__ void init(const QStack &q, int e, const RowMap &map, int Nrows, int p) {
    const int n = map(p);
    if (n < Nrows) {
      const int64_t el = ((int64_t)e * q.N + n) * q.K;
      cvoff = (uint32_t)(el / 2);
      blk0 = el >> 6;
      svoff = FMT == FMT_NF4 ? (uint32_t)(blk0 * 4) : FMT == FMT_NF4_DQ ? (uint32_t)blk0 : (uint32_t)(el >> 5);
    } else {
      cvoff = svoff = OOB;
      blk0 = 0;
    }
  }
  // loads of one slab: 2 code loads + 1 scale load (+ the second-level scale for NF4_DQ)
  static constexpr int LOADS = FMT == FMT_NF4_DQ ? 4 : 3;
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                        __amdgpu_buffer_rsrc_t rs2, int k0, uint32_t dead) {
    c0 = bload128(rc, cvoff, ((uint32_t)k0 / 2) | dead);
    c1 = bload128(rc, cvoff + 16, ((uint32_t)k0 / 2) | dead);
    if constexpr (FMT == FMT_NF4) {
      sraw = bload32(rs, svoff, ((uint32_t)(k0 / 64) * 4) | dead);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      sraw = bload8(rs, svoff, (uint32_t)(k0 / 64) | dead);
      s2 = __uint_as_float(bload32(rs2, (uint32_t)((blk0 + k0 / 64) >> 8) * 4, dead));
    } else {  // the two E8M0 bytes of the slab's two blocks of 32 (2-byte aligned)
      sraw = bload16(rs, svoff + (uint32_t)(k0 / 32), dead);
    }
  }
  // decode the slab and write tile row p: piece c (8 k) from code word c
  template <class TileT>
  __device__ __forceinline__ void decode_store(TileT &t, const DecodeTables &tb, int p) const {
    if constexpr (FMT == FMT_MXFP4) {
      const float sa = e8m0_to_f32(sraw & 0xffu), sb = e8m0_to_f32((sraw >> 8) & 0xffu);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t w = c < 4 ? c0[c] : c1[c - 4];
        st_lds16(&t.v[p][bswz(p, c)], mxfp4_word_to_bf16(w, c < 4 ? sa : sb));
      }
    } else {
      GroupDecoder<FMT> dec;
      dec.prepare(sraw, s2, tb);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t w = c < 4 ? c0[c] : c1[c - 4];
        st_lds16(&t.v[p][bswz(p, c)], dec(w));
      }
    }
  }
};

// 8-bit stacks (INT8, FP8) for the producer waves, stored [N, K]: thread p -> tile row p
// (weight row map(p)) and the whole 64-k slab: four 16-byte code loads (64 contiguous bytes)
// and the block's fp32 scale, decoded into the eight 16-byte pieces of the tile row.
template <int FMT>
struct LQuantRow8 {
  static constexpr int LOADS = 5;
  u32x4 c[4];
  uint32_t sraw;
  uint32_t cvoff, svoff;  // byte offsets at k0 = 0
  __device__ __forceinline__ void init(const QStack &q, int e, const RowMap &map, int Nrows, int p) {
    const int n = map(p);
    if (n < Nrows) {
      const int64_t el = ((int64_t)e * q.N + n) * q.K;
      cvoff = (uint32_t)el;
      svoff = (uint32_t)((el >> 6) * 4);
    } else {
      cvoff = svoff = OOB;
    }
  }
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                        __amdgpu_buffer_rsrc_t, int k0, uint32_t dead) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = bload128(rc, cvoff + 16 * i, (uint32_t)k0 | dead);
    sraw = bload32(rs, svoff, ((uint32_t)(k0 / 64) * 4) | dead);
  }
  template <class TileT>
  __device__ __forceinline__ void decode_store(TileT &t, const DecodeTables &, int p) const {
    const float sc = __uint_as_float(sraw);
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) {
      const u32x2 a = byte_word_to_bf16<FMT>(c[pc >> 1][2 * (pc & 1)], sc);
      const u32x2 b = byte_word_to_bf16<FMT>(c[pc >> 1][2 * (pc & 1) + 1], sc);
      st_lds16(&t.v[p][bswz(p, pc)], u32x4{a[0], a[1], b[0], b[1]});
    }
  }
};

// 8-bit stacks reduced over their stored row axis (dgrad), LDS tile [64 k][256 n]: virtual
// thread vt -> stored row vt / 8 and 32 stored columns (vt % 8): two 16-byte code loads and
// the scale of the 64-column block they lie in, written as four 16-byte row pieces.
template <int FMT>
struct LQuantKN8 {
  static constexpr int VTS = 2, PARTS = 4;
  static constexpr int LOADS = 3;
  u32x4 w[2];
  uint32_t sraw;
  float sc;
  uint32_t cvoff, svoff, crow, srow;
  __device__ __forceinline__ void init(const QStack &q, int e, int n0, int Nout, int vt) {
    const int kb = vt >> 3, nb = vt & 7;
    const int n = n0 + nb * 32;
    crow = (uint32_t)q.K;
    srow = (uint32_t)(q.K / 64 * 4);
    if (n < Nout) {
      const int64_t el = ((int64_t)e * q.N + kb) * q.K + n;
      cvoff = (uint32_t)el;
      svoff = (uint32_t)((el >> 6) * 4);
    } else {
      cvoff = svoff = OOB;
    }
  }
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                        __amdgpu_buffer_rsrc_t, int k0, uint32_t dead) {
    w[0] = bload128(rc, cvoff, ((uint32_t)k0 * crow) | dead);
    w[1] = bload128(rc, cvoff + 16, ((uint32_t)k0 * crow) | dead);
    sraw = bload32(rs, svoff, ((uint32_t)k0 * srow) | dead);
  }
  __device__ __forceinline__ void prepare(const DecodeTables &) { sc = __uint_as_float(sraw); }
  __device__ __forceinline__ void store(LTileKN &t, int part, int vt) const {
    const int kb = vt >> 3, nb = vt & 7;
    const u32x2 a = byte_word_to_bf16<FMT>(w[part >> 1][2 * (part & 1)], sc);
    const u32x2 b = byte_word_to_bf16<FMT>(w[part >> 1][2 * (part & 1) + 1], sc);
    st_lds16(&t.v[kb][knswz(kb, nb * 32 + part * 8)], u32x4{a[0], a[1], b[0], b[1]});
  }
};

// Dense bf16 B rows (LoRA K-extension): tile row tid -> weight row map(tid), zero past
// kbound.  Always written in the [n][k] layout.
struct LDenseNK {
  u32x4 buf[4];
  const uint16_t *row;
  bool ok;
  __device__ __forceinline__ void init(const uint16_t *__restrict__ base, int64_t ld, const RowMap &map,
                                       int Nrows) {
    const int n = map(threadIdx.x & 255);
    ok = n < Nrows;
    row = base + (int64_t)(ok ? n : 0) * ld + (threadIdx.x >> 8) * 32;
  }
  // this thread's half of the slab: k0 + 32 * (tid / 256) + 8v
  __device__ __forceinline__ void fetch(int k0, int kbound) {
    const int kh = k0 + (threadIdx.x >> 8) * 32;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      buf[v] = (ok && kh + 8 * v < kbound) ? *(const u32x4 *)(row + k0 + 8 * v) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void store(LTile &t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = threadIdx.x & 255;
      st_lds16(&t.v[row][bswz(row, (threadIdx.x >> 8) * 4 + v)], buf[v]);
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// MFMA core of the large tile: wave (wm, wn) = (w / 4, w % 4) owns rows wm*128 .. +127
// and columns wn*64 .. +63: four 32-row by two 32-column accumulator tiles.
struct LMma {
  f32x16 acc[4][2];
  __device__ __forceinline__ static int wm() { return threadIdx.x >> 8; }
  __device__ __forceinline__ static int wn() { return (threadIdx.x >> 6) & 3; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }
  // B fragments from an [n][k] tile (ds_read_b128).
  __device__ __forceinline__ static bf16x8 bfrag_nk(const LTile &B, int j, int ks) {
    const int lane = threadIdx.x & 63;
    const int row = wn() * 64 + j * 32 + (lane & 31);
    return *(const bf16x8 *)&B.v[row][bswz(row, ks * 2 + (lane >> 5))];
  }
  // B fragments from a [k][n] tile with the transposing LDS read: within each 16-lane
  // group, lane i receives element i%4 of the 8-byte pieces addressed by lanes 4j + i/4,
  // so lane (4*kr + c) addresses row kr, columns 4c..4c+3 of the group's 16 columns.
  __device__ __forceinline__ static bf16x8 bfrag_kn(const LTileKN &B, int j, int ks) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, i = lane & 15;
    const int row = ks * 16 + (G >> 1) * 8 + (i >> 2);
    const int col = wn() * 64 + j * 32 + (G & 1) * 16 + (i & 3) * 4;
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&B.v[row][knswz(row, col)]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&B.v[row + 4][knswz(row + 4, col)]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  }
  // B fragments from an unpadded [k][n] tile (LTileKD), transposing LDS read as above.
  __device__ __forceinline__ static bf16x8 bfrag_kd(const LTileKD &B, int j, int ks) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, i = lane & 15;
    const int row = ks * 16 + (G >> 1) * 8 + (i >> 2);
    const int col = wn() * 64 + j * 32 + (G & 1) * 16 + (i & 3) * 4;
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&B.v[row][kdswz(row, col)]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&B.v[row + 4][kdswz(row + 4, col)]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  }
  __device__ __forceinline__ static bf16x8 bfrag(const LTile &B, int j, int ks) { return bfrag_nk(B, j, ks); }
  __device__ __forceinline__ static bf16x8 bfrag(const LTileKN &B, int j, int ks) { return bfrag_kn(B, j, ks); }
  __device__ __forceinline__ static bf16x8 bfrag(const LTileKD &B, int j, int ks) { return bfrag_kd(B, j, ks); }
  // The operand fragments of one k-step (16 k) for this wave.
  struct Frag {
    bf16x8 a[4], b[2];
  };
  template <bool KN, class BT>
  __device__ __forceinline__ static void load(const ATile &A, const BT &B, int ks, Frag &f) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[j] = bfrag(B, j, ks);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *(const bf16x8 *)&A.v[aswz(wm() * 128 + i * 32 + r, kc)];
  }
  __device__ __forceinline__ void mma(const Frag &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  }
  // A k-step range over only the first ni (< 4) 32-row sub-tiles of this wave's 128 rows:
  // the tile's other rows are padding past the expert's rows (its last row tile), so their
  // A fragments and MFMAs are skipped (ni is the same for the whole wave).
  template <bool KN, class BT>
  __device__ __forceinline__ void step_rows(const ATile &A, const BT &B, int ksteps, int ni) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 31;
    for (int ks = 0; ks < ksteps; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = bfrag(B, j, ks);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < ni) {
          const bf16x8 a = *(const bf16x8 *)&A.v[aswz(wm() * 128 + i * 32 + r, kc)];
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  template <bool KN, class BT>
  __device__ __forceinline__ void kstep(const ATile &A, const BT &B, int ks) {
    Frag f;
    load<KN>(A, B, ks, f);
    mma(f);
  }
  template <bool KN, class BT>
  __device__ __forceinline__ void step(const ATile &A, const BT &B, int ksteps) {
    for (int ks = 0; ks < ksteps; ++ks) kstep<KN>(A, B, ks);
  }
  // tile-local (row, col) of accumulator element (i, j, v) for this lane
  __device__ __forceinline__ static int row_of(int i, int v) {
    const int lane = threadIdx.x & 63;
    return wm() * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
  }
  __device__ __forceinline__ static int col_of(int j) {
    const int lane = threadIdx.x & 63;
    return wn() * 64 + j * 32 + (lane & 31);
  }
};

// ---------------------------------------------------------------- k-major tiles
// Tiles of the weight-gradient products, whose reduction index (the routed rows) is the
// row index of both operands in memory: [64 k][W] bf16 rows copied as they are, with a
// row pitch of W + 32 elements (320 or 192 bytes), so that the four rows one 16-lane
// group of a transposing fragment read touches fall in distinct banks.
template <int W>
struct KTile {
  static constexpr int PITCH = W + 32;
  uint16_t v[BK][PITCH];
};
// MFMA fragment (32 columns at col0, k-step ks) from a KTile with the transposing LDS
// read: within each 16-lane group, lane i receives element i % 4 of the 8-byte pieces
// addressed by lanes 4 j + i / 4; lane 4 kr + c addresses row kr, columns 4 c .. 4 c + 3
// of the group's 16 columns, so lane i ends up with column i at four consecutive k.  The
// fragment layout is the same for the A and the B operand.
template <int W>
__device__ __forceinline__ bf16x8 ktile_frag(const KTile<W> &t, int ks, int col0) {
  typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, i = lane & 15;
  const int row = ks * 16 + (G >> 1) * 8 + (i >> 2);
  const int col = col0 + (G & 1) * 16 + (i & 3) * 4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&t.v[row][col]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(&t.v[row + 4][col]));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}
// Rows k0 .. k0 + 63 (of krows) of a row-major [rows][ld] bf16 matrix, columns col0 ..
// col0 + W - 1 (of ncols) into a KTile: W / 8 lanes read one row's 2 W bytes, each pass
// takes 256 / (W / 8) rows.  Row k is source row row0 + k, or gather[row0 + k] / gdiv.  The
// 128-wide operand of a weight-gradient tile is the large one, read once: non-temporal loads.
template <int W>
struct KRowLoader {
  static constexpr int LPR = W / 8, RPP = NTHREADS / LPR, PASSES = BK / RPP;
  u32x4 buf[PASSES];
  __device__ __forceinline__ void fetch(const uint16_t *__restrict__ base, int64_t ld, int col0, int ncols,
                                        int row0, int krows, const int32_t *__restrict__ gather, int gdiv, int k0) {
    const int c = threadIdx.x % LPR, r = threadIdx.x / LPR;
    const int col = col0 + c * 8;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int kk = k0 + p * RPP + r;
      const bool ok = kk < krows && col < ncols;
      int64_t src = 0;
      if (ok) src = gather ? (int64_t)(gather[row0 + kk] / gdiv) : (int64_t)(row0 + kk);
      buf[p] = ok ? (W == 128 ? __builtin_nontemporal_load((const u32x4 *)(base + src * ld + col)) : *(const u32x4 *)(base + src * ld + col)) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(KTile<W> &t) {
    const int c = threadIdx.x % LPR, r = threadIdx.x / LPR;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) st_lds16(&t.v[p * RPP + r][c * 8], buf[p]);
  }
};
// Products over KTiles: acc[i][j] += A-tile columns (wm TM + i) 32 .. x B-tile columns
// (wn TN + j) 32 .., over `ksteps` 16-row k steps.  The accumulators are those of Mma.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void mma_ktiles(Mma<BM, BN, WM, WN> &m, const KTile<BM> &A, const KTile<BN> &B,
                                           int ksteps) {
  constexpr int TM = Mma<BM, BN, WM, WN>::TM, TN = Mma<BM, BN, WM, WN>::TN;
  const int wave = threadIdx.x >> 6, wm = wave / WN, wn = wave % WN;
  for (int ks = 0; ks < ksteps; ++ks) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = ktile_frag(A, ks, (wm * TM + i) * 32);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = ktile_frag(B, ks, (wn * TN + j) * 32);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        m.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], m.acc[i][j], 0, 0, 0);
  }
}

}  // namespace e4b
