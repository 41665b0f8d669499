// gfx950 kernels of the routed-expert MoE layer: routing, the grouped MFMA
// GEMMs with in-register 4-bit decode, LoRA K-extension and SwiGLU epilogues,
// the top-k combine and its backward, the unpermute-sum, the segmented LoRA
// weight-gradient GEMMs, and the quantise / dequantise kernels.
#include <type_traits>

#include "gemm.hpp"
#include "kernels.hpp"
#include <algorithm>

namespace e4b {

__constant__ float kNF4[16] = E4B_NF4_VALUES;
__constant__ float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};


// =============================================================== routing
// One workgroup of 8 wave64s.  Wave w owns a contiguous range of flat indices.
// Pass 1 counts (expert, wave) pairs in LDS; pass 2 turns them into per-wave
// starting positions (expert-major, wave-minor) and the expert offsets; pass 3
// walks each range in order, ranking equal expert ids inside a wave64 by the
// lanes below them (bitwise key match from ballots), which keeps the grouping
// stable in the flat index t*k + j.
constexpr int RT_WAVES = 16, RT_BATCH = 8;

__global__ __launch_bounds__(RT_WAVES * 64) void route_kernel(const int32_t *__restrict__ ids, int M,
                                                              int E, int32_t *__restrict__ cnt,
                                                              int32_t *__restrict__ off,
                                                              int32_t *__restrict__ perm,
                                                              int32_t *__restrict__ inv,
                                                              int32_t *__restrict__ zero, int nzero) {
  extern __shared__ int32_t sm[];
  for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  const int KE = E + 1;  // keys 0..E-1 valid, E = dropped
  int32_t *wc = sm;                   // [RT_WAVES][KE]
  int32_t *soff = sm + RT_WAVES * KE;  // [KE]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < RT_WAVES * KE; i += blockDim.x) wc[i] = 0;
  __syncthreads();
  const int S = (((M + RT_WAVES - 1) / RT_WAVES) + 63) & ~63;
  const int f0 = min(M, w * S), f1 = min(M, f0 + S);
  // the ids of RT_BATCH 64-wide chunks are loaded together, so a wave waits for memory
  // once per batch rather than once per chunk
  int ev[RT_BATCH];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < RT_BATCH; ++u) {
      const int f = c0 + 64 * u + lane;
      ev[u] = f < f1 ? ids[f] : 0;
    }
  };
  for (int c0 = f0; c0 < f1; c0 += 64 * RT_BATCH) {
    load_batch(c0);
#pragma unroll
    for (int u = 0; u < RT_BATCH; ++u) {
      const int e = ev[u];
      if (c0 + 64 * u + lane < f1) atomicAdd(&wc[w * KE + ((e >= 0 && e < E) ? e : E)], 1);
    }
  }
  __syncthreads();
  for (int key = tid; key < KE; key += blockDim.x) {
    int run = 0;
    for (int ww = 0; ww < RT_WAVES; ++ww) {
      const int c = wc[ww * KE + key];
      wc[ww * KE + key] = run;
      run += c;
    }
    cnt[key] = run;
    soff[key] = run;
  }
  __syncthreads();
  if (w == 0) {
    int base = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      const int v = e < E ? soff[e] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      if (e < E) soff[e] = base + incl - v;
      base += __shfl(incl, 63);
    }
    if (lane == 0) soff[E] = base;
  }
  __syncthreads();
  for (int e = tid; e < KE; e += blockDim.x) off[e] = soff[e];
  const int nbits = 32 - __clz(E);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int cb = f0; cb < f1; cb += 64 * RT_BATCH) {
    load_batch(cb);
#pragma unroll
    for (int u = 0; u < RT_BATCH; ++u) {
      const int f = cb + 64 * u + lane;
      const bool act = f < f1;
      const int e = ev[u];
      const bool valid = act && e >= 0 && e < E;
      const int key = valid ? e : E;
      uint64_t eq = __ballot(act);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t m = __ballot(bit);
        eq &= bit ? m : ~m;
      }
      const int rank = __popcll(eq & lt);
      const int total = __popcll(eq);
      if (valid) {
        const int pos = soff[e] + wc[w * KE + e] + rank;
        perm[pos] = f;
        inv[f] = pos;
      } else if (act) {
        inv[f] = -1;
      }
      if (valid && rank == 0) wc[w * KE + e] += total;
    }
  }
  for (int p = soff[E] + tid; p < M; p += blockDim.x) perm[p] = -1;
}

bool launch_route(const int32_t *ids, int M, int E, int32_t *cnt, int32_t *off, int32_t *perm,
                  int32_t *inv, hipStream_t s, int32_t *zero, int nzero) {
  LaunchScope ls(FAM_ROUTE, s);
  const size_t shm = (size_t)(RT_WAVES + 1) * (E + 1) * sizeof(int32_t);
  route_kernel<<<1, RT_WAVES * 64, shm, s>>>(ids, M, E, cnt, off, perm, inv, zero, zero ? nzero : 0);
  return last_launch_ok();
}

// Per-workgroup LDS decode tables (see DecodeTables) from the stack's tables.
__device__ __forceinline__ void init_decode_tables(DecodeTables &t, const QStack &q) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    t.cb2[i] = make_float2(code_value(q.codebook, i >> 4), code_value(q.codebook, i & 15));
    t.tab8[i] = dq_value(q.dq_table, i);
    if (i < 16) t.cb[i] = code_value(q.codebook, i);
  }
}

// =============================================================== small-tile bf16 GEMM
// C = alpha * A B^T over expert segments with a dense per-expert B [N][ldb]: the
// LoRA-A projections (z = s A[e] x and u = s dG B[e]) whose N is the adapter rank.
template <int BN, int WM, int WN>
__global__ __launch_bounds__(NTHREADS) void dense_gemm_kernel(GroupedArgs g) {
  constexpr int BMt = 128;
  __shared__ LdsTile<BMt> As;
  __shared__ LdsTile<BN> Bs;
  __shared__ int tile_sh[4];
  TileM tm;
  if (!find_tile(g.off, g.E, BMt, blockIdx.y, tm, tile_sh)) return;
  const int e = tm.e;
  const int n0 = blockIdx.x * BN;
  const RowMap map{n0, 0, false};
  Mma<BMt, BN, WM, WN> mma;
  mma.zero();
  RowLoader<BMt> la;
  DenseNKLoader<BN> ld;
  const uint16_t *Bd_e = g.Bd + (int64_t)e * g.b_estride;
  // this split's slabs
  const int nall = g.K / BK, chunk = (nall + g.nsplit - 1) / g.nsplit;
  const int s0 = min(nall, (int)blockIdx.z * chunk), s1 = min(nall, s0 + chunk);
  la.init(g.lda, tm.rows, tm.row0, g.a_gather, g.a_gdiv);
  auto fetch = [&](int s) {
    la.fetch(g.A, s * BK, g.K);
    ld.fetch(Bd_e, g.ldb, map, g.N, s * BK, g.K);
  };
  if (s0 < s1) fetch(s0);
  for (int s = s0; s < s1; ++s) {
    __syncthreads();
    la.store(As);
    ld.store(Bs);
    __syncthreads();
    if (s + 1 < s1) fetch(s + 1);
    mma.step(As, Bs, 4);
  }
  if (g.nsplit > 1) {
    float *P = g.part + (int64_t)blockIdx.z * g.M * g.N;
    mma.for_each([&](int row, int col, float v) {
      const int n = n0 + col;
      if (row < tm.rows && n < g.N) P[(int64_t)(tm.row0 + row) * g.N + n] = v;
    });
  } else {
    mma.for_each([&](int row, int col, float v) {
      const int n = n0 + col;
      if (row < tm.rows && n < g.N) ((uint16_t *)g.C)[(int64_t)(tm.row0 + row) * g.ldc + n] = f2bf(g.alpha * v);
    });
  }
}

// out[row][col] = alpha * sum over s of part[s * stride + row * cols + col], added in split
// order; fp32 or bf16 output with leading dimension ldo.
__global__ void reduce_splits_kernel(const float *__restrict__ part, int nsplit, int64_t stride, int64_t count,
                                     int cols, int64_t ldo, float alpha, int out_bf16, void *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int s2 = 1; s2 < nsplit; ++s2) acc += part[s2 * stride + i];
  const int64_t o = (i / cols) * ldo + i % cols;
  if (out_bf16) ((uint16_t *)out)[o] = f2bf(alpha * acc);
  else ((float *)out)[o] = alpha * acc;
}

static bool launch_reduce_splits(const float *part, int nsplit, int64_t stride, int64_t count, int cols,
                                 int64_t ldo, float alpha, bool out_bf16, void *out, hipStream_t s) {
  if (count == 0) return true;
  reduce_splits_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(part, nsplit, stride, count, cols, ldo,
                                                                        alpha, out_bf16 ? 1 : 0, out);
  return last_launch_ok();
}

// Aim for about four workgroups per compute unit; each split keeps at least 4 slabs.
static constexpr int SPLIT_TARGET_WGS = 1024, SPLIT_MAX = 8;
static int splits_for(int64_t wgs, int64_t slabs) {
  int sp = (int)std::min<int64_t>(SPLIT_MAX, std::max<int64_t>(1, (SPLIT_TARGET_WGS + wgs - 1) / std::max<int64_t>(1, wgs)));
  return (int)std::max<int64_t>(1, std::min<int64_t>(sp, slabs / 4));
}
// LoRA-A: also at most 64 slabs per split, so that a long reduction (K = 2I in the
// backward) is not left to one workgroup per row tile and split.
int lora_a_splits(int M, int E, int N, int K) {
  if (M == 0) return 1;
  const int sp = splits_for((int64_t)cdiv(N, 64) * (cdiv(M, 128) + E), K / BK);
  return std::max(sp, (int)std::min<int64_t>(SPLIT_MAX, std::max(1, cdiv(K / BK, 64))));
}
// Upper bound on the splits of one expert's weight-gradient reduction; each expert takes
// as many as its own rows fill (wgrad_expert_splits).  With many experts the routed rows are
// skewed (a few experts hold many times the mean), and one split count for all experts
// would leave the largest as one long chain: then up to SPLIT_MAX, within a partial-sum
// buffer of at most 256 MB.
int wgrad_splits(int M, int E, int Na, int Nb) {
  if (M == 0 || E == 0) return 1;
  const int64_t tiles = Nb <= 64 ? (int64_t)cdiv(Nb, 64) * cdiv(Na, 128) : (int64_t)cdiv(Nb, 128) * cdiv(Na, 64);
  // short-wide tiles (rank rows x 128 weight columns) reach the memory rate only with
  // about three times as many workgroups in flight
  const int64_t wgs = Nb <= 64 ? tiles * E : tiles * E * SPLIT_TARGET_WGS / 3072;
  int sp = splits_for(wgs, (int64_t)M / E / BK);
  if (E >= 32) {
    const int64_t per = (int64_t)E * Na * Nb * 4;
    sp = std::max(sp, (int)std::min<int64_t>(SPLIT_MAX, std::max<int64_t>(1, ((int64_t)256 << 20) / per)));
  }
  return sp;
}

// Waits of the large-tile pipelines.  Direct-to-LDS loads count in vmcnt and are not
// covered by a barrier: every wave waits for its own before the workgroup barrier that
// publishes them.  vmcnt(n) waits until at most n vector-memory loads of this wave are
// outstanding (loads retire in order), so loads issued after the ones waited for can stay in
// flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // expcnt/lgkmcnt at their maximum: no wait
}
__device__ __forceinline__ void wait_lds_dma() { wait_vmcnt<0>(); }

// Workgroup barrier after this wave's LDS stores (lgkmcnt(0)) and all but its last N
// vector-memory loads (vmcnt(N): the direct-to-LDS A loads, issued first) completed.
// A fenced __syncthreads() would drain every outstanding load, including the B loads
// prefetched ahead; the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void slab_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}


// The same main loop over a bf16 copy of the stack (written by expand_kernel with the same
// decode functions): A and B both go HBM -> LDS by direct loads, with no decode work, and
// the MFMA sequence over identical LDS contents is that of the producer / consumer tiles,
// so the two give bit-identical accumulators.  The A rows land one slab ahead; the weight tiles, which
// other workgroups on the same L2 rarely share, land two slabs ahead in a ring of three
// LDS tiles.
union XBuf {
  LTile nk;
  LTileKD kd;
};
template <bool KN>
struct XPipe {
  using BTile = typename std::conditional<KN, LTileKD, LTile>::type;
  ATile &A0, &A1;
  XBuf &B0, &B1, &B2;
  __amdgpu_buffer_rsrc_t ra, rb;
  LDirectA la;
  typename std::conditional<KN, LDirectBKN, LDirectBNK>::type lb;
  uint32_t bstep;  // bytes of B per slab
  LMma mma;
  LMma::Frag f[2];
  __device__ __forceinline__ XPipe(ATile &a0, ATile &a1, XBuf &b0, XBuf &b1, XBuf &b2, const GroupedArgs &g,
                                   int e)
      : A0(a0), A1(a1), B0(b0), B1(b1), B2(b2),
        ra(make_rsrc(g.A, g.a_bytes)),
        rb(make_rsrc(g.Bx + (int64_t)e * g.bx_estride, g.bx_bytes)),
        bstep(KN ? (uint32_t)(BK * g.N * 2) : (uint32_t)(BK * 2)) {}
  template <int P>
  __device__ __forceinline__ ATile &atile() {
    if constexpr (P == 0) return A0;
    else return A1;
  }
  template <int Q>
  __device__ __forceinline__ BTile &btile() {
    XBuf &b = Q == 0 ? B0 : Q == 1 ? B1 : B2;
    if constexpr (KN) return b.kd;
    else return b.nk;
  }
  __device__ __forceinline__ static uint32_t dead(int slab, int nmain) { return slab < nmain ? 0u : OOB; }
  template <int P>
  __device__ __forceinline__ void issue_a(int slab, int nmain) {
    la.issue(ra, atile<P>(), (uint32_t)(slab * BK * 2) | dead(slab, nmain));
  }
  template <int Q>
  __device__ __forceinline__ void issue_b(int slab, int nmain) {
    lb.issue(rb, btile<Q>(), (uint32_t)slab * bstep | dead(slab, nmain));
  }
  // Scheduling hint for one k-step: each MFMA followed by one fragment read of the next.
  __device__ __forceinline__ static void interleave() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (q < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  }
  // Slab s computes from A tile P = s % 2 and B tile Q = s % 3.  Fragments are read one
  // k-step ahead (f[0] holds k-step 0 of slab s on entry).  The barrier sits between the
  // reads of k-step 3 and its MFMAs: past it the A rows and weights of slab s+1 are in LDS
  // and every wave has finished reading slab s, so k-step 0 of slab s+1 is read while the
  // last MFMAs of slab s run.  The B loads of slab s+2 go into the tile slab s-1 used.
  template <int P, int Q>
  __device__ __forceinline__ void body(int s, int nmain) {
    issue_a<P ^ 1>(s + 1, nmain);
    issue_b<(Q + 2) % 3>(s + 2, nmain);
    __builtin_amdgcn_sched_barrier(0);
    LMma::load<KN>(atile<P>(), btile<Q>(), 1, f[1]);
    mma.mma(f[0]);
    interleave();
    LMma::load<KN>(atile<P>(), btile<Q>(), 2, f[0]);
    mma.mma(f[1]);
    interleave();
    LMma::load<KN>(atile<P>(), btile<Q>(), 3, f[1]);
    mma.mma(f[0]);
    interleave();
    slab_barrier<4>();  // A rows and weights of slab s+1 have landed (those of s+2 may not)
    LMma::load<KN>(atile<P ^ 1>(), btile<(Q + 1) % 3>(), 0, f[0]);
    mma.mma(f[1]);
    interleave();
  }
  __device__ __forceinline__ void run(int nmain) {
    issue_a<0>(0, nmain);
    issue_b<0>(0, nmain);
    issue_b<1>(1, nmain);
    wait_lds_dma();
    __syncthreads();
    LMma::load<KN>(A0, btile<0>(), 0, f[0]);
    // six bodies cycle both tile rings
    for (int s = 0;; s += 6) {
      body<0, 0>(s, nmain);
      if (s + 1 >= nmain) break;
      body<1, 1>(s + 1, nmain);
      if (s + 2 >= nmain) break;
      body<0, 2>(s + 2, nmain);
      if (s + 3 >= nmain) break;
      body<1, 0>(s + 3, nmain);
      if (s + 4 >= nmain) break;
      body<0, 1>(s + 4, nmain);
      if (s + 5 >= nmain) break;
      body<1, 2>(s + 5, nmain);
      if (s + 6 >= nmain) break;
    }
    // the last body's weight loads (past the end) must land before B0 is reused
    wait_lds_dma();
    __syncthreads();
  }
};

// After the main loop: the LoRA K-extension into the same accumulator (through the A0 /
// B0 tiles) by the 512 threads that hold the accumulators; any other waves of the
// workgroup take part in its barriers only (lora_barriers).
__device__ __forceinline__ void lora_extension(LMma &mma, const GroupedArgs &g, const TileM &tm, int e,
                                               const RowMap &map, int Nrows, ATile &A0, LTile &B0) {
  if (g.r > 0) {  // LoRA rank as a K-extension of the same accumulator
    LRegA lx;
    LDenseNK lbd;
    lbd.init(g.xb + (int64_t)e * g.xb_estride, g.ldxb, map, Nrows);
    for (int k0 = 0; k0 < g.r; k0 += BK) {
      lx.load(g.xa, g.ldxa, tm.rows, tm.row0, k0, g.r);
      lbd.fetch(k0, g.r);
      lx.store(A0);
      lbd.store(B0);
      __syncthreads();
      mma.step<false>(A0, B0, min(4, (g.r - k0 + 15) / 16));
      __syncthreads();
    }
  }
}
__device__ __forceinline__ void lora_barriers(const GroupedArgs &g) {
  for (int k0 = 0; k0 < g.r; k0 += BK) {
    __syncthreads();
    __syncthreads();
  }
}

template <int EPI>
__device__ __forceinline__ void large_epilogue(LMma &mma, const GroupedArgs &g, const TileM &tm, int n0);

template <int EPI>
__device__ __forceinline__ void large_finish(LMma &mma, const GroupedArgs &g, const TileM &tm, int e, int n0,
                                             const RowMap &map, int Nrows, ATile &A0, LTile &B0) {
  lora_extension(mma, g, tm, e, map, Nrows, A0, B0);
  large_epilogue<EPI>(mma, g, tm, n0);
}

// The tile epilogue of the 512 accumulator threads.
template <int EPI>
__device__ __forceinline__ void large_epilogue(LMma &mma, const GroupedArgs &g, const TileM &tm, int n0) {

  // Outputs go through buffer resources over exactly this tile's rows, so the range check
  // drops the stores of rows past the tile; a lane whose column is past the end gets an
  // out-of-range offset.  Each lane's offset is fixed; the (i, v) step of the accumulator
  // element adds a multiple of the row pitch that is the same for all lanes.
  const int lane = threadIdx.x & 63;
  const int rl = LMma::wm() * 128 + (lane >> 5) * 4;  // the lane's first tile row
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    // tile rows interleave 32 gate and 32 up weight rows: the wave's pair (0, 1) holds gate
    // and up of h columns n0 + wn*32 + lane%32.  Accumulator elements v and v+1 (v even) are
    // rows r and r+1: lane pairs store two columns per 4-byte store (pair_bf16), the even
    // lane row r and the odd lane row r+1.
    const int col = n0 + LMma::wn() * 32 + (lane & 31);
    const bool odd = lane & 1;
    const int pc = col & ~1, pr = rl + (odd ? 1 : 0);
    const __amdgpu_buffer_rsrc_t rh = rows_rsrc(g.C, tm.row0, tm.rows, g.ldc, 2);
    const uint32_t hoff = col < g.I ? (uint32_t)((pr * g.ldc + pc) * 2) : OOB;
    const uint32_t hpitch = (uint32_t)(g.ldc * 2);
    if (g.act == 1) {
      // clamped GLU over interleaved rows: this lane's gate and up are stack rows 2 col and
      // 2 col + 1, so the saved pre-activation keeps the stored order and each (gate, up)
      // pair of a row is one 4-byte store (row rl + dr, no lane pairing)
      float bg = 0.0f, bu = 0.0f;
      if (g.bias && col < g.I) {
        const uint16_t *b = g.bias + (int64_t)tm.e * g.bias_estride + 2 * col;
        bg = bf2f(b[0]);
        bu = bf2f(b[1]);
      }
      const __amdgpu_buffer_rsrc_t rg = rows_rsrc(g.Gout, tm.row0, tm.rows, g.ldg, 2);
      const uint32_t goff = col < g.I ? (uint32_t)((rl * g.ldg + 2 * col) * 2) : OOB;
      const uint32_t gpitch = (uint32_t)(g.ldg * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t dr = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
          const float gt0 = mma.acc[i][0][v] + bg, up0 = mma.acc[i][1][v] + bu;
          const float gt1 = mma.acc[i][0][v + 1] + bg, up1 = mma.acc[i][1][v + 1] + bu;
          const float h0 = glu_clamped(gt0, up0, g.glu_alpha, g.glu_limit);
          const float h1 = glu_clamped(gt1, up1, g.glu_alpha, g.glu_limit);
          bstore32u(rh, pair_bf16(h0, h1, odd), hoff + dr * hpitch);
          if (g.Gout) {
            bstore32u(rg, pack_bf16x2(gt0, up0), goff + dr * gpitch);
            bstore32u(rg, pack_bf16x2(gt1, up1), goff + (dr + 1) * gpitch);
          }
        }
    } else if (g.Gout) {
      const __amdgpu_buffer_rsrc_t rg = rows_rsrc(g.Gout, tm.row0, tm.rows, g.ldg, 2);
      const uint32_t goff = col < g.I ? (uint32_t)((pr * g.ldg + pc) * 2) : OOB;
      const uint32_t gpitch = (uint32_t)(g.ldg * 2), uoff = (uint32_t)(g.I * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t dr = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
          const float gt0 = mma.acc[i][0][v], up0 = mma.acc[i][1][v];
          const float gt1 = mma.acc[i][0][v + 1], up1 = mma.acc[i][1][v + 1];
          const float h0 = gt0 * sigmoid_fast(gt0) * up0, h1 = gt1 * sigmoid_fast(gt1) * up1;
          bstore32u(rh, pair_bf16(h0, h1, odd), hoff + dr * hpitch);
          bstore32u(rg, pair_bf16(gt0, gt1, odd), goff + dr * gpitch);
          bstore32u(rg, pair_bf16(up0, up1, odd), goff + dr * gpitch + uoff);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t dr = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
          const float gt0 = mma.acc[i][0][v], up0 = mma.acc[i][1][v];
          const float gt1 = mma.acc[i][0][v + 1], up1 = mma.acc[i][1][v + 1];
          const float h0 = gt0 * sigmoid_fast(gt0) * up0, h1 = gt1 * sigmoid_fast(gt1) * up1;
          bstore32u(rh, pair_bf16(h0, h1, odd), hoff + dr * hpitch);
        }
    }
  } else if constexpr (EPI == EPI_F32) {
    // lane pairs store two columns per 8-byte store (bstore_pair_f32), as above
    const bool odd = lane & 1;
    const __amdgpu_buffer_rsrc_t rc = rows_rsrc(g.C, tm.row0, tm.rows, g.ldc, 4);
    const uint32_t pitch = (uint32_t)(g.ldc * 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + LMma::col_of(j);
      const uint32_t off = n < g.N ? (uint32_t)(((rl + (odd ? 1 : 0)) * g.ldc + (n & ~1)) * 4) : OOB;
      // per-expert bias of this lane's column (clamped GLU experts' down projection)
      const float bn = (g.bias && n < g.N) ? bf2f(g.bias[(int64_t)tm.e * g.bias_estride + n]) : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t dr = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
          bstore_pair_f32(rc, g.alpha * mma.acc[i][j][v] + bn, g.alpha * mma.acc[i][j][v + 1] + bn, odd,
                          off + dr * pitch);
        }
    }
  } else {  // EPI_SWIGLU_BWD: acc = dh; dG from the saved pre-activation G
    // G and dG are separate buffers.  The G values of a 16-row group are loaded before any
    // of them is used, so their latencies overlap; rows past the tile read zero.  Loads
    // and stores go two columns per dword through lane pairs (unpair_bf16, pair_bf16): the
    // even lane handles rows r and the odd lane rows r+1 of accumulator pairs (v, v+1).
    const bool odd = lane & 1;
    const __amdgpu_buffer_rsrc_t ri = rows_rsrc(g.Gin, tm.row0, tm.rows, g.ldg, 2);
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc(g.Gout, tm.row0, tm.rows, g.ldg, 2);
    const uint32_t pitch = (uint32_t)(g.ldg * 2), uoff = (uint32_t)(g.I * 2);
    if (g.act == 1) {
      // clamped GLU over interleaved rows: the (gate, up) pair of column n of a row is one
      // dword of G and of dG; every lane handles its own column, rows rl + dr
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + LMma::col_of(j);
        const uint32_t off = n < g.N ? (uint32_t)((rl * g.ldg + 2 * n) * 2) : OOB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t gu[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) gu[v] = bload32(ri, off + (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * pitch, 0);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float dg, du;
            glu_clamped_bwd(bf2f((uint16_t)(gu[v] & 0xffffu)), bf2f((uint16_t)(gu[v] >> 16)), g.glu_alpha,
                            g.glu_limit, mma.acc[i][j][v], dg, du);
            bstore32u(ro, pack_bf16x2(dg, du), off + (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * pitch);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + LMma::col_of(j);
      const uint32_t off = n < g.N ? (uint32_t)(((rl + (odd ? 1 : 0)) * g.ldg + (n & ~1)) * 2) : OOB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t gd[8], ud[8];
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t o = off + (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * pitch;
          gd[v / 2] = bload32(ri, o, 0);
          ud[v / 2] = bload32(ri, o + uoff, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t o = off + (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * pitch;
          float g0, g1, u0, u1;
          unpair_bf16_f32(gd[v / 2], odd, g0, g1);
          unpair_bf16_f32(ud[v / 2], odd, u0, u1);
          float dg[2], du[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float dh = mma.acc[i][j][v + q], gt = q ? g1 : g0, up = q ? u1 : u0;
            const float sg = sigmoid_fast(gt);
            dg[q] = dh * up * sg * (1.0f + gt * (1.0f - sg));
            du[q] = dh * gt * sg;
          }
          bstore32u(ro, pair_bf16(dg[0], dg[1], odd), o);
          bstore32u(ro, pair_bf16(du[0], du[1], odd), o + uoff);
        }
      }
    }
  }
}

// The large tile over a bf16 copy of the stack (XPipe).  Its LDS is the two A tiles and
// the three B tiles (160 KB): the tile lookup runs in every wave instead of through LDS.
template <bool KN, int EPI, bool SWIGLU>
__global__ __launch_bounds__(L_THREADS) void gemm_x_kernel(GroupedArgs g) {
  __shared__ ATile A0, A1;
  __shared__ XBuf B0, B1, B2;
  TileM tm;
  if (!find_tile_wave(g.off, g.E, L_BM, blockIdx.y, tm)) return;
  const int e = tm.e;
  const int n0 = blockIdx.x * (SWIGLU ? L_BN / 2 : L_BN);
  const RowMap map{n0, g.I, SWIGLU, SWIGLU && g.act == 1};
  const int Nrows = SWIGLU ? 2 * g.I : g.N;

  XPipe<KN> pipe(A0, A1, B0, B1, B2, g, e);
  pipe.mma.zero();
  pipe.la.init(tm.rows, tm.row0, g.a_gather, g.a_gdiv, g.lda);
  if constexpr (KN) pipe.lb.init(n0, g.N);
  else pipe.lb.init(map, Nrows, g.K);
  pipe.run(g.K / BK);
  large_finish<EPI>(pipe.mma, g, tm, e, n0, map, Nrows, A0, B0.nk);
}


// =============================================================== producer / consumer tiles
// The large tile with the work split by wave: eight consumer waves (two per SIMD) hold the
// 256 x 256 accumulators and only read MFMA fragments from LDS and issue MFMAs; four
// producer waves (one per SIMD) stream the A rows straight into LDS and load, decode and
// write the 4-bit B slab.  The decode's VALU work then issues beside the other waves' MFMAs
// instead of in the same instruction stream.  One workgroup barrier per slab: past barrier
// s, slab s is in LDS buffers s % 2, every consumer has finished slab s-1, and the
// producers fill buffers (s+1) % 2 with slab s+1 while the consumers compute slab s.  The
// B codes are loaded two slabs before they are decoded, in a register ring of three.
constexpr int WS_CONSUMERS = 512, WS_THREADS = 768;

// Workgroup barrier of the consumer waves: their LDS reads (MFMA fragments) completed.
__device__ __forceinline__ void consumer_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int BKIND, int FMT>
struct WSProducer {
  static constexpr bool KN = BKIND == B_QKN;
  using RowL = typename std::conditional<fmt_8bit(FMT), LQuantRow8<FMT>, LQuantRow<FMT>>::type;
  using KnL = typename std::conditional<fmt_8bit(FMT), LQuantKN8<FMT>, LQuantKN<FMT>>::type;
  // vector-memory loads of one B slab per producer thread (KnL::VTS K-major loaders, or one row)
  static constexpr int LOADS = KN ? KnL::VTS * KnL::LOADS : RowL::LOADS;
  using BTile = typename std::conditional<KN, LTileKN, LTile>::type;
  DecodeTables &tb;
  ATile &A0, &A1;
  BBuf &B0, &B1;
  __amdgpu_buffer_rsrc_t ra, rc, rs, rs2;
  LDirectAN<4> la;
  int v, p;  // producer wave (0..3) and thread (0..255)
  int sb = 0;  // first 64-wide slab of K this tile reduces over (its part of a K-split tile)
  RowL nk[3];          // NK ring: slab t in nk[t % 3]
  KnL kn[3][KnL::VTS];  // KN ring: K-major loaders of virtual threads p, p + 256

  __device__ __forceinline__ WSProducer(DecodeTables &tb_, ATile &a0, ATile &a1, BBuf &b0, BBuf &b1,
                                        const GroupedArgs &g)
      : tb(tb_), A0(a0), A1(a1), B0(b0), B1(b1),
        ra(make_rsrc(g.A, g.a_bytes)),
        rc(make_rsrc(g.q.codes, g.q.codes_bytes)),
        rs(make_rsrc(g.q.scale, g.q.scale_bytes)),
        rs2(make_rsrc(g.q.scale2, g.q.scale2_bytes)),
        v((int)(threadIdx.x - WS_CONSUMERS) >> 6),
        p((int)threadIdx.x - WS_CONSUMERS) {}

  template <int P>
  __device__ __forceinline__ ATile &atile() {
    if constexpr (P == 0) return A0;
    else return A1;
  }
  template <int P>
  __device__ __forceinline__ BTile &btile() {
    BBuf &b = P == 0 ? B0 : B1;
    if constexpr (KN) return b.kn;
    else return b.nk;
  }
  __device__ __forceinline__ static uint32_t dead(int slab, int nmain) { return slab < nmain ? 0u : OOB; }
  template <int Q>
  __device__ __forceinline__ void fetch_b(int slab, int nmain) {
    if constexpr (KN) {
#pragma unroll
      for (int h = 0; h < KnL::VTS; ++h) kn[Q][h].fetch(rc, rs, rs2, (slab + sb) * BK, dead(slab, nmain));
    } else {
      nk[Q].fetch(rc, rs, rs2, (slab + sb) * BK, dead(slab, nmain));
    }
  }
  template <int Q, int P>
  __device__ __forceinline__ void decode() {
    if constexpr (KN) {
#pragma unroll
      for (int h = 0; h < KnL::VTS; ++h) {
        kn[Q][h].prepare(tb);
#pragma unroll
        for (int part = 0; part < KnL::PARTS; ++part) kn[Q][h].store(btile<P>(), part, p + 256 * h);
      }
    } else {
      nk[Q].decode_store(btile<P>(), tb, p);
    }
  }
  __device__ __forceinline__ void issue_a(ATile &t, int slab, int nmain) {
    la.issue(ra, t, (uint32_t)((slab + sb) * BK * 2) | dead(slab, nmain), v);
  }
  // The LoRA K-extension as nl = ceil(r / 64) more slabs nmain, nmain + 1: tile rows of
  // the adapter input (xa, sorted rows) and of the adapter's B rows (xb, mapped like the
  // weight rows) go straight into the next buffers; columns at or past r read as zero.
  struct LoraCtx {
    int nl;
    int r, rows, Nrows;
    int64_t row0, ldxa, ldxb;
    RowMap map;
    __amdgpu_buffer_rsrc_t rxa, rxb;
  };
  struct RowsA {
    int rows;
    int64_t row0;
    __device__ __forceinline__ int64_t operator()(int r) const { return r < rows ? row0 + r : -1; }
  };
  struct RowsB {
    RowMap map;
    int Nrows;
    __device__ __forceinline__ int64_t operator()(int r) const {
      const int n = map(r);
      return n < Nrows ? n : -1;
    }
  };
  __device__ __forceinline__ void lora_slab(const LoraCtx &lc, int x, ATile &at, LTile &bt) {
    LDirectRows<4> da, db;
    da.init(v, RowsA{lc.rows, lc.row0}, lc.ldxa, x * BK, lc.r);
    db.init(v, RowsB{lc.map, lc.Nrows}, lc.ldxb, x * BK, lc.r);
    da.issue(lc.rxa, at.v, v);
    db.issue(lc.rxb, &bt.v[0][0], v);
    slab_barrier<0>();
  }
  // iteration s: the A rows of slab s+1, the B codes of slab s+3, and the decode of slab s+1
  // (codes loaded at iteration s-2) into buffers P = (s+1) % 2; Q = s % 3; past the main
  // slabs, LoRA slab s+1 - nmain instead.
  template <int P, int Q>
  __device__ __forceinline__ void body(int s, int nmain, const LoraCtx &lc) {
    if (s + 1 >= nmain && lc.nl > 0) {
      lora_slab(lc, s + 1 - nmain, atile<P>(), (P == 0 ? B0 : B1).nk);
      return;
    }
    issue_a(atile<P>(), s + 1, nmain);
    __builtin_amdgcn_sched_barrier(0);
    fetch_b<Q>(s + 3, nmain);
    __builtin_amdgcn_sched_barrier(0);
    decode<(Q + 1) % 3, P>();
    slab_barrier<LOADS>();  // A rows of slab s+1 landed; only the B codes of slab s+3 in flight
  }
  __device__ __forceinline__ void run(const GroupedArgs &g, int e, int n0, const RowMap &map, int Nrows,
                                      const TileM &tm, int kb0, int nmain, int nl) {
    sb = kb0;
    const LoraCtx ls{nl, g.r, tm.rows, Nrows, tm.row0, g.ldxa, g.ldxb, map,
                     make_rsrc(g.xa, (uint32_t)((int64_t)g.M * g.ldxa * 2)),
                     make_rsrc(g.xb + (int64_t)e * g.xb_estride, (uint32_t)((int64_t)Nrows * g.ldxb * 2))};
    la.init(v, tm.rows, tm.row0, g.a_gather, g.a_gdiv, g.lda);
    if constexpr (KN) {
#pragma unroll
      for (int h = 0; h < KnL::VTS; ++h) {
        kn[0][h].init(g.q, e, n0, g.N, p + 256 * h);
        kn[1][h] = kn[2][h] = kn[0][h];
      }
    } else {
      nk[0].init(g.q, e, map, Nrows, p);
      nk[1] = nk[2] = nk[0];
    }
    issue_a(A0, 0, nmain);
    __builtin_amdgcn_sched_barrier(0);
    fetch_b<0>(0, nmain);
    fetch_b<1>(1, nmain);
    fetch_b<2>(2, nmain);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * LOADS>();  // A rows and B codes of slab 0
    decode<0, 0>();
    slab_barrier<2 * LOADS>();
    // bodies 0 .. nb-1: the last prepares the last LoRA slab (slab nmain when there is none)
    const int nb = nmain + max(nl, 1) - 1;
    for (int s = 0;; s += 6) {
      body<1, 0>(s, nmain, ls);
      if (s + 1 >= nb) break;
      body<0, 1>(s + 1, nmain, ls);
      if (s + 2 >= nb) break;
      body<1, 2>(s + 2, nmain, ls);
      if (s + 3 >= nb) break;
      body<0, 0>(s + 3, nmain, ls);
      if (s + 4 >= nb) break;
      body<1, 1>(s + 4, nmain, ls);
      if (s + 5 >= nb) break;
      body<0, 2>(s + 5, nmain, ls);
      if (s + 6 >= nb) break;
    }
    wait_vmcnt<0>();  // nothing in flight past the main loop
  }
};

// ---------------------------------------------------------------- K-split of the last round
// With one workgroup per compute unit, a launch of nt tiles runs in ceil(nt / 256) rounds and
// its last round keeps only nt % 256 compute units busy.  The fp32-epilogue GEMMs (down,
// gate_up dgrad) split each tile of that round along K into q parts (q of them fit one round,
// each part keeps at least TAIL_MIN_SLABS slabs): part 0 runs in the tile's own workgroup,
// parts 1 .. q-1 in the extra grid rows, which are dispatched last.  Tiles are numbered as
// the grid deals them, t = row tile * gridDim.x + column tile.
struct TailPart {
  int ti = -1;  // index of the split tile among the split tiles, or -1: a whole tile
  int part = 0, q = 1;
};
// Row tiles of BMt rows over all expert segments (the same in every wave).
__device__ __forceinline__ int count_row_tiles(const int32_t *__restrict__ off, int E, int BMt) {
  const int lane = threadIdx.x & 63;
  int tot = 0;
  for (int c = 0; c < E; c += 64) {
    const int ee = c + lane;
    int nt = ee < E ? (off[ee + 1] - off[ee] + BMt - 1) / BMt : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) nt += __shfl_xor(nt, d);
    tot += nt;
  }
  return __builtin_amdgcn_readfirstlane(tot);
}
// This workgroup's (row tile, column tile) and part; false: nothing to do.
__device__ __forceinline__ bool tail_split(const GroupedArgs &g, int nall, int &slot, int &col, TailPart &tp) {
  const int ncol = (int)gridDim.x, nt = count_row_tiles(g.off, g.E, L_BM) * ncol;
  const int r = nt % TAIL_UNITS;  // tiles of the last, partial round
  const int q = r ? min(min(TAIL_Q, TAIL_UNITS / r), nall / TAIL_MIN_SLABS) : 1;
  const int first = nt - r;
  if (slot >= g.tail_slot0) {  // parts 1 .. q-1 of the split tiles
    const int x = (slot - g.tail_slot0) * ncol + col;
    if (q < 2 || x >= r * (q - 1)) return false;
    tp.ti = x / (q - 1);
    tp.part = 1 + x % (q - 1);
    tp.q = q;
    const int t = first + tp.ti;
    slot = t / ncol;
    col = t % ncol;
    return true;
  }
  const int t = slot * ncol + col;
  if (q > 1 && t >= first && t < nt) {
    tp.ti = t - first;
    tp.part = 0;
    tp.q = q;
  }
  return true;
}
// Accumulators 4c .. 4c+3 of this lane (c a constant in unrolled loops).
__device__ __forceinline__ f32x4 acc_piece(const LMma &m, int c) {
  const f32x16 &a = m.acc[c >> 3][(c >> 2) & 1];
  const int o = (c & 3) * 4;
  return f32x4{a[o], a[o + 1], a[o + 2], a[o + 3]};
}
// The q parts' partial tiles of this lane added in part order (base(p): the lane's pieces of
// part p) and stored as the fp32 epilogue stores them: out = alpha * sum + bias[column].
// Piece c holds accumulators (i, j, 4 (c & 3) .. +3) = rows rl + 32 i + 8 (c & 3) .. +3 of
// column n0 + col_of(j).  Branch-free over q: all TAIL_Q loads of a piece are issued (parts
// past q read part q - 1 again) and the sum takes part p only when p < q; one piece's loads
// are in flight at a time.
template <class Base>
__device__ __forceinline__ void tail_sum_store(const GroupedArgs &g, const TileM &tm, int n0, const Base &base,
                                               int q) {
  const int lane = threadIdx.x & 63;
  const int rl = LMma::wm() * 128 + (lane >> 5) * 4;
  float *C = (float *)g.C;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    f32x4 v[TAIL_Q];
#pragma unroll
    for (int p = 0; p < TAIL_Q; ++p) v[p] = *(const f32x4 *)(base(min(p, q - 1)) + c * 64 * 4);
    f32x4 sum = v[0];
#pragma unroll
    for (int p = 1; p < TAIL_Q; ++p) {
      const f32x4 t = sum + v[p];
      sum = p < q ? t : sum;
    }
    const int i = c >> 3, j = (c >> 2) & 1, r0 = rl + i * 32 + (c & 3) * 8;
    const int n = n0 + LMma::col_of(j);
    if (n < g.N) {
      const float bn = g.bias ? bf2f(g.bias[(int64_t)tm.e * g.bias_estride + n]) : 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (r0 + u < tm.rows) C[(int64_t)(tm.row0 + r0 + u) * g.ldc + n] = g.alpha * sum[u] + bn;
    }
    asm volatile("" ::: "memory");
  }
}
// The end of one part of a split tile, per consumer wave (no workgroup barrier: the producer
// waves have ended).  The wave stores its fp32 accumulators as the part's partial tile and
// counts its arrival on its (tile, wave) counter; the wave that arrives last adds the q
// partial tiles in part order, which fixes the result bit for bit whatever the arrival
// order, stores it through the tile epilogue and resets the counter for the next launch.
// Partial layout per (tile, part, wave): 32 pieces of 4 accumulators x 64 lanes.
__device__ __forceinline__ void tail_finish(LMma &mma, const GroupedArgs &g, const TileM &tm, int n0,
                                            const TailPart &tp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  auto base = [&](int p) { return g.tail + (((int64_t)(tp.ti * tp.q + p) * 8 + w) * 32 * 64 + lane) * 4; };
  {
    float *mine = base(tp.part);
#pragma unroll
    for (int c = 0; c < 32; ++c) *(f32x4 *)(mine + c * 64 * 4) = acc_piece(mma, c);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // the partial tile before the arrival
  int old = 0;
  if (lane == 0) old = atomicAdd(&g.tail_ctr[tp.ti * 8 + w], 1);
  old = __shfl(old, 0);
  if (old != tp.q - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other parts' partial tiles
  tail_sum_store(g, tm, n0, base, tp.q);  // the wave's own part is read back like the others
  if (lane == 0) g.tail_ctr[tp.ti * 8 + w] = 0;
}

template <int BKIND, int EPI, bool SWIGLU, int FMT>
__global__ __launch_bounds__(WS_THREADS) void gemm_ws_kernel(GroupedArgs g) {
  __shared__ DecodeTables tb;
  __shared__ ATile A0, A1;
  __shared__ BBuf B0, B1;
  __shared__ int tile_sh[4];
  constexpr bool KN = BKIND == B_QKN;
  init_decode_tables(tb, g.q);
  TileM tm;
  const int nall = g.K / BK;
  int slot = blockIdx.y, col = blockIdx.x;
  TailPart tp;
  if constexpr (EPI == EPI_F32) {
    if (g.tail && !tail_split(g, nall, slot, col, tp)) return;
  }
  if (!find_tile(g.off, g.E, L_BM, slot, tm, tile_sh)) return;
  const int e = tm.e;
  const int n0 = col * (SWIGLU ? L_BN / 2 : L_BN);
  const RowMap map{n0, g.I, SWIGLU, SWIGLU && g.act == 1};
  const int Nrows = SWIGLU ? 2 * g.I : g.N;
  // this tile's slabs of K: all of them, or its part of a split tile
  const int kb0 = tp.part * nall / tp.q, nmain = (tp.part + 1) * nall / tp.q - kb0;
  // the LoRA K-extension: ceil(r / 64) more slabs of the producers' pipeline (the last part)
  const int nl = tp.part == tp.q - 1 ? (g.r + BK - 1) / BK : 0;
  if (threadIdx.x >= WS_CONSUMERS) {
    // The NF4 decode is the heaviest VALU work of a slab: its waves issue first, so the
    // slab is ready sooner (measured 1-1.5% on the input-gradient GEMMs; the light MXFP4
    // decode is better left at the consumers' priority).
    if constexpr (FMT == FMT_NF4 || FMT == FMT_NF4_DQ) __builtin_amdgcn_s_setprio(2);
    WSProducer<BKIND, FMT> pr(tb, A0, A1, B0, B1, g);
    pr.run(g, e, n0, map, Nrows, tm, kb0, nmain, nl);
    return;
  }
  LMma mma;
  mma.zero();
  auto bt = [&](BBuf &b) -> auto & {
    if constexpr (KN) return b.kn;
    else return b.nk;
  };
  // 32-row sub-tiles of this wave's 128 rows that hold rows of the expert: fewer than 4 only in
  // an expert's last row tile, whose padding rows then cost no MFMAs
  const int half_rows = tm.rows - LMma::wm() * 128;
  const int ni = half_rows <= 0 ? 0 : min(4, (half_rows + 31) / 32);
  consumer_barrier();  // slab 0
  if (ni == 4) {
    for (int s = 0;; s += 2) {
      mma.step<KN>(A0, bt(B0), 4);
      consumer_barrier();
      if (s + 1 >= nmain) break;
      mma.step<KN>(A1, bt(B1), 4);
      consumer_barrier();
      if (s + 2 >= nmain) break;
    }
  } else {
    for (int s = 0;; s += 2) {
      mma.step_rows<KN>(A0, bt(B0), 4, ni);
      consumer_barrier();
      if (s + 1 >= nmain) break;
      mma.step_rows<KN>(A1, bt(B1), 4, ni);
      consumer_barrier();
      if (s + 2 >= nmain) break;
    }
  }
  for (int x = 0; x < nl; ++x) {  // LoRA slab x in buffers (nmain + x) % 2, NK layout, k < r
    const bool odd = (nmain + x) & 1;
    mma.step_rows<false>(odd ? A1 : A0, (odd ? B1 : B0).nk, min(4, (g.r - x * BK + 15) / 16), ni);
    if (x + 1 < nl) consumer_barrier();
  }
  if constexpr (EPI == EPI_F32) {
    if (tp.ti >= 0) {
      tail_finish(mma, g, tm, n0, tp);
      return;
    }
  }
  large_epilogue<EPI>(mma, g, tm, n0);
}

template <int BKIND, int EPI, bool SWIGLU>
static void launch_large(const GroupedArgs &a, dim3 grid, hipStream_t s) {
  if (a.Bx) {  // bf16 copy of the stack: no decode in the GEMM
    gemm_x_kernel<BKIND == B_QKN, EPI, SWIGLU><<<grid, L_THREADS, 0, s>>>(a);
    return;
  }
  switch (a.q.fmt) {
    case FMT_NF4: gemm_ws_kernel<BKIND, EPI, SWIGLU, FMT_NF4><<<grid, WS_THREADS, 0, s>>>(a); break;
    case FMT_NF4_DQ: gemm_ws_kernel<BKIND, EPI, SWIGLU, FMT_NF4_DQ><<<grid, WS_THREADS, 0, s>>>(a); break;
    case FMT_MXFP4: gemm_ws_kernel<BKIND, EPI, SWIGLU, FMT_MXFP4><<<grid, WS_THREADS, 0, s>>>(a); break;
    case FMT_INT8: gemm_ws_kernel<BKIND, EPI, SWIGLU, FMT_INT8><<<grid, WS_THREADS, 0, s>>>(a); break;
    default: gemm_ws_kernel<BKIND, EPI, SWIGLU, FMT_FP8><<<grid, WS_THREADS, 0, s>>>(a); break;
  }
}

static inline int m_slots(const GroupedArgs &a, int BMt) { return cdiv(a.M, BMt) + a.E; }

bool launch_gemm_gate_up(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_GATE_UP, s);
  dim3 grid(cdiv(a.I, L_BN / 2), m_slots(a, L_BM));
  launch_large<B_QNK, EPI_SWIGLU_FWD, true>(a, grid, s);
  return last_launch_ok();
}

// Grid of a large fp32-epilogue GEMM: the tile grid, plus rows for the parts of split tiles
// past the first (tail_split) when the caller gave the partial-tile workspace.
static dim3 f32_grid(GroupedArgs &b) {
  const int ncol = cdiv(b.N, L_BN), slots = m_slots(b, L_BM);
  // the bf16-copy tiles stay whole, and so do tiles too short for two parts
  if (b.Bx || b.K / BK < 2 * TAIL_MIN_SLABS) b.tail = nullptr;
  b.tail_slot0 = slots;
  return dim3(ncol, slots + (b.tail ? cdiv(TAIL_UNITS, ncol) : 0));
}

bool launch_gemm_down(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_DOWN, s);
  GroupedArgs b = a;
  const dim3 grid = f32_grid(b);
  launch_large<B_QNK, EPI_F32, false>(b, grid, s);
  return last_launch_ok();
}

bool launch_gemm_down_dgrad(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_DOWN_DGRAD, s);
  dim3 grid(cdiv(a.N, L_BN), m_slots(a, L_BM));
  launch_large<B_QKN, EPI_SWIGLU_BWD, false>(a, grid, s);
  return last_launch_ok();
}

bool launch_gemm_gate_up_dgrad(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_GATE_UP_DGRAD, s);
  GroupedArgs b = a;
  const dim3 grid = f32_grid(b);
  launch_large<B_QKN, EPI_F32, false>(b, grid, s);
  return last_launch_ok();
}

bool launch_lora_a(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_LORA_A, s);
  GroupedArgs b = a;
  if (!b.part) b.nsplit = 1;
  b.nsplit = std::max(1, b.nsplit);
  dim3 grid(cdiv(b.N, 64), m_slots(b, 128), b.nsplit);
  dense_gemm_kernel<64, 4, 1><<<grid, NTHREADS, 0, s>>>(b);
  if (!last_launch_ok()) return false;
  if (b.nsplit > 1)
    return launch_reduce_splits(b.part, b.nsplit, (int64_t)b.M * b.N, (int64_t)b.M * b.N, b.N, b.ldc, b.alpha, true,
                                b.C, s);
  return true;
}

// =============================================================== LoRA weight gradients
// Splits of one expert's reduction over its `rows` routed rows: one per four 64-row slabs,
// at least one, at most nsplit.
__device__ __forceinline__ int wgrad_expert_splits(int rows, int nsplit) {
  return max(1, min(nsplit, (rows + BK - 1) / BK / 4));
}

// C[e][a][b] = sum over the routed rows m of expert e of P[m][a] * Q[m][b].
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(NTHREADS) void wgrad_kernel(WgradArgs g) {
  // both operands stay in their memory order, [routed row][column], in LDS; the MFMA
  // fragments come out of the transposing LDS read
  __shared__ KTile<BM> As;
  __shared__ KTile<BN> Bs;
  const int e = blockIdx.z / g.nsplit, sp = blockIdx.z % g.nsplit;
  const int a0 = blockIdx.y * BM, b0 = blockIdx.x * BN;
  const int row0 = g.off[e], krows = g.off[e + 1] - g.off[e];
  // this expert's own split count: the splits past it have no rows and write nothing
  const int nsplit_e = g.nsplit > 1 ? wgrad_expert_splits(krows, g.nsplit) : 1;
  if (sp >= nsplit_e) return;
  Mma<BM, BN, WM, WN> mma;
  mma.zero();
  KRowLoader<BM> la;
  KRowLoader<BN> lb;
  // this split's slabs of the expert's rows
  const int nall = (krows + BK - 1) / BK, chunk = (nall + nsplit_e - 1) / nsplit_e;
  const int s0 = min(nall, sp * chunk), s1 = min(nall, s0 + chunk);
  auto fetch = [&](int s) {
    la.fetch(g.P, g.ldp, a0, g.Na, row0, krows, g.p_gather, g.p_gdiv, s * BK);
    lb.fetch(g.Q, g.ldq, b0, g.Nb, row0, krows, g.q_gather, g.q_gdiv, s * BK);
  };
  if (s0 < s1) fetch(s0);
  for (int s = s0; s < s1; ++s) {
    __syncthreads();
    la.store(As);
    lb.store(Bs);
    __syncthreads();
    if (s + 1 < s1) fetch(s + 1);
    mma_ktiles(mma, As, Bs, 4);
  }
  // every split of the expert writes its (possibly zero) partial sums; an expert that takes
  // one split writes C itself (the reduction leaves it alone)
  float *C = nsplit_e > 1 ? g.part + ((int64_t)sp * g.E + e) * g.Na * g.Nb : g.C + (int64_t)e * g.Na * g.Nb;
  mma.for_each([&](int row, int col, float v) {
    const int a = a0 + row, b = b0 + col;
    if (a < g.Na && b < g.Nb) C[(int64_t)a * g.Nb + b] = v;
  });
}

// C[e] = the sum of expert e's own splits of the partial sums [nsplit][E][Na * Nb], in split
// order, for the experts that take more than one split (the others wrote C directly).
__global__ void wgrad_reduce_kernel(const float *__restrict__ part, const int32_t *__restrict__ off, int nsplit,
                                    int64_t per_expert, int E, float *__restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)E * per_expert;
  if (i >= n) return;
  const int e = (int)(i / per_expert);
  const int ns = wgrad_expert_splits(off[e + 1] - off[e], nsplit);
  if (ns == 1) return;
  float acc = part[i];
  for (int s2 = 1; s2 < ns; ++s2) acc += part[s2 * n + i];
  C[i] = acc;
}

bool launch_wgrad(const WgradArgs &a, hipStream_t s) {
  if (a.E == 0) return true;
  LaunchScope ls(FAM_WGRAD, s);
  WgradArgs b = a;
  if (!b.part) b.nsplit = 1;
  b.nsplit = std::max(1, b.nsplit);
  if (b.Nb <= 64) {  // tall-skinny: rows = weight rows, cols = rank
    dim3 grid(cdiv(b.Nb, 64), cdiv(b.Na, 128), b.E * b.nsplit);
    wgrad_kernel<128, 64, 4, 1><<<grid, NTHREADS, 0, s>>>(b);
  } else {  // short-wide: rows = rank, cols = weight columns
    dim3 grid(cdiv(b.Nb, 128), cdiv(b.Na, 64), b.E * b.nsplit);
    wgrad_kernel<64, 128, 1, 4><<<grid, NTHREADS, 0, s>>>(b);
  }
  if (!last_launch_ok()) return false;
  if (b.nsplit > 1) {
    const int64_t n = (int64_t)b.E * b.Na * b.Nb;
    wgrad_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(b.part, b.off, b.nsplit, (int64_t)b.Na * b.Nb,
                                                                    b.E, b.C);
    return last_launch_ok();
  }
  return true;
}

// =============================================================== combine and friends
// y[t] = bf16(sum_j w[t,j] * O[inv[t*k+j]]), fp32 sum in j order.  One partial sum (the
// training forward): every choice's row piece is loaded before any is added, so the k
// loads of a thread are in flight together.
template <int U>  // 1024-column chunks per workgroup
__global__ void combine1_kernel(const float *__restrict__ O, const int32_t *__restrict__ inv,
                                const float *__restrict__ topw, int k, int H, uint16_t *__restrict__ y) {
  constexpr int KP = 8;  // choices held in registers (k <= KP)
  const int t = blockIdx.x;
  int pj[KP];
  float wj[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    pj[j] = j < k ? inv[(int64_t)t * k + j] : -1;
    wj[j] = j < k ? topw[(int64_t)t * k + j] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int h = (blockIdx.y * U + u) * 1024 + threadIdx.x * 4;
    if (h >= H) break;
    f32x4 o[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) o[j] = pj[j] >= 0 ? __builtin_nontemporal_load((const f32x4 *)(O + (int64_t)pj[j] * H + h)) : f32x4{0.f, 0.f, 0.f, 0.f};
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      if (pj[j] < 0) continue;
      a0 += wj[j] * o[j][0];
      a1 += wj[j] * o[j][1];
      a2 += wj[j] * o[j][2];
      a3 += wj[j] * o[j][3];
    }
    u32x2 out{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
    *(u32x2 *)(y + (int64_t)t * H + h) = out;
  }
}

// Any number of partial sums (up to COMBINE_MAX_SPLITS), added in split order first.
template <int U>  // 1024-column chunks per workgroup
__global__ void combine_kernel(const float *__restrict__ O, int nsplit, int64_t split_stride,
                               const int32_t *__restrict__ inv, const float *__restrict__ topw, int k,
                               int H, uint16_t *__restrict__ y) {
  // block (t, U chunks of 1024 columns); thread -> 4 columns of each chunk
  const int t = blockIdx.x;
  // the rows and weights of up to 8 choices first, then per choice the loads of all its
  // split partial sums at once (added in split order), so that the latencies overlap
  constexpr int KP = 8;
  int pj[KP];
  float wj[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    pj[j] = j < k ? inv[(int64_t)t * k + j] : -1;
    wj[j] = j < k ? topw[(int64_t)t * k + j] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int h = (blockIdx.y * U + u) * 1024 + threadIdx.x * 4;
    if (h >= H) break;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    auto add = [&](int p, float w) {
      f32x4 ov[COMBINE_MAX_SPLITS];
#pragma unroll
      for (int c = 0; c < COMBINE_MAX_SPLITS; ++c)
        if (c < nsplit) ov[c] = *(const f32x4 *)(O + c * split_stride + (int64_t)p * H + h);
      f32x4 o = ov[0];
#pragma unroll
      for (int c = 1; c < COMBINE_MAX_SPLITS; ++c)
        if (c < nsplit) o += ov[c];
      a0 += w * o[0];
      a1 += w * o[1];
      a2 += w * o[2];
      a3 += w * o[3];
    };
    // the first KP choices from registers (a compile-time index each), the rest from memory
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (pj[j] >= 0) add(pj[j], wj[j]);
    for (int j = KP; j < k; ++j) {
      const int p = inv[(int64_t)t * k + j];
      if (p >= 0) add(p, topw[(int64_t)t * k + j]);
    }
    u32x2 out{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
    *(u32x2 *)(y + (int64_t)t * H + h) = out;
  }
}

// ================================================================ router
// One wave per token.  Lane l holds logits l, l + 64, ... (at most 16 each).  Each of the k
// rounds takes the wave's largest remaining logit, equal logits in ascending expert id (a
// local pass, then a butterfly over the lanes), and lane j keeps round j.  The softmax over
// the chosen logits is fp32 and max-subtracted; its sum adds the lanes in a fixed tree.
__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_down(v, d);
  return __shfl(v, 0);  // lane 0's sum, the same tree for every call
}

template <int QN>  // logits per lane: E <= 64 QN
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                          int32_t *__restrict__ ids, float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *l = logits + (int64_t)t * E;
  float v[QN];
  uint32_t taken = 0;  // bit q: logit lane + 64 q is chosen or past E
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? l[e] : 0.0f;
    if (e >= E) taken |= 1u << q;
  }
  float myv = 0.0f, m = 0.0f;
  int myid = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int e = lane + 64 * q;
      if (!((taken >> q) & 1u) && (bi < 0 || v[q] > bv)) bv = v[q], bi = e;  // ascending e: ties keep the lower
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d);
      const int oi = __shfl_xor(bi, d);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) bv = ov, bi = oi;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) myv = bv, myid = bi;
    if (j == 0) m = bv;
  }
  const float ex = lane < k ? expf(myv - m) : 0.0f;
  const float den = wave_sum_fixed(ex);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myid;
    w[(int64_t)t * k + lane] = ex / den;
  }
}

bool launch_router_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t s) {
  if (T == 0) return true;
  if (E > 1024) return false;
  LaunchScope ls(FAM_ROUTER, s);
  const dim3 grid(cdiv(T, 4));
  if (E <= 64) router_topk_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128) router_topk_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256) router_topk_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, ids, w);
  else router_topk_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, ids, w);
  return last_launch_ok();
}

// d_logit[ids[t, j]] = w_j (dw_j - sum_i w_i dw_i), zero elsewhere: one wave per token.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float *__restrict__ w, const float *__restrict__ dw,
                                                         const int32_t *__restrict__ ids, int T, int E, int k,
                                                         float *__restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float wj = lane < k ? w[(int64_t)t * k + lane] : 0.0f;
  const float gj = lane < k ? dw[(int64_t)t * k + lane] : 0.0f;
  const int idj = lane < k ? ids[(int64_t)t * k + lane] : -1;
  const float dot = wave_sum_fixed(wj * gj);
  const float dj = wj * (gj - dot);
  float out[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) out[q] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int id = __shfl(idj, j);
    const float d = __shfl(dj, j);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (id == lane + 64 * q) out[q] = d;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = lane + 64 * q;
    if (e < E) dl[(int64_t)t * E + e] = out[q];
  }
}

bool launch_router_bwd(const float *w, const float *dw, const int32_t *ids, int T, int E, int k, float *dl,
                       hipStream_t s) {
  if (T == 0) return true;
  LaunchScope ls(FAM_ROUTER, s);
  router_bwd_kernel<<<cdiv(T, 4), 256, 0, s>>>(w, dw, ids, T, E, k, dl);
  return last_launch_ok();
}

bool launch_combine(const float *O, int nsplit, int64_t split_stride, const int32_t *inv, const float *topw,
                    int T, int k, int H, uint16_t *y, hipStream_t s) {
  if (T == 0) return true;
  if (nsplit < 1 || nsplit > COMBINE_MAX_SPLITS) return false;
  LaunchScope ls(FAM_COMBINE, s);
  // many tokens: a workgroup per token covers up to 4 chunks (fewer, longer workgroups)
  if (nsplit == 1 && k <= 8) {
    if (T >= 1024) combine1_kernel<4><<<dim3(T, cdiv(H, 4096)), 256, 0, s>>>(O, inv, topw, k, H, y);
    else combine1_kernel<1><<<dim3(T, cdiv(H, 1024)), 256, 0, s>>>(O, inv, topw, k, H, y);
    return last_launch_ok();
  }
  if (T >= 1024) combine_kernel<4><<<dim3(T, cdiv(H, 4096)), 256, 0, s>>>(O, nsplit, split_stride, inv, topw, k, H, y);
  else combine_kernel<1><<<dim3(T, cdiv(H, 1024)), 256, 0, s>>>(O, nsplit, split_stride, inv, topw, k, H, y);
  return last_launch_ok();
}

// dO[p] = bf16(w * dy[t]); d_topw[t,j] = <dy[t], O[p]>.
__global__ void combine_bwd_kernel(const uint16_t *__restrict__ dy, const float *__restrict__ O,
                                   const int32_t *__restrict__ inv, const float *__restrict__ topw,
                                   int k, int H, uint16_t *__restrict__ dO,
                                   float *__restrict__ d_topw) {
  const int64_t f = blockIdx.x;
  const int t = (int)(f / k);
  const int p = inv[f];
  __shared__ float red[4];
  if (p < 0) {
    if (d_topw && threadIdx.x == 0) d_topw[f] = 0.0f;
    return;
  }
  const float w = topw[f];
  float dot = 0.0f;
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    const u32x2 d = *(const u32x2 *)(dy + (int64_t)t * H + h);
    const float d0 = __uint_as_float(d[0] << 16), d1 = __uint_as_float(d[0] & 0xffff0000u);
    const float d2 = __uint_as_float(d[1] << 16), d3 = __uint_as_float(d[1] & 0xffff0000u);
    const f32x4 o = __builtin_nontemporal_load((const f32x4 *)(O + (int64_t)p * H + h));
    dot += d0 * o[0] + d1 * o[1] + d2 * o[2] + d3 * o[3];
    u32x2 out{pack_bf16x2(w * d0, w * d1), pack_bf16x2(w * d2, w * d3)};
    *(u32x2 *)(dO + (int64_t)p * H + h) = out;
  }
  if (d_topw) {
    for (int d = 32; d > 0; d >>= 1) dot += __shfl_xor(dot, d);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.0f;
      for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
      d_topw[f] = s;
    }
  }
}

bool launch_combine_bwd(const uint16_t *dy, const float *O, const int32_t *inv, const float *topw,
                        int T, int k, int H, uint16_t *dO, float *d_topw, hipStream_t s) {
  if (T == 0) return true;
  LaunchScope ls(FAM_COMBINE_BWD, s);
  combine_bwd_kernel<<<T * k, 256, 0, s>>>(dy, O, inv, topw, k, H, dO, d_topw);
  return last_launch_ok();
}

// dx[t] = bf16(sum_j dXp[inv[t*k+j]]).
__global__ void unpermute_kernel(const float *__restrict__ dXp, const int32_t *__restrict__ inv, int k,
                                 int H, uint16_t *__restrict__ dx) {
  const int t = blockIdx.x;
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < k; ++j) {
      const int p = inv[(int64_t)t * k + j];
      if (p < 0) continue;
      const f32x4 o = __builtin_nontemporal_load((const f32x4 *)(dXp + (int64_t)p * H + h));
      a0 += o[0];
      a1 += o[1];
      a2 += o[2];
      a3 += o[3];
    }
    u32x2 out{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
    *(u32x2 *)(dx + (int64_t)t * H + h) = out;
  }
}

bool launch_unpermute(const float *dXp, const int32_t *inv, int T, int k, int H, uint16_t *dx,
                      hipStream_t s) {
  if (T == 0) return true;
  LaunchScope ls(FAM_UNPERMUTE, s);
  unpermute_kernel<<<T, 256, 0, s>>>(dXp, inv, k, H, dx);
  return last_launch_ok();
}

// out[e][c][r] = in[e][r][c] (bf16), 32x32 tiles through LDS.
__global__ void transpose_kernel(const uint16_t *__restrict__ in, int R, int C, uint16_t *__restrict__ out) {
  __shared__ uint16_t t[32][33];
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const uint16_t *src = in + (int64_t)e * R * C;
  uint16_t *dst = out + (int64_t)e * R * C;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 8 rows per pass
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? src[(int64_t)r * C + c] : 0;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) dst[(int64_t)c * R + r] = t[tx][i];
  }
}

// Narrow matrices (adapter factors: one side is the rank, at most 128): a thread takes 8
// consecutive elements of one row of the narrow side (one 16-byte access), blockIdx.y the
// 8-element group, so that a wave's 2-byte accesses on the other side cover 128
// consecutive bytes.
template <bool NARROW_IN>
__global__ void transpose_narrow_kernel(const uint16_t *__restrict__ in, int R, int C, uint16_t *__restrict__ out) {
  const int e = blockIdx.z, g8 = blockIdx.y * 8;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const uint16_t *src = in + (int64_t)e * R * C;
  uint16_t *dst = out + (int64_t)e * R * C;
  if constexpr (NARROW_IN) {  // C <= 128: input row i, columns g8 .. g8 + 7
    if (i >= R) return;
    const u32x4 v = *(const u32x4 *)(src + (int64_t)i * C + g8);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[(int64_t)(g8 + q) * R + i] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
  } else {  // R <= 128: output row i, elements g8 .. g8 + 7
    if (i >= C) return;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)src[(int64_t)(g8 + 2 * q) * C + i] | ((uint32_t)src[(int64_t)(g8 + 2 * q + 1) * C + i] << 16);
    *(u32x4 *)(dst + (int64_t)i * R + g8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

bool launch_transpose(const uint16_t *in, int E, int R, int C, uint16_t *out, hipStream_t s) {
  if (E == 0 || R == 0 || C == 0) return true;
  LaunchScope ls(FAM_TRANSPOSE, s);
  // narrow forms need the narrow side a multiple of 8 (16-byte row pieces)
  if (C <= 128 && C % 8 == 0) {
    transpose_narrow_kernel<true><<<dim3(cdiv(R, 256), C / 8, E), 256, 0, s>>>(in, R, C, out);
  } else if (R <= 128 && R % 8 == 0) {
    transpose_narrow_kernel<false><<<dim3(cdiv(C, 256), R / 8, E), 256, 0, s>>>(in, R, C, out);
  } else {
    dim3 grid(cdiv(C, 32), cdiv(R, 32), E);
    transpose_kernel<<<grid, 256, 0, s>>>(in, R, C, out);
  }
  return last_launch_ok();
}

// =============================================================== quantise / dequantise
__device__ __forceinline__ uint32_t nf4_nearest_dev(float v) {
  uint32_t best = 0;
  float bestd = fabsf(v - kNF4[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    const float d = fabsf(v - kNF4[i]);
    if (d < bestd) {
      bestd = d;
      best = i;
    }
  }
  return best;
}

// One wave64 per block of 64 elements (element i of the block on lane i).
__global__ void quant_nf4_kernel(const float *__restrict__ w, int64_t nblk, uint8_t *__restrict__ codes,
                                 float *__restrict__ absmax_out) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= nblk) return;
  const float v = w[b * 64 + lane];
  float amax = fabsf(v);
  for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const uint32_t q = amax == 0.0f ? 7u : nf4_nearest_dev(v / amax);
  const uint32_t partner = __shfl_xor(q, 1);
  if ((lane & 1) == 0) codes[b * 32 + (lane >> 1)] = (uint8_t)((q << 4) | partner);
  if (lane == 0 && absmax_out) absmax_out[b] = amax;
}

// Second level of NF4_DQ: one workgroup of 256 threads per group of 256 blocks.
__global__ void quant_dq_kernel(const float *__restrict__ w, int64_t nblk, uint8_t *__restrict__ qabs,
                                float *__restrict__ scale2) {
  __shared__ float red[256];
  const int64_t g = blockIdx.x;
  const int64_t b = g * 256 + threadIdx.x;
  float amax = 0.0f;
  if (b < nblk) {
    const float *p = w + b * 64;
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(p[i]));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float s2 = red[0];
  if (threadIdx.x == 0) scale2[g] = s2;
  if (b < nblk) {
    uint8_t c = 0;
    if (s2 != 0.0f) {
      float t = amax / s2;
      t = t * 255.0f;
      c = (uint8_t)rintf(t);
    }
    qabs[b] = c;
  }
}

// One wave64 per two MXFP4 blocks of 32 (lanes 0-31 and 32-63).
__global__ void quant_mxfp4_kernel(const float *__restrict__ w, int64_t nblk, uint8_t *__restrict__ codes,
                                   uint8_t *__restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t b = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool ok = b < nblk;
  const float v = ok ? w[b * 32 + (lane & 31)] : 0.0f;
  float amax = fabsf(v);
  for (int d = 16; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  uint32_t q = 0;
  int X = 0;
  if (amax != 0.0f) {
    int ex;
    frexpf(amax, &ex);
    X = min(254, max(0, (ex - 1) - 2 + 127));
    const float s = ldexpf(v, -(X - 127));
    const float a = fabsf(s);
    if (a >= 6.0f) {
      q = 7;
    } else {
      float bestd = a;
      for (int i = 1; i < 8; ++i) {
        const float d = fabsf(a - kE2M1[i]);
        if (d < bestd || (d == bestd && (i & 1) == 0)) {
          bestd = d;
          q = i;
        }
      }
    }
    if (s < 0.0f && q != 0) q |= 8;
  }
  const uint32_t partner = __shfl_xor(q, 1);
  if (ok && (lane & 1) == 0) codes[b * 16 + ((lane & 31) >> 1)] = (uint8_t)(q | (partner << 4));
  if (ok && (lane & 31) == 0) scales[b] = (uint8_t)X;
}

// 8-bit bases: one wave64 per block of 64 (element i on lane i).  INT8: s = absmax / 127,
// q = rne(w / s) in [-127, 127].  FP8: s = absmax / 448, the hardware round-to-nearest-even
// conversion of w / s clamped to the largest finite value 448 (it would give NaN beyond).
template <int FMT>
__global__ void quant8_kernel(const float *__restrict__ w, int64_t nblk, uint8_t *__restrict__ codes,
                              float *__restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= nblk) return;
  const float v = w[b * 64 + lane];
  float amax = fabsf(v);
  for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float sc = amax / (FMT == FMT_INT8 ? 127.0f : 448.0f);
  uint32_t q = 0;
  if (sc != 0.0f) {
    const float t = v / sc;
    if constexpr (FMT == FMT_INT8) {
      q = (uint32_t)(uint8_t)(int8_t)(int)fminf(127.0f, fmaxf(-127.0f, rintf(t)));
    } else {
      const float c = fminf(448.0f, fmaxf(-448.0f, t));
      q = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
      if (q == 0x80u) q = 0;  // -0 is stored as +0
    }
  }
  codes[b * 64 + lane] = (uint8_t)q;
  if (lane == 0) scales[b] = sc;
}

bool launch_quantize(int fmt, int64_t n, const float *w, uint8_t *codes, void *scale, float *scale2,
                     hipStream_t s) {
  if (n == 0) return true;
  if (fmt < FMT_NF4 || fmt > FMT_FP8) return false;
  LaunchScope ls(FAM_QUANT, s);
  if (fmt_8bit(fmt)) {
    const int64_t nblk = n / 64;
    if (fmt == FMT_INT8) quant8_kernel<FMT_INT8><<<cdiv(nblk, 4), 256, 0, s>>>(w, nblk, codes, (float *)scale);
    else quant8_kernel<FMT_FP8><<<cdiv(nblk, 4), 256, 0, s>>>(w, nblk, codes, (float *)scale);
    return last_launch_ok();
  }
  if (fmt == FMT_MXFP4) {
    const int64_t nblk = n / 32;
    quant_mxfp4_kernel<<<cdiv(nblk, 8), 256, 0, s>>>(w, nblk, codes, (uint8_t *)scale);
    return last_launch_ok();
  }
  const int64_t nblk = n / 64;
  quant_nf4_kernel<<<cdiv(nblk, 4), 256, 0, s>>>(w, nblk, codes,
                                                 fmt == FMT_NF4 ? (float *)scale : nullptr);
  if (!last_launch_ok()) return false;
  if (fmt == FMT_NF4_DQ) {
    quant_dq_kernel<<<cdiv(nblk, 256), 256, 0, s>>>(w, nblk, (uint8_t *)scale, scale2);
    return last_launch_ok();
  }
  return true;
}

// 8 consecutive elements per thread: elements elem0 + 8*i .. +8 of the flat stack.
__global__ void dequant_kernel(QStack q, int64_t elem0, int64_t nwords, float *__restrict__ f32,
                               uint16_t *__restrict__ b16) {
  __shared__ DecodeTables tb;
  init_decode_tables(tb, q);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int64_t elem = elem0 + i * 8;
  float vals[8];
  u32x4 bits;
  if (fmt_8bit(q.fmt)) {  // 8 code bytes, one fp32 scale per 64 elements
    const u32x2 c = *(const u32x2 *)(q.codes + elem);
    const float sc = ((const float *)q.scale)[elem >> 6];
    const bool i8 = q.fmt == FMT_INT8;
    const u32x2 a = i8 ? byte_word_to_bf16<FMT_INT8>(c[0], sc) : byte_word_to_bf16<FMT_FP8>(c[0], sc);
    const u32x2 b = i8 ? byte_word_to_bf16<FMT_INT8>(c[1], sc) : byte_word_to_bf16<FMT_FP8>(c[1], sc);
    bits = u32x4{a[0], a[1], b[0], b[1]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t byte = (c[j >> 2] >> (8 * (j & 3))) & 0xffu;
      const float v = i8 ? (float)(int)(int8_t)byte : __builtin_amdgcn_cvt_pk_f32_fp8((int)byte, false)[0];
      vals[j] = v * sc;
    }
  } else if (q.fmt == FMT_MXFP4) {
    const uint32_t w = *(const uint32_t *)(q.codes + elem / 2);
    const uint32_t X = ((const uint8_t *)q.scale)[elem >> 5];
    const float sc = e8m0_to_f32(X);
    bits = mxfp4_word_to_bf16(w, sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = (w >> (4 * j)) & 15u;  // element j: byte j/2, low nibble first
      const float m = (c & 8u) ? -kE2M1[c & 7u] : kE2M1[c & 7u];
      vals[j] = m * sc;
    }
  } else {
    const uint32_t w = *(const uint32_t *)(q.codes + elem / 2);
    const float am = nf4_block_absmax(q, elem >> 6, tb);
    bits = nf4_word_to_bf16(w, am, tb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (w >> (8 * j)) & 0xffu;
      const float2 cv = tb.cb2[byte];
      vals[2 * j] = cv.x * am;
      vals[2 * j + 1] = cv.y * am;
    }
  }
  if (f32) {
    f32x4 a{vals[0], vals[1], vals[2], vals[3]}, b{vals[4], vals[5], vals[6], vals[7]};
    *(f32x4 *)(f32 + i * 8) = a;
    *(f32x4 *)(f32 + i * 8 + 4) = b;
  }
  if (b16) *(u32x4 *)(b16 + i * 8) = bits;
}

// bf16 copy of a stack in its stored layout, decoded with the large tiles' GroupDecoder.
// A workgroup covers 1024 consecutive 8-code words; load and store p of thread t handle
// word 256 p + t, so consecutive lanes read consecutive 4-byte code words and write
// consecutive 16-byte pieces.
template <int FMT>
__global__ __launch_bounds__(256) void expand_kernel(QStack q, int64_t nwords, uint16_t *__restrict__ out) {
  __shared__ DecodeTables tb;
  if constexpr (FMT != FMT_MXFP4) {
    init_decode_tables(tb, q);
    __syncthreads();
  }
  const int64_t w0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  uint32_t code[4], raw[4];
  float s2[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t w = w0 + 256 * p;
    code[p] = 0;
    raw[p] = 0;
    s2[p] = 1.0f;
    if (w < nwords) {
      code[p] = ((const uint32_t *)q.codes)[w];
      if constexpr (FMT == FMT_NF4) {
        raw[p] = ((const uint32_t *)q.scale)[w >> 3];
      } else if constexpr (FMT == FMT_NF4_DQ) {
        raw[p] = ((const uint8_t *)q.scale)[w >> 3];
        s2[p] = q.scale2[w >> 11];
      } else {
        raw[p] = ((const uint8_t *)q.scale)[w >> 2];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t w = w0 + 256 * p;
    if (w >= nwords) continue;
    GroupDecoder<FMT> dec;
    dec.prepare(raw[p], s2[p], tb);
    *(u32x4 *)(out + w * 8) = dec(code[p]);
  }
}

// The same for 8-bit stacks: thread t of a workgroup takes 8-byte piece 256 p + t (8
// elements under one fp32 scale) and writes its 16 bytes of bf16.
template <int FMT>
__global__ __launch_bounds__(256) void expand8_kernel(QStack q, int64_t npieces, uint16_t *__restrict__ out) {
  const int64_t w0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t w = w0 + 256 * p;
    if (w >= npieces) continue;
    const u32x2 c = ((const u32x2 *)q.codes)[w];
    const float sc = ((const float *)q.scale)[w >> 3];
    const u32x2 a = byte_word_to_bf16<FMT>(c[0], sc), b = byte_word_to_bf16<FMT>(c[1], sc);
    *(u32x4 *)(out + w * 8) = u32x4{a[0], a[1], b[0], b[1]};
  }
}

bool launch_expand(const QStack &q, int E, uint16_t *out, hipStream_t s) {
  const int64_t nwords = (int64_t)E * q.N * q.K / 8;
  if (nwords == 0) return true;
  if (q.fmt < FMT_NF4 || q.fmt > FMT_FP8) return false;
  LaunchScope ls(FAM_EXPAND, s);
  const unsigned grid = (unsigned)((nwords + 1023) / 1024);
  switch (q.fmt) {
    case FMT_INT8: expand8_kernel<FMT_INT8><<<grid, 256, 0, s>>>(q, nwords, out); break;
    case FMT_FP8: expand8_kernel<FMT_FP8><<<grid, 256, 0, s>>>(q, nwords, out); break;
    case FMT_NF4: expand_kernel<FMT_NF4><<<grid, 256, 0, s>>>(q, nwords, out); break;
    case FMT_NF4_DQ: expand_kernel<FMT_NF4_DQ><<<grid, 256, 0, s>>>(q, nwords, out); break;
    default: expand_kernel<FMT_MXFP4><<<grid, 256, 0, s>>>(q, nwords, out); break;
  }
  return last_launch_ok();
}

bool launch_dequant(const QStack &q, int64_t elem0, int64_t n, float *out_f32, uint16_t *out_bf16,
                    hipStream_t s) {
  if (n == 0) return true;
  if (q.fmt < FMT_NF4 || q.fmt > FMT_FP8) return false;
  LaunchScope ls(FAM_DEQUANT, s);
  const int64_t nwords = n / 8;
  dequant_kernel<<<cdiv(nwords, 256), 256, 0, s>>>(q, elem0, nwords, out_f32, out_bf16);
  return last_launch_ok();
}

}  // namespace e4b
