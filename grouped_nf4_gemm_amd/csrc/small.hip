// Decode-shaped forward: grouped 4-bit GEMMs for a few routed rows per expert.
//
// With a handful of tokens per expert the layer is bound by reading the packed weights
// once from HBM, and the large-tile kernels (256-row tiles, decode shared through LDS)
// would spend their time on padding.  Here every wave streams the codes of its own weight
// rows straight into MFMA operand registers, with no LDS staging of the weights:
//
//  * MFMA C[token][n] = X[token][k] . W[n][k] with v_mfma_f32_32x32x16_bf16, 32 tokens by
//    32 weight rows.  Lane (n, h) loads the 16 code bytes of weight row n covering
//    k = 32h .. 32h+31 of a 64-wide block and feeds them to the four MFMAs of the block
//    (MFMA s takes k = 32h + 8s .. +7); the activation fragments use the same k order.
//  * NF4 codes become bf16 code values through a table read (two codes per read) and the
//    block's absmax scales the fp32 partial sum of that block (the block of 64 lies in
//    one lane column, so the scale is one value per lane).  MXFP4 codes are converted
//    with their E8M0 scale by the hardware conversion, which is exact.
//  * Every load of a block (activation fragments, codes, scales) is issued D blocks ahead
//    in one group: vector-memory loads retire in order, so a load issued later than the
//    codes would make their wait cover the younger blocks as well.  The ring has D + 1
//    register slots and each step first refills the slot its predecessor freed, then
//    computes: loads placed after the compute of the last step would be carried around
//    the loop edge and land right before their use.
//  * gate_up rows come as 16 gate rows and the 16 up rows of the same h columns, so the
//    SwiGLU epilogue pairs lanes n and n + 16.  down splits K over workgroups and writes
//    fp32 partial sums that the combine adds in split order.
#include <type_traits>

#include "gemm.hpp"
#include "kernels.hpp"

namespace e4b {

constexpr int SM_WAVES = 8, SM_THREADS = 64 * SM_WAVES;

// 64 copies of the bf16 code-pair table, copy c for lane c: entry b of copy c at byte
// offset b * 256 + c * 4, so one byte permute forms the address and no two lanes of a
// wave share a bank.  Entry b holds bf16(nf4[b >> 4]) in its low half (element 2j, the
// high nibble) and bf16(nf4[b & 15]) in its high half.
struct SmallTables {
  uint32_t cp[256][64];
};

// Thread t of the 512 computes entry t / 2 once and writes 8 of its 16 pieces (16 bytes
// each, copies 4p .. 4p+3).  In the k-th store lane t writes piece (k + t / 2 + 8 (t & 1))
// mod 16: the 16 lanes of one store pass write 16 different pieces, so their banks differ.
__device__ __forceinline__ void init_small_tables(SmallTables &t, const float *codebook) {
  static_assert(SM_THREADS == 512, "two threads per table entry");
  const uint32_t b = threadIdx.x >> 1;
  const uint32_t v = pack_bf16x2(code_value(codebook, b >> 4), code_value(codebook, b & 15));
  const uint32_t p0 = b + 8 * (threadIdx.x & 1);
#pragma unroll
  for (uint32_t k = 0; k < 8; ++k) *(u32x4 *)&t.cp[b][4 * ((p0 + k) & 15)] = u32x4{v, v, v, v};
}

// bf16 code values of the four code bytes of word w for this lane (l4 = lane * 4).
__device__ __forceinline__ bf16x8 nf4_codes_bf16(uint32_t w, uint32_t l4, const SmallTables &t) {
  const char *base = (const char *)&t.cp[0][0];
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte 0 of the address = l4, byte 1 = code byte j of w, bytes 2-3 = 0
    const uint32_t addr = __builtin_amdgcn_perm(w, l4, 0x0C0C0400u | ((4u + j) << 8));
    r[j] = *(const uint32_t *)(base + addr);
  }
  return __builtin_bit_cast(bf16x8, r);
}

// Static LDS of the two kernels: the code table (NF4 formats only) comes first, at LDS
// address 0, so that a table address formed by a byte permute needs no base added.
template <bool TABLE, class Rest>
struct WithTable {
  SmallTables tb;
  Rest rest;
};
template <class Rest>
struct WithTable<false, Rest> {
  Rest rest;
};
template <bool TABLE, class Rest>
__device__ __forceinline__ SmallTables &table_of(WithTable<TABLE, Rest> &s) {
  if constexpr (TABLE) return s.tb;
  else return *reinterpret_cast<SmallTables *>(&s);  // not read: the formats without a table
}

constexpr int SM_BMT = 32;                  // tokens per workgroup slot
constexpr int SM_CB = 4;                    // 64-wide blocks per chunk

// Activations of one chunk for the slot's tokens in a ring of four buffers: row t = token t
// of the slot (zero past its rows), 32 pieces of 16 bytes (4 blocks of 8).  Rows are 512
// bytes apart, all starting in one bank: piece p of row t sits at p ^ (t & 15), so the
// fragment reads of 16 rows (one 16-lane pass) fall in 16 different groups of 4 banks.
struct SmallX {
  uint16_t v[4][SM_BMT][SM_CB * 64];
};
__device__ __forceinline__ int xpiece_swz(int t, int p) { return p ^ (t & 15); }

// Byte o / the dword at byte offset o (a multiple of 4) of a 16-byte window.  Byte permutes
// with per-lane selectors pick within each half and a select picks the half, so the window
// stays in registers: a chain of selects over the four words is recognised as a
// variable-index vector extract, which puts the window in a private array (scratch).
__device__ __forceinline__ uint32_t byte_at(const u32x4 &r, uint32_t o) {
  const uint32_t sel = 0x0C0C0C00u | (o & 7u);
  const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], sel), hi = __builtin_amdgcn_perm(r[3], r[2], sel);
  return (o & 8u) ? hi : lo;
}
__device__ __forceinline__ uint32_t dword_at(const u32x4 &r, uint32_t o) {
  const uint32_t sel = (o & 4u) ? 0x07060504u : 0x03020100u;
  const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], sel), hi = __builtin_amdgcn_perm(r[3], r[2], sel);
  return (o & 8u) ? hi : lo;
}

// Raw scales of one chunk (4 blocks) of one weight row, read as one 16-byte window that
// starts `sh` bytes before them (the window is moved back to stay inside the scale
// array): NF4: 4 fp32 absmax at sh + 4b; NF4_DQ: 4 absmax codes at sh + b, plus the
// second-level scales of the chunk's first and last block; MXFP4: this lane's E8M0 byte
// of block b at sh + 2b.
struct ChunkScale {
  u32x4 raw;
  uint32_t sh;
  float s2a, s2b;
};

// LDS barrier that leaves vector-memory loads in flight: waits for this wave's LDS
// accesses only (vmcnt and expcnt at their maximum, lgkmcnt(0)).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The codes of a strip are read CH blocks at a time with each lane loading 16 bytes of one
// row (2 CH lanes per row, so a load covers whole 32 CH-byte row segments), staged in a
// per-wave LDS buffer, and read back in the MFMA lane layout: loads in which the 64 lanes
// touch 32 different rows keep the vector memory unit stalled on its cache.
template <int CH>
__device__ __forceinline__ int stage_swz(int rho, int p) {
  if constexpr (CH == 4) return p ^ ((rho >> 1) & 7);  // 8 pieces per row
  else return p ^ ((rho >> 2) & 3);                      // 4 pieces per row
}
constexpr int stage_bytes(int ch) { return SM_WAVES * 32 * ch * 32; }

// ------------------------------------------------------------ two-launch decode forward
// Routing of M <= 256 routed rows inside one workgroup, with the result of the route kernel:
// per-wave counts, their scan over the waves and over the experts, then stable ranks by
// ballot.  LDS: [4][E+1] counts, [E+1] cnt, [E+1] off, [M] perm, [M] inv.
struct LdsRoute {
  int32_t *cnt, *off, *perm, *inv;
};
__host__ __device__ constexpr size_t route_lds_bytes(int E, int M) { return (size_t)(6 * (E + 1) + 2 * M) * 4; }

__device__ __forceinline__ LdsRoute route_in_lds(const int32_t *__restrict__ ids, int M, int E, int32_t *sm) {
  const int KE = E + 1, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t *wc = sm, *cnt = sm + 4 * KE, *off = cnt + KE, *perm = off + KE, *inv = perm + M;
  for (int i = tid; i < 4 * KE; i += SM_THREADS) wc[i] = 0;
  const int f = 64 * w + lane;
  const bool act = w < 4 && f < M;
  const int e = act ? ids[f] : 0;
  const bool valid = act && e >= 0 && e < E;
  const int key = valid ? e : E;
  __syncthreads();
  if (act) atomicAdd(&wc[w * KE + key], 1);
  __syncthreads();
  for (int k = tid; k < KE; k += SM_THREADS) {
    int run = 0;
    for (int ww = 0; ww < 4; ++ww) {
      const int c = wc[ww * KE + k];
      wc[ww * KE + k] = run;
      run += c;
    }
    cnt[k] = run;
  }
  __syncthreads();
  if (w == 0) {
    int base = 0;
    for (int c = 0; c < E; c += 64) {
      const int ee = c + lane;
      const int v = ee < E ? cnt[ee] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      if (ee < E) off[ee] = base + incl - v;
      base += __shfl(incl, 63);
    }
    if (lane == 0) off[E] = base;
  }
  __syncthreads();
  if (w < 4) {
    const int nbits = 32 - __clz(E);
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    uint64_t eq = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      eq &= bit ? m : ~m;
    }
    const int rank = __popcll(eq & lt);
    if (valid) {
      const int pos = off[e] + wc[w * KE + e] + rank;
      perm[pos] = f;
      inv[f] = pos;
    } else if (act) {
      inv[f] = -1;
    }
  }
  __syncthreads();
  return LdsRoute{cnt, off, perm, inv};
}

// One gate_up workgroup hands the routing to the down launch (and to the caller's
// workspace), and zeroes the down launch's arrival counters.
__device__ __forceinline__ void route_export(const LdsRoute &r, const GroupedArgs &g) {
  const int KE = g.E + 1, nvalid = r.off[g.E];
  for (int i = threadIdx.x; i < KE; i += SM_THREADS) {
    g.fz.cnt[i] = r.cnt[i];
    g.fz.off[i] = r.off[i];
  }
  for (int p = threadIdx.x; p < g.M; p += SM_THREADS) {
    g.fz.perm[p] = p < nvalid ? r.perm[p] : -1;
    g.fz.inv[p] = r.inv[p];
  }
  for (int i = threadIdx.x; i < g.fz.nctr; i += SM_THREADS) g.fz.ctr[i] = 0;
}

// z2 of the rows row0 .. row0 + rows - 1 (rows <= 32) from the gate_up launch's partial
// sums, added in part order: zs[t][j] = bf16(s2 * sum_q zp[q][row0 + t][j]) for j < r (the
// down launch's rank), zero for r <= j < 32.  Every thread takes one group of 4 adjacent
// outputs (one output when r is not a multiple of 4) and every G-th part, G = 512 / groups
// (at least 1), loading 8 parts at a time; the G sums of a group are then added in order.
// red: 2048 floats of LDS; zs: [32][32] bf16 of LDS.  Ends with a barrier.
__device__ __forceinline__ void z2_reduce(const GroupedArgs &g, int row0, int rows, float *red, uint16_t *zs) {
  const int r = g.r, P = g.fz.nparts;
  const int W = (r & 3) == 0 ? 4 : 1;  // outputs per group
  const int ng = rows * r / W;
  const int G = max(1, SM_THREADS / max(1, ng)), stride = SM_THREADS / G;
  const int64_t pstride = (int64_t)g.M * r;
  for (int o = threadIdx.x / G; o < ng; o += stride) {
    const int gi = threadIdx.x % G;
    const float *src = g.fz.zp + (int64_t)row0 * r + (int64_t)o * W;  // rows are r apart: group o at o * W
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = gi; q0 < P; q0 += 8 * G) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * G;
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (q < P) {
          if (W == 4) v[u] = *(const f32x4 *)(src + q * pstride);
          else v[u][0] = src[q * pstride];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u * G < P) acc += v[u];
    }
    for (int i = 0; i < W; ++i) red[(o * W + i) * G + gi] = acc[i];
  }
  lds_barrier();
  for (int o = threadIdx.x; o < 32 * 32; o += SM_THREADS) {
    const int t = o >> 5, j = o & 31;
    float v = 0.0f;
    if (t < rows && j < r) {
      const int oo = t * r + j;
      for (int gi = 0; gi < G; ++gi) v += red[oo * G + gi];
      v *= g.fz.s2;
    }
    zs[o] = f2bf(v);
  }
  lds_barrier();
}

// Down launch of the two-launch forward: once this workgroup's partial sums are stored it
// counts its arrival on its column range [c0, c1); the last of the range's gridDim.y *
// gridDim.z workgroups forms y there, as the combine kernel does: y[t][c] =
// bf16(sum_j w[t,j] * (sum over splits of O[s][inv[t,j]][c])), splits then choices in order.
// flag: one int of LDS.  Every wave of the workgroup calls it once.
// The workgroup barrier orders every thread's stores before thread 0's agent-scope release
// fence (an L2 writeback), and the last workgroup's acquire fence (an L2 invalidate) before
// every thread's loads: one fence per workgroup and side, not a full fence (which would do
// both on every workgroup).
// A workgroup that stored nothing (an empty slot) arrives without the release fence: the
// counter's read-modify-writes carry the release of the workgroups before it.
__device__ __forceinline__ void arrive_combine(const GroupedArgs &g, int c0, int c1, int *flag, bool stored = true) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int total = (int)(gridDim.y * gridDim.z);
    if (stored) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(&g.fz.ctr[blockIdx.x], 1) == total - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  c1 = min(c1, g.N);
  if (c0 >= c1) return;
  const int ncol4 = (c1 - c0) / 4, k = g.fz.topk, ns = g.fz.nsplit, nq = g.fz.T * ncol4;
  const float *O = (const float *)g.C;
  // four column quads per thread and step; for each choice the partial sums of every split
  // of the four quads are loaded together (their latencies overlap)
  for (int q0 = threadIdx.x; q0 < nq; q0 += 4 * SM_THREADS) {
    f32x4 a[4];
    int tq[4], cq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = min(q0 + u * SM_THREADS, nq - 1);
      tq[u] = q / ncol4;
      cq[u] = c0 + 4 * (q - tq[u] * ncol4);
      a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int j = 0; j < k; ++j) {
      int pj[4];
      float wj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pj[u] = g.fz.inv[(int64_t)tq[u] * k + j];
        wj[u] = g.fz.topw[(int64_t)tq[u] * k + j];
      }
      f32x4 ov[4][SMALL_MAX_SPLITS];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int sp = 0; sp < SMALL_MAX_SPLITS; ++sp)
          if (sp < ns && pj[u] >= 0) ov[u][sp] = *(const f32x4 *)(O + sp * g.fz.split_stride + (int64_t)pj[u] * g.ldc + cq[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pj[u] < 0) continue;
        f32x4 o = ov[u][0];
#pragma unroll
        for (int sp = 1; sp < SMALL_MAX_SPLITS; ++sp)
          if (sp < ns) o += ov[u][sp];
        a[u][0] += wj[u] * o[0];
        a[u][1] += wj[u] * o[1];
        a[u][2] += wj[u] * o[2];
        a[u][3] += wj[u] * o[3];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q0 + u * SM_THREADS < nq)
        *(u32x2 *)(g.fz.y + (int64_t)tq[u] * g.ldc + cq[u]) = u32x2{pack_bf16x2(a[u][0], a[u][1]), pack_bf16x2(a[u][2], a[u][3])};
  }
}

// FUSE (two-launch forward): 0 off; 1 or 2: on, with ranks up to 16 FUSE.
template <int FMT, int SPW, int EPI, int DC, int FUSE>
__global__ __launch_bounds__(SM_THREADS) void small_gemm_kernel(GroupedArgs g, int kb_per_split,
                                                                 int64_t split_stride) {
  constexpr bool NF4ISH = FMT != FMT_MXFP4;
  constexpr int R = DC + 1;  // chunk slots of the register ring
  static_assert(SPW == 1 && SM_CB == 4, "one strip per wave, codes staged four blocks at a time");
  // LDS: the table (64 KB), the activation ring (64 KB) and the code stages (32 KB), the
  // whole 160 KB: the tile lookup runs in each wave
  struct Rest {
    SmallX xs;
    u32x4 stage[SM_WAVES][32 * 8];  // per wave: [32 strip rows][8 swizzled 16-byte pieces]
  };
  __shared__ __attribute__((aligned(16))) WithTable<NF4ISH, Rest> sm;
  SmallTables &tb = table_of(sm);
  SmallX &xs = sm.rest.xs;
  if constexpr (NF4ISH) init_small_tables(tb, g.q.codebook);
  constexpr bool FUP = FUSE && EPI == EPI_SWIGLU_FWD, FDN = FUSE && EPI == EPI_F32;
  // two-launch forward: the gate_up launch routes in LDS (the activation ring's space)
  const int32_t *offp = g.off, *gath = g.a_gather;
  if constexpr (FUP) {
    const LdsRoute rt = route_in_lds(g.fz.ids, g.M, g.E, (int32_t *)&xs);
    if (blockIdx.x == 0 && blockIdx.y == 0) route_export(rt, g);
    offp = rt.off;
    gath = rt.perm;
  }
  TileM tm;
  if (!find_tile_wave(offp, g.E, SM_BMT, blockIdx.y, tm)) {  // the same for every wave
    if constexpr (FDN) arrive_combine(g, blockIdx.x * SM_WAVES * 32, (blockIdx.x + 1) * SM_WAVES * 32, (int *)&xs, false);
    return;
  }
  const int e = tm.e;
  // the wave index, in a scalar register: offsets derived from it are wave-uniform
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const uint32_t l4 = (uint32_t)lane * 4;
  const int N = g.q.N, K = g.q.K, KB = K / 64;
  const int kb0 = blockIdx.z * kb_per_split, kb1 = min(KB, kb0 + kb_per_split);
  const int nchunks = max(0, (kb1 - kb0 + SM_CB - 1) / SM_CB);
  // gate_up launch of the two-launch forward: z1 = s1 A1[e] x accumulates beside the main
  // product from the staged activations.  Wave w takes the 32-wide k step w of every chunk
  // (block w / 2) with 16 x 16 x 32 MFMAs: tokens 16 hf + lane % 16, adapter rows 16 jt +
  // lane % 16, k = 8 (lane / 16) .. +7 of the step; its A1 fragments ride the register ring
  // with the weights.
  constexpr int ZT = FUSE == 2 ? 2 : 1;  // adapter tiles of 16
  const bool zon = FUP && g.r > 0;
  const __amdgpu_buffer_rsrc_t ra1 =
      make_rsrc(FUP ? g.fz.a1 + (int64_t)e * g.fz.a1_estride : nullptr, FUP ? (uint32_t)(g.r * K * 2) : 0u);
  uint32_t a1v[ZT];
#pragma unroll
  for (int jt = 0; jt < ZT; ++jt)
    a1v[jt] = (zon && 16 * jt + (lane & 15) < g.r) ? (uint32_t)((16 * jt + (lane & 15)) * K * 2 + 16 * (lane >> 4)) : OOB;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.q.codes, g.q.codes_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.q.scale, g.q.scale_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(g.q.scale2, g.q.scale2_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
  // last 4-byte aligned start of a 16-byte scale window inside the scale array
  const uint32_t slast = g.q.scale_bytes >= 16 ? (g.q.scale_bytes - 16) & ~3u : 0u;

  // this lane's weight row in each strip; code and scale offsets at block kb0
  int row[SPW];
  uint32_t sbase[SPW], ssh[SPW];
  int64_t blk0[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int st = (blockIdx.x * SM_WAVES + w) * SPW + s;
    bool ok;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int i = st * 16 + (n & 15);
      ok = i < g.I;
      row[s] = gate_up_row(i, n >= 16, g.act == 1, g.I);
    } else {
      row[s] = st * 32 + n;
      ok = row[s] < N;
    }
    const int64_t el = ((int64_t)e * N + row[s]) * K;
    blk0[s] = (el >> 6) + kb0;
    // scale windows: NF4 byte 4*blk; NF4_DQ byte blk; MXFP4 byte (el >> 5) + 2 kb + h,
    // each read from the 4-byte aligned address at or below it
    const uint32_t sb = FMT == FMT_NF4 ? (uint32_t)(blk0[s] * 4)
                        : FMT == FMT_NF4_DQ ? (uint32_t)blk0[s]
                                            : (uint32_t)(el >> 5) + 2u * kb0 + hh;
    ssh[s] = sb & 3u;
    sbase[s] = ok ? (sb & ~3u) : OOB;
    if (!ok) row[s] = -1;
  }
  // staged code loads (a chunk of 4 blocks): load i reads strip row 8 i + lane / 8, piece lane % 8
  uint32_t voffc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rho = 8 * i + lane / 8;
    const int st = blockIdx.x * SM_WAVES + w;
    int r;
    bool rok;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int ii = st * 16 + (rho & 15);
      rok = ii < g.I;
      r = gate_up_row(ii, rho >= 16, g.act == 1, g.I);
    } else {
      r = st * 32 + rho;
      rok = r < N;
    }
    voffc[i] = rok ? (uint32_t)((((int64_t)e * N + r) * K) / 2) + (uint32_t)kb0 * 32 + 16u * (lane % 8) : OOB;
  }
  char *stage = (char *)&sm.rest.stage[w][0];
  // activation staging: thread -> token row t / 16, 16 elements at 16 * (t % 16) of a chunk
  const int xrow = threadIdx.x >> 4, xpiece = threadIdx.x & 15;
  uint32_t xoff = OOB;
  if (xrow < tm.rows) {
    const int64_t p = tm.row0 + xrow;
    const int64_t src = gath ? (int64_t)(gath[p] / g.a_gdiv) : p;
    xoff = (uint32_t)((src * g.lda + (int64_t)kb0 * 64 + 16 * xpiece) * 2);
  }

  u32x4 cw[R][SPW][SM_CB];
  ChunkScale cs[R][SPW];
  u32x4 xr[R][2];  // activation pieces ride the same ring as the weights
  u32x4 a1r[FUP ? R : 1][ZT];
  f32x4 zacc[2][ZT];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int jt = 0; jt < ZT; ++jt) zacc[hf][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x16 acc[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[s][v] = 0.0f;

  auto load_x = [&](int slot, int c) {
    const uint32_t dead = c < nchunks ? 0u : OOB;
    xr[slot][0] = bload128(ra, xoff, ((uint32_t)c * SM_CB * 128) | dead);
    xr[slot][1] = bload128(ra, xoff, ((uint32_t)c * SM_CB * 128 + 16) | dead);
  };
  auto store_x = [&](int slot, int c) {
    uint16_t *row = &xs.v[c & 3][xrow][0];
    *(u32x4 *)(row + 8 * xpiece_swz(xrow, 2 * xpiece)) = xr[slot][0];
    *(u32x4 *)(row + 8 * xpiece_swz(xrow, 2 * xpiece + 1)) = xr[slot][1];
  };
  auto load_w = [&](int slot, int c) {
    if constexpr (FUP) {  // this wave's A1 fragments of chunk c (k step w: block w / 2)
      const int kb = kb0 + c * SM_CB + (w >> 1);
      const uint32_t zdead = (c < nchunks && kb < kb1) ? 0u : OOB;
#pragma unroll
      for (int jt = 0; jt < ZT; ++jt)
        a1r[slot][jt] = bload128(ra1, a1v[jt], ((uint32_t)(kb0 + c * SM_CB) * 128 + 64u * w) | zdead);
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      // the chunk's codes, 32 rows x 128 bytes (a chunk past the split reads zero; blocks of a
      // chunk past kb1 read bytes that their zero scale cancels)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cw[slot][s][i] = bload128_stream(rc, voffc[i], ((uint32_t)(c * SM_CB) * 32) | (c < nchunks ? 0u : OOB));
      const uint32_t dead = c < nchunks ? 0u : OOB;
      const uint32_t step = FMT == FMT_NF4 ? SM_CB * 4 : FMT == FMT_NF4_DQ ? SM_CB : SM_CB * 2;
      uint32_t win = OOB, sh = 0;
      if (sbase[s] != OOB) {
        const uint32_t at = sbase[s] + (uint32_t)c * step;
        win = min(at, slast);
        sh = ssh[s] + (at - win);
      }
      cs[slot][s].raw = bload128(rs, win, dead);
      cs[slot][s].sh = sh;
      if constexpr (FMT == FMT_NF4_DQ) {
        const uint32_t s2off = sbase[s] == OOB ? OOB : (uint32_t)((blk0[s] + c * SM_CB) >> 8) * 4;
        const uint32_t s2offb = sbase[s] == OOB ? OOB : (uint32_t)((blk0[s] + c * SM_CB + SM_CB - 1) >> 8) * 4;
        cs[slot][s].s2a = __uint_as_float(bload32(rs2, s2off, dead));
        cs[slot][s].s2b = __uint_as_float(bload32(rs2, s2offb, dead));
      }
    }
  };
  // scale of block b of the chunk in `slot` for strip s
  auto scale_of = [&](int slot, int s, int b, int c) -> float {
    if constexpr (FMT == FMT_NF4) {
      return __uint_as_float(dword_at(cs[slot][s].raw, cs[slot][s].sh + 4 * b));  // a multiple of 4
    } else if constexpr (FMT == FMT_NF4_DQ) {
      const uint32_t code = byte_at(cs[slot][s].raw, cs[slot][s].sh + b);
      const bool second = ((blk0[s] + c * SM_CB + b) >> 8) != ((blk0[s] + c * SM_CB) >> 8);
      return dq_value(g.q.dq_table, code) * (second ? cs[slot][s].s2b : cs[slot][s].s2a);
    } else {
      return e8m0_to_f32(byte_at(cs[slot][s].raw, cs[slot][s].sh + 2 * b));
    }
  };

  // prologue: the activations and weights of chunks 0 .. DC-1 in slot order (activations
  // first in each group: they are waited for one step before the weights)
#pragma unroll
  for (int d = 0; d < DC; ++d) {
    __builtin_amdgcn_sched_barrier(0);
    load_x(d, d);
    load_w(d, d);
  }
  __builtin_amdgcn_sched_barrier(0);
  // this lane's operand pieces of the LoRA K-extension in the two-launch forward (token n,
  // adapter columns 16 q + 8 h .. +7): z1 (gate_up) or z2 (down, first split)
  u32x4 zf[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
  if constexpr (FUP) lds_barrier();  // the routing in the activation ring's space has been read
  if constexpr (FDN) {
    if (g.r > 0 && blockIdx.z == 0) {
      uint16_t *zs = (uint16_t *)((char *)&xs + 8192);
      z2_reduce(g, tm.row0, tm.rows, (float *)&xs, zs);
#pragma unroll
      for (int q = 0; q < 2; ++q) zf[q] = *(const u32x4 *)(zs + n * 32 + 16 * q + 8 * hh);
      lds_barrier();
    }
  }
  store_x(0, 0);
  store_x(1, 1);
  lds_barrier();

  static_assert(R % 2 == 0, "a barrier after every odd chunk");
  for (int cb = 0; cb < nchunks; cb += R) {
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int c = cb + d;  // chunk c sits in slot d; its activations in xs.v[c & 3]
      // loads of chunk c+DC (activations, then weights) into the slot the previous step
      // freed; the activations of chunk c+2, loaded a step ago, are staged at the end
      __builtin_amdgcn_sched_barrier(0);
      load_x((d + DC) % R, c + DC);
      load_w((d + DC) % R, c + DC);
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t *xb = &xs.v[c & 3][n][0];
      // this chunk's codes to the wave's stage (the previous chunk's reads came first)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rho = 8 * i + lane / 8;
        *(u32x4 *)(stage + rho * 128 + stage_swz<4>(rho, lane % 8) * 16) = cw[d][0][i];
      }
#pragma unroll
      for (int b = 0; b < SM_CB; ++b) {
        const u32x4 cwb = *(const u32x4 *)(stage + n * 128 + stage_swz<4>(n, 2 * b + hh) * 16);
        bf16x8 af[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) af[s4] = *(const bf16x8 *)(xb + 8 * xpiece_swz(n, 8 * b + 4 * hh + s4));
        if constexpr (FUP) {
          if (zon && b == (w >> 1)) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int m = 16 * hf + (lane & 15);
              const bf16x8 xa = *(const bf16x8 *)(&xs.v[c & 3][m][0] + 8 * xpiece_swz(m, 4 * w + (lane >> 4)));
#pragma unroll
              for (int jt = 0; jt < ZT; ++jt)
                zacc[hf][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, a1r[d][jt]),
                                                                       zacc[hf][jt], 0, 0, 0);
            }
          }
        }
        // a block past kb1 reads zero codes, which are nf4 code 0 (-1), against staged
        // activations that are not zero: its scale is set to zero instead
        const bool live = kb0 + c * SM_CB + b < kb1;
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          const float sc = live ? scale_of(d, s, b, c) : 0.0f;
          if constexpr (NF4ISH) {
            f32x16 blk = {};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const uint32_t cw4 = cwb[s4];
              blk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s4], nf4_codes_bf16(cw4, l4, tb), blk, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[s][v] += sc * blk[v];
            // keeps the scaling of this block's partial sum here: sunk to the end of the
            // step, the partial sums of all its blocks stay live and spill, and the spill
            // reloads (vector-memory loads) then wait for every weight load in flight
            asm volatile("" : "+v"(acc[s]));
          } else {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const uint32_t cw4 = cwb[s4];
              acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  af[s4], __builtin_bit_cast(bf16x8, mxfp4_word_to_bf16(cw4, sc)), acc[s], 0, 0, 0);
            }
          }
        }
      }
      // The activations of chunk c+2 (loaded a step ago) go to buffer (c+2) & 3, last read
      // at chunk c-2; a barrier after every odd chunk separates each buffer's writes from
      // its earlier reads and from its later reads.
      store_x((d + 2) % R, c + 2);
      if (d & 1) lds_barrier();
    }
  }

  // z1 of the two-launch forward: the eight waves' partial products added in wave order
  if constexpr (FUP) {
    if (zon) {
      float *red = (float *)&xs;  // [8 waves][32 tokens][32]; the ring is no longer read
      uint16_t *zs = (uint16_t *)((char *)&xs + 32768);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int jt = 0; jt < ZT; ++jt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(w * 32 + 16 * hf + 4 * (lane >> 4) + v) * 32 + 16 * jt + (lane & 15)] = zacc[hf][jt][v];
      if (ZT == 1) {  // adapter rows 16 .. 31 are zero
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[(w * 32 + 16 * hf + 4 * (lane >> 4) + v) * 32 + 16 + (lane & 15)] = 0.0f;
      }
      lds_barrier();
      for (int o = threadIdx.x; o < 32 * 32; o += SM_THREADS) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < SM_WAVES; ++ww) v += red[(ww * 32 + (o >> 5)) * 32 + (o & 31)];
        zs[o] = f2bf((o & 31) < g.r ? g.fz.s1 * v : 0.0f);
      }
      lds_barrier();
#pragma unroll
      for (int q = 0; q < 2; ++q) zf[q] = *(const u32x4 *)(zs + n * 32 + 16 * q + 8 * hh);
    }
  }
  // the down LoRA-A fragment of this wave's h columns (z2 partial sums, two-launch forward)
  u32x4 a2f = {0, 0, 0, 0};
  if constexpr (FUP) {
    const int i0 = (blockIdx.x * SM_WAVES + w) * 16;
    if (n < g.fz.r2 && i0 < g.I) a2f = *(const u32x4 *)(g.fz.a2 + (int64_t)e * g.fz.a2_estride + (int64_t)n * g.I + i0 + 8 * hh);
  }

  // LoRA K-extension (first split only): acc += z . B[e]^T over the adapter rank
  const int tok = n;
  if (g.r > 0 && blockIdx.z == 0) {
    for (int kk = 0; kk < g.r; kk += 16) {
      const int kc = kk + 8 * hh;
      u32x4 za = {0, 0, 0, 0};
      if constexpr (FUSE) za = kk == 0 ? zf[0] : zf[1];
      else if (tok < tm.rows && kc < g.r) za = *(const u32x4 *)(g.xa + (tm.row0 + tok) * g.ldxa + kc);
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        u32x4 zb = {0, 0, 0, 0};
        if (row[s] >= 0 && kc < g.r) zb = *(const u32x4 *)(g.xb + e * g.xb_estride + (int64_t)row[s] * g.ldxb + kc);
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, za),
                                                         __builtin_bit_cast(bf16x8, zb), acc[s], 0, 0, 0);
      }
    }
  }

  // epilogue: acc[s][v] is C[token 8(v/4) + 4h + v%4][n]
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int i = ((blockIdx.x * SM_WAVES + w) * SPW + s) * 16 + (n & 15);
      float bg = 0.0f, bu = 0.0f;
      if (g.bias && n < 16 && i < g.I) {
        bg = bf2f(g.bias[e * g.bias_estride + gate_up_row(i, false, g.act == 1, g.I)]);
        bu = bf2f(g.bias[e * g.bias_estride + gate_up_row(i, true, g.act == 1, g.I)]);
      }
      uint16_t *hT = (uint16_t *)stage;  // two-launch forward: h of the tile, [32 tokens][16]
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float mine = acc[s][v];
        const float other = __shfl_xor(mine, 16);
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        uint16_t hb = 0;
        if (n < 16 && i < g.I && t < tm.rows) {
          const int64_t p = tm.row0 + t;
          const float gt = mine + bg, up = other + bu;
          const float h = g.act == 1 ? glu_clamped(gt, up, g.glu_alpha, g.glu_limit) : gt * sigmoid_fast(gt) * up;
          hb = f2bf(h);
          ((uint16_t *)g.C)[p * g.ldc + i] = hb;
          if (g.Gout) {
            g.Gout[p * g.ldg + gate_up_row(i, false, g.act == 1, g.I)] = f2bf(gt);
            g.Gout[p * g.ldg + gate_up_row(i, true, g.act == 1, g.I)] = f2bf(up);
          }
        }
        if constexpr (FUP) {
          if (n < 16) hT[t * 16 + n] = hb;
        }
      }
      if constexpr (FUP) {
        // z2 partial sums over this workgroup's h columns: the tile's h (tokens x 16) times
        // this wave's A2 fragment, then the eight waves added in wave order
        if (g.fz.r2 > 0) {
          asm volatile("" ::: "memory");
          const bf16x8 hf = *(const bf16x8 *)(hT + n * 16 + 8 * hh);
          const f32x16 zp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, __builtin_bit_cast(bf16x8, a2f), f32x16{}, 0, 0, 0);
          float *red = (float *)&xs;  // [8 waves][32 tokens][32]
#pragma unroll
          for (int v = 0; v < 16; ++v) red[(w * 32 + 8 * (v >> 2) + 4 * hh + (v & 3)) * 32 + n] = zp[v];
          lds_barrier();
          const int r2 = g.fz.r2;
          for (int o = threadIdx.x; o < 32 * 32; o += SM_THREADS) {
            const int t = o >> 5, j = o & 31;
            if (t < tm.rows && j < r2) {
              float v = 0.0f;
#pragma unroll
              for (int ww = 0; ww < SM_WAVES; ++ww) v += red[(ww * 32 + t) * 32 + j];
              g.fz.zp[((int64_t)blockIdx.x * g.M + tm.row0 + t) * r2 + j] = v;
            }
          }
        }
      }
    } else {
      if (row[s] < 0) continue;
      float *out = (float *)g.C + blockIdx.z * split_stride;
      // the first split also adds the per-expert bias (clamped GLU experts' down projection)
      const float bn = (g.bias && blockIdx.z == 0) ? bf2f(g.bias[e * g.bias_estride + row[s]]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (t < tm.rows) out[(tm.row0 + t) * g.ldc + row[s]] = acc[s][v] + bn;
      }
    }
  }
  if constexpr (FDN) arrive_combine(g, blockIdx.x * SM_WAVES * 32, (blockIdx.x + 1) * SM_WAVES * 32, (int *)&xs);
}

// Variant for few tokens per expert: workgroup slots of at most XMAX tokens, whose
// activation rows over the whole K range of the split are staged in LDS once; the lanes
// of the other token rows read a zero line (one address for all of them, a broadcast),
// so the loop streams only codes and scales: one 16-byte code load per block and one
// scale window per 4 blocks, in a ring of 8 block slots loaded 7 blocks ahead.  The
// operands of block j+1 (activation fragments, table reads, scale) are read while the
// MFMAs of block j run.  Eight waves per workgroup, one strip each.
constexpr int XMAX = 8;
// (the block scaling touches accumulator values v < 4 only: C rows 8(v/4) + 4h + v%4 < 8)
static_assert(XMAX == 8, "token rows of a direct slot");
constexpr int XPT = 8;  // staged 16-byte activation pieces per thread: rows x blocks <= 512

template <int FMT, int EPI, int CH, bool SEQ, int FUSE>
__global__ __launch_bounds__(SM_THREADS) void small_direct_kernel(GroupedArgs g, int kb_per_split,
                                                                   int64_t split_stride, int nseq) {
  constexpr bool NF4ISH = FMT != FMT_MXFP4;
  constexpr int D = 7, R = 8;
  static_assert(CH == 2 || CH == 4, "staged chunk");
  constexpr int LPR = 2 * CH, RPI = 64 / LPR, NI = 32 / RPI, CS = R / CH;  // lanes/row, rows/load, loads, slots
  // static LDS: only the code table (NF4 formats), at LDS address 0; dynamic LDS: the
  // staged activation rows [rows][blocks of the split][64], then the code stages.  With 8
  // staged rows of 4096 and four-block stages this is the whole 160 KB.
  __shared__ __attribute__((aligned(16))) SmallTables direct_tb;
  extern __shared__ __attribute__((aligned(16))) uint32_t small_lds[];
  SmallTables &tb = direct_tb;  // read by the NF4 formats only
  uint16_t *xs = (uint16_t *)small_lds;
  constexpr bool FUP = FUSE && EPI == EPI_SWIGLU_FWD, FDN = FUSE && EPI == EPI_F32;
  // two-launch forward: the gate_up launch routes in LDS (the staged activations' space)
  const int32_t *offp = g.off, *gath = g.a_gather;
  if constexpr (FUP) {
    const LdsRoute rt = route_in_lds(g.fz.ids, g.M, g.E, (int32_t *)small_lds);
    if (blockIdx.x == 0 && blockIdx.y == 0) route_export(rt, g);
    offp = rt.off;
    gath = rt.perm;
  }
  TileM tm;
  if (!find_tile_wave(offp, g.E, XMAX, blockIdx.y, tm)) {  // the same for every wave
    if constexpr (FDN) arrive_combine(g, blockIdx.x * nseq * SM_WAVES * 32, (blockIdx.x + 1) * nseq * SM_WAVES * 32, (int *)small_lds, false);
    return;
  }
  const int e = tm.e;
  // the wave index, in a scalar register: offsets derived from it are wave-uniform
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const uint32_t l4 = (uint32_t)lane * 4;
  const int N = g.q.N, K = g.q.K, KB = K / 64;
  const int kb0 = blockIdx.z * kb_per_split, kb1 = min(KB, kb0 + kb_per_split);
  const int nblk = max(0, kb1 - kb0);

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.q.codes, g.q.codes_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.q.scale, g.q.scale_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(g.q.scale2, g.q.scale2_bytes);
  const uint32_t slast = g.q.scale_bytes >= 16 ? (g.q.scale_bytes - 16) & ~3u : 0u;

  // Each wave computes a sequence of nseq strips of 32 weight rows, strip k being
  // (blockIdx.x nseq + k) SM_WAVES + w: the table, the staged activations and the start-up
  // latency are paid once per workgroup.  Strip state: the output row of this lane, the
  // scale windows and the staged code load offsets.
  int row = -1;
  int64_t blk0 = 0;
  uint32_t ssh = 0, sbase = OOB;
  uint32_t voffc[NI];
  auto strip_of = [&](int k) { return (blockIdx.x * nseq + k) * SM_WAVES + w; };
  auto strip_valid = [&](int st) { return EPI == EPI_SWIGLU_FWD ? st * 16 < g.I : st * 32 < N; };
  auto setup_strip = [&](int st) {
    bool ok;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int i = st * 16 + (n & 15);
      ok = i < g.I;
      row = gate_up_row(i, n >= 16, g.act == 1, g.I);
    } else {
      row = st * 32 + n;
      ok = row < N;
    }
    const int64_t el = ((int64_t)e * N + row) * K;
    blk0 = (el >> 6) + kb0;
    const uint32_t sb = FMT == FMT_NF4 ? (uint32_t)(blk0 * 4)
                        : FMT == FMT_NF4_DQ ? (uint32_t)blk0
                                            : (uint32_t)(el >> 5) + 2u * kb0 + hh;
    ssh = sb & 3u;
    sbase = ok ? (sb & ~3u) : OOB;
    if (!ok) row = -1;
    // staged code loads: load i of a chunk reads strip row RPI i + lane / LPR, piece lane % LPR
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rho = RPI * i + lane / LPR;
      int r;
      bool rok;
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        const int ii = st * 16 + (rho & 15);
        rok = ii < g.I;
        r = gate_up_row(ii, rho >= 16, g.act == 1, g.I);
      } else {
        r = st * 32 + rho;
        rok = r < N;
      }
      voffc[i] = rok ? (uint32_t)((((int64_t)e * N + r) * K) / 2) + (uint32_t)kb0 * 32 + 16u * (lane % LPR) : OOB;
    }
  };
  setup_strip(strip_of(0));

  {
    const int t0 = 0, xrows = tm.rows;
    const int xrow_len = nblk * 64;  // staged elements per token row
    // Start-up latency is overlapped: the activation pieces are loaded first, then the
    // first D blocks of codes, then the table is built, and only then do the pieces go
    // to LDS (waiting for them does not wait for the younger code loads).
    u32x4 xp[XPT];
    const int npieces = xrows * nblk * 8;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = threadIdx.x + u * SM_THREADS;
      xp[u] = u32x4{0, 0, 0, 0};
      if (i < npieces) {
        const int xr = i / (nblk * 8), piece = i - xr * (nblk * 8);
        const int64_t p = tm.row0 + xr;
        const int64_t src = gath ? (int64_t)(gath[p] / g.a_gdiv) : p;
        xp[u] = *(const u32x4 *)(g.A + src * g.lda + (int64_t)kb0 * 64 + piece * 8);
      }
    }
    const int tok = n;
    const bool xlane = tok >= t0 && tok < t0 + xrows;
    // fragment source of this lane: its token row; a lane without a token reads token 0's
    // row (its accumulator row is never stored, and rows do not mix in the product)
    // Staged rows are 128 n bytes apart, so all start in the same LDS bank: the 16-byte
    // piece c of a block of row t sits at piece c ^ (t & 7), and the fragment reads of up
    // to 8 token rows fall in different banks.
    const int xrow = xlane ? tok - t0 : 0;
    const uint16_t *xsrc = xs + xrow * xrow_len;
    int xpc[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) xpc[s4] = ((4 * hh + s4) ^ (xrow & 7)) * 8;
    // the LoRA operands of the first 16 adapter columns, loaded now so that their latency
    // is not paid after the loop
    const bool lora = g.r > 0 && blockIdx.z == 0;
    u32x4 za0 = {0, 0, 0, 0}, zb0 = {0, 0, 0, 0};
    auto load_zb0 = [&]() {
      zb0 = u32x4{0, 0, 0, 0};
      if (lora && row >= 0 && 8 * hh < g.r) zb0 = *(const u32x4 *)(g.xb + e * g.xb_estride + (int64_t)row * g.ldxb + 8 * hh);
    };
    if (!FUSE && lora && xlane && 8 * hh < g.r) za0 = *(const u32x4 *)(g.xa + (tm.row0 + tok) * g.ldxa + 8 * hh);
    load_zb0();
    // two-launch forward, gate_up: this wave's down LoRA-A fragment of its strip's h columns
    u32x4 a2f = {0, 0, 0, 0};
    float zsum[4] = {0.f, 0.f, 0.f, 0.f};  // z2 partial sums, tokens 4 h + v (v < 4)
    auto load_a2f = [&](int st) {
      if constexpr (FUP) {
        a2f = u32x4{0, 0, 0, 0};
        if (n < g.fz.r2 && st * 16 < g.I)
          a2f = *(const u32x4 *)(g.fz.a2 + (int64_t)e * g.fz.a2_estride + (int64_t)n * g.I + st * 16 + 8 * hh);
      }
    };
    load_a2f(strip_of(0));
    u32x4 zf1 = {0, 0, 0, 0};  // the second 16 adapter columns (two-launch forward)
    // z1 of the two-launch forward (gate_up): wave w takes the 32-wide k steps w, w + 8, ...
    // with 16 x 16 x 32 MFMAs (tokens lane % 16, adapter rows 16 jt + lane % 16, k = 8 (lane
    // / 16) .. +7 of the step), ZI = 16 (step, tile) items per round; the first round's A1
    // fragments are loaded before the codes, so that waiting for them does not wait for the codes
    constexpr int ZT = FUSE == 2 ? 2 : 1, ZI = 16;
    const int KS32 = K / 32, zitems = FUP && lora ? ZT * ((KS32 - w + SM_WAVES - 1) / SM_WAVES) : 0;
    const __amdgpu_buffer_rsrc_t ra1 =
        make_rsrc(FUP ? g.fz.a1 + (int64_t)e * g.fz.a1_estride : nullptr, FUP ? (uint32_t)(g.r * K * 2) : 0u);
    u32x4 a1f[FUP ? ZI : 1];
    auto load_a1_round = [&](int i0) {
#pragma unroll
      for (int i = 0; i < ZI; ++i) {
        const int it = i0 + i, jt = it % ZT, st = w + SM_WAVES * (it / ZT);
        const int j = 16 * jt + (lane & 15);
        const uint32_t voff = j < g.r ? (uint32_t)(j * K * 2 + 16 * (lane >> 4)) : OOB;
        a1f[i] = bload128(ra1, voff, it < zitems ? (uint32_t)st * 64 : OOB);
      }
    };
    if constexpr (FUP) {
      if (zitems > 0) load_a1_round(0);
    }
    // the code stages: [waves][32 strip rows][2 CH pieces of 16 bytes], pieces swizzled
    char *stage0 = (char *)small_lds + ((xrows * xrow_len * 2 + 15) & ~15);
    char *stage = stage0 + w * (32 * CH * 32);

    u32x4 craw[CS][NI];
    // scale windows, and the four block scales of the window in use, taken out of it as
    // it comes into use: the windows are then never copied (a copy of a window whose load
    // is in flight waits for every load issued before it)
    ChunkScale sq[R / 4];
    float scur[4];
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

    auto load_blk = [&](int slot, int j) {
      const uint32_t dead = j < nblk ? 0u : OOB;
      if (slot % CH == 0) {  // the codes of blocks j .. j+CH-1, 32 rows
#pragma unroll
        for (int i = 0; i < NI; ++i) craw[slot / CH][i] = bload128_stream(rc, voffc[i], ((uint32_t)j * 32) | dead);
      }
      if (slot % 4 == 0) {  // the scales of blocks j .. j+3
        const uint32_t step = FMT == FMT_NF4 ? 16u : FMT == FMT_NF4_DQ ? 4u : 8u;
        ChunkScale &q = sq[slot / 4];
        uint32_t win = OOB, sh = 0;
        if (sbase != OOB) {
          const uint32_t at = sbase + (uint32_t)(j / 4) * step;
          win = min(at, slast);
          sh = ssh + (at - win);
        }
        q.raw = bload128(rs, win, dead);
        q.sh = sh;
        if constexpr (FMT == FMT_NF4_DQ) {
          q.s2a = __uint_as_float(bload32(rs2, sbase == OOB ? OOB : (uint32_t)((blk0 + j) >> 8) * 4, dead));
          q.s2b = __uint_as_float(bload32(rs2, sbase == OOB ? OOB : (uint32_t)((blk0 + j + 3) >> 8) * 4, dead));
        }
      }
    };
    // scale of block j (slot d) from the quad window `q`, block b = j % 4 of it
    auto scale_in = [&](const ChunkScale &q, int b, int j) -> float {
      if constexpr (FMT == FMT_NF4) {
        return __uint_as_float(dword_at(q.raw, q.sh + 4 * b));
      } else if constexpr (FMT == FMT_NF4_DQ) {
        const uint32_t code = byte_at(q.raw, q.sh + b);
        const bool second = ((blk0 + j) >> 8) != ((blk0 + j - b) >> 8);
        return dq_value(g.q.dq_table, code) * (second ? q.s2b : q.s2a);
      } else {
        return e8m0_to_f32(byte_at(q.raw, q.sh + 2 * b));
      }
    };
    // chunk slot cs -> this wave's stage (after the previous chunk's reads, in LDS order)
    auto stage_write = [&](int cs) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rho = RPI * i + lane / LPR;
        *(u32x4 *)(stage + rho * (CH * 32) + stage_swz<CH>(rho, lane % LPR) * 16) = craw[cs][i];
      }
    };
    // the codes of block b of the staged chunk in the MFMA layout: row n, piece 2 b + h
    auto stage_read = [&](int b) -> u32x4 {
      return *(const u32x4 *)(stage + n * (CH * 32) + stage_swz<CH>(n, 2 * b + hh) * 16);
    };
    // operands of block j in slot d: activation fragments, B fragments, scale
    struct Ops {
      bf16x8 a[4], b[4];
      float sc;
    };
    // cwb: the block's codes, read from the stage a step earlier than the rest
    auto prepare = [&](int d, int j, Ops &o, const u32x4 &cwb) {
      // blocks past the range (the ring runs up to R - 1 blocks beyond it) read the last
      // staged block (LDS past the staged rows is not initialised and could hold NaN,
      // which their zero scale would not cancel)
      const uint16_t *xb = xsrc + 64 * max(0, min(j, nblk - 1));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) o.a[s4] = *(const bf16x8 *)(xb + xpc[s4]);
      if (d % 4 == 0) {  // block j starts a window: take out its four scales
#pragma unroll
        for (int b = 0; b < 4; ++b) scur[b] = scale_in(sq[d / 4], b, j + b);
      }
      const float sc = scur[d % 4];
      // a block past the range has zero codes (nf4 code 0 = -1): zero its scale
      o.sc = j < nblk ? sc : 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const uint32_t cw4 = cwb[s4];
        if constexpr (NF4ISH) o.b[s4] = nf4_codes_bf16(cw4, l4, tb);
        else o.b[s4] = __builtin_bit_cast(bf16x8, mxfp4_word_to_bf16(cw4, o.sc));
      }
    };
    auto compute = [&](const Ops &o) {
      if constexpr (NF4ISH) {
        f32x16 blk = {};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) blk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[s4], o.b[s4], blk, 0, 0, 0);
        // only C rows 8(v/4) + 4h + v%4 < XMAX hold tokens of the slot: v < 4
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += o.sc * blk[v];
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[s4], o.b[s4], acc, 0, 0, 0);
      }
    };

#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_barrier(0);
      load_blk(d, d);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NF4ISH) init_small_tables(tb, g.q.codebook);
    if constexpr (FUP) lds_barrier();  // the routing in the staged activations' space has been read
    if constexpr (FDN) {
      if (lora) {  // z2 of the slot's rows from the gate_up launch's partial sums
        uint16_t *zs = (uint16_t *)(stage0 + 8192);
        z2_reduce(g, tm.row0, xrows, (float *)stage0, zs);
        za0 = *(const u32x4 *)(zs + xrow * 32 + 8 * hh);
        zf1 = *(const u32x4 *)(zs + xrow * 32 + 16 + 8 * hh);
      }
    }
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = threadIdx.x + u * SM_THREADS;
      if (i < npieces) {  // piece i: row i / (8 nblk), block q / 8, piece q % 8 (swizzled)
        const int xr = i / (nblk * 8), q = i - xr * (nblk * 8);
        *(u32x4 *)(xs + xr * xrow_len + (q & ~7) * 8 + ((q & 7) ^ (xr & 7)) * 8) = xp[u];
      }
    }
    lds_barrier();
    if constexpr (FUP) {
      // z1 = s1 A1[e] x of the slot's rows from the staged activations: wave w takes the
      // 16-wide k steps w, w + 8, ... (32 tokens x 32 adapter rows per MFMA), 16 A1
      // fragments in flight per round; then the waves' products are added in wave order
      if (lora) {
        const int m = lane & 15, xr16 = m < xrows ? m : 0;  // token row of this lane's A fragment
        const uint16_t *xs16 = xs + xr16 * xrow_len;
        f32x4 zacc[ZT];
#pragma unroll
        for (int jt = 0; jt < ZT; ++jt) zacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i0 = 0; i0 < zitems; i0 += ZI) {
          if (i0 > 0) load_a1_round(i0);
#pragma unroll
          for (int i = 0; i < ZI; ++i) {
            const int it = i0 + i, jt = it % ZT, st = w + SM_WAVES * (it / ZT);
            if (it < zitems) {
              const int c = 4 * (st & 1) + (lane >> 4);  // 8-element piece of block st / 2
              const bf16x8 xa = *(const bf16x8 *)(xs16 + (st >> 1) * 64 + ((c ^ (xr16 & 7)) * 8));
              zacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, a1f[i]), zacc[jt], 0, 0, 0);
            }
          }
        }
        float *red = (float *)stage0;  // [8 waves][8 tokens][32]
        uint16_t *zs = (uint16_t *)(stage0 + SM_WAVES * XMAX * 32 * 4);
        if ((lane >> 4) < 2) {  // tokens 4 (lane / 16) + v < 8
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              red[(w * XMAX + 4 * (lane >> 4) + v) * 32 + 16 * jt + (lane & 15)] = jt < ZT ? zacc[jt % ZT][v] : 0.0f;
        }
        lds_barrier();
        if (threadIdx.x < XMAX * 32) {
          float v = 0.0f;
#pragma unroll
          for (int ww = 0; ww < SM_WAVES; ++ww) v += red[(ww * XMAX + (threadIdx.x >> 5)) * 32 + (threadIdx.x & 31)];
          zs[threadIdx.x] = f2bf((threadIdx.x & 31) < g.r ? g.fz.s1 * v : 0.0f);
        }
        lds_barrier();
        za0 = *(const u32x4 *)(zs + xrow * 32 + 8 * hh);
        zf1 = *(const u32x4 *)(zs + xrow * 32 + 16 + 8 * hh);
        lds_barrier();  // the main loop writes the code stages
      }
    }

    for (int k = 0;;) {
    Ops ops[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    stage_write(0);
    prepare(0, 0, ops[0], stage_read(0));
    u32x4 ccur = stage_read(1);  // block 1 (chunk 0 holds at least two blocks)
    for (int jb = 0; jb < nblk; jb += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int j = jb + d;  // block j sits in slot d; its operands are in ops[d & 1]
        __builtin_amdgcn_sched_barrier(0);
        load_blk((d + D) % R, j + D);
        __builtin_amdgcn_sched_barrier(0);
        // block j+2 starts a chunk: stage it (block j+1's codes were read a step ago), then
        // read block j+2's codes, a step before their table reads
        if ((d + 2) % CH == 0) stage_write(((d + 2) % R) / CH);
        const u32x4 cn = stage_read((d + 2) % CH);
        prepare((d + 1) % R, j + 1, ops[(d + 1) & 1], ccur);
        compute(ops[d & 1]);
        ccur = cn;
      }
    }

    const int row_done = row, st_done = strip_of(k);
    const u32x4 zb_done = zb0;

    if (lora) {
      for (int kk = 0; kk < g.r; kk += 16) {
        const int kc = kk + 8 * hh;
        u32x4 za = za0, zb = zb_done;
        if (kk > 0) {
          za = zb = u32x4{0, 0, 0, 0};
          if constexpr (FUSE) za = zf1;
          else if (xlane && kc < g.r) za = *(const u32x4 *)(g.xa + (tm.row0 + tok) * g.ldxa + kc);
          if (row_done >= 0 && kc < g.r) zb = *(const u32x4 *)(g.xb + e * g.xb_estride + (int64_t)row_done * g.ldxb + kc);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, za), __builtin_bit_cast(bf16x8, zb),
                                                      acc, 0, 0, 0);
      }
    }
    // accumulator rows are the slot's tokens: write those of this pass
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int i = st_done * 16 + (n & 15);
      float bg = 0.0f, bu = 0.0f;
      if (g.bias && n < 16 && i < g.I) {
        bg = bf2f(g.bias[e * g.bias_estride + gate_up_row(i, false, g.act == 1, g.I)]);
        bu = bf2f(g.bias[e * g.bias_estride + gate_up_row(i, true, g.act == 1, g.I)]);
      }
      uint16_t *hT = (uint16_t *)stage;  // two-launch forward: h of the strip, [32 tokens][16]
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float mine = acc[v];
        const float other = __shfl_xor(mine, 16);
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        uint16_t hb = 0;
        if (n < 16 && i < g.I && t >= t0 && t < t0 + xrows) {
          const int64_t p = tm.row0 + t;
          const float gt = mine + bg, up = other + bu;
          const float h = g.act == 1 ? glu_clamped(gt, up, g.glu_alpha, g.glu_limit) : gt * sigmoid_fast(gt) * up;
          hb = f2bf(h);
          ((uint16_t *)g.C)[p * g.ldc + i] = hb;
          if (g.Gout) {
            g.Gout[p * g.ldg + gate_up_row(i, false, g.act == 1, g.I)] = f2bf(gt);
            g.Gout[p * g.ldg + gate_up_row(i, true, g.act == 1, g.I)] = f2bf(up);
          }
        }
        if constexpr (FUP) {
          if (n < 16) hT[t * 16 + n] = hb;
        }
      }
      if constexpr (FUP) {
        // z2 partial sums over the strip's 16 h columns (tokens < XMAX: accumulator v < 4)
        if (g.fz.r2 > 0 && row_done >= 0) {
          asm volatile("" ::: "memory");
          const bf16x8 hf = *(const bf16x8 *)(hT + n * 16 + 8 * hh);
          const f32x16 zp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, __builtin_bit_cast(bf16x8, a2f), f32x16{}, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) zsum[v] += zp[v];
        }
      }
    } else if (row_done >= 0) {
      float *out = (float *)g.C + blockIdx.z * split_stride;
      // the first split also adds the per-expert bias (clamped GLU experts' down projection)
      const float bn = (g.bias && blockIdx.z == 0) ? bf2f(g.bias[e * g.bias_estride + row_done]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (t >= t0 && t < t0 + xrows) out[(tm.row0 + t) * g.ldc + row_done] = acc[v] + bn;
      }
    }
    // the next strip: its first loads
    ++k;
    if (!SEQ || k >= nseq || !strip_valid(strip_of(k))) break;
    setup_strip(strip_of(k));
    load_zb0();
    load_a2f(strip_of(k));
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_barrier(0);
      load_blk(d, d);
    }
    __builtin_amdgcn_sched_barrier(0);
    }  // strips
    if constexpr (FUP) {
      // the workgroup's z2 partial sums: the waves' sums added in wave order
      if (g.fz.r2 > 0) {
        float *red = (float *)stage0;  // [8 waves][8 tokens][32]
        lds_barrier();  // every wave is past its last strip's tile
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(w * XMAX + 4 * hh + v) * 32 + n] = zsum[v];
        lds_barrier();
        const int t = threadIdx.x >> 5, j = threadIdx.x & 31, r2 = g.fz.r2;
        if (t < xrows && j < r2) {
          float v = 0.0f;
#pragma unroll
          for (int ww = 0; ww < SM_WAVES; ++ww) v += red[(ww * XMAX + t) * 32 + j];
          g.fz.zp[((int64_t)blockIdx.x * g.M + tm.row0 + t) * r2 + j] = v;
        }
      }
    }
  }
  if constexpr (FDN) arrive_combine(g, blockIdx.x * nseq * SM_WAVES * 32, (blockIdx.x + 1) * nseq * SM_WAVES * 32, (int *)small_lds);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Strips (32 weight rows) per wave.  One: a second strip would double the register ring
// and spill.
static int pick_spw(int64_t) { return 1; }

// Upper bound on the workgroup slots of bmt tokens over the experts' row segments.
static int small_slots(int M, int E, int bmt) { return cdiv(M, bmt) + min(E, M); }

// Few tokens per touched expert (at most 2 on average) and staged activations that fit
// the per-thread pieces: the direct variant.
static int direct_rows(const GroupedArgs &a) { return min(XMAX, a.M); }
static bool use_direct(const GroupedArgs &a, int kbs) {
  return a.M <= 2 * min(a.E, a.M) && direct_rows(a) * kbs * 8 <= XPT * SM_THREADS;
}

// Launch shape of one decode-shaped GEMM: the direct variant (staged activation rows, nseq
// strips per wave) or the 32-token slots.
struct SmallPlan {
  bool direct, four;
  int nseq;
  dim3 grid;
  size_t lds;
};
template <int FMT>
static SmallPlan small_plan(const GroupedArgs &a, int strips_per_expert, int splits, int kbs) {
  SmallPlan p{};
  p.direct = use_direct(a, kbs);
  if (p.direct) {
    // strips per wave: the fewest with which the workgroups of the touched experts (at most
    // min(E, M)) fit on the compute units at once
    const int cus = device_cus();
    p.nseq = 1;
    while (p.nseq < 16 && (int64_t)cdiv(strips_per_expert, SM_WAVES * p.nseq) * min(a.E, a.M) * splits > cus) ++p.nseq;
    p.grid = dim3(cdiv(strips_per_expert, SM_WAVES * p.nseq), small_slots(a.M, a.E, XMAX), splits);
    const size_t xlds = ((size_t)direct_rows(a) * kbs * 64 * 2 + 15) & ~(size_t)15;
    // four-block stages when they fit beside the table and the staged activations
    constexpr size_t STATIC_LDS = FMT != FMT_MXFP4 ? sizeof(SmallTables) : 0;
    p.four = STATIC_LDS + xlds + stage_bytes(4) <= 160 * 1024;
    p.lds = xlds + stage_bytes(p.four ? 4 : 2);
  } else {
    p.nseq = 1;
    p.grid = dim3(cdiv(strips_per_expert, SM_WAVES), small_slots(a.M, a.E, SM_BMT), splits);
    p.lds = 0;
  }
  return p;
}

template <int FMT, int EPI, int FUSE>
static void launch_small_plan(const GroupedArgs &a, const SmallPlan &p, int kbs, int64_t split_stride, hipStream_t s) {
  if (p.direct) {
    if (p.nseq > 1) {
      if (p.four) small_direct_kernel<FMT, EPI, 4, true, FUSE><<<p.grid, SM_THREADS, p.lds, s>>>(a, kbs, split_stride, p.nseq);
      else small_direct_kernel<FMT, EPI, 2, true, FUSE><<<p.grid, SM_THREADS, p.lds, s>>>(a, kbs, split_stride, p.nseq);
    } else {
      if (p.four) small_direct_kernel<FMT, EPI, 4, false, FUSE><<<p.grid, SM_THREADS, p.lds, s>>>(a, kbs, split_stride, 1);
      else small_direct_kernel<FMT, EPI, 2, false, FUSE><<<p.grid, SM_THREADS, p.lds, s>>>(a, kbs, split_stride, 1);
    }
  } else {
    small_gemm_kernel<FMT, 1, EPI, 3, FUSE><<<p.grid, SM_THREADS, 0, s>>>(a, kbs, split_stride);
  }
}

template <int EPI>
static SmallPlan launch_small(const GroupedArgs &a, int strips_per_expert, int splits, int kbs, int64_t split_stride,
                              hipStream_t s, bool launch = true) {
  auto go = [&](auto fmt_tag) {
    constexpr int FMT = decltype(fmt_tag)::value;
    const SmallPlan p = small_plan<FMT>(a, strips_per_expert, splits, kbs);
    if (launch) {
      if (!a.fz.on) launch_small_plan<FMT, EPI, 0>(a, p, kbs, split_stride, s);
      else if (a.r <= 16) launch_small_plan<FMT, EPI, 1>(a, p, kbs, split_stride, s);
      else launch_small_plan<FMT, EPI, 2>(a, p, kbs, split_stride, s);
    }
    return p;
  };
  switch (a.q.fmt) {
    case FMT_NF4: return go(std::integral_constant<int, FMT_NF4>{});
    case FMT_NF4_DQ: return go(std::integral_constant<int, FMT_NF4_DQ>{});
    default: return go(std::integral_constant<int, FMT_MXFP4>{});
  }
}

bool launch_small_gate_up(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_GATE_UP, s);
  launch_small<EPI_SWIGLU_FWD>(a, cdiv(a.I, 16), 1, a.K / 64, 0, s);
  return last_launch_ok();
}

int small_gate_up_parts(const GroupedArgs &a) {
  return (int)launch_small<EPI_SWIGLU_FWD>(a, cdiv(a.I, 16), 1, a.K / 64, 0, nullptr, false).grid.x;
}

// K splits of down: enough waves for the device, each split a whole number of chunks.  With
// few tokens per expert, also enough splits for the staged activation rows of a split to
// fit the direct variant.
int small_down_splits(int M, int E, int N, int K) {
  const int64_t strips = (int64_t)cdiv(N, 32) * min(E, M);
  const int64_t waves = strips / pick_spw(strips);
  int splits = (int)((2048 + waves - 1) / waves);
  const int chunks = cdiv(K / 64, SM_CB);
  if (M <= 2 * min(E, M)) {
    const int max_kbs = (XPT * SM_THREADS) / (8 * min(XMAX, M));  // staged pieces per thread
    splits = max(splits, cdiv(K / 64, max_kbs / SM_CB * SM_CB));
  }
  splits = max(1, min(splits, min(SMALL_MAX_SPLITS, chunks / 4)));
  return splits;
}

static int small_down_kbs(const GroupedArgs &a, int splits) {
  return cdiv(cdiv(a.K / 64, splits), SM_CB) * SM_CB;
}

bool launch_small_down(const GroupedArgs &a, int splits, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_DOWN, s);
  launch_small<EPI_F32>(a, cdiv(a.N, 32), splits, small_down_kbs(a, splits), (int64_t)a.M * a.ldc, s);
  return last_launch_ok();
}

int small_down_ranges(const GroupedArgs &a, int splits) {
  return (int)launch_small<EPI_F32>(a, cdiv(a.N, 32), splits, small_down_kbs(a, splits), (int64_t)a.M * a.ldc,
                                    nullptr, false).grid.x;
}

// z[p][j] = alpha * <B[e_p][j], A[src(p)]> for the routed rows p of the valid experts: one
// workgroup of four waves per row and four adapter rows; each thread takes 8-element
// pieces of K, fp32 products, reduced across the wave and then the workgroup.
__global__ __launch_bounds__(256) void small_lora_a_kernel(GroupedArgs g) {
  const int p = blockIdx.x, j0 = blockIdx.y * 4, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float red[4][4];
  // the row's source index is loaded alongside the expert lookup (the two are independent),
  // so the operand loads wait for one round of memory latency, not two
  const int32_t gsrc = g.a_gather ? g.a_gather[p] : 0;
  int e = -1;
  for (int c = 0; c < g.E; c += 64) {
    const int ee = c + lane;
    const bool hit = ee < g.E && g.off[ee] <= p && p < g.off[ee + 1];
    const uint64_t m = __ballot(hit);
    if (m) {
      e = c + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  if (e < 0) return;  // past the valid rows (uniform over the workgroup)
  const int64_t src = g.a_gather ? (int64_t)(gsrc / g.a_gdiv) : p;
  const uint16_t *xr = g.A + src * g.lda;
  const uint16_t *br[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) br[jj] = g.Bd + e * g.b_estride + (int64_t)min(j0 + jj, g.N - 1) * g.ldb;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // one round of loads covers K up to 16384 (the same k order per thread for any K)
  for (int k0 = tid * 8; k0 < g.K; k0 += 8 * 2048) {
    u32x4 xv[8], bv[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u * 2048;
      const bool ok = k < g.K;
      xv[u] = ok ? *(const u32x4 *)(xr + k) : u32x4{0, 0, 0, 0};
      // the first workgroup of the row keeps the gathered row for the gate_up GEMM
      if (ok && g.xg_out && blockIdx.y == 0) *(u32x4 *)(g.xg_out + (int64_t)p * g.K + k) = xv[u];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bv[u][jj] = ok ? *(const u32x4 *)(br[jj] + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[jj] += __uint_as_float(xv[u][q] << 16) * __uint_as_float(bv[u][jj][q] << 16);
          acc[jj] += __uint_as_float(xv[u][q] & 0xffff0000u) * __uint_as_float(bv[u][jj][q] & 0xffff0000u);
        }
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc[jj] += __shfl_xor(acc[jj], d);
  if (lane == 0)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) red[w][jj] = acc[jj];
  __syncthreads();
  if (tid < 4 && j0 + tid < g.N) {
    const float v = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    ((uint16_t *)g.C)[(int64_t)p * g.ldc + j0 + tid] = f2bf(g.alpha * v);
  }
}

bool launch_small_lora_a(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_LORA_A, s);
  small_lora_a_kernel<<<dim3(a.M, cdiv(a.N, 4)), 256, 0, s>>>(a);
  return last_launch_ok();
}

}  // namespace e4b
