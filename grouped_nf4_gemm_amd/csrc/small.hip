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
#include "gemm.hpp"
#include "kernels.hpp"

namespace e4b {

// 64 copies of the bf16 code-pair table, copy c for lane c: entry b of copy c at byte
// offset b * 256 + c * 4, so one byte permute forms the address and no two lanes of a
// wave share a bank.  Entry b holds bf16(nf4[b >> 4]) in its low half (element 2j, the
// high nibble) and bf16(nf4[b & 15]) in its high half.
struct SmallTables {
  uint32_t cp[256][64];
};

// thread t builds entry t % 256 and writes its 64 copies (16 bytes at a time)
__device__ __forceinline__ void init_small_tables(SmallTables &t) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    const uint32_t v = pack_bf16x2(nf4_value(b >> 4), nf4_value(b & 15));
#pragma unroll
    for (int c = 0; c < 64; c += 4) *(u32x4 *)&t.cp[b][c] = u32x4{v, v, v, v};
  }
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

constexpr int SM_THREADS = 256;  // four waves
constexpr int SM_BMT = 32;       // tokens per workgroup slot

template <int FMT>
struct SmallScale {
  uint32_t raw;
  float s2;
};

template <int FMT, int SPW, int EPI, int D>
__global__ __launch_bounds__(SM_THREADS) void small_gemm_kernel(GroupedArgs g, int kb_per_split,
                                                                 int64_t split_stride) {
  constexpr bool NF4ISH = FMT != FMT_MXFP4;
  // the table lives in dynamic LDS, sized at launch: NF4 formats only
  extern __shared__ __attribute__((aligned(16))) uint32_t small_lds[];
  SmallTables &tb = *reinterpret_cast<SmallTables *>(small_lds);
  __shared__ int tile_sh[4];
  if constexpr (NF4ISH) init_small_tables(tb);
  TileM tm;
  if (!find_tile(g.off, g.E, SM_BMT, blockIdx.y, tm, tile_sh)) return;  // (synchronises)
  const int e = tm.e;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const uint32_t l4 = (uint32_t)lane * 4;
  const int N = g.q.N, K = g.q.K, KB = K / 64;
  const int kb0 = blockIdx.z * kb_per_split, kb1 = min(KB, kb0 + kb_per_split);

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.q.codes, g.q.codes_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.q.scale, g.q.scale_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(g.q.scale2, g.q.scale2_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);

  // this lane's weight row in each strip, its code and scale offsets at block 0
  int row[SPW];
  uint32_t cbase[SPW], sbase[SPW];
  int64_t blk0[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int st = (blockIdx.x * 4 + w) * SPW + s;
    bool ok;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int i = st * 16 + (n & 15);
      ok = i < g.I;
      row[s] = n < 16 ? i : g.I + i;
    } else {
      row[s] = st * 32 + n;
      ok = row[s] < N;
    }
    const int64_t el = ((int64_t)e * N + row[s]) * K;
    blk0[s] = el >> 6;
    cbase[s] = ok ? (uint32_t)(el / 2) + 16 * hh : OOB;
    sbase[s] = !ok ? OOB
               : FMT == FMT_NF4 ? (uint32_t)(blk0[s] * 4)
               : FMT == FMT_NF4_DQ ? (uint32_t)blk0[s]
                                   : (uint32_t)(el >> 5) + hh;
    if (!ok) row[s] = -1;
  }
  // activation row of this lane (token n of the slot)
  const int tok = n;
  uint32_t avoff = OOB;
  if (tok < tm.rows) {
    const int64_t p = tm.row0 + tok;
    const int64_t src = g.a_gather ? (int64_t)(g.a_gather[p] / g.a_gdiv) : p;
    avoff = (uint32_t)((src * g.lda + 32 * hh) * 2);
  }

  constexpr int R = D + 1;  // ring slots
  u32x4 cw[R][SPW];
  SmallScale<FMT> sr[R][SPW];
  bf16x8 av[R][4];
  f32x16 acc[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[s][v] = 0.0f;

  auto load_b = [&](int slot, int kb) {
    const uint32_t dead = kb < kb1 ? 0u : OOB;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      cw[slot][s] = bload128(rc, cbase[s], ((uint32_t)kb * 32) | dead);
      if constexpr (FMT == FMT_NF4) {
        sr[slot][s].raw = bload32(rs, sbase[s], ((uint32_t)kb * 4) | dead);
      } else if constexpr (FMT == FMT_NF4_DQ) {
        sr[slot][s].raw = bload8(rs, sbase[s], (uint32_t)kb | dead);
        const uint32_t s2off = sbase[s] == OOB ? OOB : (uint32_t)((blk0[s] + kb) >> 8) * 4;
        sr[slot][s].s2 = __uint_as_float(bload32(rs2, s2off, dead));
      } else {
        sr[slot][s].raw = bload8(rs, sbase[s], ((uint32_t)kb * 2) | dead);
      }
    }
  };
  auto load_a = [&](int slot, int kb) {
    const uint32_t dead = kb < kb1 ? 0u : OOB;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      av[slot][s4] = __builtin_bit_cast(bf16x8, bload128(ra, avoff, ((uint32_t)kb * 128 + s4 * 16) | dead));
  };

  // prologue: the first D blocks
#pragma unroll
  for (int d = 0; d < D; ++d) {
    __builtin_amdgcn_sched_barrier(0);  // in slot order, as in the loop
    load_a(d, kb0 + d);
    load_b(d, kb0 + d);
  }
  __builtin_amdgcn_sched_barrier(0);

  // The body is straight-line: a block past kb1 has zero codes, scales and activations
  // (out-of-range loads) and adds nothing, and the exact wait counts survive.
  for (int kb = kb0; kb < kb1; kb += R) {
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int k = kb + d;  // block k sits in slot d
      {
        __builtin_amdgcn_sched_barrier(0);
        load_a((d + D) % R, k + D);
        load_b((d + D) % R, k + D);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          if constexpr (NF4ISH) {
            float sc;
            if constexpr (FMT == FMT_NF4) sc = __uint_as_float(sr[d][s].raw);
            else sc = ((float)sr[d][s].raw / 255.0f) * sr[d][s].s2;
            f32x16 blk = {};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
              blk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[d][s4], nf4_codes_bf16(cw[d][s][s4], l4, tb),
                                                            blk, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[s][v] += sc * blk[v];
          } else {
            const float sc = e8m0_to_f32(sr[d][s].raw);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
              acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[d][s4], __builtin_bit_cast(bf16x8,
                           mxfp4_word_to_bf16(cw[d][s][s4], sc)), acc[s], 0, 0, 0);
          }
        }
      }
    }
  }

  // LoRA K-extension (first split only): acc += z . B[e]^T over the adapter rank
  if (g.r > 0 && blockIdx.z == 0) {
    for (int kk = 0; kk < g.r; kk += 16) {
      const int kc = kk + 8 * hh;
      u32x4 za = {0, 0, 0, 0};
      if (tok < tm.rows && kc < g.r) za = *(const u32x4 *)(g.xa + (tm.row0 + tok) * g.ldxa + kc);
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
      const int i = ((blockIdx.x * 4 + w) * SPW + s) * 16 + (n & 15);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float mine = acc[s][v];
        const float other = __shfl_xor(mine, 16);
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (n < 16 && i < g.I && t < tm.rows) {
          const int64_t p = tm.row0 + t;
          const float gt = mine, up = other;
          const float act = gt / (1.0f + expf(-gt));
          ((uint16_t *)g.C)[p * g.ldc + i] = f2bf(act * up);
          if (g.Gout) {
            g.Gout[p * g.ldg + i] = f2bf(gt);
            g.Gout[p * g.ldg + g.I + i] = f2bf(up);
          }
        }
      }
    } else {
      if (row[s] < 0) continue;
      float *out = (float *)g.C + blockIdx.z * split_stride;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (t < tm.rows) out[(tm.row0 + t) * g.ldc + row[s]] = acc[s][v];
      }
    }
  }
}

// Strips per wave: the largest of 4, 2, 1 that still gives about two waves per SIMD.
static int pick_spw(int64_t strips) {
  if (strips / 4 >= 2048) return 4;
  if (strips / 2 >= 2048) return 2;
  return 1;
}

template <int FMT, int EPI>
static void launch_small_fmt(const GroupedArgs &a, int spw, int strips_per_expert, int slots, int splits,
                             int kbs, int64_t split_stride, hipStream_t s) {
  // codes in flight per wave: D blocks of SPW strips
  const int per_wg = 4 * spw;
  const dim3 grid(cdiv(strips_per_expert, per_wg), slots, splits);
  const size_t lds = FMT == FMT_MXFP4 ? 0 : sizeof(SmallTables);
  switch (spw) {
    case 4: small_gemm_kernel<FMT, 4, EPI, 2><<<grid, SM_THREADS, lds, s>>>(a, kbs, split_stride); break;
    case 2: small_gemm_kernel<FMT, 2, EPI, 4><<<grid, SM_THREADS, lds, s>>>(a, kbs, split_stride); break;
    default: small_gemm_kernel<FMT, 1, EPI, 6><<<grid, SM_THREADS, lds, s>>>(a, kbs, split_stride); break;
  }
}

template <int EPI>
static void launch_small(const GroupedArgs &a, int spw, int strips_per_expert, int slots, int splits, int kbs,
                         int64_t split_stride, hipStream_t s) {
  switch (a.q.fmt) {
    case FMT_NF4: launch_small_fmt<FMT_NF4, EPI>(a, spw, strips_per_expert, slots, splits, kbs, split_stride, s); break;
    case FMT_NF4_DQ: launch_small_fmt<FMT_NF4_DQ, EPI>(a, spw, strips_per_expert, slots, splits, kbs, split_stride, s); break;
    default: launch_small_fmt<FMT_MXFP4, EPI>(a, spw, strips_per_expert, slots, splits, kbs, split_stride, s); break;
  }
}

static int small_slots(int M, int E) { return cdiv(M, SM_BMT) + min(E, M); }

bool launch_small_gate_up(const GroupedArgs &a, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_GATE_UP, s);
  const int strips_per_expert = cdiv(a.I, 16);
  const int64_t strips = (int64_t)strips_per_expert * min(a.E, a.M);
  const int KB = a.K / 64;
  launch_small<EPI_SWIGLU_FWD>(a, pick_spw(strips), strips_per_expert, small_slots(a.M, a.E), 1, KB, 0, s);
  return last_launch_ok();
}

int small_down_splits(int M, int E, int N, int K) {
  const int64_t strips = (int64_t)cdiv(N, 32) * min(E, M);
  const int spw = pick_spw(strips);
  const int64_t waves = strips / spw;
  int splits = (int)((2048 + waves - 1) / waves);
  splits = max(1, min(splits, min(SMALL_MAX_SPLITS, K / 64 / 8)));
  return splits;
}

bool launch_small_down(const GroupedArgs &a, int splits, hipStream_t s) {
  if (a.M == 0) return true;
  LaunchScope ls(FAM_DOWN, s);
  const int strips_per_expert = cdiv(a.N, 32);
  const int64_t strips = (int64_t)strips_per_expert * min(a.E, a.M);
  const int KB = a.K / 64;
  const int kbs = cdiv(KB, splits);
  launch_small<EPI_F32>(a, pick_spw(strips), strips_per_expert, small_slots(a.M, a.E), splits, kbs,
                        (int64_t)a.M * a.ldc, s);
  return last_launch_ok();
}

// z[p][j] = alpha * <B[e_p][j], A[src(p)]> for the routed rows p of the valid experts: one
// workgroup of four waves per row and four adapter rows; each thread takes 8-element
// pieces of K, fp32 products, reduced across the wave and then the workgroup.
__global__ __launch_bounds__(256) void small_lora_a_kernel(GroupedArgs g) {
  const int p = blockIdx.x, j0 = blockIdx.y * 4, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float red[4][4];
  if (p >= g.off[g.E]) return;  // past the valid rows (uniform over the workgroup)
  int e = 0;
  for (int c = 0; c < g.E; c += 64) {
    const int ee = c + lane;
    const bool hit = ee < g.E && g.off[ee] <= p && p < g.off[ee + 1];
    const uint64_t m = __ballot(hit);
    if (m) {
      e = c + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  const int64_t src = g.a_gather ? (int64_t)(g.a_gather[p] / g.a_gdiv) : p;
  const uint16_t *xr = g.A + src * g.lda;
  const uint16_t *br[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) br[jj] = g.Bd + e * g.b_estride + (int64_t)min(j0 + jj, g.N - 1) * g.ldb;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = tid * 8; k0 < g.K; k0 += 4 * 2048) {
    u32x4 xv[4], bv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 2048;
      const bool ok = k < g.K;
      xv[u] = ok ? *(const u32x4 *)(xr + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bv[u][jj] = ok ? *(const u32x4 *)(br[jj] + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
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
