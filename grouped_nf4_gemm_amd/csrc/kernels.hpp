// Host-side launch interface of the gfx950 kernels (internal to libe4b).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace e4b {

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Kernel families for launch counting and event timing.
enum Family : int {
  FAM_ROUTE = 0,
  FAM_LORA_A,
  FAM_GATE_UP,
  FAM_DOWN,
  FAM_COMBINE,
  FAM_COMBINE_BWD,
  FAM_DOWN_DGRAD,
  FAM_GATE_UP_DGRAD,
  FAM_UNPERMUTE,
  FAM_WGRAD,
  FAM_QUANT,
  FAM_DEQUANT,
  FAM_TRANSPOSE,
  FAM_EXPAND,
  FAM_ROUTER,
  FAM_COUNT
};
const char *family_name(int f);

// Brackets one launch: counts it and, while timing is on, records events.
struct LaunchScope {
  int fam;
  hipStream_t s;
  int slot;
  LaunchScope(int fam, hipStream_t s);
  ~LaunchScope();
};
bool last_launch_ok();

// Two-launch decode forward (few routed rows, inference).  The gate_up launch also routes
// the raw ids inside every workgroup, forms z1 = s1 A1[e] x for the workgroup's own rows and
// writes the workgroup's partial sums of z2 = s2 A2[e] h over its h columns; the down launch
// adds those partial sums (split 0) and the last of its workgroups to finish a column range
// forms y over that range.  on = 0: every operand comes from the grouped-GEMM fields.
struct DecodeFuse {
  int on;
  const int32_t *ids;               // [M] expert of routed row f = t * topk + j
  int topk;
  int32_t *cnt, *off, *perm, *inv;  // routing, written by one gate_up workgroup
  int32_t *ctr;                     // down launch: one arrival counter per column range
  int nctr;                         // zeroed by the gate_up launch
  const uint16_t *a1;               // gate_up LoRA A [E][r1][H] (r1 = the launch's r)
  int64_t a1_estride;
  float s1;
  const uint16_t *a2;               // down LoRA A [E][r2][I]
  int64_t a2_estride;
  int r2;
  float s2;
  float *zp;                        // z2 partial sums [nparts][M][r2]
  int nparts;
  const float *topw;                // combine: [T][topk]
  int T;
  uint16_t *y;                      // [T][ldc of the down launch]
  int64_t split_stride;             // floats between the down launch's split partial sums
  int nsplit;
};
// Fused decode limits: workgroup routing scratch in LDS and one 32-wide MFMA tile of rank.
constexpr int FUSE_E_MAX = 256, FUSE_R_MAX = 32;

// Operands of one grouped GEMM over expert segments (see gemm.hpp).
struct GroupedArgs {
  const int32_t *off;
  int E;
  int M;   // total routed rows (grid sizing)
  int N;   // output columns (per expert); for SwiGLU: I (h columns)
  int K;   // main reduction length, multiple of 64
  // A operand: row-major bf16, sorted row p -> source row p (or gather[p] / gdiv)
  const uint16_t *A;
  int64_t lda;
  const int32_t *a_gather;
  int a_gdiv;
  uint32_t a_bytes;  // extent of A (large-tile buffer loads)
  // B operand
  QStack q;            // 4-bit stack (NK: [N, K] rows; KN: stored [K, N])
  // bf16 copy of q in its stored layout (nullable): the large tiles then load it directly
  // instead of decoding; bx_estride elements and bx_bytes bytes per expert
  const uint16_t *Bx;
  int64_t bx_estride;
  uint32_t bx_bytes;
  const uint16_t *Bd;  // dense bf16 [E][N][ldb]
  int64_t b_estride, ldb;
  // LoRA K-extension: xa [M][ldxa] sorted rows, xb [E][N][ldxb]; r = 0 disables
  const uint16_t *xa;
  int64_t ldxa;
  const uint16_t *xb;
  int64_t xb_estride, ldxb;
  int r;
  // epilogue
  void *C;
  int64_t ldc;
  float alpha;
  uint16_t *Gout;       // SwiGLU fwd: saved pre-activation [M][2I] (nullable); bwd: dG out
  const uint16_t *Gin;  // SwiGLU bwd: saved pre-activation
  int64_t ldg;
  int I;
  // small-N dense GEMM only: with nsplit > 1 the reduction is split nsplit ways and the
  // fp32 partial sums [nsplit][M][N] go to `part`, then are added in split order
  float *part;
  int nsplit;
  // few-row LoRA-A only (nullable): also write the gathered activation rows, [M][K] in
  // sorted-row order, for the GEMM that follows
  uint16_t *xg_out;
  // activation of the gate_up epilogues: 0 = act(gate) * up over rows [0, I) / [I, 2I);
  // 1 = clamped GLU over interleaved rows (2i, 2i+1), see glu_clamped
  int act;
  float glu_alpha, glu_limit;
  // per-expert bias added to the output columns (nullable): gate_up [E][2I] in stored row
  // order, down [E][H]
  const uint16_t *bias;
  int64_t bias_estride;
  DecodeFuse fz;
  // large fp32-epilogue tiles (down, gate_up dgrad): with `tail` set, the tiles of the last,
  // partial round of workgroups are split along K (tail_split); grid rows from tail_slot0 on
  // run the split parts past the first.  tail: fp32 partial tiles; tail_ctr: one arrival
  // counter per split tile and consumer wave, zero between launches.
  float *tail;
  int32_t *tail_ctr;
  int tail_slot0;
};

// K-split of the last round of large fp32-epilogue tiles: at most TAIL_UNITS workgroup units
// (the compute units of one round), at most TAIL_Q parts per tile and at least TAIL_MIN_SLABS
// 64-wide slabs per part (shorter parts do not repay their start-up, partial store and
// fences).  Workspace: TAIL_UNITS partial tiles (256 x 256 fp32) and TAIL_CTRS counters.
constexpr int TAIL_UNITS = 256, TAIL_Q = 8, TAIL_MIN_SLABS = 64, TAIL_CTRS = TAIL_UNITS * 8;
constexpr size_t TAIL_BYTES = (size_t)TAIL_UNITS * 256 * 256 * 4;

enum BKind : int { B_QNK = 0, B_QKN = 1, B_DENSE = 2 };
enum EpiKind : int { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU_FWD = 2, EPI_SWIGLU_BWD = 3 };

// Launchers (return false if the launch failed).
// zero (nullable): nzero ints set to 0 by the same launch (the tail-split arrival counters)
bool launch_route(const int32_t *ids, int M, int E, int32_t *cnt, int32_t *off, int32_t *perm,
                  int32_t *inv, hipStream_t s, int32_t *zero = nullptr, int nzero = 0);
// gate_up forward: h = swiglu(X W1^T + z1 B1^T) (+ G saved)
bool launch_gemm_gate_up(const GroupedArgs &a, hipStream_t s);
// down forward: O = h W2^T + z2 B2^T (fp32)
bool launch_gemm_down(const GroupedArgs &a, hipStream_t s);
// dgrad through down (stored [H, I] reduced over H) + SwiGLU backward -> dG
bool launch_gemm_down_dgrad(const GroupedArgs &a, hipStream_t s);
// dgrad through gate_up (stored [2I, H] reduced over 2I) -> dXp (fp32)
bool launch_gemm_gate_up_dgrad(const GroupedArgs &a, hipStream_t s);
// small-N dense GEMM: C = alpha * A B^T (bf16 out), B per expert [N][K]
bool launch_lora_a(const GroupedArgs &a, hipStream_t s);

struct WgradArgs {
  const int32_t *off;
  int E;
  const uint16_t *P;  // rows a: P[row][a]
  int64_t ldp;
  int Na;
  const int32_t *p_gather;
  int p_gdiv;
  const uint16_t *Q;  // cols b: Q[row][b]
  int64_t ldq;
  int Nb;
  const int32_t *q_gather;
  int q_gdiv;
  float *C;  // [E][Na][Nb]
  // with nsplit > 1 each expert's rows are split nsplit ways; the fp32 partial sums
  // [nsplit][E][Na][Nb] go to `part` and are added in split order
  float *part;
  int nsplit;
};
bool launch_wgrad(const WgradArgs &a, hipStream_t s);
// Reduction splits that give the skinny GEMMs enough workgroups to fill the device.
int lora_a_splits(int M, int E, int N, int K);
int wgrad_splits(int M, int E, int Na, int Nb);

// y[t] = bf16(sum_j w[t,j] * O[inv[t,j]]); O holds `nsplit` (at most COMBINE_MAX_SPLITS)
// partial sums, split_stride floats apart, that are added in split order first.
bool launch_combine(const float *O, int nsplit, int64_t split_stride, const int32_t *inv, const float *topw,
                    int T, int k, int H, uint16_t *y, hipStream_t s);

// Decode-shaped forward (few routed rows per expert), see small.hip.  Used when the routed
// rows of a call are at most SMALL_M_MAX.
constexpr int SMALL_M_MAX = 256;
constexpr int SMALL_MAX_SPLITS = 8;
constexpr int COMBINE_MAX_SPLITS = SMALL_MAX_SPLITS;
bool launch_small_lora_a(const GroupedArgs &a, hipStream_t s);
bool launch_small_gate_up(const GroupedArgs &a, hipStream_t s);
int small_down_splits(int M, int E, int N, int K);
bool launch_small_down(const GroupedArgs &a, int splits, hipStream_t s);
// Workgroups along the strip dimension of the decode-shaped gate_up and down launches (the
// z2 partial-sum count and the arrival-counter count of the two-launch forward).
int small_gate_up_parts(const GroupedArgs &a);
int small_down_ranges(const GroupedArgs &a, int splits);
// Router: top-k ids (larger logit first, ties to the lower id) and the fp32 softmax over
// them, E <= 1024, k <= 64; its gradient to the logits with the ids held fixed.
bool launch_router_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t s);
bool launch_router_bwd(const float *w, const float *dw, const int32_t *ids, int T, int E, int k, float *dl,
                       hipStream_t s);
bool launch_combine_bwd(const uint16_t *dy, const float *O, const int32_t *inv, const float *topw,
                        int T, int k, int H, uint16_t *dO, float *d_topw, hipStream_t s);
bool launch_unpermute(const float *dXp, const int32_t *inv, int T, int k, int H, uint16_t *dx,
                      hipStream_t s);
bool launch_transpose(const uint16_t *in, int E, int R, int C, uint16_t *out, hipStream_t s);
bool launch_quantize(int fmt, int64_t n, const float *w, uint8_t *codes, void *scale, float *scale2,
                     hipStream_t s);
bool launch_dequant(const QStack &q, int64_t elem0, int64_t n, float *out_f32, uint16_t *out_bf16,
                    hipStream_t s);
// bf16 copy of a whole stack [E][N][K] in its stored layout, decoded exactly as the GEMM
// tiles decode it.
bool launch_expand(const QStack &q, int E, uint16_t *out, hipStream_t s);

}  // namespace e4b
