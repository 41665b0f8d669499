// C ABI of libe4b: argument validation, workspace layout, the three layer calls
// (forward, input gradient, LoRA weight gradients) as stream-ordered kernel
// sequences, and the verification / observability exports.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "e4b.h"
#include "kernels.hpp"

namespace e4b {

// ------------------------------------------------------------------ launch bookkeeping
static std::atomic<int64_t> g_count[FAM_COUNT];
static std::atomic<int64_t> g_total{0};
static std::mutex g_tmu;
static bool g_timing = false;
struct TimedLaunch {
  hipEvent_t a, b;
  int fam;
};
static std::vector<TimedLaunch> g_pending;
// Set on the calling thread for the duration of an allocation-free call: its launches are
// counted but not bracketed by events (creating events is left to calls that may allocate).
static thread_local bool t_noalloc = false;
static int64_t g_tl[FAM_COUNT];
static double g_tms[FAM_COUNT];

const char *family_name(int f) {
  static const char *names[FAM_COUNT] = {"route",          "lora_a",       "gemm_gate_up",
                                         "gemm_down",      "combine",      "combine_bwd",
                                         "gemm_down_dgrad", "gemm_gate_up_dgrad", "unpermute",
                                         "wgrad",          "quant",        "dequant",
                                         "transpose",      "expand",       "router"};
  return (f >= 0 && f < FAM_COUNT) ? names[f] : "?";
}

LaunchScope::LaunchScope(int f, hipStream_t st) : fam(f), s(st), slot(-1) {
  g_count[f]++;
  g_total++;
  if (g_timing && !t_noalloc) {
    TimedLaunch t{};
    t.fam = f;
    if (hipEventCreate(&t.a) == hipSuccess && hipEventCreate(&t.b) == hipSuccess &&
        hipEventRecord(t.a, s) == hipSuccess) {
      std::lock_guard<std::mutex> lk(g_tmu);
      slot = (int)g_pending.size();
      g_pending.push_back(t);
    }
  }
}

LaunchScope::~LaunchScope() {
  if (slot >= 0) {
    std::lock_guard<std::mutex> lk(g_tmu);
    (void)hipEventRecord(g_pending[slot].b, s);
  }
}

bool last_launch_ok() { return hipGetLastError() == hipSuccess; }

// ------------------------------------------------------------------ workspace layout
struct Layout {
  size_t cnt, off, perm, inv, z1, z2, G, h, O, dO, u2, dG, u1, dXp, A1T, B1T, A2T, B2T, part, W1x, W2x,
      zp, ctr, tail, tail_ctr, total;
};
static constexpr size_t NONE = ~(size_t)0;
// Activations and stacks that the 4-bit GEMMs stream with buffer loads must each stay
// below 2 GiB (32-bit per-lane byte offsets).
static constexpr int64_t BUF_LIMIT = ((int64_t)1 << 31) - 1;

// The large-tile GEMMs decode the packed stacks inside the tile, once per 256-row tile, in the
// forward and again in the dgrad (nothing dequantised is held between the calls).  A caller
// can ask the forward to write bf16 copies of both stacks into the workspace first and stream
// those (E4B_EXPAND: 2 bytes per weight of workspace); the results are bit-identical.  The
// decode-shaped path (few rows) never expands.
static bool use_expand(const e4b_moe_desc &d) {
  const int64_t M = (int64_t)d.T * d.topk;
  if (M <= SMALL_M_MAX || !(d.flags & E4B_EXPAND)) return false;
  return (int64_t)2 * d.I * d.H * 2 <= BUF_LIMIT;  // one expert's copy: 32-bit offsets
}

static Layout layout(const e4b_moe_desc &d, int r1, int r2) {
  Layout L;
  const size_t M = (size_t)d.T * d.topk, E = d.E, H = d.H, I = d.I;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = (o + bytes + 255) & ~(size_t)255;
    return at;
  };
  const bool train = d.flags & E4B_TRAIN;
  L.cnt = take((E + 1) * 4);
  L.off = take((E + 1) * 4);
  L.perm = take(M * 4);
  L.inv = take(M * 4);
  L.z1 = take(M * r1 * 2);
  L.z2 = take(M * r2 * 2);
  L.G = train ? take(M * 2 * I * 2) : NONE;
  L.h = take(M * I * 2);
  // the decode-shaped forward keeps up to SMALL_MAX_SPLITS partial sums of O (inference only)
  const bool decode = M <= (size_t)SMALL_M_MAX && !train;
  L.O = take((decode ? SMALL_MAX_SPLITS : 1) * M * H * 4);
  // two-launch decode forward: z2 partial sums of the gate_up workgroups (at most one per 8
  // strips of 16 h columns) and one arrival counter per 256 output columns of down
  L.zp = decode ? take((size_t)cdiv(cdiv(I, 16), 8) * M * r2 * 4) : NONE;
  L.ctr = decode ? take((size_t)cdiv(H, 256) * 4) : NONE;
  if (train) {
    L.dO = take(M * H * 2);
    L.u2 = take(M * r2 * 2);
    L.dG = take(M * 2 * I * 2);
    L.u1 = take(M * r1 * 2);
    L.dXp = take(M * H * 4);
    L.A1T = take(E * H * r1 * 2);
    L.B1T = take(E * r1 * 2 * I * 2);
    L.A2T = take(E * I * r2 * 2);
    L.B2T = take(E * r2 * H * 2);
  } else {
    L.dO = L.u2 = L.dG = L.u1 = L.dXp = L.A1T = L.B1T = L.A2T = L.B2T = NONE;
  }
  // fp32 partial sums of the split skinny GEMMs (LoRA-A projections, LoRA weight gradients),
  // sized for the largest of them
  size_t part = 0;
  auto lora = [&](int r, int K) {
    const int sp = r ? lora_a_splits((int)M, (int)E, r, K) : 1;
    if (sp > 1) part = std::max(part, (size_t)sp * M * r * 4);
  };
  auto wgrad = [&](int Na, int Nb) {
    const int sp = Na && Nb ? wgrad_splits((int)M, (int)E, Na, Nb) : 1;
    if (sp > 1) part = std::max(part, (size_t)sp * E * Na * Nb * 4);
  };
  lora(r1, (int)H);
  lora(r2, (int)I);
  if (train) {
    lora(r2, (int)H);
    lora(r1, (int)(2 * I));
    if (r1) { wgrad((int)(2 * I), r1); wgrad(r1, (int)H); }
    if (r2) { wgrad((int)H, r2); wgrad(r2, (int)I); }
  }
  L.part = part ? take(part) : NONE;
  // training: the K-split of the last round of the large fp32-epilogue GEMMs (down, gate_up
  // dgrad): partial tiles and arrival counters (zeroed by the forward's routing launch)
  L.tail = train ? take(TAIL_BYTES) : NONE;
  L.tail_ctr = train ? take((size_t)TAIL_CTRS * 4) : NONE;
  if (use_expand(d)) {
    L.W1x = take(E * 2 * I * H * 2);
    L.W2x = take(E * H * I * 2);
  } else {
    L.W1x = L.W2x = NONE;
  }
  L.total = o;
  return L;
}

template <class T>
static T *at(void *ws, size_t off) {
  return (T *)((char *)ws + off);
}

// ------------------------------------------------------------------ validation

static e4b_status check_desc(const e4b_moe_desc *d) {
  if (!d) return E4B_ERR_INVALID_ARG;
  if (d->E < 1 || d->E > 1024 || d->topk < 1 || d->topk > d->E || d->T < 0) return E4B_ERR_INVALID_ARG;
  if (d->H <= 0 || d->I <= 0 || d->H % 64 || d->I % 64) return E4B_ERR_INVALID_ARG;
  if ((int64_t)d->T * d->topk > (int64_t)1 << 30) return E4B_ERR_INVALID_ARG;
  const int64_t M = (int64_t)d->T * d->topk;
  if ((int64_t)d->T * d->H * 2 > BUF_LIMIT || M * d->H * 4 > BUF_LIMIT || M * 2 * d->I * 2 > BUF_LIMIT)
    return E4B_ERR_INVALID_ARG;
  if (d->flags & ~(E4B_TRAIN | E4B_EXPAND | E4B_SEPARATE)) return E4B_ERR_INVALID_ARG;
  if (const e4b_act *a = d->act) {
    if (a->kind == E4B_ACT_SWIGLU) {
      if (a->b_gu || a->b_dn) return E4B_ERR_INVALID_ARG;  // the stock epilogue has no biases
    } else if (a->kind == E4B_ACT_CLAMPED_GLU) {
      if (!std::isfinite(a->alpha) || !std::isfinite(a->limit) || !(a->limit > 0.0f)) return E4B_ERR_INVALID_ARG;
    } else {
      return E4B_ERR_UNSUPPORTED;
    }
  }
  return E4B_OK;
}

// Activation of the gate_up epilogues, and the biases, into the GEMM arguments.
static void set_act(const e4b_moe_desc &d, GroupedArgs &a, const uint16_t *bias, int64_t bias_estride) {
  const e4b_act *act = d.act;
  a.act = act && act->kind == E4B_ACT_CLAMPED_GLU ? 1 : 0;
  a.glu_alpha = a.act ? act->alpha : 0.0f;
  a.glu_limit = a.act ? act->limit : 0.0f;
  a.bias = bias;
  a.bias_estride = bias_estride;
}

static e4b_status check_lora(const e4b_lora *l, int *r) {
  *r = 0;
  if (!l || !l->A) return (l && l->B) ? E4B_ERR_INVALID_ARG : E4B_OK;
  if (!l->B) return E4B_ERR_INVALID_ARG;
  if (l->r < 8 || l->r > 128 || l->r % 8) return E4B_ERR_INVALID_ARG;
  if (!(l->scaling == l->scaling)) return E4B_ERR_INVALID_ARG;
  *r = l->r;
  return E4B_OK;
}

static e4b_status check_q(const e4b_qweight *q, int E, int N, int K) {
  if (!q || !q->codes || !q->scale) return E4B_ERR_INVALID_ARG;
  if (q->fmt < E4B_FMT_NF4 || q->fmt > E4B_FMT_FP8) return E4B_ERR_UNSUPPORTED;
  if (q->fmt == E4B_FMT_NF4_DQ && !q->scale2) return E4B_ERR_INVALID_ARG;
  if (q->fmt != E4B_FMT_NF4_DQ && q->dq_table) return E4B_ERR_INVALID_ARG;
  if (q->fmt != E4B_FMT_NF4 && q->fmt != E4B_FMT_NF4_DQ && q->codebook) return E4B_ERR_INVALID_ARG;
  if (q->E != E || q->N != N || q->K != K) return E4B_ERR_INVALID_ARG;
  if ((int64_t)E * N * K / (fmt_8bit(q->fmt) ? 1 : 2) > BUF_LIMIT) return E4B_ERR_INVALID_ARG;
  return E4B_OK;
}

static QStack qstack(const e4b_qweight *q) {
  QStack s;
  s.codes = q->codes;
  s.scale = q->scale;
  s.scale2 = q->scale2;
  s.codebook = q->codebook;
  s.dq_table = q->dq_table;
  s.fmt = q->fmt;
  s.N = q->N;
  s.K = q->K;
  const int64_t n = (int64_t)q->E * q->N * q->K;
  s.codes_bytes = (uint32_t)(fmt_8bit(q->fmt) ? n : n / 2);
  s.scale_bytes = (uint32_t)(q->fmt == E4B_FMT_NF4_DQ ? n / 64 : q->fmt == E4B_FMT_MXFP4 ? n / 32 : n / 64 * 4);
  s.scale2_bytes = q->fmt == E4B_FMT_NF4_DQ ? (uint32_t)((n / 64 + 255) / 256 * 4) : 0;
  return s;
}

#define E4B_TRY(x)                       \
  do {                                   \
    e4b_status st_ = (x);                \
    if (st_ != E4B_OK) return st_;       \
  } while (0)
#define E4B_LAUNCH(x)                    \
  do {                                   \
    if (!(x)) return E4B_ERR_HIP;        \
  } while (0)

}  // namespace e4b

using namespace e4b;

extern "C" {

int32_t e4b_version(void) { return 100; }

const char *e4b_status_str(int32_t s) {
  switch (s) {
    case E4B_OK: return "ok";
    case E4B_ERR_INVALID_ARG: return "invalid argument";
    case E4B_ERR_UNSUPPORTED: return "unsupported format";
    case E4B_ERR_WORKSPACE: return "workspace too small";
    case E4B_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

e4b_status e4b_moe_workspace_size(const e4b_moe_desc *desc, const e4b_lora *l_gu,
                                  const e4b_lora *l_dn, size_t *bytes) {
  int r1, r2;
  E4B_TRY(check_desc(desc));
  E4B_TRY(check_lora(l_gu, &r1));
  E4B_TRY(check_lora(l_dn, &r2));
  if (!bytes) return E4B_ERR_INVALID_ARG;
  *bytes = layout(*desc, r1, r2).total;
  return E4B_OK;
}

static e4b_status validate_layer(const e4b_moe_desc *d, const e4b_qweight *w_gu,
                                 const e4b_qweight *w_dn, const e4b_lora *l_gu,
                                 const e4b_lora *l_dn, int *r1, int *r2) {
  E4B_TRY(check_desc(d));
  E4B_TRY(check_q(w_gu, d->E, 2 * d->I, d->H));
  E4B_TRY(check_q(w_dn, d->E, d->H, d->I));
  if (w_gu->fmt != w_dn->fmt) return E4B_ERR_UNSUPPORTED;
  E4B_TRY(check_lora(l_gu, r1));
  E4B_TRY(check_lora(l_dn, r2));
  return E4B_OK;
}

// Decode-shaped inference forward as two launches (see E4B_SEPARATE): the gate_up launch
// routes inside each workgroup, forms z1 for its rows and the z2 partial sums over its h
// columns, and zeroes the down launch's arrival counters; the down launch adds the z2
// partial sums (first split) and forms y in the last workgroup of each column range.
static e4b_status moe_fwd_two_launch(const e4b_moe_desc &d, const e4b_qweight *w_gu, const e4b_qweight *w_dn,
                                     const e4b_lora *l_gu, const e4b_lora *l_dn, const uint16_t *x,
                                     const int32_t *ids, const float *topw, uint16_t *y, void *ws, const Layout &L,
                                     int r1, int r2, hipStream_t s) {
  const int M = d.T * d.topk, E = d.E, H = d.H, I = d.I;
  GroupedArgs gu{};
  gu.off = nullptr; gu.E = E; gu.M = M; gu.N = I; gu.K = H;
  gu.A = x; gu.lda = H; gu.a_gather = nullptr; gu.a_gdiv = d.topk;
  gu.a_bytes = (uint32_t)((int64_t)d.T * H * 2);
  gu.q = qstack(w_gu);
  gu.xb = r1 ? l_gu->B : nullptr; gu.xb_estride = (int64_t)2 * I * r1; gu.ldxb = r1; gu.r = r1;
  gu.C = at<uint16_t>(ws, L.h); gu.ldc = I; gu.alpha = 1.0f;
  gu.Gout = nullptr; gu.ldg = 2 * I; gu.I = I;
  set_act(d, gu, d.act ? d.act->b_gu : nullptr, (int64_t)2 * I);

  GroupedArgs dn{};
  dn.off = at<int32_t>(ws, L.off); dn.E = E; dn.M = M; dn.N = H; dn.K = I;
  dn.A = at<uint16_t>(ws, L.h); dn.lda = I; dn.a_gdiv = 1;
  dn.a_bytes = (uint32_t)((int64_t)M * I * 2);
  dn.q = qstack(w_dn);
  dn.xb = r2 ? l_dn->B : nullptr; dn.xb_estride = (int64_t)H * r2; dn.ldxb = r2; dn.r = r2;
  dn.C = at<float>(ws, L.O); dn.ldc = H; dn.alpha = 1.0f; dn.I = I;
  set_act(d, dn, d.act ? d.act->b_dn : nullptr, H);
  const int nsplit = small_down_splits(M, E, H, I);

  DecodeFuse f{};
  f.on = 1;
  f.ids = ids; f.topk = d.topk;
  f.cnt = at<int32_t>(ws, L.cnt); f.off = at<int32_t>(ws, L.off);
  f.perm = at<int32_t>(ws, L.perm); f.inv = at<int32_t>(ws, L.inv);
  f.ctr = at<int32_t>(ws, L.ctr);
  f.a1 = r1 ? l_gu->A : nullptr; f.a1_estride = (int64_t)r1 * H; f.s1 = r1 ? l_gu->scaling : 0.0f;
  f.a2 = r2 ? l_dn->A : nullptr; f.a2_estride = (int64_t)r2 * I; f.r2 = r2; f.s2 = r2 ? l_dn->scaling : 0.0f;
  f.zp = at<float>(ws, L.zp);
  f.topw = topw; f.T = d.T; f.y = y;
  f.split_stride = (int64_t)M * H; f.nsplit = nsplit;
  gu.fz = f;
  dn.fz = f;
  f.nparts = small_gate_up_parts(gu);
  f.nctr = small_down_ranges(dn, nsplit);
  if (f.nparts > cdiv(cdiv(I, 16), 8) || f.nctr > cdiv(H, 256)) return E4B_ERR_UNSUPPORTED;  // the layout's bounds
  gu.fz = f;
  dn.fz = f;
  E4B_LAUNCH(launch_small_gate_up(gu, s));
  E4B_LAUNCH(launch_small_down(dn, nsplit, s));
  return E4B_OK;
}

// The forward as a stream-ordered kernel sequence over a workspace of ws_bytes bytes.
static e4b_status moe_fwd(const e4b_moe_desc *desc, const e4b_qweight *w_gu, const e4b_qweight *w_dn,
                          const e4b_lora *l_gu, const e4b_lora *l_dn, const uint16_t *x, const int32_t *ids,
                          const float *topw, uint16_t *y, void *ws, size_t ws_bytes, void *stream) {
  int r1, r2;
  E4B_TRY(validate_layer(desc, w_gu, w_dn, l_gu, l_dn, &r1, &r2));
  const e4b_moe_desc &d = *desc;
  const Layout L = layout(d, r1, r2);
  if (!ws || ws_bytes < L.total) return E4B_ERR_WORKSPACE;
  if (d.T > 0 && (!x || !ids || !topw || !y)) return E4B_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int M = d.T * d.topk, E = d.E, H = d.H, I = d.I;
  int32_t *cnt = at<int32_t>(ws, L.cnt), *off = at<int32_t>(ws, L.off);
  int32_t *perm = at<int32_t>(ws, L.perm), *inv = at<int32_t>(ws, L.inv);
  uint16_t *z1 = at<uint16_t>(ws, L.z1), *z2 = at<uint16_t>(ws, L.z2), *h = at<uint16_t>(ws, L.h);
  float *O = at<float>(ws, L.O);
  uint16_t *G = L.G == NONE ? nullptr : at<uint16_t>(ws, L.G);
  float *part = L.part == NONE ? nullptr : at<float>(ws, L.part);
  uint16_t *W1x = L.W1x == NONE ? nullptr : at<uint16_t>(ws, L.W1x);
  uint16_t *W2x = L.W2x == NONE ? nullptr : at<uint16_t>(ws, L.W2x);

  if (M <= SMALL_M_MAX && !fmt_8bit(w_gu->fmt) && !(d.flags & (E4B_TRAIN | E4B_SEPARATE)) && E <= FUSE_E_MAX &&
      r1 <= FUSE_R_MAX && r2 <= FUSE_R_MAX)
    return M == 0 ? E4B_OK : moe_fwd_two_launch(d, w_gu, w_dn, l_gu, l_dn, x, ids, topw, y, ws, L, r1, r2, s);
  float *tail = L.tail == NONE ? nullptr : at<float>(ws, L.tail);
  int32_t *tail_ctr = L.tail_ctr == NONE ? nullptr : at<int32_t>(ws, L.tail_ctr);
  E4B_LAUNCH(launch_route(ids, M, E, cnt, off, perm, inv, s, tail_ctr, TAIL_CTRS));
  if (M == 0) return E4B_OK;
  if (W1x) {
    E4B_LAUNCH(launch_expand(qstack(w_gu), E, W1x, s));
    E4B_LAUNCH(launch_expand(qstack(w_dn), E, W2x, s));
  }
  // few routed rows: weight-streaming kernels (small.hip); otherwise the large tiles
  const bool small = M <= SMALL_M_MAX && !fmt_8bit(w_gu->fmt);  // 8-bit bases: large tiles at any size
  const bool train = d.flags & E4B_TRAIN;
  auto lora_a = [&](const GroupedArgs &a) { return small ? launch_small_lora_a(a, s) : launch_lora_a(a, s); };

  if (r1) {  // z1 = s1 * A1[e] x
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = r1; a.K = H;
    a.A = x; a.lda = H; a.a_gather = perm; a.a_gdiv = d.topk;
    a.Bd = l_gu->A; a.b_estride = (int64_t)r1 * H; a.ldb = H;
    a.C = z1; a.ldc = r1; a.alpha = l_gu->scaling;
    a.part = part; a.nsplit = lora_a_splits(M, E, a.N, a.K);
    // few rows: the LoRA-A kernel also writes the gathered rows of x into the O region
    // (written only later, by down), so gate_up reads them without a dependent gather
    if (small) a.xg_out = (uint16_t *)O;
    E4B_LAUNCH(lora_a(a));
  }
  {  // h = silu(G_gate) * G_up, G = W1 x + B1 z1
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = I; a.K = H;
    a.A = x; a.lda = H; a.a_gather = perm; a.a_gdiv = d.topk;
    a.a_bytes = (uint32_t)((int64_t)d.T * H * 2);
    if (small && r1) {  // the gathered copy: M rows in sorted order
      a.A = (const uint16_t *)O, a.a_gather = nullptr, a.a_gdiv = 1;
      a.a_bytes = (uint32_t)((int64_t)M * H * 2);
    }
    a.q = qstack(w_gu);
    a.Bx = W1x; a.bx_estride = (int64_t)2 * I * H; a.bx_bytes = (uint32_t)(a.bx_estride * 2);
    a.xa = z1; a.ldxa = r1; a.xb = r1 ? l_gu->B : nullptr; a.xb_estride = (int64_t)2 * I * r1;
    a.ldxb = r1; a.r = r1;
    a.C = h; a.ldc = I; a.alpha = 1.0f;
    a.Gout = G; a.ldg = 2 * I; a.I = I;
    set_act(d, a, d.act ? d.act->b_gu : nullptr, (int64_t)2 * I);
    E4B_LAUNCH(small ? launch_small_gate_up(a, s) : launch_gemm_gate_up(a, s));
  }
  if (r2) {  // z2 = s2 * A2[e] h
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = r2; a.K = I;
    a.A = h; a.lda = I; a.a_gdiv = 1;
    a.Bd = l_dn->A; a.b_estride = (int64_t)r2 * I; a.ldb = I;
    a.C = z2; a.ldc = r2; a.alpha = l_dn->scaling;
    a.part = part; a.nsplit = lora_a_splits(M, E, a.N, a.K);
    E4B_LAUNCH(lora_a(a));
  }
  int nsplit = 1;
  {  // O = W2 h + B2 z2
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = H; a.K = I;
    a.A = h; a.lda = I; a.a_gdiv = 1;
    a.a_bytes = (uint32_t)((int64_t)M * I * 2);
    a.q = qstack(w_dn);
    a.Bx = W2x; a.bx_estride = (int64_t)H * I; a.bx_bytes = (uint32_t)(a.bx_estride * 2);
    a.xa = z2; a.ldxa = r2; a.xb = r2 ? l_dn->B : nullptr; a.xb_estride = (int64_t)H * r2;
    a.ldxb = r2; a.r = r2;
    a.C = O; a.ldc = H; a.alpha = 1.0f; a.I = I;
    set_act(d, a, d.act ? d.act->b_dn : nullptr, H);
    if (small) {
      nsplit = train ? 1 : small_down_splits(M, E, H, I);
      E4B_LAUNCH(launch_small_down(a, nsplit, s));
    } else {
      a.tail = tail; a.tail_ctr = tail_ctr;
      E4B_LAUNCH(launch_gemm_down(a, s));
    }
  }
  E4B_LAUNCH(launch_combine(O, nsplit, (int64_t)M * H, inv, topw, d.T, d.topk, H, y, s));
  return E4B_OK;
}

e4b_status e4b_moe_fwd(const e4b_moe_desc *desc, const e4b_qweight *w_gu, const e4b_qweight *w_dn,
                       const e4b_lora *l_gu, const e4b_lora *l_dn, const uint16_t *x,
                       const int32_t *ids, const float *topw, uint16_t *y, void *ws,
                       size_t ws_bytes, void *stream) {
  return moe_fwd(desc, w_gu, w_dn, l_gu, l_dn, x, ids, topw, y, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ allocation-free forward
// One device-resident scratch array per GPU takes the place of the caller's workspace.  In
// host code the array's name is not a device address: its address on a device is looked up
// once, with that device current (hipGetSymbolAddress), kept in g_scratch, and only that
// address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[E4B_NOALLOC_SCRATCH_BYTES];
static constexpr int MAX_DEVICES = 64;
static void *g_scratch[MAX_DEVICES];
static std::mutex g_scratch_mu;

static e4b_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return E4B_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return E4B_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return E4B_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return E4B_OK;
}

e4b_status e4b_moe_fwd_noalloc(const e4b_moe_desc *desc, const e4b_qweight *w_gu, const e4b_qweight *w_dn,
                               const e4b_lora *l_gu, const e4b_lora *l_dn, const uint16_t *x,
                               const int32_t *ids, const float *topw, uint16_t *y, void *stream) {
  int r1, r2;
  E4B_TRY(validate_layer(desc, w_gu, w_dn, l_gu, l_dn, &r1, &r2));
  if (desc->flags & ~E4B_SEPARATE) return E4B_ERR_INVALID_ARG;  // inference only, no bf16 stack copies
  if (layout(*desc, r1, r2).total > (size_t)E4B_NOALLOC_SCRATCH_BYTES) return E4B_ERR_WORKSPACE;
  if (desc->T > 0 && (!x || !ids || !topw || !y)) return E4B_ERR_INVALID_ARG;
  void *ws = nullptr;
  E4B_TRY(scratch_of_current_device(&ws));
  t_noalloc = true;
  const e4b_status st = moe_fwd(desc, w_gu, w_dn, l_gu, l_dn, x, ids, topw, y, ws,
                                (size_t)E4B_NOALLOC_SCRATCH_BYTES, stream);
  t_noalloc = false;
  return st;
}

e4b_status e4b_moe_dgrad(const e4b_moe_desc *desc, const e4b_qweight *w_gu, const e4b_qweight *w_dn,
                         const e4b_lora *l_gu, const e4b_lora *l_dn, const int32_t *ids,
                         const float *topw, const uint16_t *dy, uint16_t *dx, float *d_topw,
                         void *ws, size_t ws_bytes, void *stream) {
  int r1, r2;
  E4B_TRY(validate_layer(desc, w_gu, w_dn, l_gu, l_dn, &r1, &r2));
  const e4b_moe_desc &d = *desc;
  if (!(d.flags & E4B_TRAIN)) return E4B_ERR_INVALID_ARG;
  const Layout L = layout(d, r1, r2);
  if (!ws || ws_bytes < L.total) return E4B_ERR_WORKSPACE;
  if (d.T > 0 && (!ids || !topw || !dy || !dx)) return E4B_ERR_INVALID_ARG;
  (void)ids;
  hipStream_t s = (hipStream_t)stream;
  const int M = d.T * d.topk, E = d.E, H = d.H, I = d.I;
  if (M == 0) return E4B_OK;
  int32_t *off = at<int32_t>(ws, L.off), *inv = at<int32_t>(ws, L.inv);
  uint16_t *G = at<uint16_t>(ws, L.G), *dO = at<uint16_t>(ws, L.dO), *dG = at<uint16_t>(ws, L.dG);
  uint16_t *u1 = at<uint16_t>(ws, L.u1), *u2 = at<uint16_t>(ws, L.u2);
  float *O = at<float>(ws, L.O), *dXp = at<float>(ws, L.dXp);
  float *part = L.part == NONE ? nullptr : at<float>(ws, L.part);
  uint16_t *A1T = at<uint16_t>(ws, L.A1T), *B1T = at<uint16_t>(ws, L.B1T);
  uint16_t *A2T = at<uint16_t>(ws, L.A2T), *B2T = at<uint16_t>(ws, L.B2T);
  // the base is decoded from the packed stacks again (the forward's bf16 copies, if it made
  // any, are not read)
  const uint16_t *W1x = nullptr, *W2x = nullptr;

  E4B_LAUNCH(launch_combine_bwd(dy, O, inv, topw, d.T, d.topk, H, dO, d_topw, s));
  if (r2) {
    E4B_LAUNCH(launch_transpose(l_dn->B, E, H, r2, B2T, s));  // [E,H,r] -> [E,r,H]
    E4B_LAUNCH(launch_transpose(l_dn->A, E, r2, I, A2T, s));  // [E,r,I] -> [E,I,r]
    GroupedArgs a{};  // u2 = s2 * dO B2
    a.off = off; a.E = E; a.M = M; a.N = r2; a.K = H;
    a.A = dO; a.lda = H; a.a_gdiv = 1;
    a.Bd = B2T; a.b_estride = (int64_t)r2 * H; a.ldb = H;
    a.C = u2; a.ldc = r2; a.alpha = l_dn->scaling;
    a.part = part; a.nsplit = lora_a_splits(M, E, a.N, a.K);
    E4B_LAUNCH(launch_lora_a(a, s));
  }
  {  // dH = dO W2 + u2 A2 -> SwiGLU backward -> dG
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = I; a.K = H;
    a.A = dO; a.lda = H; a.a_gdiv = 1;
    a.a_bytes = (uint32_t)((int64_t)M * H * 2);
    a.q = qstack(w_dn);
    a.Bx = W2x; a.bx_estride = (int64_t)H * I; a.bx_bytes = (uint32_t)(a.bx_estride * 2);
    a.xa = u2; a.ldxa = r2; a.xb = r2 ? A2T : nullptr; a.xb_estride = (int64_t)I * r2;
    a.ldxb = r2; a.r = r2;
    a.Gin = G; a.Gout = dG; a.ldg = 2 * I; a.I = I;
    set_act(d, a, nullptr, 0);
    E4B_LAUNCH(launch_gemm_down_dgrad(a, s));
  }
  if (r1) {
    E4B_LAUNCH(launch_transpose(l_gu->B, E, 2 * I, r1, B1T, s));  // [E,2I,r] -> [E,r,2I]
    E4B_LAUNCH(launch_transpose(l_gu->A, E, r1, H, A1T, s));      // [E,r,H] -> [E,H,r]
    GroupedArgs a{};  // u1 = s1 * dG B1
    a.off = off; a.E = E; a.M = M; a.N = r1; a.K = 2 * I;
    a.A = dG; a.lda = 2 * I; a.a_gdiv = 1;
    a.Bd = B1T; a.b_estride = (int64_t)r1 * 2 * I; a.ldb = 2 * I;
    a.C = u1; a.ldc = r1; a.alpha = l_gu->scaling;
    a.part = part; a.nsplit = lora_a_splits(M, E, a.N, a.K);
    E4B_LAUNCH(launch_lora_a(a, s));
  }
  {  // dXp = dG W1 + u1 A1
    GroupedArgs a{};
    a.off = off; a.E = E; a.M = M; a.N = H; a.K = 2 * I;
    a.A = dG; a.lda = 2 * I; a.a_gdiv = 1;
    a.a_bytes = (uint32_t)((int64_t)M * 2 * I * 2);
    a.q = qstack(w_gu);
    a.Bx = W1x; a.bx_estride = (int64_t)2 * I * H; a.bx_bytes = (uint32_t)(a.bx_estride * 2);
    a.xa = u1; a.ldxa = r1; a.xb = r1 ? A1T : nullptr; a.xb_estride = (int64_t)H * r1;
    a.ldxb = r1; a.r = r1;
    a.C = dXp; a.ldc = H; a.alpha = 1.0f; a.I = I;
    a.tail = L.tail == NONE ? nullptr : at<float>(ws, L.tail);
    a.tail_ctr = L.tail_ctr == NONE ? nullptr : at<int32_t>(ws, L.tail_ctr);
    E4B_LAUNCH(launch_gemm_gate_up_dgrad(a, s));
  }
  E4B_LAUNCH(launch_unpermute(dXp, inv, d.T, d.topk, H, dx, s));
  return E4B_OK;
}

e4b_status e4b_lora_wgrad(const e4b_moe_desc *desc, const e4b_lora *l_gu, const e4b_lora *l_dn,
                          const uint16_t *x, void *ws, size_t ws_bytes, float *dA_gu, float *dB_gu,
                          float *dA_dn, float *dB_dn, void *stream) {
  int r1, r2;
  E4B_TRY(check_desc(desc));
  E4B_TRY(check_lora(l_gu, &r1));
  E4B_TRY(check_lora(l_dn, &r2));
  const e4b_moe_desc &d = *desc;
  if (!(d.flags & E4B_TRAIN)) return E4B_ERR_INVALID_ARG;
  const Layout L = layout(d, r1, r2);
  if (!ws || ws_bytes < L.total) return E4B_ERR_WORKSPACE;
  if (r1 && (!dA_gu || !dB_gu || (d.T > 0 && !x))) return E4B_ERR_INVALID_ARG;
  if (r2 && (!dA_dn || !dB_dn)) return E4B_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int E = d.E, H = d.H, I = d.I;
  int32_t *off = at<int32_t>(ws, L.off), *perm = at<int32_t>(ws, L.perm);
  float *part = L.part == NONE ? nullptr : at<float>(ws, L.part);
  const int M = d.T * d.topk;
  auto split = [&](WgradArgs &w) {
    w.part = part;
    w.nsplit = wgrad_splits(M, E, w.Na, w.Nb);
  };
  if (r1) {
    WgradArgs a{};  // dB1[e] = dG_e^T z1_e
    a.off = off; a.E = E;
    a.P = at<uint16_t>(ws, L.dG); a.ldp = 2 * I; a.Na = 2 * I; a.p_gdiv = 1;
    a.Q = at<uint16_t>(ws, L.z1); a.ldq = r1; a.Nb = r1; a.q_gdiv = 1;
    a.C = dB_gu;
    split(a);
    E4B_LAUNCH(launch_wgrad(a, s));
    WgradArgs b{};  // dA1[e] = u1_e^T X_e
    b.off = off; b.E = E;
    b.P = at<uint16_t>(ws, L.u1); b.ldp = r1; b.Na = r1; b.p_gdiv = 1;
    b.Q = x; b.ldq = H; b.Nb = H; b.q_gather = perm; b.q_gdiv = d.topk;
    b.C = dA_gu;
    split(b);
    E4B_LAUNCH(launch_wgrad(b, s));
  }
  if (r2) {
    WgradArgs a{};  // dB2[e] = dO_e^T z2_e
    a.off = off; a.E = E;
    a.P = at<uint16_t>(ws, L.dO); a.ldp = H; a.Na = H; a.p_gdiv = 1;
    a.Q = at<uint16_t>(ws, L.z2); a.ldq = r2; a.Nb = r2; a.q_gdiv = 1;
    a.C = dB_dn;
    split(a);
    E4B_LAUNCH(launch_wgrad(a, s));
    WgradArgs b{};  // dA2[e] = u2_e^T h_e
    b.off = off; b.E = E;
    b.P = at<uint16_t>(ws, L.u2); b.ldp = r2; b.Na = r2; b.p_gdiv = 1;
    b.Q = at<uint16_t>(ws, L.h); b.ldq = I; b.Nb = I; b.q_gdiv = 1;
    b.C = dA_dn;
    split(b);
    E4B_LAUNCH(launch_wgrad(b, s));
  }
  return E4B_OK;
}

e4b_status e4b_moe_route(const e4b_moe_desc *desc, const int32_t *ids, int32_t *cnt, int32_t *off,
                         int32_t *perm, int32_t *inv, void *stream) {
  E4B_TRY(check_desc(desc));
  const int M = desc->T * desc->topk;
  if (!cnt || !off || (M > 0 && (!ids || !perm || !inv))) return E4B_ERR_INVALID_ARG;
  E4B_LAUNCH(launch_route(ids, M, desc->E, cnt, off, perm, inv, (hipStream_t)stream));
  return E4B_OK;
}

e4b_status e4b_router_topk(const float *logits, int32_t T, int32_t E, int32_t topk, int32_t *ids, float *topw,
                           void *stream) {
  if (T < 0 || E < 1 || E > E4B_ROUTER_MAX_E || topk < 1 || topk > E || topk > E4B_ROUTER_MAX_K)
    return E4B_ERR_INVALID_ARG;
  if (T == 0) return E4B_OK;
  if (!logits || !ids || !topw) return E4B_ERR_INVALID_ARG;
  E4B_LAUNCH(launch_router_topk(logits, T, E, topk, ids, topw, (hipStream_t)stream));
  return E4B_OK;
}

e4b_status e4b_router_bwd(const float *topw, const float *d_topw, const int32_t *ids, int32_t T, int32_t E,
                          int32_t topk, float *d_logits, void *stream) {
  if (T < 0 || E < 1 || E > E4B_ROUTER_MAX_E || topk < 1 || topk > E || topk > E4B_ROUTER_MAX_K)
    return E4B_ERR_INVALID_ARG;
  if (T == 0) return E4B_OK;
  if (!topw || !d_topw || !ids || !d_logits) return E4B_ERR_INVALID_ARG;
  E4B_LAUNCH(launch_router_bwd(topw, d_topw, ids, T, E, topk, d_logits, (hipStream_t)stream));
  return E4B_OK;
}

e4b_status e4b_dequant(const e4b_qweight *w, int32_t expert, float *out_f32, uint16_t *out_bf16,
                       void *stream) {
  if (!w || w->E < 1 || w->N < 1 || w->K < 64 || w->K % 64) return E4B_ERR_INVALID_ARG;
  E4B_TRY(check_q(w, w->E, w->N, w->K));
  if (expert >= w->E) return E4B_ERR_INVALID_ARG;
  if (!out_f32 && !out_bf16) return E4B_ERR_INVALID_ARG;
  const int64_t per = (int64_t)w->N * w->K;
  const int64_t e0 = expert < 0 ? 0 : expert;
  const int64_t n = expert < 0 ? per * w->E : per;
  E4B_LAUNCH(launch_dequant(qstack(w), e0 * per, n, out_f32, out_bf16, (hipStream_t)stream));
  return E4B_OK;
}

e4b_status e4b_quantize(int32_t fmt, int32_t E, int32_t N, int32_t K, const float *w, uint8_t *codes,
                        void *scale, float *scale2, void *stream) {
  if (fmt < E4B_FMT_NF4 || fmt > E4B_FMT_FP8) return E4B_ERR_UNSUPPORTED;
  if (E < 1 || N < 1 || K < 64 || K % 64) return E4B_ERR_INVALID_ARG;
  if (!w || !codes || !scale || (fmt == E4B_FMT_NF4_DQ && !scale2)) return E4B_ERR_INVALID_ARG;
  const int64_t n = (int64_t)E * N * K;
  E4B_LAUNCH(launch_quantize(fmt, n, w, codes, scale, scale2, (hipStream_t)stream));
  return E4B_OK;
}

e4b_status e4b_moe_check(const e4b_moe_desc *desc, const void *ws, void *stream, int32_t *dropped) {
  E4B_TRY(check_desc(desc));
  if (!ws || !dropped) return E4B_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return E4B_ERR_HIP;
  const Layout L = layout(*desc, 0, 0);
  int32_t v = 0;
  if (hipMemcpy(&v, (const char *)ws + L.cnt + (size_t)desc->E * 4, 4, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return E4B_ERR_HIP;
  *dropped = v;
  return E4B_OK;
}

e4b_status e4b_get_stats(e4b_stats *out) {
  if (!out) return E4B_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  out->launches_total = g_total.load();
  out->route = g_count[FAM_ROUTE].load();
  out->lora_a = g_count[FAM_LORA_A].load();
  out->gemm_gate_up = g_count[FAM_GATE_UP].load();
  out->gemm_down = g_count[FAM_DOWN].load();
  out->combine = g_count[FAM_COMBINE].load();
  out->combine_bwd = g_count[FAM_COMBINE_BWD].load();
  out->gemm_down_dgrad = g_count[FAM_DOWN_DGRAD].load();
  out->gemm_gate_up_dgrad = g_count[FAM_GATE_UP_DGRAD].load();
  out->unpermute = g_count[FAM_UNPERMUTE].load();
  out->wgrad = g_count[FAM_WGRAD].load();
  out->quant = g_count[FAM_QUANT].load();
  out->dequant = g_count[FAM_DEQUANT].load();
  out->expand = g_count[FAM_EXPAND].load();
  out->router = g_count[FAM_ROUTER].load();
  out->fallbacks = 0;
  return E4B_OK;
}

void e4b_reset_stats(void) {
  for (int i = 0; i < FAM_COUNT; ++i) g_count[i] = 0;
  g_total = 0;
}

e4b_status e4b_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return E4B_OK;
}

e4b_status e4b_timing_read(int32_t max, char (*names)[32], int64_t *launches, double *ms,
                           int32_t *n_out) {
  if (!n_out) return E4B_ERR_INVALID_ARG;
  std::vector<TimedLaunch> pend;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    pend.swap(g_pending);
  }
  for (auto &t : pend) {
    float el = 0.0f;
    if (hipEventSynchronize(t.b) != hipSuccess) return E4B_ERR_HIP;
    if (hipEventElapsedTime(&el, t.a, t.b) != hipSuccess) return E4B_ERR_HIP;
    g_tl[t.fam]++;
    g_tms[t.fam] += el;
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  int n = 0;
  for (int f = 0; f < FAM_COUNT; ++f) {
    if (g_tl[f] == 0) continue;
    if (n < max) {
      if (names) {
        std::strncpy(names[n], family_name(f), 31);
        names[n][31] = 0;
      }
      if (launches) launches[n] = g_tl[f];
      if (ms) ms[n] = g_tms[f];
    }
    ++n;
    g_tl[f] = 0;
    g_tms[f] = 0.0;
  }
  *n_out = n;
  return E4B_OK;
}

}  // extern "C"
