/*
 * CPU oracle -- TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load
 * or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the HIP library.
 *
 * What it computes, and where the pages fix it:
 *  - The expert layer: for each routed expert e of a token, act(W_e x + s*B[e]A[e]x)
 *    on the fused gate_up stack [E,2I,H], then down_proj [E,H,I] plus its own
 *    LoRA delta, weighted by the router weight and summed over the token's top-k
 *    (solution page "How do I QLoRA-train the fused experts of a MoE", section
 *    "The abstraction that fails, and what replaces it": stacked shapes, the
 *    delta per routed expert before the activation; section "Why it happens":
 *    the term scaling * (x A[e]^T) B[e]^T with stacked per-expert A/B, the base
 *    re-dequantised in backward).
 *  - The epilogue act(gate) * up with SiLU (same page, "Limitations": the
 *    stock-epilogue contract; README "Supported scope": SwiGLU families).
 *  - Weights come from 4-bit packed stacks decoded with a per-block scale (README,
 *    "The package family": 4-bit-packed expert stacks, in-register decode).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - NF4: the 16-value NormalFloat table of the QLoRA paper; blocks of 64
 *    contiguous elements along the reduction axis with an fp32 absmax; element 2j
 *    in the high nibble; nearest code with ties to the lower index; zero block ->
 *    code 7 and absmax 0.  Dequant = one fp32 multiply fp32(code) * absmax.
 *  - Double quantisation: absmax codes c = rne(255 * absmax/scale2) per group of
 *    256 blocks, scale2 = group max; absmax' = fp32(c/255) * scale2.  A stack may
 *    carry its own 8-bit code table instead (absmax' = fp32(table[c] * scale2), e.g.
 *    QLoRA's dynamic 8-bit code) and its own sixteen 4-bit code values; the
 *    quantisers always target the built-in tables.
 *  - MXFP4: E2M1 elements (element 2j in the low nibble), one E8M0 scale per 32
 *    elements along the reduction axis, scale exponent floor(log2(amax)) - 2.
 *  - scaling s = alpha / r; gate = rows [0, I) of gate_up, up = rows [I, 2I).
 *  - gpt-oss experts (README "Scope": MXFP4 experts with per-expert biases and a
 *    clamped GLU; project record "limitations": the faithful clamped GLU and biases):
 *    the pages give no formula, so the reading is that model family's published expert
 *    function: gate/up interleaved by row (2i, 2i+1), biases added before the clamp,
 *    gate clamped from above and up from both sides at `limit`, h = (up + 1) * gate *
 *    sigmoid(alpha * gate), down bias added after the down projection.  The LoRA delta
 *    enters before the activation as for the stock epilogue; the biases are frozen.
 *  - 8-bit bases (README, opening section: int8 and fp8 storage modes of the fused stack;
 *    the pages fix neither scheme): blocks of 64 elements along the reduction axis with one
 *    fp32 scale, symmetric linear INT8 (scale = absmax / 127) and OCP FP8 E4M3 without
 *    infinities (largest finite 448, scale = absmax / 448), nearest value with ties to even.
 *    Dequant is the same single fp32 multiply as for NF4.
 *  - Routing grouped by expert, stable in the flat index t*k + j.
 *
 * Precision: weights dequantise exactly per the fp32 contract; everything after
 * that is fp64.  Sums run in ascending index order, one accumulator each.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int32_t orc_version(void) { return 1; }

/* NormalFloat-4 values, index 0..15 (QLoRA paper, NF4 data type table). */
static const float NF4[16] = {
    -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
    -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
    0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f, 0.33791524171829224f,
    0.44070982933044434f, 0.5626170039176941f, 0.7229568362236023f, 1.0f};

/* FP4 E2M1 magnitudes for codes 0..7 (OCP Microscaling formats v1.0). */
static const float E2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

void orc_nf4_codebook(float out[16]) { memcpy(out, NF4, sizeof(NF4)); }

/* fp32 -> bf16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

void orc_bf16_round(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}

/* ---------------------------------------------------------------- quantisers */

static uint8_t nf4_nearest(float v) {
  uint8_t best = 0;
  float bestd = fabsf(v - NF4[0]);
  for (int i = 1; i < 16; ++i) {
    float d = fabsf(v - NF4[i]);
    if (d < bestd) { bestd = d; best = (uint8_t)i; }
  }
  return best;
}

void orc_quant_nf4(const float *w, int64_t n, uint8_t *codes, float *absmax) {
  int64_t nb = n / 64;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    const float *blk = w + b * 64;
    float amax = 0.0f;
    for (int i = 0; i < 64; ++i) {
      float a = fabsf(blk[i]);
      if (a > amax) amax = a;
    }
    absmax[b] = amax;
    uint8_t q[64];
    for (int i = 0; i < 64; ++i) q[i] = (amax == 0.0f) ? 7 : nf4_nearest(blk[i] / amax);
    for (int j = 0; j < 32; ++j) codes[b * 32 + j] = (uint8_t)((q[2 * j] << 4) | q[2 * j + 1]);
  }
}

void orc_quant_nf4_dq(const float *w, int64_t n, uint8_t *codes, uint8_t *qabsmax, float *scale2) {
  int64_t nb = n / 64;
  float *am = (float *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(float));
  orc_quant_nf4(w, n, codes, am);
  int64_t ng = (nb + 255) / 256;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < ng; ++g) {
    int64_t b0 = g * 256, b1 = b0 + 256 < nb ? b0 + 256 : nb;
    float s = 0.0f;
    for (int64_t b = b0; b < b1; ++b)
      if (am[b] > s) s = am[b];
    scale2[g] = s;
    for (int64_t b = b0; b < b1; ++b) {
      if (s == 0.0f) { qabsmax[b] = 0; continue; }
      float t = am[b] / s;
      t = t * 255.0f;
      qabsmax[b] = (uint8_t)nearbyintf(t);
    }
  }
  free(am);
}

static uint8_t e2m1_nearest(float a) { /* a >= 0; ties to the even code */
  if (a >= 6.0f) return 7;
  uint8_t best = 0;
  float bestd = a;
  for (int i = 1; i < 8; ++i) {
    float d = fabsf(a - E2M1[i]);
    if (d < bestd || (d == bestd && (i & 1) == 0)) { bestd = d; best = (uint8_t)i; }
  }
  return best;
}

void orc_quant_mxfp4(const float *w, int64_t n, uint8_t *codes, uint8_t *scales) {
  int64_t nb = n / 32;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    const float *blk = w + b * 32;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(blk[i]);
      if (a > amax) amax = a;
    }
    uint8_t q[32];
    if (amax == 0.0f) {
      scales[b] = 0;
      memset(q, 0, sizeof(q));
    } else {
      int ex;
      frexpf(amax, &ex);            /* amax = m * 2^ex, m in [0.5, 1) */
      int e = (ex - 1) - 2;         /* floor(log2 amax) - emax(E2M1) */
      int X = e + 127;
      if (X < 0) X = 0;
      if (X > 254) X = 254;
      e = X - 127;
      scales[b] = (uint8_t)X;
      for (int i = 0; i < 32; ++i) {
        float v = ldexpf(blk[i], -e);
        uint8_t c = e2m1_nearest(fabsf(v));
        if (v < 0.0f && c != 0) c |= 8;
        q[i] = c;
      }
    }
    for (int j = 0; j < 16; ++j) codes[b * 16 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
  }
}

/* FP8 E4M3 (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
 * subnormals m * 2^-9; 0x7F and 0xFF are NaN (there is no infinity). */
float orc_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 15, m = code & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexpf((float)m, -9);
  else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return (code & 0x80) ? -v : v;
}

/* Nearest E4M3 code to a finite v with |v| <= 448, ties to the even code (the one whose last
 * mantissa bit is 0). */
static uint8_t e4m3_nearest(float v) {
  uint8_t sign = v < 0.0f ? 0x80 : 0;
  float a = fabsf(v);
  uint8_t best = 0;
  float bestd = a;  /* code 0 = +0 */
  for (int c = 1; c < 127; ++c) {  /* every finite positive code, ascending value */
    float d = fabsf(a - orc_e4m3_value((uint8_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) { bestd = d; best = (uint8_t)c; }
  }
  return (uint8_t)(best | (best ? sign : 0));
}

void orc_quant_int8(const float *w, int64_t n, uint8_t *codes, float *scales) {
  int64_t nb = n / 64;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    const float *blk = w + b * 64;
    float amax = 0.0f;
    for (int i = 0; i < 64; ++i) if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
    float s = amax / 127.0f;
    scales[b] = s;
    for (int i = 0; i < 64; ++i) {
      long q = 0;
      if (s != 0.0f) {
        float t = blk[i] / s;
        q = lrintf(t);  /* current rounding mode: to nearest, ties to even */
        if (q > 127) q = 127;
        if (q < -127) q = -127;
      }
      codes[b * 64 + i] = (uint8_t)(int8_t)q;
    }
  }
}

void orc_quant_fp8(const float *w, int64_t n, uint8_t *codes, float *scales) {
  int64_t nb = n / 64;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    const float *blk = w + b * 64;
    float amax = 0.0f;
    for (int i = 0; i < 64; ++i) if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
    float s = amax / 448.0f;
    scales[b] = s;
    for (int i = 0; i < 64; ++i) {
      float t = s != 0.0f ? blk[i] / s : 0.0f;
      if (t > 448.0f) t = 448.0f;
      if (t < -448.0f) t = -448.0f;
      codes[b * 64 + i] = e4m3_nearest(t);
    }
  }
}

/* ------------------------------------------------------------------- dequant */

static float deq_one(int32_t fmt, int64_t i, const uint8_t *codes, const void *scale,
                     const float *scale2, const float *dq_table, const float *codebook) {
  if (fmt == ORC_FMT_INT8) return (float)(int8_t)codes[i] * ((const float *)scale)[i / 64];
  if (fmt == ORC_FMT_FP8) return orc_e4m3_value(codes[i]) * ((const float *)scale)[i / 64];
  uint8_t byte = codes[i >> 1];
  if (fmt == ORC_FMT_MXFP4) {
    uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
    float m = E2M1[c & 7];
    if (c & 8) m = -m;
    int X = ((const uint8_t *)scale)[i / 32];
    return ldexpf(m, X - 127);
  }
  uint8_t c = (i & 1) ? (byte & 15) : (byte >> 4);
  int64_t b = i / 64;
  float amax;
  if (fmt == ORC_FMT_NF4) {
    amax = ((const float *)scale)[b];
  } else {
    uint8_t qa = ((const uint8_t *)scale)[b];
    float t = dq_table ? dq_table[qa] : (float)qa / 255.0f;
    amax = t * scale2[b / 256];
  }
  float v = codebook ? codebook[c] : NF4[c];
  return v * amax;
}

void orc_dequant(int32_t fmt, int64_t n, const uint8_t *codes, const void *scale,
                 const float *scale2, const float *dq_table, const float *codebook,
                 float *out_f32, uint16_t *out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float v = deq_one(fmt, i, codes, scale, scale2, dq_table, codebook);
    if (out_f32) out_f32[i] = v;
    if (out_bf16) out_bf16[i] = bf16_rne(v);
  }
}

/* ------------------------------------------------------------------- routing */

void orc_route(int32_t T, int32_t k, int32_t E, const int32_t *ids,
               int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv) {
  int64_t M = (int64_t)T * k;
  for (int e = 0; e <= E; ++e) cnt[e] = 0;
  for (int64_t f = 0; f < M; ++f) {
    int e = ids[f];
    if (e >= 0 && e < E) cnt[e]++;
    else cnt[E]++;
  }
  off[0] = 0;
  for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];
  int32_t *next = (int32_t *)malloc((size_t)(E > 0 ? E : 1) * sizeof(int32_t));
  for (int e = 0; e < E; ++e) next[e] = off[e];
  for (int64_t p = 0; p < M; ++p) perm[p] = -1;
  for (int64_t f = 0; f < M; ++f) {
    int e = ids[f];
    if (e >= 0 && e < E) {
      perm[next[e]] = (int32_t)f;
      inv[f] = next[e]++;
    } else {
      inv[f] = -1;
    }
  }
  free(next);
}

/* ------------------------------------------------------------ expert MLP rows */

typedef struct {
  const float *W1, *W2; /* this expert, dense fp32: [2I, H], [H, I] */
  const uint16_t *A1, *B1, *A2, *B2;
  const uint16_t *b1, *b2; /* this expert's biases [2I], [H] (clamped GLU only; nullable) */
} expert_view;

/* Router (the frozen router of the method page, "Which project solves it": top-k expert
 * ids and their weights are inputs to the layer; this is that step on its own).  For token
 * t: the k largest logits, larger first, equal logits in ascending expert id; then the
 * softmax over the k chosen, max-subtracted, in double precision, stored as float. */
void orc_router_topk(int32_t T, int32_t E, int32_t k, const float *logits, int32_t *ids, float *w) {
  for (int32_t t = 0; t < T; ++t) {
    const float *l = logits + (int64_t)t * E;
    int32_t *id = ids + (int64_t)t * k;
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        int taken = 0;
        for (int32_t q = 0; q < j; ++q) taken |= id[q] == e;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      id[j] = best;
    }
    const double m = (double)l[id[0]];
    double den = 0.0;
    for (int32_t j = 0; j < k; ++j) den += exp((double)l[id[j]] - m);
    for (int32_t j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(exp((double)l[id[j]] - m) / den);
  }
}

/* Gradient of the router weights with respect to the logits, the chosen experts held fixed:
 * d_logit[ids[j]] = w_j (dw_j - sum_i w_i dw_i) (softmax Jacobian), zero for the others. */
void orc_router_bwd(int32_t T, int32_t E, int32_t k, const float *w, const float *dw, const int32_t *ids,
                    float *dlogits) {
  for (int32_t t = 0; t < T; ++t) {
    const float *wt = w + (int64_t)t * k, *gt = dw + (int64_t)t * k;
    float *d = dlogits + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) d[e] = 0.0f;
    double dot = 0.0;
    for (int32_t j = 0; j < k; ++j) dot += (double)wt[j] * (double)gt[j];
    for (int32_t j = 0; j < k; ++j) d[ids[(int64_t)t * k + j]] = (float)((double)wt[j] * ((double)gt[j] - dot));
  }
}

static double silu(double g) { return g / (1.0 + exp(-g)); }
static double sigm(double g) { return 1.0 / (1.0 + exp(-g)); }

/* Clamped GLU (act == 1): h and its partial derivatives at (gate, up).  The clamps pass the
 * gradient where the argument lies inside the closed interval. */
static double cglu(const orc_layer *L, double g, double u, double *dh_dg, double *dh_du) {
  const double gc = g < L->limit ? g : L->limit;
  const double uc = u < -L->limit ? -L->limit : (u > L->limit ? L->limit : u);
  const double sg = sigm(L->alpha * gc);
  if (dh_dg) *dh_dg = g <= L->limit ? (uc + 1.0) * (sg + L->alpha * gc * sg * (1.0 - sg)) : 0.0;
  if (dh_du) *dh_du = (u >= -L->limit && u <= L->limit) ? gc * sg : 0.0;
  return (uc + 1.0) * gc * sg;
}
static double bias_of(const uint16_t *b, int64_t i) { return b ? bf16_to_double(b[i]) : 0.0; }

/* Forward of one routed row.  Fills z1[r1], gu[2I], hh[I], z2[r2], o[H]. */
static void row_forward(const orc_layer *L, const expert_view *X, const double *x,
                        double *z1, double *gu, double *hh, double *z2, double *o) {
  const int H = L->H, I = L->I, r1 = L->r1, r2 = L->r2;
  const int lora1 = X->A1 != NULL, lora2 = X->A2 != NULL;
  /* z1 = A1 x */
  for (int j = 0; j < r1 && lora1; ++j) {
    double acc = 0.0;
    for (int h = 0; h < H; ++h) acc += bf16_to_double(X->A1[(int64_t)j * H + h]) * x[h];
    z1[j] = acc;
  }
  /* gu = W1 x + s1 * B1 z1 */
  for (int n = 0; n < 2 * I; ++n) {
    const float *wr = X->W1 + (int64_t)n * H;
    double acc = 0.0;
    for (int h = 0; h < H; ++h) acc += (double)wr[h] * x[h];
    double d = 0.0;
    for (int j = 0; j < r1 && lora1; ++j) d += bf16_to_double(X->B1[(int64_t)n * r1 + j]) * z1[j];
    gu[n] = L->post_act_delta ? acc : acc + L->s1 * d; /* planted variant re-adds it below */
    if (L->act == 1) gu[n] += bias_of(X->b1, n);
  }
  /* h = silu(gate) * up, or the clamped GLU over interleaved rows */
  for (int i = 0; i < I; ++i) {
    if (L->act == 1) {
      hh[i] = cglu(L, gu[2 * i], gu[2 * i + 1], NULL, NULL);
    } else if (!L->post_act_delta) {
      hh[i] = silu(gu[i]) * gu[I + i];
    } else {
      /* planted variant: act(W x) + d on the activated half */
      double dg = 0.0, du = 0.0;
      for (int j = 0; j < r1 && lora1; ++j) {
        dg += bf16_to_double(X->B1[(int64_t)i * r1 + j]) * z1[j];
        du += bf16_to_double(X->B1[(int64_t)(I + i) * r1 + j]) * z1[j];
      }
      hh[i] = (silu(gu[i]) + L->s1 * dg) * (gu[I + i] + L->s1 * du);
    }
  }
  /* z2 = A2 h */
  for (int j = 0; j < r2 && lora2; ++j) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += bf16_to_double(X->A2[(int64_t)j * I + i]) * hh[i];
    z2[j] = acc;
  }
  /* o = W2 h + s2 * B2 z2 */
  for (int n = 0; n < H; ++n) {
    const float *wr = X->W2 + (int64_t)n * I;
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += (double)wr[i] * hh[i];
    double d = 0.0;
    for (int j = 0; j < r2 && lora2; ++j) d += bf16_to_double(X->B2[(int64_t)n * r2 + j]) * z2[j];
    o[n] = acc + L->s2 * d;
    if (L->act == 1) o[n] += bias_of(X->b2, n);
  }
}

/* Dense fp32 weights of expert e: the caller's, or expert e of the packed stack
 * dequantised through the flat element index (double-quantised scales group 256
 * blocks over the whole flat stack, so the flat index is the plain addressing). */
static const float *expert_weights_any(const float *dense, const orc_qweight *q, int e,
                                       int64_t per, float *buf) {
  if (dense) return dense + (int64_t)e * per;
  int64_t base = (int64_t)e * per;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < per; ++i)
    buf[i] = deq_one(q->fmt, base + i, q->codes, q->scale, q->scale2, q->dq_table, q->codebook);
  return buf;
}

static expert_view make_view(const orc_layer *L, int e, const float *W1, const float *W2) {
  expert_view v;
  v.W1 = W1;
  v.W2 = W2;
  v.A1 = L->A1 ? L->A1 + (int64_t)e * L->r1 * L->H : NULL;
  v.B1 = L->A1 ? L->B1 + (int64_t)e * 2 * L->I * L->r1 : NULL;
  v.A2 = L->A2 ? L->A2 + (int64_t)e * L->r2 * L->I : NULL;
  v.B2 = L->A2 ? L->B2 + (int64_t)e * L->H * L->r2 : NULL;
  v.b1 = L->b1 ? L->b1 + (int64_t)e * 2 * L->I : NULL;
  v.b2 = L->b2 ? L->b2 + (int64_t)e * L->H : NULL;
  return v;
}

/* Rows routed to expert e among the selected tokens, ascending flat index. */
static int64_t rows_of(const orc_layer *L, const uint8_t *mask, int e, int64_t *out) {
  int64_t M = (int64_t)L->T * L->k, n = 0;
  for (int64_t f = 0; f < M; ++f)
    if (L->ids[f] == e && (!mask || mask[f / L->k])) out[n++] = f;
  return n;
}

int32_t orc_moe_fwd(const orc_layer *L, const uint8_t *tok_mask, double *y, double *O) {
  const int E = L->E, H = L->H, I = L->I, T = L->T, k = L->k;
  const int r1 = L->r1 > 0 ? L->r1 : 1, r2 = L->r2 > 0 ? L->r2 : 1;
  const int64_t M = (int64_t)T * k, per1 = (int64_t)2 * I * H, per2 = (int64_t)H * I;
  double *Orow = O ? O : (double *)calloc((size_t)(M > 0 ? M : 1) * H, sizeof(double));
  if (O) memset(O, 0, (size_t)M * H * sizeof(double));
  int64_t *rows = (int64_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
  float *buf1 = L->W1f ? NULL : (float *)malloc((size_t)per1 * sizeof(float));
  float *buf2 = L->W2f ? NULL : (float *)malloc((size_t)per2 * sizeof(float));
  for (int e = 0; e < E; ++e) {
    int64_t nr = rows_of(L, tok_mask, e, rows);
    if (nr == 0) continue;
    const float *W1 = expert_weights_any(L->W1f, L->w_gu, e, per1, buf1);
    const float *W2 = expert_weights_any(L->W2f, L->w_dn, e, per2, buf2);
    expert_view V = make_view(L, e, W1, W2);
#pragma omp parallel
    {
      double *x = (double *)malloc(sizeof(double) * H);
      double *z1 = (double *)malloc(sizeof(double) * r1);
      double *gu = (double *)malloc(sizeof(double) * 2 * I);
      double *hh = (double *)malloc(sizeof(double) * I);
      double *z2 = (double *)malloc(sizeof(double) * r2);
#pragma omp for schedule(dynamic, 1)
      for (int64_t q = 0; q < nr; ++q) {
        int64_t f = rows[q];
        const uint16_t *xr = L->x + (f / k) * (int64_t)H;
        for (int h = 0; h < H; ++h) x[h] = bf16_to_double(xr[h]);
        row_forward(L, &V, x, z1, gu, hh, z2, Orow + f * (int64_t)H);
      }
      free(x); free(z1); free(gu); free(hh); free(z2);
    }
  }
  /* y[t] = sum_j w[t,j] * o[t,j], j ascending */
  for (int t = 0; t < T; ++t) {
    double *yt = y + (int64_t)t * H;
    for (int h = 0; h < H; ++h) yt[h] = 0.0;
    if (tok_mask && !tok_mask[t]) continue;
    for (int j = 0; j < k; ++j) {
      int64_t f = (int64_t)t * k + j;
      int e = L->ids[f];
      if (e < 0 || e >= E) continue;
      double w = (double)L->topw[f];
      const double *o = Orow + f * (int64_t)H;
      for (int h = 0; h < H; ++h) yt[h] += w * o[h];
    }
  }
  free(rows); free(buf1); free(buf2);
  if (!O) free(Orow);
  return 0;
}

int32_t orc_moe_bwd(const orc_layer *L, const uint8_t *tok_mask, const uint16_t *dy,
                    double *dx, double *dw, double *dA1, double *dB1, double *dA2, double *dB2) {
  const int E = L->E, H = L->H, I = L->I, T = L->T, k = L->k;
  const int R1 = L->r1, R2 = L->r2;
  const int r1 = R1 > 0 ? R1 : 1, r2 = R2 > 0 ? R2 : 1;
  const int lora1 = L->A1 != NULL, lora2 = L->A2 != NULL;
  const int64_t M = (int64_t)T * k, per1 = (int64_t)2 * I * H, per2 = (int64_t)H * I;
  double *dxp = (double *)calloc((size_t)(M > 0 ? M : 1) * H, sizeof(double));
  int64_t *rows = (int64_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
  float *buf1 = L->W1f ? NULL : (float *)malloc((size_t)per1 * sizeof(float));
  float *buf2 = L->W2f ? NULL : (float *)malloc((size_t)per2 * sizeof(float));
  if (dw) for (int64_t f = 0; f < M; ++f) dw[f] = 0.0;
  if (dA1 && lora1) memset(dA1, 0, sizeof(double) * (size_t)E * R1 * H);
  if (dB1 && lora1) memset(dB1, 0, sizeof(double) * (size_t)E * 2 * I * R1);
  if (dA2 && lora2) memset(dA2, 0, sizeof(double) * (size_t)E * R2 * I);
  if (dB2 && lora2) memset(dB2, 0, sizeof(double) * (size_t)E * H * R2);

  for (int e = 0; e < E; ++e) {
    int64_t nr = rows_of(L, tok_mask, e, rows);
    if (nr == 0) continue;
    const float *W1 = expert_weights_any(L->W1f, L->w_gu, e, per1, buf1);
    const float *W2 = expert_weights_any(L->W2f, L->w_dn, e, per2, buf2);
    expert_view V = make_view(L, e, W1, W2);
    /* per-row vectors kept for the weight-gradient reductions */
    double *Sx = (double *)malloc(sizeof(double) * nr * H);
    double *Sz1 = (double *)malloc(sizeof(double) * nr * r1);
    double *Sdz1 = (double *)malloc(sizeof(double) * nr * r1);
    double *Sdgu = (double *)malloc(sizeof(double) * nr * 2 * I);
    double *Shh = (double *)malloc(sizeof(double) * nr * I);
    double *Sz2 = (double *)malloc(sizeof(double) * nr * r2);
    double *Sdz2 = (double *)malloc(sizeof(double) * nr * r2);
    double *Sdo = (double *)malloc(sizeof(double) * nr * H);
#pragma omp parallel
    {
      double *gu = (double *)malloc(sizeof(double) * 2 * I);
      double *o = (double *)malloc(sizeof(double) * H);
      double *dhh = (double *)malloc(sizeof(double) * I);
      double *u2 = (double *)malloc(sizeof(double) * r2);
      double *u1 = (double *)malloc(sizeof(double) * r1);
#pragma omp for schedule(dynamic, 1)
      for (int64_t q = 0; q < nr; ++q) {
        int64_t f = rows[q];
        int64_t t = f / k;
        double *x = Sx + q * H, *z1 = Sz1 + q * r1, *dz1 = Sdz1 + q * r1;
        double *dgu = Sdgu + q * 2 * I, *hh = Shh + q * I, *z2 = Sz2 + q * r2;
        double *dz2 = Sdz2 + q * r2, *dO = Sdo + q * H;
        for (int h = 0; h < H; ++h) x[h] = bf16_to_double(L->x[t * H + h]);
        row_forward(L, &V, x, z1, gu, hh, z2, o);
        double w = (double)L->topw[f];
        const uint16_t *dyt = dy + t * (int64_t)H;
        /* d topk weight and the gradient into the expert output */
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += bf16_to_double(dyt[h]) * o[h];
        if (dw) dw[f] = acc;
        for (int h = 0; h < H; ++h) dO[h] = w * bf16_to_double(dyt[h]);
        /* down: u2 = B2^T dO, dz2 = s2 u2, dh = W2^T dO + A2^T dz2 */
        for (int j = 0; j < r2; ++j) u2[j] = 0.0;
        for (int j = 0; j < R2 && lora2; ++j) {
          double a = 0.0;
          for (int n = 0; n < H; ++n) a += bf16_to_double(V.B2[(int64_t)n * R2 + j]) * dO[n];
          u2[j] = a;
          dz2[j] = L->s2 * a;
        }
        for (int i = 0; i < I; ++i) dhh[i] = 0.0;
        for (int n = 0; n < H; ++n) {
          const float *wr = W2 + (int64_t)n * I;
          double g = dO[n];
          for (int i = 0; i < I; ++i) dhh[i] += (double)wr[i] * g;
        }
        for (int j = 0; j < R2 && lora2; ++j)
          for (int i = 0; i < I; ++i) dhh[i] += bf16_to_double(V.A2[(int64_t)j * I + i]) * dz2[j];
        /* activation backward */
        for (int i = 0; i < I; ++i) {
          if (L->act == 1) {
            double dg, du;
            (void)cglu(L, gu[2 * i], gu[2 * i + 1], &dg, &du);
            dgu[2 * i] = dhh[i] * dg;
            dgu[2 * i + 1] = dhh[i] * du;
          } else {
            double g = gu[i], u = gu[I + i], sg = sigm(g);
            dgu[i] = dhh[i] * u * sg * (1.0 + g * (1.0 - sg));
            dgu[I + i] = dhh[i] * silu(g);
          }
        }
        /* gate_up: u1 = B1^T dgu, dz1 = s1 u1, dx_row = W1^T dgu + A1^T dz1 */
        for (int j = 0; j < R1 && lora1; ++j) {
          double a = 0.0;
          for (int n = 0; n < 2 * I; ++n) a += bf16_to_double(V.B1[(int64_t)n * R1 + j]) * dgu[n];
          u1[j] = a;
          dz1[j] = L->s1 * a;
        }
        double *dxr = dxp + f * (int64_t)H;
        for (int h = 0; h < H; ++h) dxr[h] = 0.0;
        for (int n = 0; n < 2 * I; ++n) {
          const float *wr = W1 + (int64_t)n * H;
          double g = dgu[n];
          for (int h = 0; h < H; ++h) dxr[h] += (double)wr[h] * g;
        }
        for (int j = 0; j < R1 && lora1; ++j)
          for (int h = 0; h < H; ++h) dxr[h] += bf16_to_double(V.A1[(int64_t)j * H + h]) * dz1[j];
      }
      free(gu); free(o); free(dhh); free(u2); free(u1);
    }
    /* weight gradients: reductions over this expert's rows, ascending */
    if (lora1 && dB1) {
      double *D = dB1 + (int64_t)e * 2 * I * R1;
#pragma omp parallel for schedule(static)
      for (int n = 0; n < 2 * I; ++n)
        for (int64_t q = 0; q < nr; ++q)
          for (int j = 0; j < R1; ++j) D[(int64_t)n * R1 + j] += L->s1 * Sdgu[q * 2 * I + n] * Sz1[q * r1 + j];
    }
    if (lora1 && dA1) {
      double *D = dA1 + (int64_t)e * R1 * H;
#pragma omp parallel for schedule(static)
      for (int h = 0; h < H; ++h)
        for (int64_t q = 0; q < nr; ++q)
          for (int j = 0; j < R1; ++j) D[(int64_t)j * H + h] += Sdz1[q * r1 + j] * Sx[q * H + h];
    }
    if (lora2 && dB2) {
      double *D = dB2 + (int64_t)e * H * R2;
#pragma omp parallel for schedule(static)
      for (int n = 0; n < H; ++n)
        for (int64_t q = 0; q < nr; ++q)
          for (int j = 0; j < R2; ++j) D[(int64_t)n * R2 + j] += L->s2 * Sdo[q * H + n] * Sz2[q * r2 + j];
    }
    if (lora2 && dA2) {
      double *D = dA2 + (int64_t)e * R2 * I;
#pragma omp parallel for schedule(static)
      for (int i = 0; i < I; ++i)
        for (int64_t q = 0; q < nr; ++q)
          for (int j = 0; j < R2; ++j) D[(int64_t)j * I + i] += Sdz2[q * r2 + j] * Shh[q * I + i];
    }
    free(Sx); free(Sz1); free(Sdz1); free(Sdgu); free(Shh); free(Sz2); free(Sdz2); free(Sdo);
  }
  /* dx[t] = sum_j dx_row[t,j], j ascending */
  for (int t = 0; t < T; ++t) {
    double *d = dx + (int64_t)t * H;
    for (int h = 0; h < H; ++h) d[h] = 0.0;
    if (tok_mask && !tok_mask[t]) continue;
    for (int j = 0; j < k; ++j) {
      int64_t f = (int64_t)t * k + j;
      int e = L->ids[f];
      if (e < 0 || e >= E) continue;
      const double *s = dxp + f * (int64_t)H;
      for (int h = 0; h < H; ++h) d[h] += s[h];
    }
  }
  free(dxp); free(rows); free(buf1); free(buf2);
  return 0;
}
