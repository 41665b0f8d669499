/*
 * Test infrastructure only: the CPU oracle for the routed-expert MoE layer with
 * per-expert pre-activation LoRA over a frozen 4-bit fused expert stack.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or helper with the HIP
 * library; the product never calls it.
 *
 * Source pages: "How do I QLoRA-train the fused experts of a MoE" (solution
 * page, sections "The abstraction that fails, and what replaces it" and "Why it
 * happens"), and the experts4bit-qlora package README ("The package family").
 *
 * Precision: dequantised weights follow the fp32 contract exactly (one fp32
 * multiply of the code value by its block scale); every other quantity of the
 * layer (products, sums, activation, gradients) is computed in fp64 and
 * returned unrounded.
 */
#ifndef E4B_ORACLE_H
#define E4B_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FMT_NF4 = 0, ORC_FMT_NF4_DQ = 1, ORC_FMT_MXFP4 = 2, ORC_FMT_INT8 = 3, ORC_FMT_FP8 = 4 };

/* One 4-bit expert stack [E, N, K], K contiguous, as bytes + scales. */
typedef struct {
  int32_t fmt;
  int32_t E, N, K;
  const uint8_t *codes;   /* [E*N*K/2] (4-bit formats) or [E*N*K] (INT8, FP8) */
  const void *scale;      /* NF4, INT8, FP8: float[E*N*K/64]; NF4_DQ: uint8[E*N*K/64]; MXFP4: uint8[E*N*K/32] */
  const float *scale2;    /* NF4_DQ: float[ceil(E*N*K/64/256)]; else unused */
  const float *dq_table;  /* NF4_DQ: value of each 8-bit absmax code [256]; NULL = c/255 */
  const float *codebook;  /* NF4 formats: value of each 4-bit code [16]; NULL = NormalFloat */
} orc_qweight;

/* The layer: weights either packed (w_gu/w_dn) or dense fp32 (W1f/W2f, for
 * identities that need weights outside the 4-bit grid). */
typedef struct {
  int32_t E, H, I, T, k;
  const orc_qweight *w_gu;  /* gate_up_proj [E, 2I, H] */
  const orc_qweight *w_dn;  /* down_proj    [E, H, I]  */
  const float *W1f;         /* optional dense [E, 2I, H] (overrides w_gu) */
  const float *W2f;         /* optional dense [E, H, I]  (overrides w_dn) */
  const uint16_t *A1, *B1;  /* bf16 [E, r1, H], [E, 2I, r1]; A1 == NULL: no adapter */
  int32_t r1; double s1;
  const uint16_t *A2, *B2;  /* bf16 [E, r2, I], [E, H, r2]; A2 == NULL: no adapter */
  int32_t r2; double s2;
  const uint16_t *x;        /* bf16 [T, H] */
  const int32_t *ids;       /* [T, k] */
  const float *topw;        /* [T, k] */
  int32_t post_act_delta;   /* test hook: 1 = act(Wx) + delta instead of act(Wx + delta) */
  /* Expert activation.  0: stock act(gate) * up with gate rows [0, I), up rows [I, 2I).
   * 1: the clamped GLU of gpt-oss's experts: gate = row 2i, up = row 2i+1 (interleaved),
   *    g' = min(gate, limit), u' = clamp(up, -limit, limit), h = (u' + 1) * g' * sigmoid(alpha g'),
   *    with per-expert biases b1 [E, 2I] (added before the activation, with the LoRA delta)
   *    and b2 [E, H] (added to the down projection); bf16, either may be NULL. */
  int32_t act;
  double alpha, limit;
  const uint16_t *b1, *b2;
} orc_layer;

int32_t orc_version(void);
void orc_nf4_codebook(float out[16]);
void orc_bf16_round(const float *in, uint16_t *out, int64_t n);

void orc_quant_nf4(const float *w, int64_t n, uint8_t *codes, float *absmax);
void orc_quant_nf4_dq(const float *w, int64_t n, uint8_t *codes, uint8_t *qabsmax, float *scale2);
void orc_quant_mxfp4(const float *w, int64_t n, uint8_t *codes, uint8_t *scales);
/* 8-bit bases, blocks of 64 along K with an fp32 scale: INT8 q = rne(w / s) in [-127, 127],
 * s = absmax / 127; FP8 E4M3 (OCP, finite, max 448) q = rne(w / s) with s = absmax / 448. */
void orc_quant_int8(const float *w, int64_t n, uint8_t *codes, float *scales);
void orc_quant_fp8(const float *w, int64_t n, uint8_t *codes, float *scales);
float orc_e4m3_value(uint8_t code);
/* Dequantise n elements (flat) to fp32 and/or bf16 (either pointer may be NULL).
 * dq_table / codebook: the stack's own code tables (NULL = the built-in ones). */
void orc_dequant(int32_t fmt, int64_t n, const uint8_t *codes, const void *scale,
                 const float *scale2, const float *dq_table, const float *codebook,
                 float *out_f32, uint16_t *out_bf16);

void orc_route(int32_t T, int32_t k, int32_t E, const int32_t *ids,
               int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv);
/* Router: top-k ids (larger logit first, ties to the lower id) and the softmax over them;
   its gradient with respect to the logits, the chosen ids held fixed. */
void orc_router_topk(int32_t T, int32_t E, int32_t k, const float *logits, int32_t *ids, float *w);
void orc_router_bwd(int32_t T, int32_t E, int32_t k, const float *w, const float *dw, const int32_t *ids,
                    float *dlogits);

/* Forward.  tok_mask[T] (NULL = all tokens) selects the tokens whose rows are
 * computed.  y: fp64 [T, H] (unselected tokens get 0).  O (nullable): fp64
 * per-routed-row expert outputs [T*k, H] in flat (t*k+j) order. Returns 0. */
int32_t orc_moe_fwd(const orc_layer *L, const uint8_t *tok_mask, double *y, double *O);

/* Backward of sum(dy * y) with the routing held fixed.  dy: bf16 [T, H]; only
 * masked tokens contribute.  Outputs (any nullable except dx): dx [T, H],
 * dw [T, k], dA1 [E, r1, H], dB1 [E, 2I, r1], dA2 [E, r2, I], dB2 [E, H, r2]. */
int32_t orc_moe_bwd(const orc_layer *L, const uint8_t *tok_mask, const uint16_t *dy,
                    double *dx, double *dw, double *dA1, double *dB1, double *dA2, double *dB2);

#ifdef __cplusplus
}
#endif
#endif
