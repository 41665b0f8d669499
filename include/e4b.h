/*
 * libe4b -- routed-expert MoE layer over a frozen 4-bit fused expert stack with a
 * trainable per-expert LoRA delta before the activation, on AMD Instinct MI355X
 * (gfx950).  Plain C ABI: host or device pointers and sizes only.
 *
 * The operation (solution page "How do I QLoRA-train the fused experts of a MoE",
 * section "The abstraction that fails, and what replaces it", and section "Why it
 * happens"):  for token t and each routed expert e = ids[t,j] with weight w[t,j],
 *     z1 = A1[e] x_t                       (LoRA A of gate_up, [r, H])
 *     G  = W1[e] x_t + s1 * B1[e] z1       (gate_up_proj [2I, H], B1 [2I, r])
 *     h  = silu(G[0:I]) * G[I:2I]          (stock epilogue act(gate) * up)
 *     z2 = A2[e] h ;  O = W2[e] h + s2 * B2[e] z2   (down_proj [H, I])
 *     y_t = sum_j w[t,j] * O_{t,j}
 * W1/W2 are frozen 4-bit stacks decoded in-kernel (README of the runtime package,
 * "The package family": one launch over 4-bit-packed expert stacks, in-register
 * decode, fp32 accumulation).  The backward re-decodes the packed base (solution
 * page, "Why it happens") and gives dx (the input gradient, with the router
 * weights held fixed), optionally d w[t,j], and the LoRA gradients dA/dB.
 *
 * Conventions used by every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - Device pointers unless stated otherwise.  The caller owns all memory; the
 *    library never allocates device memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues
 *    work and returns; nothing synchronises except e4b_moe_check.
 *  - Invalid arguments are rejected on the host before anything is enqueued
 *    (status != E4B_OK, no kernel launched).  E4B_ERR_HIP reports a failed launch.
 *  - Shapes: H % 64 == 0, I % 64 == 0, 1 <= topk <= E <= 1024, T >= 0,
 *    LoRA rank r % 8 == 0 and 8 <= r <= 128 (or no adapter: A == NULL).
 */
#ifndef E4B_H
#define E4B_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  E4B_OK = 0,
  E4B_ERR_INVALID_ARG = 1,
  E4B_ERR_UNSUPPORTED = 2,
  E4B_ERR_WORKSPACE = 3,
  E4B_ERR_HIP = 4
} e4b_status;

/* 4-bit storage formats of a frozen stack.
 *  NF4:    16-value NormalFloat code (QLoRA table), blocks of 64 consecutive
 *          elements along K with one fp32 absmax; element 2j in the HIGH nibble of
 *          byte j.  w = fp32(nf4[q]) * absmax.
 *  NF4_DQ: NF4 whose absmax is itself 8-bit: absmax = fp32(c / 255) * scale2[b / 256]
 *          with b the flat block index over the whole stack.
 *  MXFP4:  FP4 E2M1 elements (element 2j in the LOW nibble) with one E8M0 scale byte
 *          per 32 consecutive elements along K: w = e2m1[q] * 2^(X - 127). */
typedef enum { E4B_FMT_NF4 = 0, E4B_FMT_NF4_DQ = 1, E4B_FMT_MXFP4 = 2 } e4b_fmt;

/* A frozen stack [E, N, K] (K contiguous) in one of the formats above.
 *  codes : uint8 [E, N, K/2]
 *  scale : NF4: float [E, N, K/64]; NF4_DQ: uint8 [E, N, K/64]; MXFP4: uint8 [E, N, K/32]
 *  scale2: NF4_DQ only: float [ceil(E*N*K/64 / 256)]; NULL otherwise. */
typedef struct {
  int32_t fmt;
  int32_t E, N, K;
  const uint8_t *codes;
  const void *scale;
  const float *scale2;
} e4b_qweight;

/* Stacked per-expert adapter of one projection [E, N, K]:
 *  A bf16 [E, r, K], B bf16 [E, N, r], delta = scaling * B[e] (A[e] v).
 *  A == NULL (and B == NULL) disables the adapter. */
typedef struct {
  const uint16_t *A;
  const uint16_t *B;
  int32_t r;
  float scaling;
} e4b_lora;

#define E4B_TRAIN 1u /* forward keeps what dgrad and wgrad read, in the workspace */
/* The 4-bit GEMMs of a call with more than 256 routed rows either decode the stacks
 * inside the GEMM tiles, once per 256-row tile, or -- by default when there are at
 * least 1024 routed rows per expert on average -- first write bf16 copies of both
 * stacks into the workspace (decoded by the same rules; 2 bytes per weight, kept from a
 * training forward for its dgrad) and stream those.  Results are bit-identical either
 * way.  These flags force the choice (not both; ignored at 256 rows or fewer). */
#define E4B_EXPAND 2u
#define E4B_NO_EXPAND 4u

typedef struct {
  int32_t E, H, I, T, topk;
  uint32_t flags;
} e4b_moe_desc;

int32_t e4b_version(void);
const char *e4b_status_str(int32_t status);

/* Bytes of caller-owned device workspace that e4b_moe_fwd / e4b_moe_dgrad /
 * e4b_lora_wgrad need for this layer (adapters may be NULL).  Host call. */
e4b_status e4b_moe_workspace_size(const e4b_moe_desc *desc, const e4b_lora *l_gu,
                                  const e4b_lora *l_dn, size_t *bytes);

/* Forward.  w_gu: gate_up stack [E, 2I, H]; w_dn: down stack [E, H, I] (same fmt).
 *  x bf16 [T, H]; ids int32 [T, topk]; topw fp32 [T, topk]; y bf16 [T, H] (written).
 *  ws: workspace of e4b_moe_workspace_size bytes.  With E4B_TRAIN the workspace
 *  then holds the routing and activations that dgrad and wgrad read: keep it and
 *  the inputs unchanged until those calls are enqueued on the same stream.
 *  Expert ids outside [0, E) are dropped rows (they add nothing to y); their count
 *  is reported by e4b_moe_check. */
e4b_status e4b_moe_fwd(const e4b_moe_desc *desc, const e4b_qweight *w_gu,
                       const e4b_qweight *w_dn, const e4b_lora *l_gu, const e4b_lora *l_dn,
                       const uint16_t *x, const int32_t *ids, const float *topw, uint16_t *y,
                       void *ws, size_t ws_bytes, void *stream);

/* Input gradient after a training forward with the same arguments.
 *  dy bf16 [T, H] -> dx bf16 [T, H] (overwritten); d_topw fp32 [T, topk]
 *  (nullable; d(sum dy*y)/d topw).  Writes the dgrad activations that
 *  e4b_lora_wgrad reads into ws. */
e4b_status e4b_moe_dgrad(const e4b_moe_desc *desc, const e4b_qweight *w_gu,
                         const e4b_qweight *w_dn, const e4b_lora *l_gu, const e4b_lora *l_dn,
                         const int32_t *ids, const float *topw, const uint16_t *dy,
                         uint16_t *dx, float *d_topw, void *ws, size_t ws_bytes, void *stream);

/* LoRA weight gradients after e4b_moe_dgrad, overwritten, fp32:
 *  dA_gu [E, r1, H], dB_gu [E, 2I, r1], dA_dn [E, r2, I], dB_dn [E, H, r2].
 *  Experts that received no rows get zeros.  x is the forward's input. */
e4b_status e4b_lora_wgrad(const e4b_moe_desc *desc, const e4b_lora *l_gu, const e4b_lora *l_dn,
                          const uint16_t *x, void *ws, size_t ws_bytes, float *dA_gu,
                          float *dB_gu, float *dA_dn, float *dB_dn, void *stream);

/* Routing metadata (stable grouping of the T*topk routed rows by expert):
 *  cnt int32 [E+1] (cnt[E] = rows with an id outside [0, E)); off int32 [E+1]
 *  (exclusive scan, off[E] = valid rows); perm int32 [T*topk] (sorted position ->
 *  flat index t*topk+j, ascending flat index within an expert, -1 past off[E]);
 *  inv int32 [T*topk] (flat index -> sorted position, -1 if dropped). */
e4b_status e4b_moe_route(const e4b_moe_desc *desc, const int32_t *ids, int32_t *cnt,
                         int32_t *off, int32_t *perm, int32_t *inv, void *stream);

/* Router (method page, "Which project solves it": the router is frozen and outside the
 * layer, whose inputs are the top-k ids and weights; this is that step on the device).
 *  logits fp32 [T, E] row-major (device); ids int32 [T, topk] and topw fp32 [T, topk]
 *  (device, written): per token the topk largest logits, larger first, equal logits in
 *  ascending expert id, and the softmax over them (fp32, max-subtracted).  Logits must be
 *  finite.  E <= E4B_ROUTER_MAX_E, 1 <= topk <= min(E, E4B_ROUTER_MAX_K); otherwise
 *  E4B_ERR_INVALID_ARG before any launch.  T = 0 launches nothing. */
#define E4B_ROUTER_MAX_E 1024
#define E4B_ROUTER_MAX_K 64
e4b_status e4b_router_topk(const float *logits, int32_t T, int32_t E, int32_t topk, int32_t *ids, float *topw,
                           void *stream);

/* Gradient of the router weights with respect to the logits, the chosen ids held fixed:
 * d_logits[t, ids[t, j]] = topw[t, j] (d_topw[t, j] - sum_i topw[t, i] d_topw[t, i]),
 * zero for the other experts.  topw, d_topw fp32 [T, topk], ids int32 [T, topk] (as
 * e4b_router_topk wrote them), d_logits fp32 [T, E] (written in full).  Limits and errors
 * as for e4b_router_topk. */
e4b_status e4b_router_bwd(const float *topw, const float *d_topw, const int32_t *ids, int32_t T, int32_t E,
                          int32_t topk, float *d_logits, void *stream);

/* Decode expert `expert` of a stack (or the whole stack if expert < 0) to fp32
 * and/or bf16 [N, K] row-major (either output nullable). */
e4b_status e4b_dequant(const e4b_qweight *w, int32_t expert, float *out_f32,
                       uint16_t *out_bf16, void *stream);

/* Quantise an fp32 stack w [E, N, K] into codes/scale/scale2 laid out as in
 * e4b_qweight (nearest code, ties to the lower NF4 index / the even E2M1 code). */
e4b_status e4b_quantize(int32_t fmt, int32_t E, int32_t N, int32_t K, const float *w,
                        uint8_t *codes, void *scale, float *scale2, void *stream);

/* Synchronises `stream` and returns the number of routed rows that the last
 * forward on this workspace dropped for an out-of-range expert id. */
e4b_status e4b_moe_check(const e4b_moe_desc *desc, const void *ws, void *stream,
                         int32_t *dropped_rows);

/* Observability: kernel launches since the last reset, per kernel family. */
typedef struct {
  int64_t launches_total;
  int64_t route, lora_a, gemm_gate_up, gemm_down, combine;
  int64_t combine_bwd, gemm_down_dgrad, gemm_gate_up_dgrad, unpermute, wgrad, quant, dequant;
  int64_t expand;    /* bf16 copies of stacks written by large-batch calls */
  int64_t fallbacks; /* always 0: there is no slower path to fall back to */
} e4b_stats;
e4b_status e4b_get_stats(e4b_stats *out);
void e4b_reset_stats(void);

/* Optional per-kernel timing with HIP events on the caller's stream.  While
 * enabled, every launch is bracketed by two events; e4b_timing_read synchronises
 * and returns, per kernel family name, the number of launches and the summed
 * milliseconds since the last read.  Host calls. */
e4b_status e4b_timing_enable(int32_t on);
e4b_status e4b_timing_read(int32_t max, char (*names)[32], int64_t *launches, double *ms,
                           int32_t *n_out);

#ifdef __cplusplus
}
#endif
#endif
