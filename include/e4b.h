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

/* Storage formats of a frozen stack.
 *  NF4:    16-value NormalFloat code (QLoRA table), blocks of 64 consecutive
 *          elements along K with one fp32 absmax; element 2j in the HIGH nibble of
 *          byte j.  w = fp32(nf4[q]) * absmax.
 *  NF4_DQ: NF4 whose absmax is itself 8-bit: absmax = fp32(c / 255) * scale2[b / 256]
 *          with b the flat block index over the whole stack.
 *  MXFP4:  FP4 E2M1 elements (element 2j in the LOW nibble) with one E8M0 scale byte
 *          per 32 consecutive elements along K: w = e2m1[q] * 2^(X - 127).
 *  INT8:   one signed byte per element, blocks of 64 along K with an fp32 scale:
 *          w = fp32(q) * scale (the library's quantiser: scale = absmax / 127).
 *  FP8:    one OCP FP8 E4M3 byte per element (finite, largest 448), blocks of 64 along K
 *          with an fp32 scale: w = fp32(e4m3(q)) * scale (quantiser: scale = absmax / 448).
 * The 8-bit formats are the int8 / fp8 storage modes of the fused-stack base (README,
 * opening section); their GEMMs run on the large tiles at every batch size. */
typedef enum {
  E4B_FMT_NF4 = 0,
  E4B_FMT_NF4_DQ = 1,
  E4B_FMT_MXFP4 = 2,
  E4B_FMT_INT8 = 3,
  E4B_FMT_FP8 = 4
} e4b_fmt;

/* A frozen stack [E, N, K] (K contiguous) in one of the formats above: the packed codes
 * plus per-block scales that the method page ("The abstraction that fails, and what
 * replaces it") names as the frozen packed base.  All pointers are device pointers owned
 * by the caller.
 *  codes   : uint8 [E, N, K/2] (4-bit formats) or [E, N, K] (INT8, FP8)
 *  scale   : NF4, INT8, FP8: float [E, N, K/64]; NF4_DQ: uint8 [E, N, K/64];
 *            MXFP4: uint8 [E, N, K/32]
 *  scale2  : NF4_DQ only: float [ceil(E*N*K/64 / 256)]; NULL otherwise.
 *  dq_table: NF4_DQ only: float [256], the value of each 8-bit absmax code:
 *            absmax = fp32(dq_table[c] * scale2[b / 256]).  NULL = the built-in linear
 *            code fp32(c / 255).  Must be NULL for the other formats.
 *  codebook: NF4 and NF4_DQ: float [16], the value of each 4-bit code,
 *            w = bf16(fp32(codebook[q] * absmax)).  NULL = the built-in NormalFloat
 *            table.  Must be NULL for the other formats (their code values are fixed).
 * A non-NULL table for a format that has none is E4B_ERR_INVALID_ARG. */
typedef struct {
  int32_t fmt;
  int32_t E, N, K;
  const uint8_t *codes;
  const void *scale;
  const float *scale2;
  const float *dq_table;
  const float *codebook;
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
/* The 4-bit GEMMs decode the packed stacks inside the GEMM tiles (README, "The package
 * family"), in the forward and again in the dgrad, so no dequantised copy of the base is
 * held between the calls (method page, "Why it happens").  E4B_EXPAND asks a forward with
 * more than 256 routed rows to first write bf16 copies of both stacks into the workspace
 * (2 bytes per weight; workspace_size grows accordingly) and stream those instead; the
 * results are bit-identical, and the dgrad still decodes the packed stacks. */
#define E4B_EXPAND 2u
/* An inference forward of at most 256 routed rows (decode) runs as two launches (project
 * record, "entry_points": the captured decode step): the gate_up launch routes the ids in
 * each workgroup, forms z1 = s1 A1 x for its own rows and the partial sums of z2 over its h
 * columns; the down launch adds those partial sums and its last workgroup over each column
 * range forms y there.  This applies with E <= 256 and adapter ranks <= 32 and for the 4-bit
 * formats; E4B_SEPARATE runs the same forward as six launches instead (route, LoRA-A,
 * gate_up, LoRA-A, down, combine).  Both agree to rounding (z1 is summed in another order). */
#define E4B_SEPARATE 4u

/* Expert activation between the two projections.
 *  E4B_ACT_SWIGLU: the stock epilogue act(gate) * up with SiLU (method page, "Limitations":
 *    the stock-epilogue contract); gate = rows [0, I) of gate_up, up = rows [I, 2I).
 *  E4B_ACT_CLAMPED_GLU: the clamped GLU of gpt-oss's MXFP4 experts (README, "Scope": per-expert
 *    biases and a clamped GLU; project record, "limitations"): gate = row 2i and up = row
 *    2i+1 of gate_up (interleaved); G = W1 x + b_gu + s1 B1 A1 x; g' = min(gate, limit),
 *    u' = clamp(up, -limit, limit), h = (u' + 1) * g' * sigmoid(alpha * g');
 *    O = W2 h + s2 B2 A2 h + b_dn.  The clamps pass gradient inside the closed interval.
 *    b_gu bf16 [E, 2I] (stored row order) and b_dn bf16 [E, H] are frozen device tensors,
 *    either may be NULL.  alpha and limit must be finite, limit > 0. */
#define E4B_ACT_SWIGLU 0
#define E4B_ACT_CLAMPED_GLU 1
typedef struct {
  int32_t kind;
  float alpha, limit;
  const uint16_t *b_gu;
  const uint16_t *b_dn;
} e4b_act;

/* One layer call: E experts, hidden H, intermediate I, T tokens, topk experts per token,
 * E4B_* flags, and the activation (act == NULL: E4B_ACT_SWIGLU, no biases; a host pointer). */
typedef struct {
  int32_t E, H, I, T, topk;
  uint32_t flags;
  const e4b_act *act;
} e4b_moe_desc;

int32_t e4b_version(void);
const char *e4b_status_str(int32_t status);

/* Bytes of caller-owned device workspace that e4b_moe_fwd / e4b_moe_dgrad /
 * e4b_lora_wgrad need for this layer (adapters may be NULL).  Host call, no device work;
 * bad shapes or adapters give E4B_ERR_INVALID_ARG and leave *bytes untouched.  With
 * E4B_TRAIN it includes 64 MiB + 8 KiB of partial tiles and arrival counters for the K-split
 * of the last round of the large down and input-gradient GEMMs (the training forward zeroes
 * the counters; every call leaves them zero).  Calls on one workspace must be ordered on
 * one stream.  (The workspace is this library's own contract: the pages leave memory
 * management to the caller's framework.) */
e4b_status e4b_moe_workspace_size(const e4b_moe_desc *desc, const e4b_lora *l_gu,
                                  const e4b_lora *l_dn, size_t *bytes);

/* Forward (method page, "The abstraction that fails, and what replaces it": each routed
 * expert's frozen packed projection plus its own low-rank delta, added before the
 * activation, act(W_e x + B[e] A[e] x); "Why it happens": the trainable term is
 * scaling * (x A[e]^T) B[e]^T; README, "The package family": one grouped launch over the
 * 4-bit-packed stacks with in-register decode and fp32 accumulation).
 *  w_gu: gate_up stack [E, 2I, H]; w_dn: down stack [E, H, I] (same fmt).
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

/* Allocation-free forward, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The same forward as
 * e4b_moe_fwd, inference only (desc->flags must be 0), with its workspace taken from one
 * device-resident scratch array of E4B_NOALLOC_SCRATCH_BYTES per GPU (held from the first
 * call on a device until the process ends) instead of a caller buffer.  Layers whose
 * e4b_moe_workspace_size exceeds it get E4B_ERR_WORKSPACE before any launch.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (different streams, or other
 * threads) race; calls ordered on one stream do not.  Nothing in the array needs to start at
 * zero.  The call itself allocates nothing (event timing is skipped for it). */
#define E4B_NOALLOC_SCRATCH_BYTES (64u << 20)
e4b_status e4b_moe_fwd_noalloc(const e4b_moe_desc *desc, const e4b_qweight *w_gu,
                               const e4b_qweight *w_dn, const e4b_lora *l_gu, const e4b_lora *l_dn,
                               const uint16_t *x, const int32_t *ids, const float *topw, uint16_t *y,
                               void *stream);

/* Input gradient after a training forward with the same arguments (method page, "The
 * abstraction that fails, and what replaces it": the grouped forward with optional dgrad;
 * "Why it happens": the base projection is dequantised again in the backward, so nothing
 * dequantised is held between the calls).  Needs E4B_TRAIN in desc->flags and the
 * forward's workspace (else E4B_ERR_INVALID_ARG / E4B_ERR_WORKSPACE, nothing enqueued).
 *  dy bf16 [T, H] -> dx bf16 [T, H] (overwritten); d_topw fp32 [T, topk]
 *  (nullable; d(sum dy*y)/d topw).  Writes the dgrad activations that
 *  e4b_lora_wgrad reads into ws. */
e4b_status e4b_moe_dgrad(const e4b_moe_desc *desc, const e4b_qweight *w_gu,
                         const e4b_qweight *w_dn, const e4b_lora *l_gu, const e4b_lora *l_dn,
                         const int32_t *ids, const float *topw, const uint16_t *dy,
                         uint16_t *dx, float *d_topw, void *ws, size_t ws_bytes, void *stream);

/* Gradients of the trainable per-expert adapters (method page, "The abstraction that
 * fails, and what replaces it": A[e] / B[e] trainable, the packed base frozen), after
 * e4b_moe_dgrad on the same workspace; overwritten, fp32, device:
 *  dA_gu [E, r1, H], dB_gu [E, 2I, r1], dA_dn [E, r2, I], dB_dn [E, H, r2].
 *  Experts that received no rows get zeros.  x is the forward's input. */
e4b_status e4b_lora_wgrad(const e4b_moe_desc *desc, const e4b_lora *l_gu, const e4b_lora *l_dn,
                          const uint16_t *x, void *ws, size_t ws_bytes, float *dA_gu,
                          float *dB_gu, float *dA_dn, float *dB_dn, void *stream);

/* Routing metadata, the grouping that lets one launch serve every expert's rows (README,
 * "The package family": one launch over the expert stacks; method page, "Why it
 * happens": the delta is applied per routed expert).  Stable grouping of the T*topk routed
 * rows by expert, device outputs, overwritten:
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

/* Dequantise (method page, "The abstraction that fails, and what replaces it": the packed
 * expert base, NF4 by default; README, opening section: the storage modes of the base):
 * expert `expert` of a stack (or the whole stack if expert < 0) to fp32 and/or bf16
 * [N, K] row-major, device, overwritten (either output nullable).  The values are those
 * the GEMM tiles use.  An expert index >= E, no output or a malformed stack:
 * E4B_ERR_INVALID_ARG (an unknown format: E4B_ERR_UNSUPPORTED), nothing enqueued. */
e4b_status e4b_dequant(const e4b_qweight *w, int32_t expert, float *out_f32,
                       uint16_t *out_bf16, void *stream);

/* Quantise (README, opening section: NF4 / FP4 / int8 / fp8 storage of the frozen base;
 * method page, "The abstraction that fails, and what replaces it": quant_type chooses it
 * at load) an fp32 stack w [E, N, K] (device) into codes / scale / scale2 laid out as in
 * e4b_qweight (device, caller-allocated, overwritten): nearest code, ties to the lower NF4
 * index / the even E2M1 code; INT8 and FP8 round to nearest even.  An unknown format is
 * E4B_ERR_UNSUPPORTED. */
e4b_status e4b_quantize(int32_t fmt, int32_t E, int32_t N, int32_t K, const float *w,
                        uint8_t *codes, void *scale, float *scale2, void *stream);

/* Synchronises `stream` and returns the number of routed rows that the last
 * forward on this workspace dropped for an out-of-range expert id.  (A diagnostic of this
 * library, no passage of the pages; the routed rows themselves are defined above.) */
e4b_status e4b_moe_check(const e4b_moe_desc *desc, const void *ws, void *stream,
                         int32_t *dropped_rows);

/* Observability: kernel launches since the last reset, per kernel family (this library's
 * own; README, "What is measured", is what its figures are compared with). */
typedef struct {
  int64_t launches_total;
  int64_t route, lora_a, gemm_gate_up, gemm_down, combine;
  int64_t combine_bwd, gemm_down_dgrad, gemm_gate_up_dgrad, unpermute, wgrad, quant, dequant;
  int64_t expand;    /* bf16 copies of stacks written by large-batch calls */
  int64_t router;    /* e4b_router_topk and e4b_router_bwd launches */
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
