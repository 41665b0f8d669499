// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA fragment
// types, and the 4-bit decode rules of the three frozen-stack formats.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e4b {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Fmt : int { FMT_NF4 = 0, FMT_NF4_DQ = 1, FMT_MXFP4 = 2, FMT_INT8 = 3, FMT_FP8 = 4 };
// One byte per element (INT8, FP8 E4M3) rather than a 4-bit code.
constexpr bool fmt_8bit(int fmt) { return fmt == FMT_INT8 || fmt == FMT_FP8; }

// NormalFloat-4 code values (QLoRA), index 0..15.
#define E4B_NF4_VALUES                                                                    \
  {-1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,              \
   -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,              \
   0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f, 0.33791524171829224f, \
   0.44070982933044434f, 0.5626170039176941f, 0.7229568362236023f, 1.0f}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// nf4[q] without a memory access (a select chain over the literal values), for building
// the per-workgroup LDS tables at kernel start without a global-memory round trip.
__device__ __forceinline__ float nf4_value(uint32_t q) {
  constexpr float v[16] = E4B_NF4_VALUES;
  float r = v[15];
#pragma unroll
  for (int i = 14; i >= 0; --i) r = q == (uint32_t)i ? v[i] : r;
  return r;
}
// Code value q of a stack: its own table, or the built-in one.
__device__ __forceinline__ float code_value(const float *codebook, uint32_t q) {
  return codebook ? codebook[q] : nf4_value(q);
}
// Absmax code c of a double-quantised stack: its own table, or the built-in fp32(c / 255).
__device__ __forceinline__ float dq_value(const float *dq_table, uint32_t c) {
  return dq_table ? dq_table[c] : (float)c / 255.0f;
}

// Logistic sigmoid 1 / (1 + e^-x) from the hardware base-2 exponential and reciprocal
// (each within about one ulp); saturates to 0 and 1 for large |x|.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// Weight row of h column c in the gate_up stack: the gate (up = false) or up row.  Stock
// layout: gate rows [0, I), up rows [I, 2I); interleaved (clamped GLU): rows 2c and 2c + 1.
__device__ __forceinline__ int gate_up_row(int c, bool up, bool interleaved, int I) {
  return interleaved ? 2 * c + (up ? 1 : 0) : (up ? I : 0) + c;
}

// Clamped GLU (gpt-oss experts): h = (u' + 1) * g' * sigmoid(alpha g'), g' = min(g, limit),
// u' = clamp(u, -limit, limit); its partial derivatives pass through the clamps inside the
// closed interval.
__device__ __forceinline__ float glu_clamped(float g, float u, float alpha, float limit) {
  const float gc = fminf(g, limit), uc = fminf(fmaxf(u, -limit), limit);
  return (uc + 1.0f) * gc * sigmoid_fast(alpha * gc);
}
__device__ __forceinline__ void glu_clamped_bwd(float g, float u, float alpha, float limit, float dh, float &dg,
                                                float &du) {
  const float gc = fminf(g, limit), uc = fminf(fmaxf(u, -limit), limit);
  const float sg = sigmoid_fast(alpha * gc);
  dg = g <= limit ? dh * (uc + 1.0f) * (sg + alpha * gc * sg * (1.0f - sg)) : 0.0f;
  du = (u >= -limit && u <= limit) ? dh * gc * sg : 0.0f;
}

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// E8M0 scale byte -> fp32 2^(X-127) (X = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t X) {
  return X == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(X << 23);
}

// Per-workgroup decode tables in LDS, filled from the stack's own tables (or the built-in
// ones when it passes none).
//  cb2[b]  = {nf4[b >> 4], nf4[b & 15]}: the two code values of code byte b, element 2j
//            (high nibble) first, so one 8-byte LDS read serves two codes.
//  tab8[c] = the 8-bit absmax code table of the double-quantised format (built-in:
//            fp32(c / 255)).
//  cb[q]   = the sixteen code values, read by the register (byte-plane) decode.
struct DecodeTables {
  float2 cb2[256];
  float tab8[256];
  float cb[16];
};

// The NF4 values of the 8 codes of one 32-bit word (bytes in memory order; element 2j in
// the high nibble of byte j).
__device__ __forceinline__ void nf4_lookup(uint32_t w, const DecodeTables &t, float (&v)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float2 x = t.cb2[(w >> (8 * b)) & 0xffu];
    v[2 * b] = x.x;
    v[2 * b + 1] = x.y;
  }
}
// w = bf16(fp32(nf4[q]) * absmax), packed in pairs.
__device__ __forceinline__ u32x4 nf4_scale_pack(const float (&v)[8], float absmax) {
  u32x4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) r[b] = pack_bf16x2(v[2 * b] * absmax, v[2 * b + 1] * absmax);
  return r;
}
// Decode the 8 NF4 codes of one 32-bit word to 8 bf16 values.
__device__ __forceinline__ u32x4 nf4_word_to_bf16(uint32_t w, float absmax, const DecodeTables &t) {
  float v[8];
  nf4_lookup(w, t, v);
  return nf4_scale_pack(v, absmax);
}

// Register-resident decode table of one NF4 block: the sixteen values e[q] = bf16(v[q] *
// absmax) (the same rounding as nf4_scale_pack) split into byte planes, so that byte permutes
// can look up four codes at a time without touching LDS.  Codes q < 8 form table A, q >= 8
// table B; code q sits at position (q + 5) & 7 of its table (the position the decode below
// reads).  pl[0..1]: low bytes of table A (positions 0-3, 4-7), pl[2..3]: low bytes of
// table B, pl[4..7]: the high bytes likewise.  v: the code values of the stack.
__device__ __forceinline__ void nf4_planes(float absmax, const float *v, uint32_t (&pl)[8]) {
  // the code at table position t: (t + 3) & 7 in table A, 8 + ((t + 3) & 7) in table B
  auto code_at = [](int t) { return (t & 8) | ((t + 3) & 7); };
  uint32_t e[8];  // e[k]: positions 2k, 2k + 1 (of A for k < 4, of B for k >= 4)
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = pack_bf16x2(v[code_at(2 * k)] * absmax, v[code_at(2 * k + 1)] * absmax);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pl[i] = __builtin_amdgcn_perm(e[2 * i + 1], e[2 * i], 0x06040200u);
    pl[4 + i] = __builtin_amdgcn_perm(e[2 * i + 1], e[2 * i], 0x07050301u);
  }
}
// The 8 codes of one 32-bit word (element 2j in the high nibble of byte j) to 8 bf16 values
// through the planes of nf4_planes.  v_perm_b32 picks byte s (0..7) of the pair {S0:S1}; for
// selector values 8-11 it replicates a sign bit, for 12 it gives 0x00 and for 13 and up 0xFF.
// With x = q + 5 per byte: x & 7 is the code's table position, and perm(0, 0, x) is 0xFF
// exactly where q >= 8 (x = 13..20; x = 5..12 gives 0x00 from zero bytes, zero sign bits and
// the constant 12), the mask that picks table B.
__device__ __forceinline__ u32x4 nf4_decode_planes(uint32_t w, const uint32_t (&pl)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 2j+1, codes 2j
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t q = __builtin_amdgcn_perm(lo, hi, p == 0 ? 0x05010400u : 0x07030602u);  // codes 4p..4p+3
    const uint32_t x = q + 0x05050505u;
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, x);  // 0xFF in bytes with q >= 8
    const uint32_t s = x & 0x07070707u;
    const uint32_t L = (__builtin_amdgcn_perm(pl[3], pl[2], s) & m) | (__builtin_amdgcn_perm(pl[1], pl[0], s) & ~m);
    const uint32_t H = (__builtin_amdgcn_perm(pl[7], pl[6], s) & m) | (__builtin_amdgcn_perm(pl[5], pl[4], s) & ~m);
    out[2 * p] = __builtin_amdgcn_perm(H, L, 0x05010400u);
    out[2 * p + 1] = __builtin_amdgcn_perm(H, L, 0x07030602u);
  }
  return out;
}

// Decode the 8 E2M1 codes of one 32-bit word (element 2j in the low nibble of
// byte j) times 2^(X-127) to 8 bf16 values (exact).
__device__ __forceinline__ u32x4 mxfp4_word_to_bf16(uint32_t w, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

// The 4 elements of one 32-bit word of an 8-bit stack (element 4j + b in byte b) times the
// block scale, as 4 bf16 values: bf16(fp32(code) * scale).
//  INT8: (byte ^ 0x80) read unsigned is q + 128, and fma(u, s, -128 s) rounds (u - 128) s
//        exactly once (-128 s is exact), which is the fp32 product q * s.
//  FP8 (OCP E4M3): the hardware conversion of two codes to fp32 (exact), then the product.
template <int FMT>
__device__ __forceinline__ u32x2 byte_word_to_bf16(uint32_t w, float sc) {
  float f[4];
  if constexpr (FMT == FMT_INT8) {
    const uint32_t x = w ^ 0x80808080u;
    const float nb = -128.0f * sc;
#pragma unroll
    for (int b = 0; b < 4; ++b) f[b] = __builtin_fmaf((float)((x >> (8 * b)) & 0xffu), sc, nb);
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0] * sc;
    f[1] = lo[1] * sc;
    f[2] = hi[0] * sc;
    f[3] = hi[1] * sc;
  }
  return u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
}

// A frozen stack (4-bit or 8-bit codes) as the kernels see it.
struct QStack {
  const uint8_t *codes;
  const void *scale;
  const float *scale2;
  const float *codebook;  // NF4 formats: 16 code values (nullptr: the built-in NormalFloat table)
  const float *dq_table;  // NF4_DQ: 256 absmax code values (nullptr: the built-in c / 255)
  int fmt;
  int N, K;  // per-expert matrix [N, K], K contiguous
  uint32_t codes_bytes, scale_bytes, scale2_bytes;  // extents (buffer range checks)
};

// Block scale for NF4 / NF4_DQ element block `b` (flat over the whole stack).
__device__ __forceinline__ float nf4_block_absmax(const QStack &q, int64_t b, const DecodeTables &t) {
  if (q.fmt == FMT_NF4) return ((const float *)q.scale)[b];
  return t.tab8[((const uint8_t *)q.scale)[b]] * q.scale2[b >> 8];
}

}  // namespace e4b
