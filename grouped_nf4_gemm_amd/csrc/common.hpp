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

enum Fmt : int { FMT_NF4 = 0, FMT_NF4_DQ = 1, FMT_MXFP4 = 2 };

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

// Logistic sigmoid 1 / (1 + e^-x) from the hardware base-2 exponential and reciprocal
// (each within about one ulp); saturates to 0 and 1 for large |x|.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
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

// Per-workgroup decode tables in LDS.
//  cb2[b]  = {nf4[b >> 4], nf4[b & 15]}: the two NF4 values of code byte b, element 2j
//            (high nibble) first, so one 8-byte LDS read serves two codes.
//  tab8[c] = fp32(c / 255): the 8-bit absmax code of the double-quantised format.
struct DecodeTables {
  float2 cb2[256];
  float tab8[256];
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

// Register-resident decode table of one NF4 block: the sixteen values e[q] = bf16(nf4[q] *
// absmax) (the same rounding as nf4_scale_pack) split into byte planes, pl[i] = low bytes of
// e[4i .. 4i+3] and pl[4 + i] = their high bytes (i < 4), so that byte permutes can look up
// four codes at a time without touching LDS.
__device__ __forceinline__ void nf4_planes(float absmax, uint32_t (&pl)[8]) {
  constexpr float v[16] = E4B_NF4_VALUES;
  uint32_t e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = pack_bf16x2(v[2 * k] * absmax, v[2 * k + 1] * absmax);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pl[i] = __builtin_amdgcn_perm(e[2 * i + 1], e[2 * i], 0x06040200u);
    pl[4 + i] = __builtin_amdgcn_perm(e[2 * i + 1], e[2 * i], 0x07050301u);
  }
}
// The 8 codes of one 32-bit word (element 2j in the high nibble of byte j) to 8 bf16 values
// through the planes of nf4_planes.  v_perm_b32 picks byte s (0..7) of the pair {S0:S1}, so a
// code q reads entry q & 7 of planes 0-1 or of planes 2-3, chosen per byte by q >= 8.  For the
// choice, q + 0x78 has bit 7 set exactly when q >= 8, and the selectors 8..11 of v_perm_b32
// replicate bit 7 of bytes 1, 3, 5, 7 of the pair into a whole byte.
__device__ __forceinline__ u32x4 nf4_decode_planes(uint32_t w, const uint32_t (&pl)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 2j+1, codes 2j
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t q = __builtin_amdgcn_perm(lo, hi, p == 0 ? 0x05010400u : 0x07030602u);  // codes 4p..4p+3
    const uint32_t x = q + 0x78787878u;
    const uint32_t m = __builtin_amdgcn_perm(x, x << 8, 0x0B090A08u);  // 0xFF in bytes with q >= 8
    const uint32_t s = q & 0x07070707u;
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

// A frozen 4-bit stack as the kernels see it.
struct QStack {
  const uint8_t *codes;
  const void *scale;
  const float *scale2;
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
