// nvfp4_device.h -- gfx950 device helpers for the NVFP4 kernels: bf16
// unpacking, E4M3 and E2M1 codecs, Philox4x32-10 and the 16-point Hadamard
// butterfly.  Every routine is IEEE binary32 with round-to-nearest-even; the
// kernels are built with -ffp-contract=off so no multiply-add is fused.
//
// Sources (web pages, cited by title and section):
//  [PAPER] "Pretraining Large Language Models with NVFP4", summary page:
//          format paragraph (E2M1 elements, E4M3 per 16, FP32 tensor scale).
//  [BLOG]  "NVFP4 Trains with Precision of 16-Bit and Speed and Efficiency of
//          4-Bit": E4M3 scale factors; Hadamard transforms; stochastic
//          rounding.
//  [SC11]  Salmon et al., "Parallel random numbers: as easy as 1, 2, 3".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Plain clang vector types (HIP's uint4 & co. are structs, which the memory
// builtins do not take).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Global memory access points of the streaming kernels: non-temporal (each
// byte is touched once per pass, so it should not displace cached data).
template <class T>
__device__ __forceinline__ T ld_(const T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_(T v, T* p) { __builtin_nontemporal_store(v, p); }

// Tensor scale maps the tensor amax onto the largest block scale:
// 6 (largest E2M1 magnitude) * 448 (largest E4M3 value).
constexpr float kScaleDen = 2688.0f;

// Bit casts usable on the host as well, so the pure bit-level routines below
// (the E4M3 and E2M1 definitions, the stochastic-rounding decision) also
// compile for the CPU, where the tests run them against the CPU reference.
__host__ __device__ __forceinline__ uint32_t f32_bits(float x) {
  return __builtin_bit_cast(uint32_t, x);
}
__host__ __device__ __forceinline__ float f32_from(uint32_t u) {
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// E4M3 (OCP E4M3FN) -- [BLOG] E4M3 scale factors
// ---------------------------------------------------------------------------
// Non-negative binary32 -> E4M3FN code, round-to-nearest-even, saturating at
// 448 (code 0x7E).  Subnormal range (x < 2^-6): the code is rint(x * 2^9),
// an exact scaling; 8 there is the smallest normal.  Normal range: round the
// binary32 mantissa to 3 bits (add half-ulp-minus-one plus the kept lsb) and
// rebias the exponent from 127 to 7.  This is the bit-level definition; the
// kernels take the same codes from the hardware encode (e4m3_code below).
__host__ __device__ __forceinline__ uint32_t e4m3_from_float(float x) {
  if (!(x > 0.0f)) return 0u;
  if (x >= 448.0f) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)__builtin_rintf(x * 512.0f);
  uint32_t u = f32_bits(x);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t e = (u >> 23) - 120u;  // 127 - 7
  uint32_t m = (u >> 20) & 7u;
  uint32_t c = (e << 3) | m;
  return c > 0x7Eu ? 0x7Eu : c;
}

// The same encode by the gfx950 FP8 convert (OCP E4M3, round to nearest
// even, subnormals kept) after clamping to 448: equal to e4m3_from_float for
// every binary32 in [0, 448] (all 1.14e9 patterns compared on MI355X), and
// both give 0x7E above.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  // x >= 0 here; the mask keeps any code a 7-bit table index
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(x, 448.0f), 0.0f, 0, false) & 0x7Fu;
}

// E4M3FN code (0..0x7E) -> binary32 (branch-free: both forms are computed
// and the exponent field selects; the subnormal form is m * 2^-9, exact).
__device__ __forceinline__ float e4m3_to_float(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0.001953125f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0u ? sub : nrm;
}

// ---------------------------------------------------------------------------
// E2M1 -- [PAPER] format paragraph: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
// ---------------------------------------------------------------------------
// Round-to-nearest-even magnitude index of a >= 0, saturating at 6.  The
// decision points are the midpoints between grid values; at a midpoint the
// even index wins, so the comparison is >= where the upper neighbour has an
// even index and > where it has an odd one.  This is the bit-level
// definition; the kernels take the same decision from the hardware FP4
// encode (encode8_rtn below).
__host__ __device__ __forceinline__ uint32_t e2m1_rtn_index(float a) {
  uint32_t i = 0;
  i += (a > 0.25f);
  i += (a >= 0.75f);
  i += (a > 1.25f);
  i += (a >= 1.75f);
  i += (a > 2.5f);
  i += (a >= 3.5f);
  i += (a > 5.0f);
  return i;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 -- [SC11]
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    u32x4 n;
    // three-input XOR in one instruction (truth table 0x96)
    n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);
    n.y = (uint32_t)p1;
    n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words for the 8 elements n0 .. n0+7 (n0 a multiple of 8).
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint32_t stream_id, uint64_t n0) {
  uint64_t g = n0 >> 3;
  u32x4 c = {(uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u};
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t rht_sign_bits(uint64_t rht_seed) {
  u32x4 c = {0u, 0u, 0u, 1u};
  return philox4x32_10(c, (uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)).x & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// 16-point Hadamard -- [BLOG] Hadamard transforms
// ---------------------------------------------------------------------------
// v <- 1/4 * H16 * D * v: sign flips, then butterflies over index bits
// 0, 1, 2, 3 (pairs j, j + h with bit h of j clear), then the exact * 1/4.
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((signs >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] *= 0.25f;
}

// The same transform of a 16-block held by two lanes of a wave, 8 elements
// each: the lane with hi == false holds elements 0..7, its partner (lane ^ 1)
// elements 8..15.  Sign flips and the butterflies over index bits 0..2 run
// inside each lane; the last stage pairs element j with j + 8 across the two
// lanes (the low lane keeps the sum, the high lane the difference); then the
// exact * 1/4.  Every output is the same chain of binary32 operations as in
// rht16.  Both lanes of a pair must execute this together.
__device__ __forceinline__ void rht16_pair(float (&v)[8], uint32_t signs, bool hi) {
  const uint32_t s = hi ? signs >> 8 : signs;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((s >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
      float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __shfl_xor(v[j], 1, 64);
    v[j] = hi ? p - v[j] : v[j] + p;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= 0.25f;
}

// ---------------------------------------------------------------------------
// Encoding one group of 8 elements given the block's reciprocal scale
// ---------------------------------------------------------------------------
// Codes of z[0..7] (element j in nibble j), round-to-nearest-even.  The
// gfx950 FP4 encode (scale 1.0: no scaling) rounds a binary32 to the nearest
// E2M1 value with ties to the even code, saturates beyond 6 and keeps the
// sign of zero -- the same decision as e2m1_rtn_index, taken on the same
// binary32 v = z * r (compared on MI355X with the nearest-value definition
// on every binary32 in [-8, 8]); it packs two codes per byte, first operand
// in the low nibble.
__device__ __forceinline__ uint32_t encode8_rtn(const float* z, float r) {
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[0] * r, z[1] * r, 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[2] * r, z[3] * r, 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[4] * r, z[5] * r, 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[6] * r, z[7] * r, 1.0f, 3);
  return out;
}

// Stochastic rounding of v onto the E2M1 grid, returned as the grid value
// itself (sign of v kept), with 16 random bits u: with lo <= |v| < hi the
// neighbouring grid values and p = (|v| - lo)/(hi - lo), round away from zero
// iff u < p * 65536; |v| >= 6 gives 6.  Above 0.5 the grid spacing within a
// binade is a power of two, so the decision is an add-and-truncate on the
// binary32 bits of a = min(|v|, 6):
//   1 <= a < 6: the grid keeps 1 mantissa bit (2^e, 1.5 * 2^e).  The low 22
//     bits f are p * 2^22, and f > u * 2^6  <=>  f + (2^22 - 1 - u * 2^6)
//     carries into bit 22; clearing the low 22 bits then leaves hi or lo
//     (the carry may run into the exponent: 1.75.. -> 2, and a < 6 tops out
//     at 6).
//   0.5 <= a < 1: no mantissa bit is kept (grid 0.5, 1): the same with 23
//     bits and u * 2^7.
//   a < 0.5 (grid 0, 0.5): p * 65536 = a * 2^17, an exact float; compared
//     with u as a float.
// The hardware FP4 encode then maps each grid value to its code exactly.
__host__ __device__ __forceinline__ float e2m1_sr_value(float v, uint32_t u) {
  const float a = __builtin_fminf(__builtin_fabsf(v), 6.0f);
  const uint32_t bits = f32_bits(a);
  // g = 1 for a >= 1 (22 dropped bits), 0 in [0.5, 1) (23): the top bit of
  // bits + (2^31 - 1.0f's pattern) -- no compare, so no mask register
  const uint32_t g = (bits + 0x40800000u) >> 31;
  // the 23-bit form of the addend, 2^23 - 1 - u * 2^7; shifted right by g it
  // is the 22-bit one (2^22 - 1 - u * 2^6) exactly, its low bit being 1.
  // Adding it to bits shifted left by g puts the carry at bit 23 in both
  // binades; clearing bits 0..22 and shifting back leaves the grid value.
  const uint32_t t7 = 0x7FFFFFu - (u << 7);
  const uint32_t rounded = (((bits << g) + t7) & 0xFF800000u) >> g;
  // a < 0.5 (grid 0, 0.5): up iff u < a * 2^17, an exact float compare
  const uint32_t small = ((float)u < a * 131072.0f) ? 0x3F000000u : 0u;
  const uint32_t mag = bits < 0x3F000000u ? small : rounded;
  return f32_from(mag | (f32_bits(v) & 0x80000000u));
}

// Stochastic rounding with the 8 16-bit halves of w (element j takes word
// j/2, low half for even j); codes packed as in encode8_rtn.
__device__ __forceinline__ uint32_t encode8_sr(const float* z, float r, u32x4 w) {
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_value(z[0] * r, w.x & 0xFFFFu), e2m1_sr_value(z[1] * r, w.x >> 16), 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_value(z[2] * r, w.y & 0xFFFFu), e2m1_sr_value(z[3] * r, w.y >> 16), 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_value(z[4] * r, w.z & 0xFFFFu), e2m1_sr_value(z[5] * r, w.z >> 16), 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_value(z[6] * r, w.w & 0xFFFFu), e2m1_sr_value(z[7] * r, w.w >> 16), 1.0f, 3);
  return out;
}

__device__ __forceinline__ float tensor_scale_from_amax(float amax_t) {
  return amax_t > 0.0f ? amax_t / kScaleDen : 1.0f;
}

// Block scale code and reciprocal element scale from a block amax.
struct BlockScale { uint32_t code; float r; };

// Per-tensor constants of the block-scale step.  rtab (LDS) holds the
// reciprocals r = 1 / (float(E) * s_t) of the E4M3 codes 1 .. 0x7E (and of
// 0x7F, which no scale takes: a 7-bit code always indexes the table), each
// computed exactly as the per-block formula would, so a lookup returns the
// same binary32 as the division it replaces.  Code 0 (a block whose scale
// underflows, or an all-zero block) gets r = 0: every element then scales to
// a zero with its own sign, which both encodes turn into the sign-only code
// such a block takes -- no separate path for zero blocks.
constexpr int kE4m3Codes = 128;

struct ScaleCtx {
  float s_t, t6, rt6;  // tensor scale, 6 * s_t, and the rounded 1 / t6
  bool divide;         // 1 / t6 overflowed (amax_t below ~1.3e-36): divide every block
  const float* rtab;
};

// Every thread gets the constants; the thread with slot e < 128 fills
// rtab[e].  The caller synchronises the workgroup before the first lookup.
__device__ __forceinline__ ScaleCtx scale_ctx(float amax_t, float* rtab, int slot) {
  ScaleCtx c;
  c.s_t = tensor_scale_from_amax(amax_t);
  c.t6 = 6.0f * c.s_t;
  c.rt6 = 1.0f / c.t6;
  c.divide = !(c.rt6 <= 3.40282347e38f);
  c.rtab = rtab;
  if (slot >= 0 && slot < kE4m3Codes)
    rtab[slot] = slot == 0 ? 0.0f : 1.0f / (e4m3_to_float((uint32_t)slot) * c.s_t);
  return c;
}

// E4M3 code of the correctly rounded quotient q = amax_b / t6.  q' =
// amax_b * fl(1/t6) is within 3 ulps of q (two roundings of relative size
// 2^-24 each, plus q's own half ulp), so the two give the same code unless a
// point where the code changes lies between them.  Those points are the
// midpoints between E4M3 values: binary32 patterns whose low 20 bits are
// 0x80000 above 2^-6 (3 significand bits kept) and 0 below it (the
// subnormal steps of 2^-9 put the midpoints at odd multiples of 2^-10).  If
// q' lies within 8 patterns of such a point (about one block in 2^16), the
// quotient is taken by the correctly rounded division instead.  So is every
// block's when 1/t6 is not finite (a tensor amax below 448 / FLT_MAX): there
// q' would be inf for every non-zero block and NaN for a zero one.
__device__ __forceinline__ uint32_t scale_code(float amax_b, const ScaleCtx& c) {
  float q = amax_b * c.rt6;
  const uint32_t b = __float_as_uint(q);
  const uint32_t centre = b < 0x3C800000u ? 0u : 0x80000u;
  // a real branch (the division is rare): if-converted, its ~10 instructions
  // would run for every block
  if (__builtin_expect(((b - centre + 8u) & 0xFFFFFu) < 16u || c.divide, 0)) q = amax_b / c.t6;
  return e4m3_code(q);
}

__device__ __forceinline__ BlockScale block_scale(float amax_b, const ScaleCtx& c) {
  BlockScale b;
  b.code = scale_code(amax_b, c);
  b.r = c.rtab[b.code];
  return b;
}

// ---------------------------------------------------------------------------
// Wave reductions (max of non-negative floats)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace nvfp4
