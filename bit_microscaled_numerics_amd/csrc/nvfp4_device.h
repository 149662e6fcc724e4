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
  // x >= 0 here, so the clamp is an integer min of the bit patterns (no
  // quieting of x first; a NaN pattern would clamp to 448 too); the convert
  // writes the low half-word, so the preserved high half-word can be
  // anything (here x's own bits: no register to clear)
  const uint32_t xb = min(__float_as_uint(x), 0x43E00000u);  // 448.0f
  // the low half-word is the code and the code of +0 (0x00): a table index
  // below 0x7F, taken with a half-word select
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(xb), 0.0f, (int)xb, false) & 0xFFFFu;
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

// UNIFORM: every input is the same across the wave (the RHT signs), so
// plain XORs keep all ten rounds on the scalar unit.
template <bool UNIFORM = false>
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    u32x4 n;
    if (UNIFORM || r == 0) {
      // plain XORs: where the counter's words are the same across the wave
      // (the stream word, the zero word, the high index word), the first
      // round and the product that follows it stay on the scalar unit
      n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
      n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
    } else {
      // three-input XOR in one instruction (truth table 0x96)
      n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);
      n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
    }
    n.y = (uint32_t)p1;
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words for the 8 elements 8g .. 8g+7 (counter g = n / 8).
__device__ __forceinline__ u32x4 sr_words_g(uint64_t seed, uint32_t stream_id, uint64_t g) {
  u32x4 c = {(uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u};
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}
// The same for the 8 elements n0 .. n0+7 (n0 a multiple of 8).
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint32_t stream_id, uint64_t n0) {
  return sr_words_g(seed, stream_id, n0 >> 3);
}

__device__ __forceinline__ uint32_t rht_sign_bits(uint64_t rht_seed) {
  u32x4 c = {0u, 0u, 0u, 1u};
  return philox4x32_10<true>(c, (uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)).x & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// 16-point Hadamard -- [BLOG] Hadamard transforms
// ---------------------------------------------------------------------------
// v <- 1/4 * H16 * D * v in two parts.  D (the sign flips) is applied where
// the bf16 inputs are unpacked to binary32: the sign bit of element j is
// flipped where bit j of the 16 sign bits is set, in the same instruction as
// the unpack (bf16_lo_flip / bf16_hi_flip).  Then butterflies over index
// bits 0, 1, 2, 3 (pairs j, j + h with bit h of j clear: sum to j,
// difference to j + h) and the exact * 1/4 (rht16_butterflies).
__device__ __forceinline__ uint32_t flip_bit(uint32_t signs, int j) {
  return ((signs >> j) & 1u) << 31;
}
// bf16 -> binary32 with bit 31 xor-ed with flip (0 or 0x80000000): for the
// low half an add of 2^31 to the shifted word changes bit 31 alone.
__device__ __forceinline__ float bf16_lo_flip(uint32_t w, uint32_t flip) {
  return __uint_as_float((w << 16) + flip);
}
__device__ __forceinline__ float bf16_hi_flip(uint32_t w, uint32_t flip) {
  return __uint_as_float((w & 0xFFFF0000u) ^ flip);
}
// The 8 elements of a 16-byte bf16 vector, element j with flip_bit(s, j).
__device__ __forceinline__ void unpack8_flip(const v4u w, uint32_t s, float (&z)[8]) {
  z[0] = bf16_lo_flip(w.x, flip_bit(s, 0));
  z[1] = bf16_hi_flip(w.x, flip_bit(s, 1));
  z[2] = bf16_lo_flip(w.y, flip_bit(s, 2));
  z[3] = bf16_hi_flip(w.y, flip_bit(s, 3));
  z[4] = bf16_lo_flip(w.z, flip_bit(s, 4));
  z[5] = bf16_hi_flip(w.z, flip_bit(s, 5));
  z[6] = bf16_lo_flip(w.w, flip_bit(s, 6));
  z[7] = bf16_hi_flip(w.w, flip_bit(s, 7));
}

// QUARTER = false leaves out the * 1/4: the caller gets 4 times the
// transform, exactly (the butterfly outputs are sums of bf16 values, whose
// quarter is always a binary32), and applies the 1/4 where it is cheaper.
template <bool QUARTER = true>
__device__ __forceinline__ void rht16_butterflies(float (&v)[16]) {
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
  if (QUARTER) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= 0.25f;
  }
}

// The same transform of a 16-block held by two lanes of a wave, 8 elements
// each: the lane with hi == false holds elements 0..7 (flipped with sign bits
// 0..7), its partner (lane ^ 1) elements 8..15 (sign bits 8..15).  The
// butterflies over index bits 0..2 run inside each lane; the last stage
// pairs element j with j + 8 across the two lanes (the low lane keeps the
// sum, the high lane the difference); then the exact * 1/4.  Every output is
// the same chain of binary32 operations as in rht16_butterflies.  The
// partner's value p comes by a DPP quad permutation [1,0,3,2]; each lane then
// forms p + v * sign with one fused multiply-add, sign = +1 on the low lane
// (v_lo + v_hi) and -1 on the high one (v_lo - v_hi): the product is exact,
// so the single rounding gives the binary32 sum or difference itself, signed
// zeros included.  Both lanes of a pair must be active.
template <bool QUARTER = true>
__device__ __forceinline__ void rht16_pair_butterflies(float (&v)[8], bool hi) {
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
  const float sign = hi ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[j]), 0xB1, 0xF, 0xF, false));
    v[j] = __builtin_fmaf(v[j], sign, p);
  }
  if (QUARTER) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= 0.25f;
  }
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
  // the four converts overwrite all four bytes: any start value will do
  uint32_t out = f32_bits(z[0]);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[0] * r, z[1] * r, 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[2] * r, z[3] * r, 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[4] * r, z[5] * r, 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, z[6] * r, z[7] * r, 1.0f, 3);
  return out;
}

// Stochastic rounding of v onto the E2M1 grid with 16 random bits u: with
// lo <= |v| < hi the neighbouring grid values and p = (|v| - lo)/(hi - lo),
// round away from zero iff u < p * 65536; |v| >= 6 gives 6.  Returned as
// TWICE the chosen grid value, with the sign of v (the FP4 encode below
// divides by its scale 2, exactly).  Two exact forms, one per range of
// a = |v|, chosen by a < 1:
//   1 <= a <= 6: within a binade the grid keeps 1 mantissa bit (2^e,
//     1.5 * 2^e, the next binade's 2^(e+1)).  The low 22 bits f are p * 2^22,
//     and f > u * 2^6  <=>  f + (2^22 - 1 - u * 2^6) carries into bit 22;
//     clearing the low 22 bits then leaves hi or lo (the carry may run into
//     the exponent: 1.75.. -> 2; a = 6 has f = 0 and stays).  The bits are
//     taken from a clamped to [1, 6]; the addend also carries 2^23, one more
//     on the exponent field, which doubles the result.  u * 2^6 has bits in
//     6..21 only, so 2^23 + 2^22 - 1 - u * 2^6 is an exclusive-or.
//   0 <= a < 1: the grid 0, 0.5, 1 has the one step 0.5, so with
//     s = a * 2^17 - u the doubled result is ceil(s / 2^16): for
//     a in [0.5, 1), s lies in (0, 2^17) and exceeds 2^16 iff
//     u < (2a - 1) * 65536; below 0.5 it is positive iff u < 2a * 65536.
//     The fused multiply-add gives s exactly on [0.5, 1) (a multiple of 2^-7
//     below 2^17) and with its sign and zero exact below 0.5, which is all
//     that the ceiling there depends on; the scaling by 2^-16 is exact.
__host__ __device__ __forceinline__ float e2m1_sr_twice(float v, uint32_t u) {
  const float a = __builtin_fabsf(v);
  const uint32_t bits = f32_bits(__builtin_fminf(__builtin_fmaxf(a, 1.0f), 6.0f));
  const float upper = f32_from((bits + ((u << 6) ^ 0xBFFFFFu)) & 0xFFC00000u);
  const float s = __builtin_fmaf(a, 131072.0f, -(float)u);
  const float lower = __builtin_ceilf(s * 0x1p-16f);
  const float mag = a < 1.0f ? lower : upper;
  // the magnitude's own sign bit is dropped: the ceiling of a negative
  // fraction is -0
  return f32_from((f32_bits(mag) & 0x7FFFFFFFu) | (f32_bits(v) & 0x80000000u));
}

// Stochastic rounding with the 8 16-bit halves of w (element j takes word
// j/2, low half for even j); codes packed as in encode8_rtn, the FP4 encode
// taking the doubled grid values with scale 2.
__device__ __forceinline__ uint32_t encode8_sr(const float* z, float r, u32x4 w) {
  uint32_t out = f32_bits(z[0]);  // every byte is written below
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_twice(z[0] * r, w.x & 0xFFFFu), e2m1_sr_twice(z[1] * r, w.x >> 16), 2.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_twice(z[2] * r, w.y & 0xFFFFu), e2m1_sr_twice(z[3] * r, w.y >> 16), 2.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_twice(z[4] * r, w.z & 0xFFFFu), e2m1_sr_twice(z[5] * r, w.z >> 16), 2.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
      out, e2m1_sr_twice(z[6] * r, w.w & 0xFFFFu), e2m1_sr_twice(z[7] * r, w.w >> 16), 2.0f, 3);
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
  // every reciprocal's quarter r / 4 is a normal binary32 (amax_t <= 2^125:
  // the smallest r, 6 / amax_t, then exceeds 2^-123), so y * (r / 4) is the
  // one rounding of (y / 4) * r -- the RHT kernels' fold of the 1/4
  bool quarter_folds;
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
  c.quarter_folds = amax_t <= 0x1p125f;
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
// q' lies within 8 patterns of such a point (about one block in 2^15 with
// the wider test below), the quotient is taken by the correctly rounded
// division instead.  So is every
// block's when 1/t6 is not finite (a tensor amax below 448 / FLT_MAX): there
// q' would be inf for every non-zero block and NaN for a zero one.
__device__ __forceinline__ uint32_t scale_code(float amax_b, const ScaleCtx& c) {
  float q = amax_b * c.rt6;
  // within 8 patterns of a pattern whose low 19 bits are zero: both kinds of
  // midpoint, plus the exact E4M3 values above 2^-6 and the half-way
  // patterns below it, which merely take the exact division as well
  const uint32_t b = __float_as_uint(q);
  // a real branch (the division is rare): if-converted, its ~10 instructions
  // would run for every block
  if (__builtin_expect(((b + 8u) & 0x7FFFFu) < 16u || c.divide, 0)) q = amax_b / c.t6;
  return e4m3_code(q);
}

// The RHT encoders hold y = 4 * the transform (rht16_butterflies<false>):
// the block amax takes the 1/4 once (exact), and the element scale takes it
// where that is exact (quarter_folds: y * (r / 4) is then the one rounding of
// (y / 4) * r); otherwise each element is quartered first, as in the plain
// transform.  Returns the reciprocal to encode y with.
template <int N>
__device__ __forceinline__ float quarter_fold(float (&y)[N], float r, const ScaleCtx& c) {
  if (__builtin_expect(c.quarter_folds, 1)) return r * 0.25f;
#pragma unroll
  for (int j = 0; j < N; ++j) y[j] *= 0.25f;
  return r;
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
// Max over lanes l and l ^ 1 (PAIR) or l ^ 2 of a non-negative binary32: a
// DPP quad permutation ([1,0,3,2] or [2,3,0,1]) feeding an integer max --
// non-negative floats order like their bit patterns, so no quieting step.
// Both lanes must be active.
template <int XOR>
__device__ __forceinline__ float quad_xor_max(float m) {
  static_assert(XOR == 1 || XOR == 2, "quad permutations only");
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(m), ctrl, 0xF, 0xF, false);
  return __uint_as_float(max(__float_as_uint(m), o));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace nvfp4
