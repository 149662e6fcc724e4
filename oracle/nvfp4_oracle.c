/*
 * nvfp4_oracle.c -- CPU oracle for the NVFP4 quantize + NVFP4-linear GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant generator with the HIP library, and it never
 * includes or calls anything from it.
 *
 * Sources (web pages, cited by title and section):
 *  [PAPER] "Pretraining Large Language Models with NVFP4" (NVIDIA, arXiv
 *          2509.25149), summary page: format paragraph (NVFP4 vs MXFP4),
 *          recipe paragraph, limitations paragraph.
 *  [BLOG]  "NVFP4 Trains with Precision of 16-Bit and Speed and Efficiency of
 *          4-Bit" (NVIDIA technical blog, Chinese rendering), section on the
 *          NVFP4 pretraining method: micro-block scaling, E4M3 scale factors,
 *          Hadamard transforms, 2D block quantization, stochastic rounding.
 *  [NEWS]  "Soumith Chintala 发布 NVFP4 训练详解文章" (news item): spec table
 *          (section 一) and technique list (section 三).
 *  [SC11]  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *          1, 2, 3", SC'11 -- Philox4x32-10.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, subnormals kept, no
 * FMA contraction (build with -ffp-contract=off, never -ffast-math).  Where
 * floating point decides a code the decision is taken in binary32, the
 * precision the GPU kernels use; the GEMM reference is exact (int64).
 *
 * Readings of points the pages leave open (all are listed in the design notes):
 *  - tensor scale s_t = amax_t / (6*448); s_t = 1 when amax_t == 0;
 *  - block scale E = E4M3FN(amax_b / (6*s_t)), RNE incl. subnormals,
 *    saturating at 448;
 *  - element scale: r = 1/(E*s_t) once per block, v = z*r per element;
 *  - E2M1 RTN: nearest grid value, ties to the even code, saturate at 6;
 *  - E2M1 SR: round away from zero iff u16 < p*65536, p = (|v|-lo)/(hi-lo);
 *  - random bits: Philox4x32-10, key = seed, counter = (n/8, stream_id, 0),
 *    16 bits per element, n = index in the K-contiguous output operand;
 *  - RHT: y = 1/4 * H16 * D * x along K, FP32 butterfly h = 1,2,4,8, sign
 *    vector D from Philox(key = rht_seed, counter = (0,0,0,1)) word 0;
 *  - sign of a zero code = sign bit of z; low nibble = even k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* bf16 / binary32 bit helpers                                         */
/* ------------------------------------------------------------------ */
static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the upper half of a binary32; widening is exact. */
ORC_API float orc_bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

/* ------------------------------------------------------------------ */
/* Philox4x32-10 [SC11]                                                */
/* ------------------------------------------------------------------ */
/* One round: two 32x32->64 multiplies of counter words 0 and 2 by the
 * round multipliers; the high halves are mixed with the other counter words
 * and the key, the low halves pass through.  The key is bumped by the Weyl
 * constants (golden ratio and sqrt(3)-1 in 32-bit fixed point) between
 * rounds. */
ORC_API void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                               uint32_t out[4]) {
  const uint32_t mul0 = 0xD2511F53u, mul1 = 0xCD9E8D57u;
  const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += weyl0; k1 += weyl1; }
    uint64_t p0 = (uint64_t)mul0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)mul1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16 random bits for the element at K-contiguous operand index n.
 * Eight elements share one Philox call: counter = (n/8 low, n/8 high,
 * stream_id, 0), word (n%8)/2, low half for even n, high half for odd n. */
ORC_API uint16_t orc_sr_bits(uint64_t seed, uint32_t stream_id, uint64_t n) {
  uint64_t g = n / 8u;
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  uint32_t w = out[(n % 8u) / 2u];
  return (n % 2u) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
}

/* RHT sign vector: bit j set means the j-th of the 16 inputs is negated. */
ORC_API uint16_t orc_rht_signs(uint64_t rht_seed) {
  uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  uint32_t key[2] = {(uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (uint16_t)(out[0] & 0xFFFFu);
}

/* ------------------------------------------------------------------ */
/* E4M3 (OCP E4M3FN) block scale -- [BLOG] E4M3 scale factors,         */
/* [PAPER] format paragraph                                            */
/* ------------------------------------------------------------------ */
/* Decode by definition: bias 7, 3 mantissa bits, exponent field 0 is
 * subnormal (m/8 * 2^-6), code 0x7F/0xFF is NaN (never produced here). */
ORC_API float orc_e4m3_decode(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  float mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = ldexpf((float)m, -9);          /* (m/8) * 2^-6 */
  else mag = ldexpf((float)(8 + m), e - 7 - 3);    /* (1+m/8) * 2^(e-7) */
  return s ? -mag : mag;
}

/* Encode a non-negative binary32 to the nearest finite E4M3FN value (codes
 * 0x00..0x7E), ties to the even code, values above 448 saturate to 448.
 * The 127 finite non-negative values increase with the code, so the nearest
 * one is found by bisection over the decoded table and one comparison with
 * each neighbour. */
static float e4m3_tab[127];
__attribute__((constructor)) static void e4m3_tab_init(void) {
  for (int c = 0; c < 127; ++c) e4m3_tab[c] = orc_e4m3_decode((uint8_t)c);
}

ORC_API uint8_t orc_e4m3_encode(float x) {
  const float* tab = e4m3_tab;
  if (!(x > 0.0f)) return 0;        /* zero (and the unused negative range) */
  if (x >= 448.0f) return 0x7E;
  /* largest code with tab[c] <= x */
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (tab[mid] <= x) lo = mid; else hi = mid - 1;
  }
  if (tab[lo] == x) return (uint8_t)lo;
  /* x lies strictly between tab[lo] and tab[lo+1]; compare distances exactly
     in double (both distances are exact there). */
  double dlo = (double)x - (double)tab[lo];
  double dhi = (double)tab[lo + 1] - (double)x;
  if (dlo < dhi) return (uint8_t)lo;
  if (dhi < dlo) return (uint8_t)(lo + 1);
  return (uint8_t)((lo % 2 == 0) ? lo : lo + 1);
}

/* Element-wise over an array (for exhaustive checks). */
ORC_API void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

/* ------------------------------------------------------------------ */
/* E2M1 element -- [PAPER] format paragraph: 0, +-0.5 ... +-6           */
/* ------------------------------------------------------------------ */
static const float kE2M1Mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

ORC_API float orc_e2m1_decode(uint8_t code) {
  float m = kE2M1Mag[code & 7];
  return (code & 8) ? -m : m;
}

/* Round-to-nearest: the grid point at least distance from a = |v|, ties to the
 * even magnitude index (the index's low bit is the E2M1 mantissa bit); values
 * beyond 6 saturate to 6.  [BLOG] stochastic-rounding paragraph contrasts this
 * "nearest representable value" rounding. */
ORC_API uint8_t orc_e2m1_rtn(float v) {
  float a = fabsf(v);
  int best = 0;
  for (int i = 1; i < 8; ++i) {
    float db = fabsf(a - kE2M1Mag[best]);
    float di = fabsf(a - kE2M1Mag[i]);
    if (di < db || (di == db && (i % 2 == 0) && (best % 2 == 1))) best = i;
  }
  if (a > 6.0f) best = 7;
  return (uint8_t)((signbit(v) ? 8 : 0) | best);
}

/* Stochastic rounding: between the neighbouring grid values lo <= a <= hi the
 * larger one is taken with probability (a-lo)/(hi-lo), decided by 16 random
 * bits u16: up iff u16 < p * 65536.  [BLOG] stochastic-rounding paragraph:
 * up or down with probability given by the distances, so the result is
 * unbiased in expectation.  |v| > 6 saturates to 6. */
ORC_API uint8_t orc_e2m1_sr(float v, uint16_t u16) {
  float a = fabsf(v);
  if (a > 6.0f) a = 6.0f;
  int lo = 0;
  for (int i = 0; i < 8; ++i) if (kE2M1Mag[i] <= a) lo = i;
  int idx = lo;
  if (kE2M1Mag[lo] != a) {
    int hi = lo + 1;
    float p = (a - kE2M1Mag[lo]) / (kE2M1Mag[hi] - kE2M1Mag[lo]);
    if ((float)u16 < p * 65536.0f) idx = hi;
  }
  return (uint8_t)((signbit(v) ? 8 : 0) | idx);
}

ORC_API void orc_e2m1_rtn_array(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_rtn(v[i]);
}

ORC_API void orc_e2m1_sr_array(const float* v, const uint16_t* u16, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_sr(v[i], u16[i]);
}

ORC_API void orc_sr_bits_array(uint64_t seed, uint32_t stream_id, uint64_t n0, int64_t n,
                               uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_bits(seed, stream_id, n0 + (uint64_t)i);
}

/* ------------------------------------------------------------------ */
/* 16-point random Hadamard transform -- [BLOG] Hadamard paragraph,     */
/* [NEWS] section 三 (RHT on weight-gradient GEMM inputs)               */
/* ------------------------------------------------------------------ */
/* out = 1/4 * H16 * D * in, H16 the Sylvester Hadamard matrix, D = diag of
 * +-1 from the sign bits.  Fast Walsh-Hadamard butterflies with strides
 * 1, 2, 4, 8 in binary32, then the exact scaling by 1/4. */
ORC_API void orc_rht16(const float in[16], uint16_t signs, float out[16]) {
  float w[16];
  for (int j = 0; j < 16; ++j) w[j] = ((signs >> j) & 1) ? -in[j] : in[j];
  for (int h = 1; h < 16; h *= 2) {
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      float a = w[j], b = w[j + h];
      w[j] = a + b;
      w[j + h] = a - b;
    }
  }
  for (int j = 0; j < 16; ++j) out[j] = w[j] * 0.25f;
}

/* ------------------------------------------------------------------ */
/* Operand view                                                        */
/* ------------------------------------------------------------------ */
/* The quantized operand z[i][k] is K-contiguous:
 *   mode 0 (1D rowwise): z = x,   I = rows, K = cols, blocks 1x16 along K
 *   mode 1 (1D colwise): z = x^T, I = cols, K = rows, blocks 1x16 along K
 *   mode 2 (2D):         z = x,   I = rows, K = cols, blocks 16x16
 * [NEWS] section 三 and [BLOG] 2D block quantization: weights use 2D blocks,
 * activations and gradients 1D blocks.  With use_rht, every 16 consecutive k
 * of a row of z are replaced by their RHT (1D modes only). */
typedef struct {
  const uint16_t* x; int64_t rows, cols; int mode;
  int use_rht; uint16_t signs;
} orc_view;

static int64_t view_I(const orc_view* v) { return v->mode == 1 ? v->cols : v->rows; }
static int64_t view_K(const orc_view* v) { return v->mode == 1 ? v->rows : v->cols; }

/* z[i][16g .. 16g+15] into out[16]. */
static void view_group(const orc_view* v, int64_t i, int64_t g, float out[16]) {
  float t[16];
  for (int j = 0; j < 16; ++j) {
    int64_t k = 16 * g + j;
    uint16_t h = (v->mode == 1) ? v->x[k * v->cols + i] : v->x[i * v->cols + k];
    t[j] = orc_bf16_to_f32(h);
  }
  if (v->use_rht) orc_rht16(t, v->signs, out);
  else memcpy(out, t, sizeof t);
}

/* ------------------------------------------------------------------ */
/* Tensor amax and scale -- [PAPER] format and limitations paragraphs   */
/* ------------------------------------------------------------------ */
static float view_amax(const orc_view* v) {
  int64_t I = view_I(v), G = view_K(v) / 16;
  float amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
  for (int64_t i = 0; i < I; ++i) {
    for (int64_t g = 0; g < G; ++g) {
      float z[16];
      view_group(v, i, g, z);
      for (int j = 0; j < 16; ++j) { float a = fabsf(z[j]); if (a > amax) amax = a; }
    }
  }
  return amax;
}

ORC_API float orc_amax(const uint16_t* x, int64_t rows, int64_t cols) {
  orc_view v = {x, rows, cols, 0, 0, 0};
  return view_amax(&v);
}

/* amax of RHT(x^T): the statistic the RHT quantizer scales by. */
ORC_API float orc_amax_rht(const uint16_t* x, int64_t rows, int64_t cols, uint64_t rht_seed) {
  orc_view v = {x, rows, cols, 1, 1, orc_rht_signs(rht_seed)};
  return view_amax(&v);
}

/* FP32 tensor scale: the largest block maps onto the largest E4M3 value. */
ORC_API float orc_tensor_scale(float amax_t) {
  return amax_t > 0.0f ? amax_t / (6.0f * 448.0f) : 1.0f;
}

/* ------------------------------------------------------------------ */
/* One block: amax -> E4M3 scale -> E2M1 codes                          */
/* ------------------------------------------------------------------ */
/* Block scale: the E4M3 code of amax_b / (6 s_t), so that the block's
 * largest magnitude lands on the largest E2M1 value, 6 ([BLOG] E4M3 scale
 * factors; [PAPER] format paragraph: one E4M3 scale per 16 values). */
ORC_API uint8_t orc_block_scale(float amax_b, float s_t) {
  float t6 = 6.0f * s_t;
  float e_f = amax_b / t6;
  return orc_e4m3_encode(e_f);
}

/* Element scale of a block with scale code E: r = 1 / (E * s_t), once per
 * block; the encode multiplies every element by it. */
ORC_API float orc_block_recip(uint8_t E, float s_t) {
  float d = orc_e4m3_decode(E) * s_t;
  return 1.0f / d;
}

/* z[] holds the n (16 or 256) values of the block, idx[] their operand
 * indices (for the random bits).  Returns the E4M3 scale code. */
static uint8_t quant_block(const float* z, const uint64_t* idx, int n, float s_t,
                           int use_sr, uint64_t seed, uint32_t stream_id, uint8_t* code) {
  float amax_b = 0.0f;
  for (int j = 0; j < n; ++j) { float a = fabsf(z[j]); if (a > amax_b) amax_b = a; }
  uint8_t E = orc_block_scale(amax_b, s_t);
  if (E == 0) {
    /* the block's scale underflowed (or the block is all zero): every
       element becomes a signed zero */
    for (int j = 0; j < n; ++j) code[j] = (uint8_t)(signbit(z[j]) ? 8 : 0);
    return E;
  }
  float r = orc_block_recip(E, s_t);
  for (int j = 0; j < n; ++j) {
    float v = z[j] * r;
    code[j] = use_sr ? orc_e2m1_sr(v, orc_sr_bits(seed, stream_id, idx[j])) : orc_e2m1_rtn(v);
  }
  return E;
}

static void put_code(uint8_t* codes, int64_t ld, int64_t i, int64_t k, uint8_t c) {
  uint8_t* b = &codes[i * ld + k / 2];
  if (k % 2 == 0) *b = (uint8_t)((*b & 0xF0) | c);
  else *b = (uint8_t)((*b & 0x0F) | (c << 4));
}

/* ------------------------------------------------------------------ */
/* Whole quantizer                                                      */
/* ------------------------------------------------------------------ */
/* x: bf16 [rows][cols] row-major.  mode as in orc_view.  Outputs:
 *   codes   [I][K/2]    (2 codes per byte, even k in the low nibble)
 *   codes_t [K][I/2]    (mode 2 only, nullable: the same codes transposed)
 *   scales  [I][K/16] for 1D, [rows/16][cols/16] for 2D
 *   *amax_io: input when amax_given, else written with amax of z
 *   *s_t_out: tensor scale
 * Returns 0, or -2 when a dimension is not a positive multiple of 16. */
ORC_API int orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int mode,
                         int use_rht, uint64_t rht_seed,
                         int use_sr, uint64_t sr_seed, uint32_t stream_id,
                         int amax_given, float* amax_io,
                         uint8_t* codes, uint8_t* codes_t, uint8_t* scales, float* s_t_out) {
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return -2;
  if (mode < 0 || mode > 2) return -4;
  if (use_rht && mode == 2) return -4;
  orc_view v = {x, rows, cols, mode, use_rht, use_rht ? orc_rht_signs(rht_seed) : (uint16_t)0};
  int64_t I = view_I(&v), K = view_K(&v);
  float amax_t = amax_given ? *amax_io : view_amax(&v);
  if (!amax_given) *amax_io = amax_t;
  float s_t = orc_tensor_scale(amax_t);
  *s_t_out = s_t;

  if (mode != 2) {
    int64_t G = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
      for (int64_t g = 0; g < G; ++g) {
        float z[16]; uint64_t idx[16]; uint8_t c[16];
        view_group(&v, i, g, z);
        for (int j = 0; j < 16; ++j) idx[j] = (uint64_t)(i * K + 16 * g + j);
        scales[i * G + g] = quant_block(z, idx, 16, s_t, use_sr, sr_seed, stream_id, c);
        for (int j = 0; j < 16; ++j) put_code(codes, K / 2, i, 16 * g + j, c[j]);
      }
    }
  } else {
    int64_t TR = rows / 16, TC = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t tr = 0; tr < TR; ++tr) {
      for (int64_t tc = 0; tc < TC; ++tc) {
        float z[256]; uint64_t idx[256]; uint8_t c[256];
        for (int a = 0; a < 16; ++a) {
          int64_t i = 16 * tr + a;
          float row[16];
          view_group(&v, i, tc, row);
          for (int b = 0; b < 16; ++b) {
            z[a * 16 + b] = row[b];
            idx[a * 16 + b] = (uint64_t)(i * K + 16 * tc + b);
          }
        }
        scales[tr * TC + tc] = quant_block(z, idx, 256, s_t, use_sr, sr_seed, stream_id, c);
        for (int a = 0; a < 16; ++a)
          for (int b = 0; b < 16; ++b) {
            int64_t i = 16 * tr + a, k = 16 * tc + b;
            put_code(codes, K / 2, i, k, c[a * 16 + b]);
            if (codes_t) put_code(codes_t, I / 2, k, i, c[a * 16 + b]);
          }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Quantized operand, decode, dequantize                                */
/* ------------------------------------------------------------------ */
/* Logical [rows][k], K-contiguous.  The scale of element (r, k) is
 * scales[(r / blk_rows) * ss_row + (k / 16) * ss_k]. */
typedef struct {
  const uint8_t* codes; int64_t ld_codes;
  const uint8_t* scales; int64_t ss_row, ss_k;
  int32_t blk_rows;
  float tensor_scale;
  int64_t rows, k;
} orc_operand;

static uint8_t op_code(const orc_operand* q, int64_t r, int64_t k) {
  uint8_t b = q->codes[r * q->ld_codes + k / 2];
  return (k % 2 == 0) ? (uint8_t)(b & 0xF) : (uint8_t)(b >> 4);
}
static uint8_t op_scale(const orc_operand* q, int64_t r, int64_t k) {
  return q->scales[(r / q->blk_rows) * q->ss_row + (k / 16) * q->ss_k];
}

/* x_hat = (code value * E) * s_t in binary32: the first product is exact,
 * the second rounds once.  The dequantize step multiplies the 4-bit value by
 * its block scale (and the tensor scale) to recover the real value. */
ORC_API void orc_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                            int64_t ss_row, int64_t ss_k, int32_t blk_rows, float tensor_scale,
                            int64_t rows, int64_t k, float* out) {
  orc_operand q = {codes, ld_codes, scales, ss_row, ss_k, blk_rows, tensor_scale, rows, k};
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < k; ++c) {
      float qe = orc_e2m1_decode(op_code(&q, r, c)) * orc_e4m3_decode(op_scale(&q, r, c));
      out[r * k + c] = qe * tensor_scale;
    }
}

/* ------------------------------------------------------------------ */
/* GEMM -- C[m][n] = s_a*s_b * sum_k A[m,k]*B[n,k]                      */
/* ------------------------------------------------------------------ */
/* Each decoded value (E2M1 value) * (E4M3 value) is an integer multiple of
 * 2^-10 below 2^22 in magnitude, so products are exact integers in units of
 * 2^-20 and the K-sum is exact in int64.  The result is scaled to double
 * once.  T[m][n] = sum_k |A[m,k]*B[n,k]| is the error scale of the
 * tolerance. */
static int64_t dec_int(const orc_operand* q, int64_t r, int64_t k) {
  uint8_t c = op_code(q, r, k);
  int64_t twoq = (int64_t)(2.0f * kE2M1Mag[c & 7]);                 /* 0..12 */
  int64_t e512 = (int64_t)ldexp((double)orc_e4m3_decode(op_scale(q, r, k)), 9); /* E * 2^9 */
  int64_t v = twoq * e512;                                              /* value * 2^10 */
  return (c & 8) ? -v : v;
}

static void gemm_one(const orc_operand* a, const orc_operand* b, int64_t m, int64_t n,
                     double* c, double* t) {
  int64_t acc = 0, abs_acc = 0;
  for (int64_t k = 0; k < a->k; ++k) {
    int64_t p = dec_int(a, m, k) * dec_int(b, n, k);
    acc += p;
    abs_acc += p < 0 ? -p : p;
  }
  double scale = ldexp(1.0, -20) * (double)a->tensor_scale * (double)b->tensor_scale;
  *c = (double)acc * scale;
  if (t) *t = (double)abs_acc * scale;
}

#define ORC_OPERAND_ARGS(p)                                                           \
  const uint8_t *p##_codes, int64_t p##_ld, const uint8_t *p##_scales, int64_t p##_ssr, \
      int64_t p##_ssk, int32_t p##_blk, float p##_st, int64_t p##_rows
#define ORC_OPERAND(p, K) {p##_codes, p##_ld, p##_scales, p##_ssr, p##_ssk, p##_blk, p##_st, p##_rows, K}

/* Full product: c and t are [M][N] row-major (t nullable). */
ORC_API int orc_gemm(ORC_OPERAND_ARGS(a), ORC_OPERAND_ARGS(b), int64_t K, double* c, double* t) {
  orc_operand A = ORC_OPERAND(a, K), B = ORC_OPERAND(b, K);
  if (K % 16) return -2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < A.rows; ++m)
    for (int64_t n = 0; n < B.rows; ++n)
      gemm_one(&A, &B, m, n, &c[m * B.rows + n], t ? &t[m * B.rows + n] : NULL);
  return 0;
}

/* Selected entries: (ms[j], ns[j]) for j < count. */
ORC_API int orc_gemm_entries(ORC_OPERAND_ARGS(a), ORC_OPERAND_ARGS(b), int64_t K,
                             const int64_t* ms, const int64_t* ns, int64_t count,
                             double* c, double* t) {
  orc_operand A = ORC_OPERAND(a, K), B = ORC_OPERAND(b, K);
  if (K % 16) return -2;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < count; ++j) gemm_one(&A, &B, ms[j], ns[j], &c[j], t ? &t[j] : NULL);
  return 0;
}

/* The decoded operand q * E (E2M1 value times E4M3 block scale, without
 * the tensor scale) as double, [rows][K] row-major: exact, being a multiple
 * of 2^-10 below 2^22 in magnitude.  With it a float64 matrix product is the
 * fast form of the GEMM above: its summation error, at most about
 * K * 2^-53 * T, is far inside the GEMM's tolerance of 1e-5 * T. */
ORC_API int orc_decode_exact(ORC_OPERAND_ARGS(q), int64_t K, double* out) {
  orc_operand Q = ORC_OPERAND(q, K);
  if (K % 16) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < Q.rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = (double)dec_int(&Q, r, k) * ldexp(1.0, -10);
  return 0;
}

/* Thread count of the OpenMP loops from here on (for timing the reference
 * single-threaded and on all cores); n <= 0 leaves it unchanged. */
ORC_API void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
