/*
 * mxfp4_oracle.c -- CPU oracle for the MXFP4 comparison format and its GEMM.
 *
 * TEST INFRASTRUCTURE ONLY, like nvfp4_oracle.c (built into the same
 * liboracle.so): the plain reference the GPU library is checked against.  It
 * shares nothing with the HIP library.
 *
 * Source (web page, cited by title and section):
 *  [PAPER] "Pretraining Large Language Models with NVFP4" (NVIDIA, arXiv
 *          2509.25149), summary page, format paragraph: NVFP4 differs from
 *          OCP MXFP4 in three ways -- MXFP4 blocks hold 32 elements, its block
 *          scale is a power of two (UE8M0), and it has no tensor-level FP32
 *          scale; with a power-of-two scale the worst case leaves the +-4 and
 *          +-6 levels unused, nearly a binade of range.
 *  [BLOG]  "NVFP4 Trains with Precision of 16-Bit and Speed and Efficiency of
 *          4-Bit", micro-block scaling and E4M3 scale-factor sections (MXFP4:
 *          32-element blocks, power-of-two E8M0 scales).
 *
 * Readings (listed in the design notes):
 *  - block: 32 consecutive elements of a row (the K-contiguous operand);
 *  - scale: E = 2^e with e the smallest integer such that amax_b <= 6 * 2^e,
 *    clamped to [-127, 127], stored as the E8M0 byte e + 127.  Rounding the
 *    exponent up keeps every block's largest |v| inside (3, 6], which is the
 *    rule whose worst case wastes +-4 and +-6 ([PAPER] format paragraph).  An
 *    all-zero block gets the smallest scale, byte 0.
 *  - element: v = z * 2^-e in binary32, then the same E2M1 RTN / SR as NVFP4
 *    (orc_e2m1_rtn / orc_e2m1_sr, Philox bits of the element index).
 *  - GEMM: C[m][n] = sum_k (q_a 2^e_a)(q_b 2^e_b) in float64; every product is
 *    exact in float64 (at most 4 significant bits, exponent within range).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* From nvfp4_oracle.c (same library). */
float orc_bf16_to_f32(uint16_t h);
float orc_e2m1_decode(uint8_t code);
uint8_t orc_e2m1_rtn(float v);
uint8_t orc_e2m1_sr(float v, uint16_t u16);
uint16_t orc_sr_bits(uint64_t seed, uint32_t stream_id, uint64_t n);

/* E8M0 byte of a block whose largest magnitude is amax (>= 0). */
ORC_API uint8_t orc_e8m0_encode(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  frexp((double)amax, &x);          /* 2^(x-1) <= amax < 2^x */
  int e = x - 4;                    /* 6 * 2^(x-4) = 0.375 * 2^x < amax: too small */
  while (6.0 * ldexp(1.0, e) < (double)amax) ++e;   /* first e with amax <= 6 * 2^e */
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (uint8_t)(e + 127);
}

ORC_API void orc_e8m0_encode_array(const float* amax, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_encode(amax[i]);
}

/* 2^(code - 127) as binary32 (exact: 2^-127 is a binary32 subnormal). */
ORC_API float orc_e8m0_decode(uint8_t code) { return ldexpf(1.0f, (int)code - 127); }

/* Rowwise MXFP4 quantization of bf16 x [rows][cols] (cols % 32 == 0):
 * codes [rows][cols/2] (low nibble = even k), scales [rows][cols/32]. */
ORC_API int orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int use_sr,
                            uint64_t sr_seed, uint32_t stream_id, uint8_t* codes,
                            uint8_t* scales) {
  if (rows <= 0 || cols <= 0 || cols % 32) return -2;
  const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      float z[32], amax = 0.0f;
      for (int j = 0; j < 32; ++j) {
        z[j] = orc_bf16_to_f32(x[r * cols + 32 * b + j]);
        float a = fabsf(z[j]);
        if (a > amax) amax = a;
      }
      const uint8_t sc = orc_e8m0_encode(amax);
      scales[r * nb + b] = sc;
      const float inv = ldexpf(1.0f, 127 - (int)sc);   /* 2^-e, a power of two */
      for (int j = 0; j < 32; ++j) {
        const float v = z[j] * inv;
        const int64_t k = 32 * b + j;
        uint8_t c;
        if (use_sr)
          c = orc_e2m1_sr(v, orc_sr_bits(sr_seed, stream_id, (uint64_t)(r * cols + k)));
        else
          c = orc_e2m1_rtn(v);
        uint8_t* byte = &codes[r * (cols / 2) + k / 2];
        if (k % 2 == 0) *byte = (uint8_t)((*byte & 0xF0) | c);
        else *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
      }
    }
  }
  return 0;
}

/* x_hat[r][k] = E2M1(code) * 2^(e - 127) in binary32 (exact unless the result
 * is below the binary32 subnormal range, where it rounds once). */
ORC_API void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t k, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const uint8_t b = codes[r * (k / 2) + c / 2];
      const uint8_t q = (c % 2 == 0) ? (uint8_t)(b & 0xF) : (uint8_t)(b >> 4);
      out[r * k + c] = orc_e2m1_decode(q) * orc_e8m0_decode(scales[r * (k / 32) + c / 32]);
    }
}

static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t k_total, int64_t r,
                       int64_t k) {
  const uint8_t b = codes[r * (k_total / 2) + k / 2];
  const uint8_t q = (k % 2 == 0) ? (uint8_t)(b & 0xF) : (uint8_t)(b >> 4);
  return (double)orc_e2m1_decode(q) * ldexp(1.0, (int)scales[r * (k_total / 32) + k / 32] - 127);
}

static void mx_one(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                   int64_t K, int64_t m, int64_t n, double* c, double* t) {
  double acc = 0.0, abs_acc = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double p = mx_value(ac, as, K, m, k) * mx_value(bc, bs, K, n, k);
    acc += p;
    abs_acc += fabs(p);
  }
  *c = acc;
  if (t) *t = abs_acc;
}

/* Every decoded value q * 2^(e - 127) as double, [rows][K] row-major
 * (exact: a power of two times a value with two significant bits).  A
 * float64 matrix product of these is the fast form of the GEMM below. */
ORC_API int orc_mx_decode_exact(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t K, double* out) {
  if (K <= 0 || K % 32) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = mx_value(codes, scales, K, r, k);
  return 0;
}

/* C[m][n] = sum_k A[m,k] * B[n,k]; A [M][K], B [N][K] MXFP4 (rowwise);
 * c, t [M][N] (t nullable). */
ORC_API int orc_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t M, const uint8_t* bc,
                        const uint8_t* bs, int64_t N, int64_t K, double* c, double* t) {
  if (K <= 0 || K % 32) return -2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      mx_one(ac, as, bc, bs, K, m, n, &c[m * N + n], t ? &t[m * N + n] : NULL);
  return 0;
}

ORC_API int orc_mx_gemm_entries(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                                const uint8_t* bs, int64_t K, const int64_t* ms,
                                const int64_t* ns, int64_t count, double* c, double* t) {
  if (K <= 0 || K % 32) return -2;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < count; ++j) mx_one(ac, as, bc, bs, K, ms[j], ns[j], &c[j], &t[j]);
  return 0;
}
