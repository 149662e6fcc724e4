/* oracle_driver.c -- runs the CPU reference (nvfp4_oracle.c, mxfp4_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: every quantizer mode
 * (rowwise, colwise, 2D with transposed codes, RHT along either axis, RTN and
 * SR), dequantize, the exact GEMM and its entry sampler, and the MXFP4
 * functions, on exactly sized heap buffers (so a write or read past any end
 * is reported), over small shapes with all-zero, subnormal, huge, infinite
 * and NaN inputs; plus the scalar codecs over sweeps of binary32 inputs and
 * the rejected shapes.  Declares the reference's functions itself: it shares
 * no header with anything.  Exits non-zero if a call misbehaves. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_amax(const uint16_t* x, int64_t rows, int64_t cols);
float orc_amax_rht(const uint16_t* x, int64_t rows, int64_t cols, uint64_t seed);
int orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int mode, int use_rht,
                 uint64_t rht_seed, int use_sr, uint64_t sr_seed, uint32_t stream_id,
                 int amax_given, float* amax_io, uint8_t* codes, uint8_t* codes_t,
                 uint8_t* scales, float* s_t_out);
void orc_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ss_row,
                    int64_t ss_k, int32_t blk_rows, float tensor_scale, int64_t rows, int64_t k,
                    float* out);
int orc_gemm(const uint8_t* ac, int64_t ald, const uint8_t* as, int64_t assr, int64_t assk,
             int32_t ablk, float ast, int64_t arows, const uint8_t* bc, int64_t bld,
             const uint8_t* bs, int64_t bssr, int64_t bssk, int32_t bblk, float bst, int64_t brows,
             int64_t K, double* c, double* t);
int orc_gemm_entries(const uint8_t* ac, int64_t ald, const uint8_t* as, int64_t assr,
                     int64_t assk, int32_t ablk, float ast, int64_t arows, const uint8_t* bc,
                     int64_t bld, const uint8_t* bs, int64_t bssr, int64_t bssk, int32_t bblk,
                     float bst, int64_t brows, int64_t K, const int64_t* ms, const int64_t* ns,
                     int64_t count, double* c, double* t);
uint8_t orc_e4m3_encode(float x);
uint8_t orc_e2m1_rtn(float v);
uint8_t orc_e2m1_sr(float v, uint16_t u);
uint8_t orc_e8m0_encode(float amax);
int orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int use_sr, uint64_t seed,
                    uint32_t stream_id, uint8_t* codes, uint8_t* scales);
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                       float* out);
int orc_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t M, const uint8_t* bc,
                const uint8_t* bs, int64_t N, int64_t K, double* c, double* t);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (uint32_t)(rng >> 11);
}

/* bf16 pattern of one of several value kinds */
static uint16_t value(int kind) {
  uint16_t b = (uint16_t)next32();
  switch (kind) {
    case 0: return (uint16_t)(0x3C00 + (b & 0x7FF)) ^ (b & 0x8000);  /* ~[2^-7, 2^5) */
    case 1: return (uint16_t)(b & 0x807F);                           /* subnormal / zero */
    case 2: return (uint16_t)(0x7F00 + (b & 0x7F)) ^ (b & 0x8000);   /* huge, NaN */
    case 3: return (uint16_t)(b & 0x8000);                           /* signed zero */
    default: return (uint16_t)(0x7F80 | (b & 0x8000));              /* infinity */
  }
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}

static int quantize_all(int64_t R, int64_t C, int kind) {
  uint16_t* x = xmalloc((size_t)(R * C) * 2);
  for (int64_t i = 0; i < R * C; ++i) x[i] = value(i % 97 == 0 ? 4 - (kind == 0) * 4 : kind);
  int bad = 0;
  for (int mode = 0; mode < 3; ++mode)
    for (int rht = 0; rht < 2; ++rht)
      for (int sr = 0; sr < 2; ++sr)
        for (int given = 0; given < 2; ++given) {
          if (mode == 2 && rht) continue;
          const int64_t I = mode == 1 ? C : R, K = mode == 1 ? R : C;
          uint8_t* codes = xmalloc((size_t)(I * K / 2));
          uint8_t* codes_t = mode == 2 ? xmalloc((size_t)(I * K / 2)) : NULL;
          const int64_t ns = mode == 2 ? (R / 16) * (C / 16) : I * (K / 16);
          uint8_t* scales = xmalloc((size_t)ns);
          float amax = 3.5f, st = 0.0f;
          if (orc_quantize(x, R, C, mode, rht, 11, sr, 13, 2, given, &amax, codes, codes_t,
                           scales, &st) != 0) ++bad;
          if (mode != 2) {
            float* out = xmalloc((size_t)(I * K) * 4);
            orc_dequantize(codes, K / 2, scales, K / 16, 1, 1, st, I, K, out);
            free(out);
          }
          free(codes); free(codes_t); free(scales);
        }
  (void)orc_amax(x, R, C);
  (void)orc_amax_rht(x, R, C, 5);
  uint8_t* mc = xmalloc((size_t)(R * C / 2));
  uint8_t* ms = xmalloc((size_t)(R * C / 32));
  if (C % 32 == 0) {
    if (orc_mx_quantize(x, R, C, 1, 3, 0, mc, ms) != 0) ++bad;
    float* out = xmalloc((size_t)(R * C) * 4);
    orc_mx_dequantize(mc, ms, R, C, out);
    free(out);
  }
  free(mc); free(ms); free(x);
  return bad;
}

static int gemm_all(int64_t M, int64_t N, int64_t K) {
  uint8_t* ac = xmalloc((size_t)(M * K / 2));
  uint8_t* bc = xmalloc((size_t)(N * K / 2));
  uint8_t* as = xmalloc((size_t)(M * K / 16));
  uint8_t* bs = xmalloc((size_t)(N * K / 16));
  for (int64_t i = 0; i < M * K / 2; ++i) ac[i] = (uint8_t)next32();
  for (int64_t i = 0; i < N * K / 2; ++i) bc[i] = (uint8_t)next32();
  for (int64_t i = 0; i < M * K / 16; ++i) as[i] = (uint8_t)(next32() % 127);
  for (int64_t i = 0; i < N * K / 16; ++i) bs[i] = (uint8_t)(next32() % 127);
  double* c = xmalloc((size_t)(M * N) * 8);
  double* t = xmalloc((size_t)(M * N) * 8);
  int bad = orc_gemm(ac, K / 2, as, K / 16, 1, 1, 0.5f, M, bc, K / 2, bs, K / 16, 1, 1, 3.0f, N,
                     K, c, t) != 0;
  int64_t ms[5] = {0, M - 1, 0, M - 1, M / 2}, ns[5] = {0, 0, N - 1, N - 1, N / 2};
  bad += orc_gemm_entries(ac, K / 2, as, K / 16, 1, 1, 0.5f, M, bc, K / 2, bs, K / 16, 1, 1, 3.0f,
                          N, K, ms, ns, 5, c, t) != 0;
  if (K % 32 == 0) {
    uint8_t* mas = xmalloc((size_t)(M * K / 32));
    uint8_t* mbs = xmalloc((size_t)(N * K / 32));
    memcpy(mas, as, (size_t)(M * K / 32));
    memcpy(mbs, bs, (size_t)(N * K / 32));
    bad += orc_mx_gemm(ac, mas, M, bc, mbs, N, K, c, t) != 0;
    free(mas); free(mbs);
  }
  free(ac); free(bc); free(as); free(bs); free(c); free(t);
  return bad;
}

int main(void) {
  int bad = 0;
  const int64_t shapes[][2] = {{16, 16}, {32, 48}, {48, 32}, {64, 96}};
  for (int s = 0; s < 4; ++s)
    for (int kind = 0; kind < 5; ++kind) bad += quantize_all(shapes[s][0], shapes[s][1], kind);
  bad += gemm_all(16, 16, 16);
  bad += gemm_all(48, 32, 96);
  bad += gemm_all(32, 64, 128);
  /* rejected shapes: status, no access */
  uint16_t x16[256] = {0};
  uint8_t b[256];
  float f = 0, g = 0;
  bad += orc_quantize(x16, 16, 24, 0, 0, 0, 0, 0, 0, 0, &f, b, NULL, b, &g) != -2;
  bad += orc_quantize(x16, 0, 16, 0, 0, 0, 0, 0, 0, 0, &f, b, NULL, b, &g) != -2;
  bad += orc_quantize(x16, 16, 16, 3, 0, 0, 0, 0, 0, 0, &f, b, NULL, b, &g) != -4;
  bad += orc_quantize(x16, 16, 16, 2, 1, 0, 0, 0, 0, 0, &f, b, NULL, b, &g) != -4;
  /* scalar codecs over binary32 sweeps, specials included */
  for (uint64_t u = 0; u <= 0xFFFFFFFFull; u += 4093) {
    uint32_t w = (uint32_t)u;
    float v;
    memcpy(&v, &w, 4);
    (void)orc_e4m3_encode(v);
    (void)orc_e2m1_rtn(v);
    (void)orc_e2m1_sr(v, (uint16_t)w);
    (void)orc_e8m0_encode(fabsf(v));
  }
  printf("oracle driver: %d unexpected results\n", bad);
  return bad ? 1 : 0;
}
