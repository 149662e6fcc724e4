// api_driver.cpp -- drives every entry point of libnvfp4's C ABI on the host
// (the launchers are stubs, api_stubs.cpp) with valid arguments, invalid
// ones and extreme sizes, under AddressSanitizer and
// UndefinedBehaviorSanitizer: validation must return the documented status
// without reading or computing out of bounds (no overflowing size arithmetic
// on huge dimensions).  Device pointers are never dereferenced by the
// validation layer, so aligned host addresses stand in for them.  Exits
// non-zero on the first unexpected status.
#include <cstdint>
#include <cstdio>

#include "nvfp4.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, \
                   got_, (int)(want), nvfp4_last_error());                              \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

alignas(256) static unsigned char dev[1 << 16];   // stands in for device memory

int main() {
  void* X = dev;
  float* F = reinterpret_cast<float*>(dev + 256);
  uint8_t* B = dev + 512;
  uint8_t* MIS = dev + 513;
  const int64_t BIG = int64_t(1) << 62, HUGE_COLS = int64_t(1) << 28;
  const int OK = NVFP4_OK, ESHAPE = NVFP4_ERR_SHAPE, ENULL = NVFP4_ERR_NULL,
            EALIGN = NVFP4_ERR_ALIGN, EARG = NVFP4_ERR_ARG;

  // amax
  EXPECT(nvfp4_amax(X, 16, 16, F, nullptr), OK);
  EXPECT(nvfp4_amax(nullptr, 16, 16, F, nullptr), ENULL);
  EXPECT(nvfp4_amax(X, 16, 24, F, nullptr), ESHAPE);
  EXPECT(nvfp4_amax(X, BIG, HUGE_COLS, F, nullptr), ESHAPE);
  EXPECT(nvfp4_amax(X, INT64_MIN, 16, F, nullptr), ESHAPE);
  EXPECT(nvfp4_amax_rht(X, BIG, 16, 3, F, nullptr), ESHAPE);
  EXPECT(nvfp4_amax_both(X, 32, 16, 3, F, F + 1, nullptr), OK);
  EXPECT(nvfp4_amax_both(X, 32, 16, 3, F, F, nullptr), EARG);
  EXPECT(nvfp4_amax_rht1d(X, 32, 16, NVFP4_ROWWISE, 3, F, nullptr), OK);
  EXPECT(nvfp4_amax_rht1d(X, BIG, HUGE_COLS, NVFP4_ROWWISE, 3, F, nullptr), ESHAPE);
  EXPECT(nvfp4_amax_rht1d(X, 32, 16, 7, 3, F, nullptr), EARG);

  // quantizers
  for (int axis = 0; axis < 2; ++axis) {
    EXPECT(nvfp4_quantize1d_rtn(X, 64, 32, axis, F, NVFP4_AMAX_COMPUTE, B, B, F + 1, nullptr), OK);
    EXPECT(nvfp4_quantize1d_sr(X, 64, 32, axis, F, NVFP4_AMAX_GIVEN, 7, 1, B, B, F + 1, nullptr),
           OK);
    EXPECT(nvfp4_quantize1d_rtn(X, BIG, HUGE_COLS, axis, F, 0, B, B, F + 1, nullptr), ESHAPE);
    EXPECT(nvfp4_quantize1d_rtn(X, 64, 32, axis, F, 0, MIS, B, F + 1, nullptr), EALIGN);
    EXPECT(nvfp4_rht_quantize1d(X, 64, 32, axis, 5, 1, 7, 0, F, 0, B, B, F + 1, nullptr), OK);
    EXPECT(nvfp4_rht_quantize1d(X, BIG, HUGE_COLS, axis, 5, 1, 7, 0, F, 0, B, B, F + 1, nullptr),
           ESHAPE);
  }
  EXPECT(nvfp4_quantize1d_rtn(X, 64, 32, 2, F, 0, B, B, F + 1, nullptr), EARG);
  EXPECT(nvfp4_quantize2d_rtn(X, 64, 32, F, 0, B, B, B, B, F + 1, nullptr), OK);
  EXPECT(nvfp4_quantize2d_sr(X, 64, 32, F, 1, 9, 2, B, nullptr, B, nullptr, F + 1, nullptr), OK);
  EXPECT(nvfp4_quantize2d_rtn(X, BIG, HUGE_COLS, F, 0, B, B, B, B, F + 1, nullptr), ESHAPE);
  EXPECT(nvfp4_rht_quantize(X, 64, 32, 5, 0, 0, 0, F, 0, B, B, F + 1, nullptr), OK);
  EXPECT(nvfp4_rht_quantize(X, BIG, HUGE_COLS, 5, 0, 0, 0, F, 0, B, B, F + 1, nullptr), ESHAPE);
  EXPECT(nvfp4_quantize_row_rht(X, 64, 32, 5, 1, 7, 0, 1, F, F + 1, B, B, F + 2, B, B, F + 3,
                                nullptr), OK);
  EXPECT(nvfp4_quantize_row_rht(X, BIG, HUGE_COLS, 5, 1, 7, 0, 1, F, F + 1, B, B, F + 2, B, B,
                                F + 3, nullptr), ESHAPE);
  EXPECT(mxfp4_quantize(X, 64, 32, 1, 7, 0, B, B, nullptr), OK);
  EXPECT(mxfp4_quantize(X, BIG, HUGE_COLS, 1, 7, 0, B, B, nullptr), ESHAPE);

  // operands, dequantize, GEMMs
  nvfp4_operand a{B, 16, B, 2, 1, 1, F, 256, 32};
  nvfp4_operand b{B, 16, B, 2, 1, 1, F, 512, 32};
  EXPECT(nvfp4_dequantize(&a, F, nullptr), OK);
  EXPECT(nvfp4_gemm(&a, &b, F, 512, nullptr), OK);
  EXPECT(nvfp4_gemm_bf16(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, nullptr, 0, nullptr), OK);
  // the stub workspace need is 4096 bytes
  EXPECT(nvfp4_gemm_bf16(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, dev + 4096, 4096,
                         nullptr), OK);
  EXPECT(nvfp4_gemm_bf16(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, dev + 4096, 4095,
                         nullptr), EARG);
  EXPECT(nvfp4_gemm_bf16(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, dev + 4100, 4096,
                         nullptr), EALIGN);
  EXPECT(nvfp4_gemm_bf16(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, nullptr, 16, nullptr),
         EARG);
  EXPECT(nvfp4_gemm_bf16_noalloc(&a, &b, reinterpret_cast<uint16_t*>(F), 512, F, nullptr), OK);
  EXPECT(nvfp4_gemm_bf16_noalloc(&a, &b, reinterpret_cast<uint16_t*>(F), 256, F, nullptr),
         ESHAPE);
  EXPECT(nvfp4_gemm_bf16_noalloc_max_bytes(), 8192);
  EXPECT(nvfp4_gemm_bf16_workspace_bytes(256, 512, 32), 4096);
  EXPECT(nvfp4_gemm_bf16_workspace_bytes(0, 512, 32), ESHAPE);
  nvfp4_operand huge = a;
  huge.rows = BIG;
  EXPECT(nvfp4_dequantize(&huge, F, nullptr), ESHAPE);
  EXPECT(nvfp4_gemm(&huge, &b, F, 512, nullptr), ESHAPE);
  EXPECT(nvfp4_gemm(&a, &huge, F, BIG, nullptr), ESHAPE);
  nvfp4_operand wide = a;
  wide.k = BIG;
  wide.ld_codes = BIG;
  EXPECT(nvfp4_dequantize(&wide, F, nullptr), ESHAPE);
  nvfp4_operand strided = a;
  strided.ss_row = BIG;
  EXPECT(nvfp4_gemm(&strided, &b, F, 512, nullptr), ESHAPE);
  EXPECT(nvfp4_gemm(&a, &b, F, BIG, nullptr), ESHAPE);
  mxfp4_operand ma{B, 16, B, 1, 256, 32};
  mxfp4_operand mb{B, 16, B, 1, 512, 32};
  EXPECT(mxfp4_dequantize(&ma, F, nullptr), OK);
  EXPECT(mxfp4_gemm(&ma, &mb, F, 512, nullptr), OK);
  mxfp4_operand mh = ma;
  mh.rows = BIG;
  EXPECT(mxfp4_dequantize(&mh, F, nullptr), ESHAPE);
  EXPECT(mxfp4_gemm(&ma, &mb, F, BIG, nullptr), ESHAPE);

  // measurement support
  EXPECT(nvfp4_probe_mfma(1, 10, dev, nvfp4_probe_scratch_bytes(), nullptr), OK);
  EXPECT(nvfp4_probe_clock(dev, nvfp4_probe_clock_bytes(), nullptr), OK);
  EXPECT(nvfp4_probe_copy(dev, dev + 1024, 1024, nullptr), OK);
  EXPECT(nvfp4_probe_copy(dev, dev + 1024, BIG + 16, nullptr), ESHAPE);

  for (int s = -6; s <= 0; ++s)
    if (nvfp4_status_string(s) == nullptr) ++failures;
  std::printf("launches reached: %d, unexpected statuses: %d\n", g_launches, failures);
  return failures ? 1 : 0;
}
