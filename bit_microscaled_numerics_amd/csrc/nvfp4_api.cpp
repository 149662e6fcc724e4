// nvfp4_api.cpp -- the C ABI of libnvfp4.so (declared in include/nvfp4.h):
// argument validation, then kernel launches on the caller's stream.  Nothing
// here allocates, frees or synchronises.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "nvfp4_kernels.h"

namespace {

thread_local char g_last_error[256] = "";

// No tensor or buffer the library touches may exceed 2^40 elements or bytes
// (far beyond the 288 GB of one MI355X): with that bound every size, offset
// and grid computation here and in the launchers stays within int64 (and the
// grids within their 32-bit dimensions).
constexpr int64_t kMaxElems = int64_t(1) << 40;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_tensor(const void* x, int64_t rows, int64_t cols, const char* name) {
  if (x == nullptr) return fail(NVFP4_ERR_NULL, "%s is NULL", name);
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16)
    return fail(NVFP4_ERR_SHAPE, "%s: rows=%lld cols=%lld must be positive multiples of 16", name,
                (long long)rows, (long long)cols);
  if (cols > (int64_t(1) << 28))
    return fail(NVFP4_ERR_SHAPE, "%s: cols=%lld exceeds 2^28", name, (long long)cols);
  if (rows > kMaxElems / cols)
    return fail(NVFP4_ERR_SHAPE, "%s: rows*cols exceeds 2^40 elements", name);
  if (!aligned(x, 16)) return fail(NVFP4_ERR_ALIGN, "%s must be 16-byte aligned", name);
  return NVFP4_OK;
}

int check_outputs(const void* codes, const void* scales, const float* amax_io,
                  const float* ts_out) {
  if (codes == nullptr) return fail(NVFP4_ERR_NULL, "codes is NULL");
  if (scales == nullptr) return fail(NVFP4_ERR_NULL, "scales_e4m3 is NULL");
  if (amax_io == nullptr) return fail(NVFP4_ERR_NULL, "amax_io is NULL");
  if (ts_out == nullptr) return fail(NVFP4_ERR_NULL, "tensor_scale_out is NULL");
  if (!aligned(codes, 16)) return fail(NVFP4_ERR_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(amax_io, 4) || !aligned(ts_out, 4))
    return fail(NVFP4_ERR_ALIGN, "amax_io / tensor_scale_out must be 4-byte aligned");
  return NVFP4_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return NVFP4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_operand(const nvfp4_operand* q, const char* name) {
  if (q == nullptr) return fail(NVFP4_ERR_NULL, "%s is NULL", name);
  if (q->codes == nullptr || q->scales == nullptr || q->tensor_scale == nullptr)
    return fail(NVFP4_ERR_NULL, "%s: codes, scales and tensor_scale are required", name);
  if (q->rows <= 0 || q->k <= 0 || q->rows % 16 || q->k % 16)
    return fail(NVFP4_ERR_SHAPE, "%s: rows=%lld k=%lld must be positive multiples of 16", name,
                (long long)q->rows, (long long)q->k);
  if (q->ld_codes < q->k / 2)
    return fail(NVFP4_ERR_SHAPE, "%s: ld_codes=%lld < k/2", name, (long long)q->ld_codes);
  if (q->ld_codes % 8)
    return fail(NVFP4_ERR_ALIGN, "%s: ld_codes=%lld must be a multiple of 8", name,
                (long long)q->ld_codes);
  if (!aligned(q->codes, 16)) return fail(NVFP4_ERR_ALIGN, "%s: codes must be 16-byte aligned", name);
  if (q->blk_rows != 1 && q->blk_rows != 16)
    return fail(NVFP4_ERR_ARG, "%s: blk_rows must be 1 or 16", name);
  if (q->ss_row < 0 || q->ss_k < 0) return fail(NVFP4_ERR_ARG, "%s: negative scale stride", name);
  if (q->ld_codes > kMaxElems || q->rows > kMaxElems / q->ld_codes)
    return fail(NVFP4_ERR_SHAPE, "%s: rows*ld_codes exceeds 2^40 bytes", name);
  const int64_t rb = (q->rows - 1) / q->blk_rows, kb = (q->k - 1) / 16;
  if ((q->ss_row > 0 && rb > kMaxElems / q->ss_row) || (q->ss_k > 0 && kb > kMaxElems / q->ss_k))
    return fail(NVFP4_ERR_SHAPE, "%s: scale index span exceeds 2^40", name);
  return NVFP4_OK;
}

// C [M][ldc] (elements) must stay within the size bound.
int check_ldc(int64_t ldc, int64_t m, const char* name) {
  if (ldc > kMaxElems / m)
    return fail(NVFP4_ERR_SHAPE, "%s: M*ldc exceeds 2^40 elements", name);
  return NVFP4_OK;
}

nvfp4::GemmOperand to_kernel(const nvfp4_operand* q) {
  const int64_t last = ((q->rows - 1) / q->blk_rows) * q->ss_row + ((q->k - 1) / 16) * q->ss_k;
  return nvfp4::GemmOperand{q->codes, q->ld_codes, q->scales, q->ss_row, q->ss_k,
                            q->blk_rows, q->tensor_scale, q->rows, last + 1};
}

// The GEMM addresses a 256-row slab of codes and the scale array with 32-bit
// buffer offsets.
int check_gemm_extent(const nvfp4_operand* q, const char* name) {
  const int64_t last = ((q->rows - 1) / q->blk_rows) * q->ss_row + ((q->k - 1) / 16) * q->ss_k;
  if (q->ld_codes > (int64_t(1) << 22) || last >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_SHAPE, "%s: codes row pitch or scale array beyond the 32-bit offset range",
                name);
  return NVFP4_OK;
}

}  // namespace

namespace nvfp4 {
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace nvfp4

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN";
    case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG";
    case NVFP4_ERR_LAUNCH: return "NVFP4_ERR_LAUNCH";
    default: return "NVFP4_ERR_UNKNOWN";
  }
}

const char* nvfp4_last_error(void) { return g_last_error; }

int nvfp4_amax(const void* x, int64_t rows, int64_t cols, float* amax_out, void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if (amax_out == nullptr) return fail(NVFP4_ERR_NULL, "amax_out is NULL");
  if (!aligned(amax_out, 4)) return fail(NVFP4_ERR_ALIGN, "amax_out must be 4-byte aligned");
  return launched(nvfp4::launch_amax(x, rows * cols, amax_out, as_stream(stream)));
}

int nvfp4_amax_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed, float* amax_out,
                   void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if (amax_out == nullptr) return fail(NVFP4_ERR_NULL, "amax_out is NULL");
  if (!aligned(amax_out, 4)) return fail(NVFP4_ERR_ALIGN, "amax_out must be 4-byte aligned");
  return launched(nvfp4::launch_amax_rht(x, rows, cols, rht_seed, amax_out, as_stream(stream)));
}

int nvfp4_amax_both(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed, float* amax_out,
                    float* amax_rht_out, void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if (amax_out == nullptr || amax_rht_out == nullptr)
    return fail(NVFP4_ERR_NULL, "amax_out / amax_rht_out is NULL");
  if (!aligned(amax_out, 4) || !aligned(amax_rht_out, 4))
    return fail(NVFP4_ERR_ALIGN, "amax_out / amax_rht_out must be 4-byte aligned");
  if (amax_out == amax_rht_out) return fail(NVFP4_ERR_ARG, "amax_out and amax_rht_out alias");
  return launched(nvfp4::launch_amax_rht(x, rows, cols, rht_seed, amax_rht_out, as_stream(stream),
                                         amax_out));
}

static int quantize1d(const void* x, int64_t rows, int64_t cols, int axis, float* amax_io,
                      int amax_mode, bool sr, uint64_t seed, uint32_t stream_id, uint8_t* codes,
                      uint8_t* scales, float* ts_out, void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if ((st = check_outputs(codes, scales, amax_io, ts_out))) return st;
  if (axis != NVFP4_ROWWISE && axis != NVFP4_COLWISE)
    return fail(NVFP4_ERR_ARG, "axis=%d is neither NVFP4_ROWWISE nor NVFP4_COLWISE", axis);
  if (amax_mode != NVFP4_AMAX_COMPUTE && amax_mode != NVFP4_AMAX_GIVEN)
    return fail(NVFP4_ERR_ARG, "amax_mode=%d out of range", amax_mode);
  hipStream_t s = as_stream(stream);
  if (amax_mode == NVFP4_AMAX_COMPUTE) {
    hipError_t e = nvfp4::launch_amax(x, rows * cols, amax_io, s);
    if (e != hipSuccess) return launched(e);
  }
  if (axis == NVFP4_ROWWISE)
    return launched(nvfp4::launch_quant_row(x, rows, cols, amax_io, false, 0, sr, seed, stream_id,
                                            codes, scales, ts_out, s));
  return launched(nvfp4::launch_quant_col(x, rows, cols, amax_io, false, 0, sr, seed, stream_id,
                                          codes, scales, ts_out, s));
}

int nvfp4_quantize1d_rtn(const void* x, int64_t rows, int64_t cols, int axis, float* amax_io,
                         int amax_mode, uint8_t* codes, uint8_t* scales, float* ts_out,
                         void* stream) {
  return quantize1d(x, rows, cols, axis, amax_io, amax_mode, false, 0, 0, codes, scales, ts_out,
                    stream);
}

int nvfp4_quantize1d_sr(const void* x, int64_t rows, int64_t cols, int axis, float* amax_io,
                        int amax_mode, uint64_t seed, uint32_t stream_id, uint8_t* codes,
                        uint8_t* scales, float* ts_out, void* stream) {
  return quantize1d(x, rows, cols, axis, amax_io, amax_mode, true, seed, stream_id, codes, scales,
                    ts_out, stream);
}

static int quantize2d(const void* w, int64_t rows, int64_t cols, float* amax_io, int amax_mode,
                      bool sr, uint64_t seed, uint32_t stream_id, uint8_t* codes,
                      uint8_t* codes_t, uint8_t* scales, uint8_t* scales_t, float* ts_out,
                      void* stream) {
  int st = check_tensor(w, rows, cols, "w");
  if (st) return st;
  if ((st = check_outputs(codes, scales, amax_io, ts_out))) return st;
  if (codes_t != nullptr && !aligned(codes_t, 16))
    return fail(NVFP4_ERR_ALIGN, "codes_t must be 16-byte aligned");
  if (amax_mode != NVFP4_AMAX_COMPUTE && amax_mode != NVFP4_AMAX_GIVEN)
    return fail(NVFP4_ERR_ARG, "amax_mode=%d out of range", amax_mode);
  hipStream_t s = as_stream(stream);
  if (amax_mode == NVFP4_AMAX_COMPUTE) {
    hipError_t e = nvfp4::launch_amax(w, rows * cols, amax_io, s);
    if (e != hipSuccess) return launched(e);
  }
  return launched(nvfp4::launch_quant_2d(w, rows, cols, amax_io, sr, seed, stream_id, codes,
                                         codes_t, scales, scales_t, ts_out, s));
}

int nvfp4_quantize2d_rtn(const void* w, int64_t rows, int64_t cols, float* amax_io, int amax_mode,
                         uint8_t* codes, uint8_t* codes_t, uint8_t* scales, uint8_t* scales_t,
                         float* ts_out, void* stream) {
  return quantize2d(w, rows, cols, amax_io, amax_mode, false, 0, 0, codes, codes_t, scales,
                    scales_t, ts_out, stream);
}

int nvfp4_quantize2d_sr(const void* w, int64_t rows, int64_t cols, float* amax_io, int amax_mode,
                        uint64_t seed, uint32_t stream_id, uint8_t* codes, uint8_t* codes_t,
                        uint8_t* scales, uint8_t* scales_t, float* ts_out, void* stream) {
  return quantize2d(w, rows, cols, amax_io, amax_mode, true, seed, stream_id, codes, codes_t,
                    scales, scales_t, ts_out, stream);
}

int nvfp4_rht_quantize(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed, int use_sr,
                       uint64_t sr_seed, uint32_t stream_id, float* amax_io, int amax_mode,
                       uint8_t* codes, uint8_t* scales, float* ts_out, void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if ((st = check_outputs(codes, scales, amax_io, ts_out))) return st;
  if (use_sr != 0 && use_sr != 1) return fail(NVFP4_ERR_ARG, "use_sr=%d must be 0 or 1", use_sr);
  if (amax_mode != NVFP4_AMAX_COMPUTE && amax_mode != NVFP4_AMAX_GIVEN)
    return fail(NVFP4_ERR_ARG, "amax_mode=%d out of range", amax_mode);
  hipStream_t s = as_stream(stream);
  if (amax_mode == NVFP4_AMAX_COMPUTE) {
    hipError_t e = nvfp4::launch_amax_rht(x, rows, cols, rht_seed, amax_io, s);
    if (e != hipSuccess) return launched(e);
  }
  return launched(nvfp4::launch_quant_col(x, rows, cols, amax_io, true, rht_seed, use_sr == 1,
                                          sr_seed, stream_id, codes, scales, ts_out, s));
}

int nvfp4_amax_rht1d(const void* x, int64_t rows, int64_t cols, int axis, uint64_t rht_seed,
                     float* amax_out, void* stream) {
  if (axis != NVFP4_ROWWISE && axis != NVFP4_COLWISE)
    return fail(NVFP4_ERR_ARG, "axis=%d is neither NVFP4_ROWWISE nor NVFP4_COLWISE", axis);
  if (axis == NVFP4_COLWISE) return nvfp4_amax_rht(x, rows, cols, rht_seed, amax_out, stream);
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if (amax_out == nullptr) return fail(NVFP4_ERR_NULL, "amax_out is NULL");
  if (!aligned(amax_out, 4)) return fail(NVFP4_ERR_ALIGN, "amax_out must be 4-byte aligned");
  return launched(nvfp4::launch_amax_rht_row(x, rows * cols, rht_seed, amax_out,
                                             as_stream(stream)));
}

int nvfp4_rht_quantize1d(const void* x, int64_t rows, int64_t cols, int axis, uint64_t rht_seed,
                         int use_sr, uint64_t sr_seed, uint32_t stream_id, float* amax_io,
                         int amax_mode, uint8_t* codes, uint8_t* scales, float* ts_out,
                         void* stream) {
  if (axis != NVFP4_ROWWISE && axis != NVFP4_COLWISE)
    return fail(NVFP4_ERR_ARG, "axis=%d is neither NVFP4_ROWWISE nor NVFP4_COLWISE", axis);
  if (axis == NVFP4_COLWISE)
    return nvfp4_rht_quantize(x, rows, cols, rht_seed, use_sr, sr_seed, stream_id, amax_io,
                              amax_mode, codes, scales, ts_out, stream);
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if ((st = check_outputs(codes, scales, amax_io, ts_out))) return st;
  if (use_sr != 0 && use_sr != 1) return fail(NVFP4_ERR_ARG, "use_sr=%d must be 0 or 1", use_sr);
  if (amax_mode != NVFP4_AMAX_COMPUTE && amax_mode != NVFP4_AMAX_GIVEN)
    return fail(NVFP4_ERR_ARG, "amax_mode=%d out of range", amax_mode);
  hipStream_t s = as_stream(stream);
  if (amax_mode == NVFP4_AMAX_COMPUTE) {
    hipError_t e = nvfp4::launch_amax_rht_row(x, rows * cols, rht_seed, amax_io, s);
    if (e != hipSuccess) return launched(e);
  }
  return launched(nvfp4::launch_quant_row(x, rows, cols, amax_io, true, rht_seed, use_sr == 1,
                                          sr_seed, stream_id, codes, scales, ts_out, s));
}

int nvfp4_quantize_row_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed,
                           int use_sr, uint64_t sr_seed, uint32_t stream_id_row,
                           uint32_t stream_id_rht, const float* amax_row, const float* amax_rht,
                           uint8_t* codes_row, uint8_t* scales_row, float* ts_row_out,
                           uint8_t* codes_rht, uint8_t* scales_rht, float* ts_rht_out,
                           void* stream) {
  int st = check_tensor(x, rows, cols, "x");
  if (st) return st;
  if ((st = check_outputs(codes_row, scales_row, amax_row, ts_row_out))) return st;
  if ((st = check_outputs(codes_rht, scales_rht, amax_rht, ts_rht_out))) return st;
  if (use_sr != 0 && use_sr != 1) return fail(NVFP4_ERR_ARG, "use_sr=%d must be 0 or 1", use_sr);
  return launched(nvfp4::launch_quant_row_rht(x, rows, cols, rht_seed, use_sr == 1, sr_seed,
                                              stream_id_row, stream_id_rht, amax_row, amax_rht,
                                              codes_row, scales_row, ts_row_out, codes_rht,
                                              scales_rht, ts_rht_out, as_stream(stream)));
}

int nvfp4_dequantize(const nvfp4_operand* q, float* out, void* stream) {
  int st = check_operand(q, "q");
  if (st) return st;
  if (out == nullptr) return fail(NVFP4_ERR_NULL, "out is NULL");
  if (!aligned(out, 16)) return fail(NVFP4_ERR_ALIGN, "out must be 16-byte aligned");
  return launched(nvfp4::launch_dequant(q->codes, q->ld_codes, q->scales, q->ss_row, q->ss_k,
                                        q->blk_rows, q->tensor_scale, q->rows, q->k, out,
                                        as_stream(stream)));
}

int nvfp4_gemm(const nvfp4_operand* a, const nvfp4_operand* b, float* c, int64_t ldc,
               void* stream) {
  int st = check_operand(a, "a");
  if (st) return st;
  if ((st = check_operand(b, "b"))) return st;
  if ((st = check_gemm_extent(a, "a"))) return st;
  if ((st = check_gemm_extent(b, "b"))) return st;
  if (a->k != b->k)
    return fail(NVFP4_ERR_SHAPE, "a.k=%lld != b.k=%lld", (long long)a->k, (long long)b->k);
  if (c == nullptr) return fail(NVFP4_ERR_NULL, "c is NULL");
  if (!aligned(c, 4)) return fail(NVFP4_ERR_ALIGN, "c must be 4-byte aligned");
  if (ldc < b->rows) return fail(NVFP4_ERR_SHAPE, "ldc=%lld < N=%lld", (long long)ldc,
                                 (long long)b->rows);
  if ((st = check_ldc(ldc, a->rows, "c"))) return st;
  return launched(nvfp4::launch_gemm(to_kernel(a), to_kernel(b), a->k, c, ldc,
                                     as_stream(stream)));
}

// The operand and output checks shared by the two BF16-output GEMM entries.
static int check_gemm_bf16(const nvfp4_operand* a, const nvfp4_operand* b, const uint16_t* c,
                           int64_t ldc, const float* amax_out) {
  int st = check_operand(a, "a");
  if (st) return st;
  if ((st = check_operand(b, "b"))) return st;
  if ((st = check_gemm_extent(a, "a"))) return st;
  if ((st = check_gemm_extent(b, "b"))) return st;
  if (a->k != b->k)
    return fail(NVFP4_ERR_SHAPE, "a.k=%lld != b.k=%lld", (long long)a->k, (long long)b->k);
  if (c == nullptr) return fail(NVFP4_ERR_NULL, "c is NULL");
  if (!aligned(c, 2)) return fail(NVFP4_ERR_ALIGN, "c must be 2-byte aligned");
  if (amax_out != nullptr && !aligned(amax_out, 4))
    return fail(NVFP4_ERR_ALIGN, "amax_out must be 4-byte aligned");
  if (ldc < b->rows) return fail(NVFP4_ERR_SHAPE, "ldc=%lld < N=%lld", (long long)ldc,
                                 (long long)b->rows);
  return check_ldc(ldc, a->rows, "c");
}

int64_t nvfp4_gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(NVFP4_ERR_SHAPE, "M=%lld N=%lld K=%lld must be positive", (long long)M,
                (long long)N, (long long)K);
  return nvfp4::gemm_bf16_workspace_bytes(M, N, K);
}

int nvfp4_gemm_bf16(const nvfp4_operand* a, const nvfp4_operand* b, uint16_t* c, int64_t ldc,
                    float* amax_out, void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_gemm_bf16(a, b, c, ldc, amax_out);
  if (st) return st;
  if (workspace == nullptr) {
    if (workspace_bytes != 0)
      return fail(NVFP4_ERR_ARG, "workspace is NULL but workspace_bytes=%lld",
                  (long long)workspace_bytes);
  } else {
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "workspace must be 256-byte aligned");
    const int64_t need = nvfp4::gemm_bf16_workspace_bytes(a->rows, b->rows, a->k);
    if (workspace_bytes < need)
      return fail(NVFP4_ERR_ARG, "workspace_bytes=%lld < %lld (nvfp4_gemm_bf16_workspace_bytes)",
                  (long long)workspace_bytes, (long long)need);
  }
  return launched(nvfp4::launch_gemm_bf16(to_kernel(a), to_kernel(b), a->k, c, ldc, amax_out,
                                          workspace, workspace_bytes, as_stream(stream)));
}

int64_t nvfp4_gemm_bf16_noalloc_max_bytes(void) { return nvfp4::gemm_bf16_noalloc_max_bytes(); }

int nvfp4_gemm_bf16_noalloc(const nvfp4_operand* a, const nvfp4_operand* b, uint16_t* c,
                            int64_t ldc, float* amax_out, void* stream) {
  int st = check_gemm_bf16(a, b, c, ldc, amax_out);
  if (st) return st;
  const int64_t need = nvfp4::gemm_bf16_workspace_bytes(a->rows, b->rows, a->k);
  if (need > nvfp4::gemm_bf16_noalloc_max_bytes())
    return fail(NVFP4_ERR_SHAPE, "M=%lld N=%lld K=%lld needs %lld workspace bytes, above the "
                "%lld this entry point holds", (long long)a->rows, (long long)b->rows,
                (long long)a->k, (long long)need, (long long)nvfp4::gemm_bf16_noalloc_max_bytes());
  return launched(nvfp4::launch_gemm_bf16_noalloc(to_kernel(a), to_kernel(b), a->k, c, ldc,
                                                  amax_out, as_stream(stream)));
}

// ---------------------------------------------------------------- MXFP4

int mxfp4_quantize(const void* x, int64_t rows, int64_t cols, int use_sr, uint64_t seed,
                   uint32_t stream_id, uint8_t* codes, uint8_t* scales, void* stream) {
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(NVFP4_ERR_NULL, "x, codes and scales_e8m0 are required");
  if (rows <= 0 || cols <= 0 || cols % 32)
    return fail(NVFP4_ERR_SHAPE, "rows=%lld cols=%lld: rows > 0, cols a positive multiple of 32",
                (long long)rows, (long long)cols);
  if (cols > kMaxElems || rows > kMaxElems / cols)
    return fail(NVFP4_ERR_SHAPE, "rows*cols exceeds 2^40 elements");
  if (!aligned(x, 16)) return fail(NVFP4_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(codes, 4)) return fail(NVFP4_ERR_ALIGN, "codes must be 4-byte aligned");
  if (use_sr != 0 && use_sr != 1) return fail(NVFP4_ERR_ARG, "use_sr=%d must be 0 or 1", use_sr);
  return launched(nvfp4::launch_mx_quant_row(x, rows, cols, use_sr == 1, seed, stream_id, codes,
                                             scales, as_stream(stream)));
}

static int check_mx_operand(const mxfp4_operand* q, const char* name, int64_t code_align) {
  if (q == nullptr) return fail(NVFP4_ERR_NULL, "%s is NULL", name);
  if (q->codes == nullptr || q->scales == nullptr)
    return fail(NVFP4_ERR_NULL, "%s: codes and scales are required", name);
  if (q->rows <= 0 || q->k <= 0 || q->k % 32)
    return fail(NVFP4_ERR_SHAPE, "%s: rows=%lld k=%lld: rows > 0, k a positive multiple of 32",
                name, (long long)q->rows, (long long)q->k);
  if (q->ld_codes < q->k / 2 || q->ld_scales < q->k / 32)
    return fail(NVFP4_ERR_SHAPE, "%s: ld_codes >= k/2 and ld_scales >= k/32 required", name);
  if (q->ld_codes > kMaxElems || q->rows > kMaxElems / q->ld_codes ||
      q->rows > kMaxElems / q->ld_scales)
    return fail(NVFP4_ERR_SHAPE, "%s: rows*ld_codes or rows*ld_scales exceeds 2^40", name);
  if (q->ld_codes % code_align || !aligned(q->codes, (uintptr_t)code_align))
    return fail(NVFP4_ERR_ALIGN, "%s: codes and ld_codes must be %lld-byte aligned", name,
                (long long)code_align);
  if (q->ld_codes > (int64_t(1) << 22) || q->rows * q->ld_scales >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_SHAPE, "%s: codes row pitch or scale array beyond the 32-bit offset range",
                name);
  return NVFP4_OK;
}

static nvfp4::MxOperand mx_kernel(const mxfp4_operand* q) {
  return nvfp4::MxOperand{q->codes, q->ld_codes, q->scales, q->ld_scales, q->rows, q->k};
}

int mxfp4_dequantize(const mxfp4_operand* q, float* out, void* stream) {
  int st = check_mx_operand(q, "q", 4);
  if (st) return st;
  if (out == nullptr) return fail(NVFP4_ERR_NULL, "out is NULL");
  if (!aligned(out, 16)) return fail(NVFP4_ERR_ALIGN, "out must be 16-byte aligned");
  return launched(nvfp4::launch_mx_dequant(mx_kernel(q), out, as_stream(stream)));
}

int mxfp4_gemm(const mxfp4_operand* a, const mxfp4_operand* b, float* c, int64_t ldc,
               void* stream) {
  int st = check_mx_operand(a, "a", 16);
  if (st) return st;
  if ((st = check_mx_operand(b, "b", 16))) return st;
  if (a->k != b->k)
    return fail(NVFP4_ERR_SHAPE, "a.k=%lld != b.k=%lld", (long long)a->k, (long long)b->k);
  if (c == nullptr) return fail(NVFP4_ERR_NULL, "c is NULL");
  if (!aligned(c, 4)) return fail(NVFP4_ERR_ALIGN, "c must be 4-byte aligned");
  if (ldc < b->rows) return fail(NVFP4_ERR_SHAPE, "ldc=%lld < N=%lld", (long long)ldc,
                                 (long long)b->rows);
  if ((st = check_ldc(ldc, a->rows, "c"))) return st;
  return launched(nvfp4::launch_mx_gemm(mx_kernel(a), mx_kernel(b), a->k, c, ldc,
                                        as_stream(stream)));
}

int64_t nvfp4_probe_scratch_bytes(void) { return nvfp4::probe_scratch_bytes(); }

int nvfp4_probe_mfma(int mode, int iters, void* scratch, int64_t scratch_bytes, void* stream) {
  if (scratch == nullptr) return fail(NVFP4_ERR_NULL, "scratch is NULL");
  if (!aligned(scratch, 256)) return fail(NVFP4_ERR_ALIGN, "scratch must be 256-byte aligned");
  if (scratch_bytes < nvfp4::probe_scratch_bytes())
    return fail(NVFP4_ERR_SHAPE, "scratch_bytes=%lld < %lld", (long long)scratch_bytes,
                (long long)nvfp4::probe_scratch_bytes());
  if (mode < 0 || mode > 2) return fail(NVFP4_ERR_ARG, "mode=%d (0, 1 or 2)", mode);
  if (iters < 1 || iters > 1000000) return fail(NVFP4_ERR_ARG, "iters=%d (1 .. 1000000)", iters);
  return launched(nvfp4::probe_mfma(mode, iters, scratch, as_stream(stream)));
}

int nvfp4_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(NVFP4_ERR_NULL, "src / dst is NULL");
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(NVFP4_ERR_ALIGN, "src and dst must be 16-byte aligned");
  if (bytes <= 0 || bytes % 16 || bytes > kMaxElems)
    return fail(NVFP4_ERR_SHAPE, "bytes=%lld must be a positive multiple of 16, at most 2^40",
                (long long)bytes);
  return launched(nvfp4::copy_bytes(src, dst, bytes, as_stream(stream)));
}

int64_t nvfp4_probe_clock_bytes(void) { return nvfp4::clock_stamp_bytes(); }

int nvfp4_probe_clock(void* stamps, int64_t stamps_bytes, void* stream) {
  if (stamps == nullptr) return fail(NVFP4_ERR_NULL, "stamps is NULL");
  if (!aligned(stamps, 8)) return fail(NVFP4_ERR_ALIGN, "stamps must be 8-byte aligned");
  if (stamps_bytes < nvfp4::clock_stamp_bytes())
    return fail(NVFP4_ERR_SHAPE, "stamps_bytes=%lld < %lld", (long long)stamps_bytes,
                (long long)nvfp4::clock_stamp_bytes());
  return launched(nvfp4::clock_stamp(stamps, as_stream(stream)));
}

}  // extern "C"
