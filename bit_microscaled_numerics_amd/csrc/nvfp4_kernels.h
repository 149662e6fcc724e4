// nvfp4_kernels.h -- launch functions of the gfx950 kernels (internal to
// libnvfp4.so; the public interface is include/nvfp4.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace nvfp4 {

int num_cus();  // compute units of the current device (cached per device)

hipError_t launch_amax(const void* x, int64_t n_elems, float* out, hipStream_t s);
// out_plain (nullable): also max |x| from the same read
hipError_t launch_amax_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed,
                           float* out, hipStream_t s, float* out_plain = nullptr);
// amax of the transform over every 16 consecutive columns of each row
hipError_t launch_amax_rht_row(const void* x, int64_t n_elems, uint64_t rht_seed, float* out,
                               hipStream_t s);
// rowwise 1D; rht: each 16-block along the row transformed first
hipError_t launch_quant_row(const void* x, int64_t rows, int64_t cols, const float* amax,
                            bool rht, uint64_t rht_seed, bool sr, uint64_t seed,
                            uint32_t stream_id, uint8_t* codes, uint8_t* scales, float* ts_out,
                            hipStream_t s);
hipError_t launch_quant_col(const void* x, int64_t rows, int64_t cols, const float* amax,
                            bool rht, uint64_t rht_seed, bool sr, uint64_t seed,
                            uint32_t stream_id, uint8_t* codes, uint8_t* scales, float* ts_out,
                            hipStream_t s);
// rowwise 1D (amax_row given) and RHT transpose (amax_rht given) from one read
hipError_t launch_quant_row_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed,
                               bool sr, uint64_t seed, uint32_t stream_row, uint32_t stream_col,
                               const float* amax_row, const float* amax_rht, uint8_t* codes_row,
                               uint8_t* scales_row, float* ts_row, uint8_t* codes_col,
                               uint8_t* scales_col, float* ts_col, hipStream_t s);
hipError_t launch_quant_2d(const void* x, int64_t rows, int64_t cols, const float* amax, bool sr,
                           uint64_t seed, uint32_t stream_id, uint8_t* codes, uint8_t* codes_t,
                           uint8_t* scales, uint8_t* scales_t, float* ts_out, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                          int64_t ss_row, int64_t ss_k, int32_t blk_rows, const float* ts,
                          int64_t rows, int64_t k, float* out, hipStream_t s);

// One GEMM operand as the kernels see it.
struct GemmOperand {
  const uint8_t* codes;
  int64_t ld;  // bytes per row
  const uint8_t* scales;
  int64_t ss_row, ss_k;
  int32_t blk_rows;
  const float* ts;
  int64_t rows;
  int64_t scale_bytes;  // size of the scale array (last index + 1)
};

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, float* c,
                       int64_t ldc, hipStream_t s);
// BF16 output (+ max |C|); ws (nullable) of ws_bytes >= gemm_bf16_workspace_bytes
// lets the tail tiles split along K, exactly as the FP32 path's do.
hipError_t launch_gemm_bf16(const GemmOperand& a, const GemmOperand& b, int64_t K, uint16_t* c,
                            int64_t ldc, float* amax, void* ws, int64_t ws_bytes, hipStream_t s);
int64_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The same with the library's own per-device workspace (no allocation, no
// workspace argument), for shapes needing at most gemm_bf16_noalloc_max_bytes().
hipError_t launch_gemm_bf16_noalloc(const GemmOperand& a, const GemmOperand& b, int64_t K,
                                    uint16_t* c, int64_t ldc, float* amax, hipStream_t s);
int64_t gemm_bf16_noalloc_max_bytes();

// MXFP4 (comparison format): rowwise, 32-element blocks, E8M0 scales.
struct MxOperand {
  const uint8_t* codes;
  int64_t ld;          // bytes per row of codes
  const uint8_t* scales;
  int64_t ld_scales;   // bytes per row of scales
  int64_t rows, k;
};

hipError_t launch_mx_quant_row(const void* x, int64_t rows, int64_t cols, bool sr, uint64_t seed,
                               uint32_t stream_id, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);
hipError_t launch_mx_dequant(const MxOperand& q, float* out, hipStream_t s);
hipError_t launch_mx_gemm(const MxOperand& a, const MxOperand& b, int64_t K, float* c,
                          int64_t ldc, hipStream_t s);

// Measurement support: MFMA-only run on operand data of kind `mode` (0 zeros,
// 1 decoded-NVFP4-like, 2 uniform FP16), clock stamps left in the scratch.
int64_t probe_scratch_bytes();
hipError_t probe_mfma(int mode, int iters, void* scratch, hipStream_t s);
// Clock stamps {XCC id, HW_ID, shader clock, 100 MHz real time} of 256 workgroups.
int64_t clock_stamp_bytes();
hipError_t clock_stamp(void* out, hipStream_t s);
// Plain device copy of `bytes` (a multiple of 16, 16-byte aligned pointers).
hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace nvfp4
