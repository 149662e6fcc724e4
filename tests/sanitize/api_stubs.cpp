// api_stubs.cpp -- host stand-ins for everything libnvfp4's C-ABI layer
// (nvfp4_api.cpp) calls below it: the kernel launchers and three HIP runtime
// functions.  Linked with nvfp4_api.cpp into a host-only program built with
// AddressSanitizer and UndefinedBehaviorSanitizer, so the validation code
// runs on the CPU with every pointer and size check instrumented.  Each stub
// counts its calls; a launcher reached means validation accepted the call.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "nvfp4_kernels.h"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* d) {
  (void)d;
  return hipErrorNoDevice;   // num_cus() then falls back to 256
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace nvfp4 {
static hipError_t ok() {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_amax(const void*, int64_t, float*, hipStream_t) { return ok(); }
hipError_t launch_amax_rht(const void*, int64_t, int64_t, uint64_t, float*, hipStream_t, float*) {
  return ok();
}
hipError_t launch_amax_rht_row(const void*, int64_t, uint64_t, float*, hipStream_t) { return ok(); }
hipError_t launch_quant_row(const void*, int64_t, int64_t, const float*, bool, uint64_t, bool,
                            uint64_t, uint32_t, uint8_t*, uint8_t*, float*, hipStream_t) {
  return ok();
}
hipError_t launch_quant_col(const void*, int64_t, int64_t, const float*, bool, uint64_t, bool,
                            uint64_t, uint32_t, uint8_t*, uint8_t*, float*, hipStream_t) {
  return ok();
}
hipError_t launch_quant_row_rht(const void*, int64_t, int64_t, uint64_t, bool, uint64_t, uint32_t,
                                uint32_t, const float*, const float*, uint8_t*, uint8_t*, float*,
                                uint8_t*, uint8_t*, float*, hipStream_t) {
  return ok();
}
hipError_t launch_quant_2d(const void*, int64_t, int64_t, const float*, bool, uint64_t, uint32_t,
                           uint8_t*, uint8_t*, uint8_t*, uint8_t*, float*, hipStream_t) {
  return ok();
}
hipError_t launch_dequant(const uint8_t*, int64_t, const uint8_t*, int64_t, int64_t, int32_t,
                          const float*, int64_t, int64_t, float*, hipStream_t) {
  return ok();
}
hipError_t launch_gemm(const GemmOperand&, const GemmOperand&, int64_t, float*, int64_t,
                       hipStream_t) {
  return ok();
}
hipError_t launch_gemm_bf16(const GemmOperand&, const GemmOperand&, int64_t, uint16_t*, int64_t,
                            float*, void*, int64_t, hipStream_t) {
  return ok();
}
int64_t gemm_bf16_workspace_bytes(int64_t, int64_t, int64_t) { return 4096; }
hipError_t launch_gemm_bf16_noalloc(const GemmOperand&, const GemmOperand&, int64_t, uint16_t*,
                                    int64_t, float*, hipStream_t) {
  return ok();
}
int64_t gemm_bf16_noalloc_max_bytes() { return 8192; }
hipError_t launch_mx_quant_row(const void*, int64_t, int64_t, bool, uint64_t, uint32_t, uint8_t*,
                               uint8_t*, hipStream_t) {
  return ok();
}
hipError_t launch_mx_dequant(const MxOperand&, float*, hipStream_t) { return ok(); }
hipError_t launch_mx_gemm(const MxOperand&, const MxOperand&, int64_t, float*, int64_t,
                          hipStream_t) {
  return ok();
}
int64_t probe_scratch_bytes() { return 1 << 20; }
hipError_t probe_mfma(int, int, void*, hipStream_t) { return ok(); }
int64_t clock_stamp_bytes() { return 8192; }
hipError_t clock_stamp(void*, hipStream_t) { return ok(); }
hipError_t copy_bytes(const void*, void*, int64_t, hipStream_t) { return ok(); }
}  // namespace nvfp4
