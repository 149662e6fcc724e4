// mfma_probe.hip -- measurement support, not part of the quantize/GEMM path:
// the sustained throughput and shader clock of the FP16 matrix cores on
// operand data of a chosen kind, the context for reading the GEMM's roofline
// fraction.  The MI355X holds its clock only while power allows, and the
// power drawn by v_mfma_f32_32x32x16_f16 depends on the operand bits: zeros
// run near the top clock, decoded NVFP4 values (what the GEMM multiplies)
// and uniform FP16 well below it.
//
// Layout of the probe: 256 workgroups x 4 waves (one wave per SIMD on 256
// CUs), each wave 8 x 2 independent 32 x 32 accumulators fed from registers
// -- the GEMM fast path's MFMA pattern with no loads, decode or LDS.  Wave 0
// of every workgroup reads the shader-clock counter (s_memtime) and the
// 100 MHz real-time counter (s_memrealtime) around the loop.
//
// Also clock stamps for any work on a stream: taken before and after it, they
// give the average shader clock the work ran at; and a plain device copy, the
// achievable HBM bandwidth of a read + write stream.
#include <hip/hip_runtime.h>

#include "nvfp4_kernels.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kProbeWgs = 256, kProbeThreads = 256, kProbeVecs = 10;   // half8 per thread

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // integer hash (xorshift-multiply)
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

// mode 0: zeros; 1: E2M1 x E4M3-mantissa values / 16 with random signs (the
// decoded operands of the NVFP4 GEMM); 2: uniform in [-1, 1).
__global__ void k_probe_fill(_Float16* v, int64_t n, int mode) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t h = mix32((uint32_t)i * 2654435761u + 12345u);
  float x = 0.f;
  if (mode == 1) {
    const float q[8] = {0.f, .5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    x = q[h & 7] * (1.f + (float)((h >> 3) & 7) / 8.f) * ((h >> 6) & 1 ? -1.f : 1.f) / 16.f;
  } else if (mode == 2) {
    x = (float)(h >> 8) / 8388608.f - 1.f;
  }
  v[i] = (_Float16)x;
}

__global__ __launch_bounds__(kProbeThreads, 1) void k_probe_mfma(const half8* src, float* sink,
                                                                 unsigned long long* clk, int iters) {
  const int gt = blockIdx.x * kProbeThreads + threadIdx.x;
  half8 a[8], b[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = src[gt * kProbeVecs + i];
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = src[gt * kProbeVecs + 8 + j];
  float16v acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16v{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  sink[gt] = s;   // keeps the MFMAs live
  if (threadIdx.x == 0) {
    clk[4 * blockIdx.x + 0] = t0;
    clk[4 * blockIdx.x + 1] = t1;
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = r1;
  }
}

// Clock stamps: each workgroup's first lane writes {XCC id, HW_ID (its
// wave, SIMD, CU, shader-array and engine fields), shader-clock counter,
// 100 MHz real-time counter}.  Shader-clock counters of different compute
// units are not synchronised with each other, so the host pairs a stamp
// taken before some work with one taken after it on the same compute unit
// (same XCC and same CU / shader-array / engine fields); one workgroup per
// CU covers the chip.
constexpr int kStampWgs = 256;

__global__ void k_clock_stamp(unsigned long long* out) {
  if (threadIdx.x != 0) return;
  const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xFu;   // HW_REG_XCC_ID[3:0]
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);         // HW_REG_HW_ID
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  out[4 * blockIdx.x + 0] = xcc;
  out[4 * blockIdx.x + 1] = hw;
  out[4 * blockIdx.x + 2] = t;
  out[4 * blockIdx.x + 3] = r;
}

// Plain device copy: the achievable HBM bandwidth of a read + write stream,
// the reference the quantizers' bandwidth fractions and the byte counters are
// read against.  The access pattern of the amax and rowwise kernels: each
// workgroup takes whole chunks of 8 x 16-byte vectors per thread, loads them
// all, then stores them; chunks dealt to the workgroups in turn.
constexpr int kCopyU = 8, kCopyThreads = 256;
typedef uint32_t v4u_ __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void k_copy(const v4u_* __restrict__ src,
                                                        v4u_* __restrict__ dst, int64_t nvec) {
  const int64_t chunk = (int64_t)kCopyU * kCopyThreads;
  for (int64_t c = (int64_t)blockIdx.x * chunk; c < nvec; c += (int64_t)gridDim.x * chunk) {
    if (c + chunk <= nvec) {
      v4u_ v[kCopyU];
#pragma unroll
      for (int u = 0; u < kCopyU; ++u)
        v[u] = __builtin_nontemporal_load(&src[c + u * kCopyThreads + threadIdx.x]);
#pragma unroll
      for (int u = 0; u < kCopyU; ++u)
        __builtin_nontemporal_store(v[u], &dst[c + u * kCopyThreads + threadIdx.x]);
    } else {
      for (int64_t i = c + threadIdx.x; i < nvec; i += kCopyThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
    }
  }
}

}  // namespace

hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t nvec = bytes / 16, chunk = (int64_t)kCopyU * kCopyThreads;
  int64_t chunks = (nvec + chunk - 1) / chunk;
  const int64_t cap = (int64_t)num_cus() * 8;
  const int64_t trips = (chunks + cap - 1) / cap;
  const int64_t grid = trips > 0 ? (chunks + trips - 1) / trips : 1;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)(grid < 1 ? 1 : grid)), dim3(kCopyThreads), 0, s,
                     static_cast<const v4u_*>(src), static_cast<v4u_*>(dst), nvec);
  return hipGetLastError();
}

int64_t clock_stamp_bytes() { return (int64_t)kStampWgs * 32; }

hipError_t clock_stamp(void* out, hipStream_t s) {
  hipLaunchKernelGGL(k_clock_stamp, dim3(kStampWgs), dim3(64), 0, s,
                     static_cast<unsigned long long*>(out));
  return hipGetLastError();
}

// Scratch layout: operands (kProbeWgs * 256 threads * 10 half8), the sink
// (one float per thread), then the stamps (4 x uint64 per workgroup).
int64_t probe_scratch_bytes() {
  return (int64_t)kProbeWgs * kProbeThreads * (kProbeVecs * 16 + 4) + (int64_t)kProbeWgs * 32;
}

hipError_t probe_mfma(int mode, int iters, void* scratch, hipStream_t s) {
  uint8_t* base = static_cast<uint8_t*>(scratch);
  const int64_t n = (int64_t)kProbeWgs * kProbeThreads * kProbeVecs * 8;   // halves
  _Float16* src = reinterpret_cast<_Float16*>(base);
  float* sink = reinterpret_cast<float*>(base + n * 2);
  unsigned long long* clk =
      reinterpret_cast<unsigned long long*>(base + n * 2 + (int64_t)kProbeWgs * kProbeThreads * 4);
  hipLaunchKernelGGL(k_probe_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, n, mode);
  const half8* s8 = reinterpret_cast<const half8*>(src);
  // a short warm-up, then the run whose stamps stay in the scratch
  hipLaunchKernelGGL(k_probe_mfma, dim3(kProbeWgs), dim3(kProbeThreads), 0, s, s8, sink, clk,
                     iters / 8 + 1);
  hipLaunchKernelGGL(k_probe_mfma, dim3(kProbeWgs), dim3(kProbeThreads), 0, s, s8, sink, clk, iters);
  return hipGetLastError();
}

}  // namespace nvfp4
