// devtest.hip -- test-only entry points that run single device helpers of the
// NVFP4 kernels on arrays: the E4M3 block-scale encode (gfx950 FP8 convert),
// the E2M1 encodes (gfx950 FP4 convert, round-to-nearest-even and the
// stochastic-rounding decision), the block-scale step with its
// reciprocal-multiply shortcut, and the GEMM's operand decode (FP4 -> FP16
// convert times the E4M3 mantissa).  The tests compare them with the CPU
// reference over whole ranges of binary32 inputs: each helper replaces a
// bit-level definition by a hardware instruction, and these are the places
// where the two could part.  Not part of libnvfp4.so; it includes the
// library's device headers so that it runs exactly the kernels' code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_decode.h"
#include "nvfp4_device.h"

using namespace nvfp4;

namespace {

constexpr int kThreads = 256;

int grid_for(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  if (g > 4096) g = 4096;
  return (int)(g < 1 ? 1 : g);
}

__global__ void k_e4m3_code(const float* __restrict__ x, uint8_t* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    out[i] = (uint8_t)e4m3_code(x[i]);
}

// groups of 8 values, element scale 1 (v * 1 is exact): out byte j of group g
// holds elements 2j (low nibble) and 2j + 1
__global__ void k_encode_rtn(const float* __restrict__ v, uint32_t* __restrict__ out, int64_t groups) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * kThreads) {
    float z[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = v[8 * g + j];
    out[g] = encode8_rtn(z, 1.0f);
  }
}

__global__ void k_encode_sr(const float* __restrict__ v, const uint16_t* __restrict__ u,
                            uint32_t* __restrict__ out, int64_t groups) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * kThreads) {
    float z[8];
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[j] = v[8 * g + j];
      h[j] = u[8 * g + j];
    }
    const u32x4 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)};
    out[g] = encode8_sr(z, 1.0f, w);
  }
}

__global__ void k_block_scale(const float* __restrict__ amax_b, int64_t n, float amax_t,
                              uint8_t* __restrict__ code, float* __restrict__ r) {
  __shared__ float rtab[kE4m3Codes];
  const ScaleCtx sc = scale_ctx(amax_t, rtab, threadIdx.x);
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const BlockScale b = block_scale(amax_b[i], sc);
    code[i] = (uint8_t)b.code;
    r[i] = b.r;
  }
}

// one 32-bit word of 8 codes and one E4M3 scale code per item -> 8 FP16
// values q * E through the GEMM's ALU scale decode, its table decode and
// the fast path's pair decode.  For the pair decode the code sits in byte
// b = i % 2 of half h = (i / 2) % 2 of a dword whose other bytes hold other
// codes, shifted by 16 h as the fast path shifts a lane's K half.
__global__ void k_gemm_decode(const uint32_t* __restrict__ w, const uint8_t* __restrict__ sc,
                              half8* __restrict__ out_alu, half8* __restrict__ out_lut,
                              half8* __restrict__ out_pair, int64_t n) {
  __shared__ v2u lut[128];
  if (threadIdx.x < 128) lut[threadIdx.x] = scale_entry(threadIdx.x);
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const uint32_t s = sc[i];
    out_alu[i] = decode8(w[i], scale_alu(s << 8, 8));
    out_lut[i] = decode8(w[i], scale_dec(lut, s << 16, 16));
    const uint32_t b = (uint32_t)i & 1u, h = ((uint32_t)i >> 1) & 1u;
    const uint32_t other = (s + 37u) % 127u;   // a different finite code
    const uint32_t word = (other * 0x01010101u & ~(0xFFu << (8u * (b + 2u * h)))) |
                          (s << (8u * (b + 2u * h)));
    const float2v e = scale_pair(word >> (16u * h));
    out_pair[i] = decode8e(w[i], b ? e.y : e.x);
  }
}

int done() { return hipGetLastError() == hipSuccess ? 0 : -5; }

}  // namespace

extern "C" {

// out[i] = E4M3 code of x[i] >= 0 (finite) as the quantizers encode block scales.
int devtest_e4m3_code(const float* x, uint8_t* out, int64_t n, void* stream) {
  if (x == nullptr || out == nullptr || n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_e4m3_code, dim3(grid_for(n)), dim3(kThreads), 0, (hipStream_t)stream, x,
                     out, n);
  return done();
}

// Packed E2M1 codes of v[0 .. n) (n a multiple of 8), round-to-nearest-even.
int devtest_encode_rtn(const float* v, uint8_t* out, int64_t n, void* stream) {
  if (v == nullptr || out == nullptr || n < 0 || n % 8) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_encode_rtn, dim3(grid_for(n / 8)), dim3(kThreads), 0, (hipStream_t)stream,
                     v, reinterpret_cast<uint32_t*>(out), n / 8);
  return done();
}

// Packed E2M1 codes of v[0 .. n), stochastic rounding with random bits u[i].
int devtest_encode_sr(const float* v, const uint16_t* u, uint8_t* out, int64_t n, void* stream) {
  if (v == nullptr || u == nullptr || out == nullptr || n < 0 || n % 8) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_encode_sr, dim3(grid_for(n / 8)), dim3(kThreads), 0, (hipStream_t)stream,
                     v, u, reinterpret_cast<uint32_t*>(out), n / 8);
  return done();
}

// Block scale code and element reciprocal of each block amax amax_b[i] for
// a tensor with amax amax_t.
int devtest_block_scale(const float* amax_b, int64_t n, float amax_t, uint8_t* code, float* r,
                        void* stream) {
  if (amax_b == nullptr || code == nullptr || r == nullptr || n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_block_scale, dim3(grid_for(n)), dim3(kThreads), 0, (hipStream_t)stream,
                     amax_b, n, amax_t, code, r);
  return done();
}

// FP16 bit patterns of the 8 values q * E of word w[i] with scale code sc[i]
// (0 .. 0x7E), by the fast-path ALU decode (out_alu) and the table decode
// (out_lut), 8 per item, element e of the word in slot e.
int devtest_gemm_decode(const uint32_t* w, const uint8_t* sc, uint16_t* out_alu,
                        uint16_t* out_lut, uint16_t* out_pair, int64_t n, void* stream) {
  if (w == nullptr || sc == nullptr || out_alu == nullptr || out_lut == nullptr ||
      out_pair == nullptr || n < 0)
    return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_gemm_decode, dim3(grid_for(n)), dim3(kThreads), 0, (hipStream_t)stream, w,
                     sc, reinterpret_cast<half8*>(out_alu), reinterpret_cast<half8*>(out_lut),
                     reinterpret_cast<half8*>(out_pair), n);
  return done();
}

// Host: the stochastic-rounding decision of the encodes (the E2M1 grid value
// chosen for v with random bits u), compiled for the CPU from the same source.
void devtest_sr_value_host(const float* v, const uint16_t* u, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = 0.5f * e2m1_sr_twice(v[i], u[i]);  // exact halving
}

}  // extern "C"
