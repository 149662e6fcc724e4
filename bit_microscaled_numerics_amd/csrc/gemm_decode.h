// gemm_decode.h -- decoding of NVFP4 GEMM operands into FP16 on gfx950
// (internal to libnvfp4.so): an E2M1 code times its E4M3 block scale, exact
// in FP16 ("Pretraining Large Language Models with NVFP4", summary page,
// format paragraph: 4-bit E2M1 elements, E4M3 scale per 16).  The GEMM
// kernels and the tests of these helpers include it.
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

// Decoding.  The gfx950 FP4 -> FP16 convert multiplies by 2^floor(log2 s)
// of its FP32 scale argument only (an E8M0-style scale; low nibble first),
// which gives q * 2^e exactly.  One packed FP16 multiply by the E4M3
// mantissa (1 + m/8) completes q * E exactly: 2 + 4 significant bits.
struct BlockDec {
  float e;       // E4M3 value as FP32 (the convert takes its exponent)
  half2v mant;   // {mantissa, mantissa} in FP16
};

// Eight codes (one 32-bit word, element e in nibble e) -> eight FP16 values
// q * E, element e in lane-vector slot e.
__device__ __forceinline__ half8 decode8(uint32_t w, const BlockDec& d) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 3);
  p0 *= d.mant;
  p1 *= d.mant;
  p2 *= d.mant;
  p3 *= d.mant;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Scale table: E4M3 code (0..127) -> {E as FP32, FP16 mantissa pair}, 1 KiB
// of LDS filled once per workgroup (one 8-byte LDS read per block scale
// costs less VALU than decoding the code).  The gfx950 FP8 -> FP32 convert
// (OCP E4M3FN, subnormals included) gives E exactly; its FP32 mantissa bits
// give the factor (1 + m/8).
__device__ __forceinline__ v2u scale_entry(uint32_t code) {
  const float e = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
  const uint32_t mb = (__float_as_uint(e) >> 20) & 7u;
  const uint32_t h = 0x3C00u | (mb << 7);
  return v2u{__float_as_uint(e), h | (h << 16)};
}

// Decode the scale code in bits [pos, pos + 7) of w (the sign bit of an
// E4M3 code is dropped: block scales are non-negative).
__device__ __forceinline__ BlockDec scale_dec(const v2u* lut, uint32_t w, uint32_t pos) {
  const v2u e = lut[__builtin_amdgcn_ubfe(w, pos, 7)];
  // copy the lanes to scalars first: clang's __builtin_bit_cast of an
  // ext-vector element expression reads element 0
  const uint32_t ex = e.x, ey = e.y;
  BlockDec d;
  d.e = __uint_as_float(ex);
  d.mant = __builtin_bit_cast(half2v, ey);
  return d;
}

// E4M3 scale code in bits [pos, pos + 7) of w -> {E, mantissa pair} in ALU
// (the table read of scale_dec would add an LDS wait next to the operand
// reads).
__device__ __forceinline__ BlockDec scale_alu(uint32_t w, uint32_t pos) {
  const uint32_t code = __builtin_amdgcn_ubfe(w, pos, 7);
  const float e = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
  const uint32_t h = 0x3C00u | (__builtin_amdgcn_ubfe(__float_as_uint(e), 20, 3) << 7);
  BlockDec d;
  d.e = e;
  d.mant = __builtin_bit_cast(half2v, h | (h << 16));
  return d;
}

// The fast path's form.  A lane's two blocks of a K step have their scale
// codes in bytes 0 and 1 of w (after a shift by the lane's K half): one
// packed FP8 -> FP32 convert gives both E values (scale codes are 0x00..0x7E
// by contract, so the sign bit is left unmasked).
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2v scale_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// decode8 from E as FP32: the convert takes E's exponent; the FP16 factor
// (1 + m/8) is built from E's top three mantissa bits (subnormal E included,
// whose FP32 form is normalised) as one half that the packed multiply
// broadcasts.  Same products as decode8(w, scale_alu(...)).
__device__ __forceinline__ half8 decode8e(uint32_t w, float e) {
  const uint16_t h = (uint16_t)(((__float_as_uint(e) >> 13) & 0x380u) | 0x3C00u);
  const _Float16 m = __builtin_bit_cast(_Float16, h);
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e, 3);
  p0 *= m;
  p1 *= m;
  p2 *= m;
  p3 *= m;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

}  // namespace nvfp4
