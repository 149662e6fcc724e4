// nvfp4_gemm.hip -- NVFP4 x NVFP4 -> FP32 GEMM on the gfx950 matrix cores.
//
// C[m][n] = s_a * s_b * sum_k (E2M1(a) * E4M3(E_a)) * (E2M1(b) * E4M3(E_b)),
// A [M][K] and B [N][K] both K-contiguous, so one kernel serves Fprop
// (Y = X W^T), Dgrad (dX = dY W, B = the transposed 2D weight codes) and Wgrad
// (dW = dY^T X, both operands quantized along the tokens).  The linear-layer
// GEMMs are the core compute the NVFP4 recipe accelerates ("NVFP4 Trains with
// Precision of 16-Bit and Speed and Efficiency of 4-Bit", GEMM-performance
// paragraph; "Pretraining Large Language Models with NVFP4", summary page).
//
// Exactness: an E2M1 value times an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in FP16; FP16 x FP16 products are
// exact in FP32.  Each element is decoded once, in registers, straight into
// the v_mfma_f32_32x32x16_f16 operand layout; the only rounding is the FP32
// accumulation, and the tensor scales are applied once in the epilogue.
//
// Layout: a workgroup of 4 waves (2 x 2) computes a (64*WM) x (64*WN) tile;
// each wave a (32*WM) x (32*WN) sub-tile as WM x WN blocks of 32x32.  Lane l
// of a wave serves row (l % 32) of a 32-row slab and K-half (l / 32): per
// 64-wide K step it loads 16 bytes of codes (two 16-element blocks) and the
// two block scales, and feeds four MFMAs (8 codes each).  A and B use the
// same lane-to-k assignment, so every k is paired with itself.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

struct GemmArgs {
  GemmOperand a, b;
  int64_t M, N, K;
  float* c;
  int64_t ldc;
};

// Eight codes (one 32-bit word, element e in nibble e) times a block scale
// -> eight FP16 values, element e in lane-vector slot e.
//
// DECODE 0: the gfx950 FP4 -> FP16 convert multiplies by 2^floor(log2(scale))
// only (an E8M0-style scale; low nibble first), which is exact for q * 2^e.
// One packed FP16 multiply by the scale's mantissa (1 + m/8) completes
// q * E exactly: 2 + 4 significant bits.
// DECODE 1: a byte-permute decode (reference variant): FP16 of an E2M1
// magnitude has a zero low byte; its high byte comes from an 8-entry byte
// table via v_perm, the sign from bit 3 of the code; then one FP16 multiply
// by the whole E4M3 value.
struct BlockDec {
  float e;       // E4M3 value as FP32 (the convert takes its exponent)
  half2v mant;   // {mantissa, mantissa} in FP16 for DECODE 0, {E, E} for DECODE 1
};

template <int DECODE>
__device__ __forceinline__ BlockDec block_dec(uint32_t code) {
  BlockDec d;
  d.e = e4m3_to_float(code);
  if constexpr (DECODE == 0) {
    const uint32_t mb = (__float_as_uint(d.e) >> 20) & 7u;
    const uint32_t h = 0x3C00u | (mb << 7);
    d.mant = __builtin_bit_cast(half2v, h | (h << 16));
  } else {
    const _Float16 hs = (_Float16)d.e;  // E4M3 values are exact in FP16
    d.mant = half2v{hs, hs};
  }
  return d;
}

template <int DECODE>
__device__ __forceinline__ half8 decode8(uint32_t w, const BlockDec& d) {
  half2v p0, p1, p2, p3;
  if constexpr (DECODE == 0) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 0);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 1);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 2);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, d.e, 3);
  } else {
    const uint32_t tab_lo = 0x3E3C3800u;  // 0, 0.5, 1, 1.5
    const uint32_t tab_hi = 0x46444240u;  // 2, 3, 4, 6
    const uint32_t sel_e = w & 0x07070707u;          // magnitudes of nibbles 0, 2, 4, 6
    const uint32_t sel_o = (w >> 4) & 0x07070707u;   // nibbles 1, 3, 5, 7
    const uint32_t hb_e = __builtin_amdgcn_perm(tab_hi, tab_lo, sel_e) | ((w << 4) & 0x80808080u);
    const uint32_t hb_o = __builtin_amdgcn_perm(tab_hi, tab_lo, sel_o) | (w & 0x80808080u);
    // pair j: bytes {0, hb_e[j], 0, hb_o[j]} (selector 0x0C yields a zero byte)
    p0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hb_o, hb_e, 0x040C000Cu));
    p1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hb_o, hb_e, 0x050C010Cu));
    p2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hb_o, hb_e, 0x060C020Cu));
    p3 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hb_o, hb_e, 0x070C030Cu));
  }
  p0 *= d.mant;
  p1 *= d.mant;
  p2 *= d.mant;
  p3 *= d.mant;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Per-lane raw data of one 32-row slab for one 64-wide K step: 32 codes
// (k = k0 + 32*half .. +31) and the two block-scale bytes, kept raw until the
// step that consumes them so the load latency hides behind the current step.
struct Slab {
  v4u codes;
  uint32_t s0, s1;
};

// Row indices past the operand are clamped to its last row: those lanes feed
// only accumulator rows/columns that are never stored.  Full steps need no
// K checks; the tail step (K % 64 != 0) zero-fills past K.
template <bool TAIL, bool LD16>
__device__ __forceinline__ Slab load_slab(const GemmOperand& op, int64_t row, int64_t kk,
                                          int64_t K) {
  Slab s;
  const int64_t r = row < op.rows ? row : op.rows - 1;
  const uint8_t* p = op.codes + r * op.ld + kk / 2;
  const uint8_t* sp = op.scales + (r / op.blk_rows) * op.ss_row + (kk / 16) * op.ss_k;
  if (!TAIL || kk + 32 <= K) {
    if (LD16) {
      s.codes = *reinterpret_cast<const v4u*>(p);
    } else {  // K % 32 == 16: rows are 8-byte aligned
      const v2u lo = *reinterpret_cast<const v2u*>(p);
      const v2u hi = *reinterpret_cast<const v2u*>(p + 8);
      s.codes = v4u{lo.x, lo.y, hi.x, hi.y};
    }
    s.s0 = sp[0];
    s.s1 = sp[op.ss_k];
  } else if (kk + 16 <= K) {
    const v2u h = *reinterpret_cast<const v2u*>(p);
    s.codes = v4u{h.x, h.y, 0u, 0u};
    s.s0 = sp[0];
    s.s1 = 0u;
  } else {
    s.codes = v4u{0u, 0u, 0u, 0u};
    s.s0 = 0u;
    s.s1 = 0u;
  }
  return s;
}

template <int WM, int WN, int DECODE>
__device__ __forceinline__ void mma_step(float16v (&acc)[WM][WN], const Slab (&a)[WM],
                                         const Slab (&b)[WN]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    BlockDec da[WM], db[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) da[i] = block_dec<DECODE>(half ? a[i].s1 : a[i].s0);
#pragma unroll
    for (int j = 0; j < WN; ++j) db[j] = block_dec<DECODE>(half ? b[j].s1 : b[j].s0);
#pragma unroll
    for (int s = 2 * half; s < 2 * half + 2; ++s) {
      half8 av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) av[i] = decode8<DECODE>(a[i].codes[s], da[i]);
#pragma unroll
      for (int j = 0; j < WN; ++j) bv[j] = decode8<DECODE>(b[j].codes[s], db[j]);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      // keep each step's decode next to its MFMAs (bounds live FP16 operands)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Tile order: the grid is 1-D.  Workgroups are dealt round-robin to the 8
// XCDs (each with its own L2), so block b is first renumbered so that every
// XCD owns a contiguous range of tiles; inside that range tiles run in
// groups of kGroupM tile-rows, M fastest, so the workgroups resident on one
// XCD at a time share both A rows and B columns in its L2.
constexpr int kXcds = 8, kGroupM = 8;

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                            int64_t& tn) {
  const int64_t total = tiles_m * tiles_n, per = total / kXcds;
  const int64_t b = blockIdx.x;
  const int64_t t = b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t in = t - group * kGroupM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// CHECKED: K % 64 != 0; every load checks its K range and zero-fills past K.
template <int WM, int WN, int DECODE, bool LD16, bool CHECKED>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_m = (g.M + 64 * WM - 1) / (64 * WM);
  const int64_t tiles_n = (g.N + 64 * WN - 1) / (64 * WN);
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * (64 * WM) + wm * (32 * WM);
  const int64_t n0 = tn * (64 * WN) + wn * (32 * WN);
  const int lrow = lane & 31, khalf = lane >> 5;

  float16v acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t steps = (g.K + 63) / 64;
  Slab a_cur[WM], b_cur[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
    a_cur[i] = load_slab<CHECKED, LD16>(g.a, m0 + 32 * i + lrow, 32 * khalf, g.K);
#pragma unroll
  for (int j = 0; j < WN; ++j)
    b_cur[j] = load_slab<CHECKED, LD16>(g.b, n0 + 32 * j + lrow, 32 * khalf, g.K);
  // Prefetch step it+1 (the last step re-reads itself, which keeps the loop
  // free of branches), then decode and multiply step it.
  const int64_t k_last = (steps - 1) * 64 + 32 * khalf;
  for (int64_t it = 0; it < steps; ++it) {
    Slab a_nxt[WM], b_nxt[WN];
    int64_t kn = (it + 1) * 64 + 32 * khalf;
    kn = kn < k_last ? kn : k_last;
#pragma unroll
    for (int i = 0; i < WM; ++i)
      a_nxt[i] = load_slab<CHECKED, LD16>(g.a, m0 + 32 * i + lrow, kn, g.K);
#pragma unroll
    for (int j = 0; j < WN; ++j)
      b_nxt[j] = load_slab<CHECKED, LD16>(g.b, n0 + 32 * j + lrow, kn, g.K);
    mma_step<WM, WN, DECODE>(acc, a_cur, b_cur);
#pragma unroll
    for (int i = 0; i < WM; ++i) a_cur[i] = a_nxt[i];
#pragma unroll
    for (int j = 0; j < WN; ++j) b_cur[j] = b_nxt[j];
  }

  // Epilogue: lane l holds column (l % 32) of each 32x32 block; accumulator
  // slot v is row (v % 4) + 8 * (v / 4) + 4 * (l / 32).
  const float alpha = (*g.a.ts) * (*g.b.ts);
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n0 + 32 * j + lrow;
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 32 * i + (v & 3) + 8 * (v >> 2) + 4 * khalf;
        if (row < g.M) g.c[row * g.ldc + col] = acc[i][j][v] * alpha;
      }
    }
}

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, float* c,
                       int64_t ldc, int decode, hipStream_t s) {
  GemmArgs g{a, b, a.rows, b.rows, K, c, ldc};
  constexpr int WM = 4, WN = 4;
  const int64_t tiles = ((g.M + 64 * WM - 1) / (64 * WM)) * ((g.N + 64 * WN - 1) / (64 * WN));
  const dim3 grid((unsigned)tiles);
  const bool ld16 = (a.ld % 16 == 0) && (b.ld % 16 == 0);
  const bool checked = (K % 64) != 0;
#define NVFP4_GEMM_LAUNCH(D, L, C) \
  hipLaunchKernelGGL((k_gemm<WM, WN, D, L, C>), grid, dim3(256), 0, s, g)
  if (decode == 0) {
    if (checked) { if (ld16) NVFP4_GEMM_LAUNCH(0, true, true); else NVFP4_GEMM_LAUNCH(0, false, true); }
    else if (ld16) NVFP4_GEMM_LAUNCH(0, true, false);
    else NVFP4_GEMM_LAUNCH(0, false, false);
  } else {
    if (checked) { if (ld16) NVFP4_GEMM_LAUNCH(1, true, true); else NVFP4_GEMM_LAUNCH(1, false, true); }
    else if (ld16) NVFP4_GEMM_LAUNCH(1, true, false);
    else NVFP4_GEMM_LAUNCH(1, false, false);
  }
#undef NVFP4_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
