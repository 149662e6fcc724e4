// mxfp4.hip -- the MXFP4 comparison format on gfx950: rowwise quantization
// (32-element blocks, power-of-two E8M0 scale, no tensor scale), dequantize,
// and the MXFP4 x MXFP4 -> FP32 GEMM on the native scaled FP4 matrix cores.
//
// MXFP4 is what the NVFP4 pages compare against: blocks of 32 instead of 16,
// an integer-power (UE8M0) block scale instead of E4M3, no tensor scale
// ("Pretraining Large Language Models with NVFP4", summary page, format
// paragraph; "NVFP4 Trains with Precision of 16-Bit and Speed and Efficiency
// of 4-Bit", micro-block scaling and E4M3 sections).  Because its scales are
// powers of two per 32 elements, it is exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes: codes go from memory to the
// matrix cores with no decode.
//
// Scale rule: E = 2^e, e the smallest integer with amax_b <= 6 * 2^e (so every
// block's largest |v| lies in (3, 6]), clamped to [-127, 127], byte e + 127.
// From the binary32 bits of amax (exponent field x, mantissa f): for amax in
// [2^(x-127), 2^(x-126)), amax <= 6 * 2^(x-129) iff f <= 0x400000, so the
// byte is max(x - 2 + (f > 0x400000), 0) -- exact, no division (zero and
// subnormal amax give byte 0, the clamped minimum).
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "gemm_tiles.h"

namespace nvfp4 {

namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int x = (int)(u >> 23), f_big = (u & 0x7FFFFFu) > 0x400000u;
  const int b = x - 2 + f_big;
  return (uint32_t)(b > 0 ? b : 0);
}

// 2^-e for byte = e + 127, as a binary32 power of two (normal for every
// byte a finite input produces, 0..253).
__device__ __forceinline__ float e8m0_inverse(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// ---------------------------------------------------------------------------
// Rowwise quantization: 4 lanes per 32-element block, 8 elements per lane.
// ---------------------------------------------------------------------------
template <bool SR>
__global__ __launch_bounds__(kQThreads) void k_mx_quant_row(
    const v4u* __restrict__ x, int64_t nvec, uint64_t seed, uint32_t stream_id,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * kQThreads;  // a multiple of 4: lane quads stay together
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < nvec; i += stride) {
    const v4u v = ld_(&x[i]);
    float z[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(z[j]));
    m = quad_xor_max<1>(m);
    m = quad_xor_max<2>(m);
    const uint32_t byte = e8m0_from_amax(m);
    const float inv = e8m0_inverse(byte);
    const uint32_t q = SR ? encode8_sr(z, inv, sr_words_g(seed, stream_id, (uint64_t)i))
                          : encode8_rtn(z, inv);
    st_(q, &codes[i]);
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)byte;
  }
}

__global__ __launch_bounds__(kQThreads) void k_mx_dequant(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    int64_t ld_scales, int64_t rows, int64_t k, float* __restrict__ out) {
  const int64_t kv = k / 8, items = rows * kv;
  for (int64_t it = (int64_t)blockIdx.x * kQThreads + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kQThreads) {
    const int64_t r = it / kv, c8 = (it - r * kv) * 8;
    const uint32_t q = *reinterpret_cast<const uint32_t*>(codes + r * ld_codes + c8 / 2);
    const uint32_t b = scales[r * ld_scales + c8 / 32];
    const float E = b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);   // 2^(b-127)
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = (q >> (4 * j)) & 0xFu;
      const uint32_t i = c & 7u;
      const float mag = i < 4u ? 0.5f * (float)i : (i < 7u ? (float)i - 2.0f : 6.0f);
      o[j] = ((c & 8u) ? -mag : mag) * E;
    }
    float* dst = out + r * k + c8;
    *reinterpret_cast<v4f*>(dst) = v4f{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<v4f*>(dst + 4) = v4f{o[4], o[5], o[6], o[7]};
  }
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------
// C[m][n] = sum_k (q_a 2^e_a)(q_b 2^e_b), FP32 accumulate.  Workgroup tile
// 256 x 256, 512 threads (8 waves, two per SIMD), wave w computes rows
// 128*(w/4) .. +127 and columns 64*(w%4) .. +63 as 4 x 2 blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4 (both operands E2M1).  In that
// instruction lane l holds row l % 32 and the 32 elements k = 32*(l/32) ..
// +31 of a 64-wide K step (16 bytes, low nibble first) and gives the E8M0
// scale of exactly those 32 elements: one MXFP4 block per lane.  The result
// layout is that of every 32x32 MFMA.
//
// A stage is 256 K (128 bytes of every row: eight 16-byte chunks, i.e. full
// 128-byte lines), loaded global -> LDS by 16-byte buffer loads that write
// lane l's data at LDS base + 16 l.  LDS (A0 A1 B0 B1, 32 KiB each) holds
// chunk c of row r at 16-byte slot 8 r + (c ^ g(r)), g(r) = (r >> 1) & 7:
// the MFMA operand reads (16 consecutive rows, one chunk) then touch 16
// distinct bank groups; the writes are whole 1 KiB runs.  Lane l of load q
// of wave w fills slot 64 G + l, G = 8 q + w: row 8 G + l / 8, chunk
// (l % 8) ^ g(row).  Scales take the same road: the stage's 8 scale bytes of
// every row (2 KiB per operand) land in LDS as [row][8] (4-byte loads, or
// byte loads when rows are not 4-byte aligned); a lane reads its row's 8
// bytes with one 8-byte LDS read and keeps the four of its K-half.
constexpr int kMxStageK = 256;
constexpr int kMxThreads = 512;
constexpr int kMxWM = 4, kMxWN = 2;
constexpr int kMxRowBytes = kMxStageK / 2;           // 128
constexpr int kMxOpBytes = kTile * kMxRowBytes;      // 32 KiB per operand and stage
constexpr int kMxScBytes = kTile * 8;                // 2 KiB of scales per operand and stage
constexpr int kMxLdsBytes = 4 * kMxOpBytes + 4 * kMxScBytes;   // 136 KiB
constexpr uint32_t kBufFlags = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;               // an offset past every num_records

struct MxArgs {
  MxOperand a, b;
  int64_t M, N, K;
  float* c;
  int64_t ldc;
  int64_t full_tiles;
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mx_slot(int row, int chunk) {
  return (uint32_t)(row * 8 + (chunk ^ ((row >> 1) & 7))) * 16u;
}

struct MxView {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t voff_load[4];   // code loads q = 0..3: row * ld + 16 * chunk
  uint32_t voff_sc;        // 4-byte scale load: row (tid / 2) * ld_scales + 4 * (tid % 2)
};

__device__ __forceinline__ MxView mx_view(const MxOperand& op, int64_t row0, int wave) {
  MxView v;
  const int64_t rem_rows = op.rows - row0;
  const int64_t code_bytes = rem_rows * op.ld;
  const int64_t sc_base = row0 * op.ld_scales;
  const int64_t sc_bytes = op.rows * op.ld_scales - sc_base;
  v.codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(op.codes + row0 * op.ld), (short)0,
      (int)(code_bytes < 0x7FFFFFFF ? code_bytes : 0x7FFFFFFF), (int)kBufFlags);
  v.scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(op.scales + sc_base), (short)0,
      (int)(sc_bytes < 0x7FFFFFFF ? sc_bytes : 0x7FFFFFFF), (int)kBufFlags);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (8 * q + wave) + lane / 8;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    v.voff_load[q] = (uint32_t)(row * op.ld + 16 * chunk);
  }
  v.voff_sc = (uint32_t)((threadIdx.x >> 1) * op.ld_scales + 4 * (threadIdx.x & 1));
  return v;
}

// Issue the four 16-byte global -> LDS loads of this wave for one operand and
// stage.  Chunks at or past K (a partial last stage) and steps past the last
// read zero codes: their per-lane offset is 2^31, which with the scalar K
// offset (< 2^23) stays below 2^32 and past every num_records.
__device__ __forceinline__ void mx_dma(const MxView& v, uint8_t* lds_stage, int wave, int t,
                                       int64_t K, bool kill) {
  const int lane = threadIdx.x & 63;
  const uint32_t kbyte = (uint32_t)t * kMxRowBytes;
  const uint32_t kbytes_valid = (uint32_t)(K / 2);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (8 * q + wave) + lane / 8;
    const uint32_t chunk = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
    const bool dead = kill || kbyte + 16u * chunk >= kbytes_valid;
    const uint32_t voff = dead ? kOob : v.voff_load[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        v.codes, (__attribute__((address_space(3))) void*)(lds_stage + 1024 * (8 * q + wave)), 16,
        voff, kbyte, 0, 0);
  }
}

// The stage's scale bytes (k-blocks 8t .. 8t+7 of the 256 rows) into LDS as
// [row][8]; thread t covers row t / 2, bytes 4 (t % 2) .. +3.  Blocks at or
// past K, and killed steps, read 0.
//  - SB4 (scale rows 4-byte aligned): one 4-byte global -> LDS load, which
//    writes lane l's dword at LDS base + 4 l.
//  - else: four byte loads into registers (mx_scale_issue), packed and
//    written to LDS after the stage's MFMAs (mx_scale_commit).  A byte
//    global -> LDS load would also fill a whole dword per lane.
__device__ __forceinline__ uint32_t mx_scale_voff(const MxView& v, const MxOperand& op, int t,
                                                  int j, int64_t K, bool kill) {
  const int kb = 8 * t + 4 * (threadIdx.x & 1) + j;
  return (kill || kb >= K / 32) ? kOob
                                : (uint32_t)((threadIdx.x >> 1) * op.ld_scales + 4 * (threadIdx.x & 1) + j);
}

__device__ __forceinline__ void mx_scale_dma4(const MxView& v, const MxOperand& op, uint8_t* lds,
                                              int wave, int t, int64_t K, bool kill) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      v.scales, (__attribute__((address_space(3))) void*)(lds + 256 * wave), 4,
      mx_scale_voff(v, op, t, 0, K, kill), (uint32_t)(8 * t), 0, 0);
}

__device__ __forceinline__ void mx_scale_issue(const MxView& v, const MxOperand& op, int t,
                                               int64_t K, bool kill, uint32_t (&bytes)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bytes[j] = __builtin_amdgcn_raw_buffer_load_b8(v.scales, mx_scale_voff(v, op, t, j, K, kill),
                                                   (uint32_t)(8 * t), 0);
}

__device__ __forceinline__ void mx_scale_commit(uint8_t* lds, const uint32_t (&bytes)[4]) {
  *reinterpret_cast<uint32_t*>(lds + 4 * threadIdx.x) =
      bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | (bytes[3] << 24);
}

// This lane's four scale bytes of a fragment row: bytes lh, 2+lh, 4+lh, 6+lh
// of the row's 8 (k-blocks 2 s + lh of sub-steps s = 0..3), so sub-step s
// uses byte s.
__device__ __forceinline__ uint32_t mx_frag_scales(const uint8_t* sc_stage, int row, uint32_t sel) {
  const v2u w = *reinterpret_cast<const v2u*>(sc_stage + 8 * row);
  const uint32_t lo = w.x, hi = w.y;
  return __builtin_amdgcn_perm(hi, lo, sel);
}

struct MxOps {
  v4u a[kMxWM], b[kMxWN];
};

__device__ __forceinline__ v4u mx_read(const uint8_t* stage, int row, int chunk) {
  return *reinterpret_cast<const v4u*>(stage + mx_slot(row, chunk));
}

// The instruction takes 8-dword operands; with E2M1 it reads only the first 4.
__device__ __forceinline__ v8i mx_widen(const v4u d) {
  return v8i{(int)d.x, (int)d.y, (int)d.z, (int)d.w, 0, 0, 0, 0};
}

__device__ __forceinline__ void mx_read_ops(MxOps& o, const uint8_t* a_stage,
                                            const uint8_t* b_stage, int wm, int wn, int lrow,
                                            int lh, int s) {
#pragma unroll
  for (int i = 0; i < kMxWM; ++i) o.a[i] = mx_read(a_stage, wm * 128 + 32 * i + lrow, 2 * s + lh);
#pragma unroll
  for (int j = 0; j < kMxWN; ++j) o.b[j] = mx_read(b_stage, wn * 64 + 32 * j + lrow, 2 * s + lh);
}

// Sub-step S of a stage: the scale of this lane's block is byte S of its
// fragment's scale word.
template <int S>
__device__ __forceinline__ void mx_mfma8(f16v (&acc)[kMxWM][kMxWN], const MxOps& o,
                                         const uint32_t (&sa)[kMxWM], const uint32_t (&sb)[kMxWN]) {
#pragma unroll
  for (int i = 0; i < kMxWM; ++i)
#pragma unroll
    for (int j = 0; j < kMxWN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          mx_widen(o.a[i]), mx_widen(o.b[j]), acc[i][j], 4, 4, S, (int)sa[i], S, (int)sb[j]);
}

template <bool SB4>
__global__ __launch_bounds__(kMxThreads, 1) void k_mx_gemm(MxArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // the wave index is uniform: in a scalar register the LDS bases of the
  // global -> LDS loads (M0) are scalar arithmetic
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = lane & 31, lh = lane >> 5;
  const int64_t tiles_m = (g.M + kTile - 1) / kTile, tiles_n = (g.N + kTile - 1) / kTile;
  int64_t tm, tn;
  int part;
  block_tile(g.full_tiles, tiles_m, tiles_n, tm, tn, part);
  const MxView va = mx_view(g.a, tm * kTile, wave);
  const MxView vb = mx_view(g.b, tn * kTile, wave);
  const uint32_t sel = 0x06040200u + 0x01010101u * (uint32_t)lh;

  f16v acc[kMxWM][kMxWN];
#pragma unroll
  for (int i = 0; i < kMxWM; ++i)
#pragma unroll
    for (int j = 0; j < kMxWN; ++j) acc[i][j] = f16v{};

  const int stages = (int)((g.K + kMxStageK - 1) / kMxStageK), half = (stages + 1) / 2;
  const int s0 = part == 1 ? half : 0, s1 = part == 0 ? half : stages;
  uint8_t* a_st[2] = {smem, smem + kMxOpBytes};
  uint8_t* b_st[2] = {smem + 2 * kMxOpBytes, smem + 3 * kMxOpBytes};
  uint8_t* sa_st[2] = {smem + 4 * kMxOpBytes, smem + 4 * kMxOpBytes + kMxScBytes};
  uint8_t* sb_st[2] = {smem + 4 * kMxOpBytes + 2 * kMxScBytes,
                       smem + 4 * kMxOpBytes + 3 * kMxScBytes};

  // Stage t computes from buffer (t - s0) & 1 while stage t+1 loads into the
  // other.  One barrier per stage: after it, every wave has finished reading
  // the buffer stage t+1 will overwrite (it held stage t-1).  Two stages per
  // trip keep the buffers fixed; a stage past the last is a killed load (zero
  // codes and scales).
  uint32_t bya[4], byb[4];   // byte-loaded scales in flight (not SB4)
  mx_dma(va, a_st[0], wave, s0, g.K, false);
  mx_dma(vb, b_st[0], wave, s0, g.K, false);
  if (SB4) {
    mx_scale_dma4(va, g.a, sa_st[0], wave, s0, g.K, false);
    mx_scale_dma4(vb, g.b, sb_st[0], wave, s0, g.K, false);
  } else {
    mx_scale_issue(va, g.a, s0, g.K, false, bya);
    mx_scale_issue(vb, g.b, s0, g.K, false, byb);
    mx_scale_commit(sa_st[0], bya);
    mx_scale_commit(sb_st[0], byb);
  }
  for (int it = s0; it < s1; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = it + h;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of stage t (all that is outstanding)
      __syncthreads();
      const bool kill = t + 1 >= s1;
      mx_dma(va, a_st[h ^ 1], wave, t + 1, g.K, kill);
      mx_dma(vb, b_st[h ^ 1], wave, t + 1, g.K, kill);
      if (SB4) {
        mx_scale_dma4(va, g.a, sa_st[h ^ 1], wave, t + 1, g.K, kill);
        mx_scale_dma4(vb, g.b, sb_st[h ^ 1], wave, t + 1, g.K, kill);
      } else {
        mx_scale_issue(va, g.a, t + 1, g.K, kill, bya);
        mx_scale_issue(vb, g.b, t + 1, g.K, kill, byb);
      }
      uint32_t sa[kMxWM], sb[kMxWN];
#pragma unroll
      for (int i = 0; i < kMxWM; ++i) sa[i] = mx_frag_scales(sa_st[h], wm * 128 + 32 * i + lrow, sel);
#pragma unroll
      for (int j = 0; j < kMxWN; ++j) sb[j] = mx_frag_scales(sb_st[h], wn * 64 + 32 * j + lrow, sel);
      MxOps o;
      mx_read_ops(o, a_st[h], b_st[h], wm, wn, lrow, lh, 0);
      mx_mfma8<0>(acc, o, sa, sb);
      mx_read_ops(o, a_st[h], b_st[h], wm, wn, lrow, lh, 1);
      mx_mfma8<1>(acc, o, sa, sb);
      mx_read_ops(o, a_st[h], b_st[h], wm, wn, lrow, lh, 2);
      mx_mfma8<2>(acc, o, sa, sb);
      mx_read_ops(o, a_st[h], b_st[h], wm, wn, lrow, lh, 3);
      mx_mfma8<3>(acc, o, sa, sb);
      if (!SB4) {   // stage t+1's scale buffer is free (it held stage t-1)
        mx_scale_commit(sa_st[h ^ 1], bya);
        mx_scale_commit(sb_st[h ^ 1], byb);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the killed loads of the last trip

  // Epilogue as in the NVFP4 GEMM: lane l holds column l % 32 of each block,
  // slot v is row (v % 4) + 8 (v / 4) + 4 (l / 32); split tiles add into the
  // zeroed output (two addends onto zero: order-independent).
  const int64_t m0 = tm * kTile + wm * 128, n0 = tn * kTile + wn * 64;
#pragma unroll
  for (int i = 0; i < kMxWM; ++i)
#pragma unroll
    for (int j = 0; j < kMxWN; ++j) {
      const int64_t col = n0 + 32 * j + lrow;
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 32 * i + (v & 3) + 8 * (v >> 2) + 4 * lh;
        if (row >= g.M) continue;
        float* dst = &g.c[row * g.ldc + col];
        if (part < 0) *dst = acc[i][j][v];
        else atomicAdd(dst, acc[i][j][v]);
      }
    }
}

int grid_for_items(int64_t items) {
  const int64_t blocks = (items + kQThreads - 1) / kQThreads;
  const int64_t cap = (int64_t)num_cus() * 16;
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_mx_quant_row(const void* x, int64_t rows, int64_t cols, bool sr, uint64_t seed,
                               uint32_t stream_id, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
  const int64_t nvec = rows * cols / 8;
  const v4u* xv = reinterpret_cast<const v4u*>(x);
  uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
  const dim3 g((unsigned)grid_for_items(nvec)), b(kQThreads);
  if (sr) hipLaunchKernelGGL(k_mx_quant_row<true>, g, b, 0, s, xv, nvec, seed, stream_id, cv, scales);
  else hipLaunchKernelGGL(k_mx_quant_row<false>, g, b, 0, s, xv, nvec, seed, stream_id, cv, scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequant(const MxOperand& q, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_dequant, dim3((unsigned)grid_for_items(q.rows * (q.k / 8))),
                     dim3(kQThreads), 0, s, q.codes, q.ld, q.scales, q.ld_scales, q.rows, q.k,
                     out);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxOperand& a, const MxOperand& b, int64_t K, float* c,
                          int64_t ldc, hipStream_t s) {
  MxArgs g{a, b, a.rows, b.rows, K, c, ldc, 0};
  const TilePlan plan = plan_tiles(g.M, g.N, (K + kMxStageK - 1) / kMxStageK);
  g.full_tiles = plan.full_tiles;
  {
    const hipError_t e = zero_split_tiles(plan, c, ldc, g.M, g.N, s);
    if (e != hipSuccess) return e;
  }
  // 4-byte scale loads only where every dword is either wholly inside K or
  // wholly past it (K / 32 a multiple of 4): a dword straddling the end of a
  // row's blocks would bring in bytes past K (padding or the next row)
  auto sb4 = [&](const MxOperand& o) {
    return o.ld_scales % 4 == 0 && (reinterpret_cast<uintptr_t>(o.scales) & 3) == 0 &&
           (K / 32) % 4 == 0;
  };
#define NVFP4_MX_LAUNCH(SB)                                                                 \
  do {                                                                                       \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mx_gemm<SB>),       \
                                       hipFuncAttributeMaxDynamicSharedMemorySize,          \
                                       kMxLdsBytes);                                        \
    if (e != hipSuccess) return e;                                                           \
    hipLaunchKernelGGL((k_mx_gemm<SB>), dim3((unsigned)plan.grid), dim3(kMxThreads),         \
                       kMxLdsBytes, s, g);                                                   \
  } while (0)
  if (sb4(a) && sb4(b)) NVFP4_MX_LAUNCH(true);
  else NVFP4_MX_LAUNCH(false);
#undef NVFP4_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
