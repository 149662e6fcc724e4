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
// exact in FP32.  Every element is decoded once per workgroup into FP16 in
// LDS and fed to v_mfma_f32_32x32x16_f16; the only rounding is the FP32
// accumulation, and the tensor scales are applied once in the epilogue.  (The
// gfx950 scaled FP4 MFMA takes power-of-two E8M0 scales per 32 elements, so
// it cannot apply an E4M3 scale per 16 exactly.)
#include <mutex>

#include "gemm_decode.h"
#include "gemm_tiles.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

struct GemmArgs {
  GemmOperand a, b;
  int64_t M, N, K;
  float* c;             // FP32 output, or
  uint16_t* cb;         // BF16 output (with the BF16 epilogue)
  uint32_t* amax;       // BF16 epilogue: binary32 bits of max |C| (nullable)
  int64_t ldc;
  int64_t full_tiles;  // tiles computed whole; tiles past them are cut by `tail`
  int tail;            // TailMode of the tiles past full_tiles
  int vec_out;         // 16-byte output stores: ldc and base aligned, 256 rows < 2^31 B
  // BF16 epilogue with K-split tail tiles: per split slot two FP32 partial
  // buffers (one per K half, kSplitSlotFloats each) and one ticket word
  float* ws;
  uint32_t* ws_tickets;
};

constexpr uint32_t kBufFlags = 0x00020000u;  // raw 32-bit buffer descriptor word 3
constexpr int kNontemporal = 2;               // buffer store cache policy: non-temporal

// Buffer view of one operand for one workgroup: codes and scales of the
// 256-row slab starting at row0.  Loads take this thread's row part of the
// offset in a VGPR (fixed for the whole K loop) and the K part in an SGPR,
// so rows past the operand lie beyond num_records and read as zero; no row
// clamping or per-iteration address arithmetic.
struct OpView {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t voff_codes;   // row * ld + 16 * khalf
  uint32_t voff_scales;  // (row / blk) * ss_row + 2 * khalf * ss_k
  uint32_t voff_srow;     // (row / blk) * ss_row
  uint32_t ss_k;
};

// Thread t of the workgroup loads row t / 2 of the slab, K-half t % 2.
__device__ __forceinline__ OpView make_view(const GemmOperand& op, int64_t row0) {
  OpView v;
  const int64_t rem_rows = op.rows - row0;
  const int64_t code_bytes = rem_rows * op.ld;
  const uint8_t* sbase = op.scales + (row0 / op.blk_rows) * op.ss_row;
  const int64_t scale_bytes = op.scale_bytes - (row0 / op.blk_rows) * op.ss_row;
  v.codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(op.codes + row0 * op.ld), (short)0,
      (int)(code_bytes < 0x7FFFFFFF ? code_bytes : 0x7FFFFFFF), (int)kBufFlags);
  v.scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sbase), (short)0,
      (int)(scale_bytes < 0x7FFFFFFF ? scale_bytes : 0x7FFFFFFF), (int)kBufFlags);
  const int r = threadIdx.x >> 1, kh = threadIdx.x & 1;
  v.voff_codes = (uint32_t)(r * op.ld + 16 * kh);
  v.voff_srow = (uint32_t)((r / op.blk_rows) * op.ss_row);
  v.voff_scales = v.voff_srow + (uint32_t)(2 * kh * op.ss_k);
  v.ss_k = (uint32_t)op.ss_k;
  return v;
}

// Per-thread raw data of one 64-wide K step of one operand: 32 codes
// (k = k0 + 32*khalf .. +31) and the scale codes of their two 16-element
// blocks: byte 0 of s0 and of s1, or (dword scales) bytes 2*khalf and
// 2*khalf + 1 of s0 == s1.
struct Slab {
  v4u codes;
  uint32_t s0, s1;
};

// Scale addressing, two forms:
//  - bytes (any layout): two byte loads per step.
//  - dword (scales contiguous along K, rows 4-byte aligned): one 4-byte load
//    brings the step's four block scales of the row, both K-halves.
// kill adds 2^31 to the scales' scalar offset, past num_records: they read
// 0, and a zero scale decodes every code to +-0, so a step past the last one
// adds nothing.  kbyte = k0 / 2 (uniform).  Blocks at k >= K are zeroed at
// decode time through their scale (zero_tail), not here: a select on a
// loaded value would stall on the load right after issuing it.
template <bool LD16, bool SDW>
__device__ __forceinline__ Slab load_slab(const OpView& v, uint32_t kbyte, uint32_t kill) {
  Slab s;
  if (LD16) {
    s.codes = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                          v.codes, v.voff_codes, kbyte, 0));
  } else {  // K % 32 == 16: rows are 8-byte aligned
    const v2u lo = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(
                                               v.codes, v.voff_codes, kbyte, 0));
    const v2u hi = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(
                                               v.codes, v.voff_codes + 8, kbyte, 0));
    s.codes = v4u{lo.x, lo.y, hi.x, hi.y};
  }
  if (SDW) {
    s.s0 = s.s1 = __builtin_amdgcn_raw_buffer_load_b32(v.scales, v.voff_srow, kbyte / 8 + kill, 0);
  } else {
    const uint32_t sk = (kbyte / 8) * v.ss_k + kill;  // block index (k0 / 16) times its stride
    s.s0 = __builtin_amdgcn_raw_buffer_load_b8(v.scales, v.voff_scales, sk, 0);
    s.s1 = __builtin_amdgcn_raw_buffer_load_b8(v.scales, v.voff_scales + v.ss_k, sk, 0);
  }
  return s;
}

// ---------------------------------------------------------------------------
// Decode-once GEMM
// ---------------------------------------------------------------------------
// Workgroup: 512 threads = 8 waves (two per SIMD) on a 256 x 256 tile; wave w
// computes rows 128*(w/4) .. +127 and columns 64*(w%4) .. +63 as 4 x 2
// blocks of 32 x 32 (128 accumulator registers, so two waves fit a SIMD and
// each covers the other's stalls).  Every element of the A and B tiles is
// decoded exactly once per K step: thread t decodes chunk t of A and chunk t
// of B (row t/2, codes 32*(t%2) .. +31 of the step) into FP16 in LDS; the
// waves read their MFMA operands back with ds_read_b128.  The decode of K
// step it+1 is interleaved with the MFMAs of step it; raw codes are loaded
// two K steps ahead.
//
// LDS: (A, B) x 2 stages x [256 rows][128 B] = 128 KiB, ordered A0 A1 B0 B1
// so an operand's two stages lie within reach of the 16-bit LDS immediate
// offset from one address register.  A row holds 64 FP16
// values = 8 chunks of 16 B; chunk j of row r sits at position j ^ f(r),
// f(r) = ((r >> 1) ^ ((r & 1) << 1)) & 7.  On gfx950 a 16-byte LDS read
// serves 16 consecutive lanes per cycle over 256 B of banks, a 16-byte write
// only 8 lanes over 128 B (measured with SQ_LDS_BANK_CONFLICT).  The operand
// reads (16 consecutive rows, one chunk) then touch 16 distinct 16-byte bank
// groups since f is a bijection on the even rows and on the odd rows of any
// 16; the decode writes (4 rows x chunks {p, p + 4} per 8 lanes) touch 8,
// since f(r) & 3 differs across every aligned group of 4 rows.
constexpr int kBK = 64;
constexpr int kThreads = 512;
constexpr int kWM = 4, kWN = 2;                    // 32x32 blocks per wave
constexpr int kRowBytes = kBK * 2;                 // 128
constexpr int kOpBytes = kTile * kRowBytes;        // 32 KiB per operand and stage
constexpr int kLdsBytes = 4 * kOpBytes;            // 128 KiB

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  const int f = ((row >> 1) ^ ((row & 1) << 1)) & 7;
  return (uint32_t)(row * kRowBytes + ((chunk ^ f) << 4));
}

struct StepOps {
  half8 a[kWM], b[kWN];
};

__device__ __forceinline__ void mfma8(float16v (&acc)[kWM][kWN], const StepOps& o) {
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
}

// A thread's raw share of one K step: one chunk of A and one of B.
struct Raw {
  Slab a, b;
};

template <bool LD16, bool SDW>
__device__ __forceinline__ void load_raw(Raw& r, const OpView& va, const OpView& vb,
                                         uint32_t kbyte, uint32_t kill) {
  r.a = load_slab<LD16, SDW>(va, kbyte, kill);
  r.b = load_slab<LD16, SDW>(vb, kbyte, kill);
}

// K % 64 != 0: in step t, this thread's blocks start at k = 64 t + 32 khalf
// and + 16; a block at or past K gets scale code 0, so its codes (whatever
// bytes the row holds there) decode to +-0.  Byte-loaded scales only.
template <bool CHECKED>
__device__ __forceinline__ void zero_tail(Raw& r, int t, int64_t K) {
  if (!CHECKED) return;
  const int64_t kk = 64 * (int64_t)t + 32 * (threadIdx.x & 1);
  if (kk >= K) { r.a.s0 = 0u; r.b.s0 = 0u; }
  if (kk + 16 >= K) { r.a.s1 = 0u; r.b.s1 = 0u; }
}

// Decode words p0, p0+1 of this thread's chunk of operand `op` (0 = A,
// 1 = B) into an LDS stage.  The first block's scale code sits at bit pos0
// of s0, the second's at bit pos1 of s1.
__device__ __forceinline__ void store_half(uint8_t* stage, const v2u* lut, const v4u& codes,
                                           uint32_t s0, uint32_t pos0, uint32_t s1,
                                           uint32_t pos1, int op, int p0) {
  uint8_t* base = stage + op * 2 * kOpBytes;
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const BlockDec d = p0 < 2 ? scale_dec(lut, s0, pos0) : scale_dec(lut, s1, pos1);
#pragma unroll
  for (int p = p0; p < p0 + 2; ++p)
    *reinterpret_cast<half8*>(base + lds_off(row, 4 * half + p)) = decode8(codes[p], d);
}

// MFMA operands of K sub-step s (16 wide) of this wave's rows and columns.
__device__ __forceinline__ void read_ops(StepOps& o, const uint8_t* stage, int wm, int wn,
                                         int lrow, int lk, int s) {
#pragma unroll
  for (int i = 0; i < kWM; ++i)
    o.a[i] = *reinterpret_cast<const half8*>(stage + lds_off(wm * 128 + 32 * i + lrow, 2 * s + lk));
#pragma unroll
  for (int j = 0; j < kWN; ++j)
    o.b[j] = *reinterpret_cast<const half8*>(stage + 2 * kOpBytes +
                                             lds_off(wn * 64 + 32 * j + lrow, 2 * s + lk));
}

// 8 x {1 MFMA, 2 VALU}, with the LDS traffic spread in between.
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
    if (m < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if (m % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
  }
}

// Epilogue straight from the accumulators (the general kernel; on the fast
// path the split tiles and outputs that cannot take 16-byte stores): this
// lane's accumulators of WM x WN blocks starting at (m0, n0).  Lane l holds column (l % 32) of each 32x32
// block; accumulator slot v is row (v % 4) + 8 (v / 4) + 4 (l / 32).  A split
// tile adds its half into the zeroed output: with exactly two addends onto
// zero the sum does not depend on their order (fp32 addition commutes), so
// the result stays deterministic.
//
// BF16 epilogue (no split tiles): C rounds to BF16 (nearest, ties to even)
// and the largest |BF16 value| of the tile goes into *g.amax by one atomic
// max per wave on its binary32 bits (monotone for non-negative values), so
// the next quantization of C can take its amax as given.
template <bool BF16, int WM, int WN>
__device__ __forceinline__ void store_c(const GemmArgs& g, float16v (&acc)[WM][WN], int64_t m0,
                                        int64_t n0, int part, float alpha) {
  const int lane = threadIdx.x & 63, lrow = lane & 31, lk = lane >> 5;
  uint32_t mag = 0u;   // largest |bf16| bits seen by this lane
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n0 + 32 * j + lrow;
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 32 * i + (v & 3) + 8 * (v >> 2) + 4 * lk;
        if (row >= g.M) continue;
        const float val = acc[i][j][v] * alpha;
        if (BF16) {
          const uint32_t u = __float_as_uint(val);
          const uint32_t h = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
          g.cb[row * g.ldc + col] = (uint16_t)h;
          mag = max(mag, h & 0x7FFFu);
        } else {
          float* dst = &g.c[row * g.ldc + col];
          // whole tiles stream C out past the caches (it is not read again
          // here, and cached it would displace operand rows that other tiles
          // still read); a split tile adds its half into the zeroed output
          if (part < 0) __builtin_nontemporal_store(val, dst);
          else atomicAdd(dst, val);
        }
      }
    }
  if (BF16 && g.amax != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off, 64));
    if (lane == 0) atomicMax(g.amax, mag << 16);
  }
}

template <bool CHECKED, bool LD16, bool SDW, bool BF16>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ v2u lut[128];
  if (threadIdx.x < 128) lut[threadIdx.x] = scale_entry(threadIdx.x);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = lane & 31, lk = lane >> 5;
  const int64_t tiles_m = (g.M + kTile - 1) / kTile, tiles_n = (g.N + kTile - 1) / kTile;
  int64_t tm, tn;
  int part;
  block_tile(g.full_tiles, tiles_m, tiles_n, tm, tn, part);
  const OpView va = make_view(g.a, tm * kTile);
  const OpView vb = make_view(g.b, tn * kTile);
  // Bit positions of this thread's two scale codes: byte 0 of s0 / s1 for
  // byte loads; in a scale dword, this K-half's pair sits 2 bytes further in.
  const uint32_t pos0 = SDW ? 16u * (threadIdx.x & 1) : 0u, pos1 = SDW ? pos0 + 8u : 0u;

  float16v acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) acc[i][j] = float16v{};

  // K steps [s0, s1): all of them, or one half for a split tile.  32-bit
  // step arithmetic (K <= 2^23, checked on the host) stays on the scalar unit.
  const int steps = (int)((g.K + kBK - 1) / kBK), half_steps = (steps + 1) / 2;
  const int s0 = part == 1 ? half_steps : 0;
  const int s1 = part == 0 ? half_steps : steps;
  const int last = s1 - 1;
  auto kbyte = [&](int t) { return (uint32_t)((t < last ? t : last) * 32); };
  auto kill = [&](int t) { return t > last ? 0x80000000u : 0u; };

  Raw r0, r1;
  load_raw<LD16, SDW>(r0, va, vb, kbyte(s0), 0u);
  load_raw<LD16, SDW>(r1, va, vb, kbyte(s0 + 1), kill(s0 + 1));
  __syncthreads();  // scale table ready
  zero_tail<CHECKED>(r0, s0, g.K);
  store_half(smem, lut, r0.a.codes, r0.a.s0, pos0, r0.a.s1, pos1, 0, 0);
  store_half(smem, lut, r0.a.codes, r0.a.s0, pos0, r0.a.s1, pos1, 0, 2);
  store_half(smem, lut, r0.b.codes, r0.b.s0, pos0, r0.b.s1, pos1, 1, 0);
  store_half(smem, lut, r0.b.codes, r0.b.s0, pos0, r0.b.s1, pos1, 1, 2);
  load_raw<LD16, SDW>(r0, va, vb, kbyte(s0 + 2), kill(s0 + 2));
  __syncthreads();
  StepOps ops, nxt;
  read_ops(ops, smem, wm, wn, lrow, lk, 0);

  // Step it multiplies stage it&1 while decoding step it+1 (raw set
  // (it+1)&1) into the other stage; after the barrier that raw set is
  // refilled with step it+3.  Two K steps per trip keep the raw sets in fixed
  // registers; the loop body is branch-free (steps past the last are killed
  // re-reads that decode to zeros).
  for (int it = s0; it < s1; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint8_t* cur = smem + (h ? kOpBytes : 0);
      uint8_t* oth = smem + (h ? 0 : kOpBytes);
      Raw& rn = h ? r0 : r1;      // raw data of step it+h+1
      zero_tail<CHECKED>(rn, it + h + 1, g.K);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) read_ops(nxt, cur, wm, wn, lrow, lk, s + 1);
        if (s < 2) store_half(oth, lut, rn.a.codes, rn.a.s0, pos0, rn.a.s1, pos1, 0, (s & 1) * 2);
        else store_half(oth, lut, rn.b.codes, rn.b.s0, pos0, rn.b.s1, pos1, 1, (s & 1) * 2);
        mfma8(acc, ops);
        interleave();
        if (s < 3) ops = nxt;
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      load_raw<LD16, SDW>(rn, va, vb, kbyte(it + h + 3), kill(it + h + 3));
      read_ops(ops, oth, wm, wn, lrow, lk, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  store_c<BF16, kWM, kWN>(g, acc, tm * kTile + wm * 128, tn * kTile + wn * 64, part,
                          (*g.a.ts) * (*g.b.ts));
}

// ---------------------------------------------------------------------------
// Fast path: raw operands moved global -> LDS by the load unit
// ---------------------------------------------------------------------------
// Used when both operands have K-contiguous, 16-byte aligned scale rows
// (dword scales), rows a multiple of 16 bytes and K / 64 steps a multiple of
// 4 (of 8 when the last round of tiles is split).  Same tile (256 x 256) and
// decode as above, different division of work:
//  - 4 waves, one per SIMD.  Wave w owns B rows 64w .. +63 of the tile and
//    all 256 A rows: 8 x 2 blocks of 32 x 32, 256 FP32 accumulators per lane
//    (they live in the accumulation registers).  A is decoded once per
//    workgroup into FP16 in LDS as above; B is private to its wave, so each
//    lane decodes its own B fragments straight into MFMA operand registers.
//    LDS traffic per step: 32 KiB of decoded A written, 128 KiB read (the
//    8-wave kernel: 64 KiB and 192 KiB).
//  - Inside a 64-wide K step, lane half lk takes K 32 lk .. +31, 8 per
//    16-wide sub-step.  The same permutation on A and B leaves the sum
//    unchanged, and a lane's B operand for a step is one 16-byte chunk of
//    codes and one scale dword.
//  - Raw codes reach LDS through buffer loads that write LDS directly, two K
//    steps (64 bytes of a row) at a time, so one load instruction covers 16
//    rows x 64 B instead of 32 rows x 32 B: half the cache lines per byte.
//    Scales come four steps (16 bytes of a row) per load, one row per lane,
//    and each thread keeps its rows' 4-step group in registers.  Each wave
//    loads exactly the A rows it decodes and the B rows it multiplies, so the
//    raw data is wave-private: no barrier, only the wave's own load counter.
//    Two code slots per operand, refilled two steps before they are read;
//    one scale slot per operand, refilled right after the wave has read it
//    into registers, four steps before it is needed.
constexpr int kThreads4 = 256;
constexpr int kMB = 8, kNB = 2;              // 32 x 32 blocks per wave
constexpr int kStage4 = kTile * kRowBytes;   // 32 KiB of decoded A per stage
constexpr int kRawRow = 64;                  // bytes of a row per 2-step group
constexpr int kRawBytes = kTile * kRawRow;   // 16 KiB per operand and slot
constexpr int kScRow = 16;                   // scale bytes of a row per 4-step group
constexpr int kScBytes = kTile * kScRow;     // 4 KiB
// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt not waited on
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw layout [row][4 chunks of 16 B], chunk c of row r at position
// c ^ rg(r): the 16-byte reads of the A decode (8 rows x 2 chunks per 16
// lanes) and of the B fragments (16 rows x 1 chunk) then hit distinct banks.
__device__ __forceinline__ int raw_g(int r) { return ((r >> 1) & 2) | ((r >> 3) & 1); }
__device__ __forceinline__ uint32_t raw_off(int r, int c) {
  return (uint32_t)(r * kRawRow + ((c ^ raw_g(r)) << 4));
}

struct DmaOp {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t voff_c[4];   // this wave's 16-row code loads
  uint32_t voff_s;      // this wave's 64-row scale load
};

// Code load q covers rows crow[q] .. +15 (lane l: row + l / 4, position
// l % 4); the scale load covers 64 rows, lane l row srow(l) (16 bytes: the
// scale dwords of 4 steps), written to scale slot row 64 w + l.
__device__ __forceinline__ DmaOp make_dma(const GemmOperand& op, int64_t row0, const int (&crow)[4],
                                          int srow_l) {
  DmaOp v;
  const int64_t rem_rows = op.rows - row0;
  const int64_t code_bytes = rem_rows * op.ld;
  const uint8_t* sbase = op.scales + (row0 / op.blk_rows) * op.ss_row;
  const int64_t scale_bytes = op.scale_bytes - (row0 / op.blk_rows) * op.ss_row;
  v.codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(op.codes + row0 * op.ld), (short)0,
      (int)(code_bytes < 0x7FFFFFFF ? code_bytes : 0x7FFFFFFF), (int)kBufFlags);
  v.scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sbase), (short)0,
      (int)(scale_bytes < 0x7FFFFFFF ? scale_bytes : 0x7FFFFFFF), (int)kBufFlags);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = crow[q] + (lane >> 2);
    v.voff_c[q] = (uint32_t)(r * op.ld + 16 * ((lane & 3) ^ raw_g(r)));
  }
  v.voff_s = (uint32_t)((srow_l / op.blk_rows) * op.ss_row);
  return v;
}

// Steps x0, x0 + 1 of this wave's rows' codes into a slot (4 load
// instructions); the code offset is clamped to the last step.
template <int NQ>
__device__ __forceinline__ void dma_codes(const DmaOp& v, uint8_t* raw, const int (&crow)[4], int x0,
                                          int last) {
  const uint32_t kb = (uint32_t)((x0 < last ? x0 : last) * 32);
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(v.codes, (lds_ptr_t)(raw + crow[q] * kRawRow), 16,
                                             v.voff_c[q], kb, 0, 0);
}

// Scale dwords of steps x0 .. x0 + 3 of this wave's 64 rows into the scale
// slot (one 16-byte load per lane).  Groups past the last step read 0
// (offset 2^31, past num_records): their blocks decode to zero.
__device__ __forceinline__ void dma_scales(const DmaOp& v, uint8_t* sc, int wave, int x0, int last) {
  const uint32_t dead = x0 > last ? 0x80000000u : 0u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(v.scales, (lds_ptr_t)(sc + 64 * wave * kScRow), 16,
                                           v.voff_s + dead, (uint32_t)(4 * x0), 0, 0);
}

// A thread's raw share of one step, read back from a slot: two rows' 16-byte
// chunks (K-half kh of group step u) and their scale dwords.
struct RawRegs {
  v4u codes[2];
  uint32_t sc[2];
};

// codes of group step u; scale dwords of 4-step group step u4 from the
// registers that hold the group (read from the scale slot once per group)
__device__ __forceinline__ void read_raw(RawRegs& r, const uint8_t* raw, const v4u (&sg)[2],
                                         int row0, int row1, int kh, int u, int u4) {
  r.codes[0] = *reinterpret_cast<const v4u*>(raw + raw_off(row0, 2 * u + kh));
  r.codes[1] = *reinterpret_cast<const v4u*>(raw + raw_off(row1, 2 * u + kh));
  r.sc[0] = sg[0][u4];
  r.sc[1] = sg[1][u4];
}

// The 4-step scale group of two slot rows into registers.
__device__ __forceinline__ void read_sg(v4u (&sg)[2], const uint8_t* sc, int idx0) {
  sg[0] = *reinterpret_cast<const v4u*>(sc + idx0 * kScRow);
  sg[1] = *reinterpret_cast<const v4u*>(sc + (idx0 + 32) * kScRow);
}

// Decode word p of A row (t / 2) + 128 q into a stage (chunk 4 (t % 2) + p).
// pos0: bit offset of the thread's first block scale in the step's dword.
__device__ __forceinline__ void store_a(uint8_t* stage, const RawRegs& r, int q, int p,
                                        uint32_t pos0) {
  const int row = (threadIdx.x >> 1) + 128 * q, h = threadIdx.x & 1;
  const float2v e = scale_pair(r.sc[q] >> pos0);
  *reinterpret_cast<half8*>(stage + lds_off(row, 4 * h + p)) =
      decode8e(r.codes[q][p], p < 2 ? e.x : e.y);
}

struct OpsA { half8 a[kMB]; };
struct OpsB { half8 b[kNB]; };

// B fragments of sub-step s: word s of each of the NB blocks' chunks.
template <int NB>
__device__ __forceinline__ void dec_b(OpsB& o, const RawRegs& r, int s, uint32_t pos0) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float2v e = scale_pair(r.sc[j] >> pos0);
    o.b[j] = decode8e(r.codes[j][s], s < 2 ? e.x : e.y);
  }
}

// A fragments of sub-step s (chunk 4 lk + s of rows 32 i + lane % 32).
__device__ __forceinline__ void read_a(OpsA& o, const uint8_t* stage, int lrow, int lk, int s) {
#pragma unroll
  for (int i = 0; i < kMB; ++i)
    o.a[i] = *reinterpret_cast<const half8*>(stage + lds_off(32 * i + lrow, 4 * lk + s));
}

template <int NB>
__device__ __forceinline__ void mfma16(float16v (&acc)[kMB][NB], const OpsA& a, const OpsB& b) {
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.a[i], b.b[j], acc[i][j], 0, 0, 0);
}

// The MFMAs of a sub-step from linear block index FROM on (block m is
// i = m / NB, j = m % NB, the order of mfma16).
template <int NB, int FROM>
__device__ __forceinline__ void mfma_from(float16v (&acc)[kMB][NB], const OpsA& a, const OpsB& b) {
#pragma unroll
  for (int m = FROM; m < kMB * NB; ++m)
    acc[m / NB][m % NB] =
        __builtin_amdgcn_mfma_f32_32x32x16_f16(a.a[m / NB], b.b[m % NB], acc[m / NB][m % NB], 0, 0, 0);
}

// The first 4 MFMAs of the last sub-step of a K step, after the workgroup
// barrier, with the NQ code loads of a slot refill (steps x0, x0 + 1, as
// dma_codes) issued one after each.  The four waves leave the barrier
// together and share the compute unit's load unit: issued back to back, the
// loads stalled each wave at issue while its matrix core had nothing queued;
// between MFMAs whose operands are already in registers the wait overlaps
// the matrix-core work.
template <int NB, int NQ>
__device__ __forceinline__ void mfma4_dma(float16v (&acc)[kMB][NB], const OpsA& a, const OpsB& b,
                                          const DmaOp& v, uint8_t* raw, const int (&crow)[4],
                                          int x0, int last) {
  const uint32_t kb = (uint32_t)((x0 < last ? x0 : last) * 32);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[m / NB][m % NB] =
        __builtin_amdgcn_mfma_f32_32x32x16_f16(a.a[m / NB], b.b[m % NB], acc[m / NB][m % NB], 0, 0, 0);
    if (m < NQ)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v.codes, (lds_ptr_t)(raw + crow[m] * kRawRow), 16,
                                               v.voff_c[m], kb, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 16 x {1 MFMA, 3 VALU}, with the LDS reads and writes spread in between.
__device__ __forceinline__ void interleave16() {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
    if (m < 9) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    if (m % 5 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
  }
}

// Epilogue of a whole fast-path tile through LDS.  The accumulator layout
// gives each lane one column of 4-row runs, so written straight out every
// store instruction carries 4 bytes per lane, and a wave can keep only 63
// of them in flight: the store phase then took 16 us per tile, about 12%
// of a short-K GEMM.  Here each wave writes its accumulators times the
// tensor scales (FP32, or rounded to BF16) into its own 16 KiB of the
// decoded-A stages (free after the K loop), 4 (FP32) or 8 (BF16) 32 x 32
// blocks at a time, reads them back as 16-byte pieces of rows (4 FP32 or
// 8 BF16 values) and stores those.  Physical LDS row of block row r:
// r ^ ((r >> 2) & 1).  A wave's 2- or 4-byte writes touch rows r and r + 4
// (r % 8 < 4), which this puts in different bank groups; its 16-byte reads
// cover consecutive rows.  Stores go through a buffer resource based at the
// wave's first output element: rows at or past M lie past num_records and a
// piece at or past column N gets an offset of 2^31, so both are dropped with
// no branch (the accumulators there are zero, as operand rows past M and N
// read as zero, so the BF16 amax may take them in).  Needs 256 rows of C
// within 2^31 bytes (checked on the host).  Values, rounding and the amax
// are those of store_c.
template <bool BF16, int NB>
__device__ __forceinline__ void store_c_lds(const GemmArgs& g, float16v (&acc)[kMB][NB],
                                            int64_t m0, int64_t n0, uint8_t* smem, int wave,
                                            float alpha) {
  const int lane = threadIdx.x & 63, lrow = lane & 31, lk = lane >> 5;
  uint8_t* region = smem + wave * 16384;
  constexpr int kEs = BF16 ? 2 : 4;                  // output element bytes
  constexpr int kRowB = 32 * kEs;                    // bytes of a block row in LDS
  constexpr int kBlockB = 32 * kRowB;                // bytes of a block in LDS
  constexpr int kPer = 16384 / kBlockB;              // blocks per pass
  constexpr int kVals = 16 / kEs;                    // values per 16-byte piece
  constexpr int kPieces = 32 / kVals;                // pieces per block row
  constexpr int kRowsPer = 64 / kPieces;             // block rows per store instruction
  constexpr int kBlocks = kMB * NB;
  uint8_t* obase = BF16 ? reinterpret_cast<uint8_t*>(g.cb + m0 * g.ldc + n0)
                        : reinterpret_cast<uint8_t*>(g.c + m0 * g.ldc + n0);
  const int64_t span = (g.M - m0) * g.ldc * kEs;
  const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
      obase, (short)0, (int)(span < 0x7FFFFFFF ? span : 0x7FFFFFFF), (int)kBufFlags);
  const int pr_row = lane / kPieces, pc = lane % kPieces;
  const uint32_t lane_off = (uint32_t)(pr_row * g.ldc + pc * kVals) * kEs;
  uint32_t voff[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    voff[j] = lane_off + (n0 + 32 * j + pc * kVals < g.N ? 0u : 0x80000000u);
  uint32_t mag = 0u;
#pragma unroll
  for (int pass = 0; pass < kBlocks / kPer; ++pass) {
#pragma unroll
    for (int b = 0; b < kPer; ++b) {
      const int idx = pass * kPer + b, i = idx / NB, j = idx % NB;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = (v & 3) + 8 * (v >> 2) + 4 * lk;
        uint8_t* dst = region + b * kBlockB + (r ^ ((r >> 2) & 1)) * kRowB + lrow * kEs;
        const float val = acc[i][j][v] * alpha;
        if (BF16) {
          const uint32_t u = __float_as_uint(val);
          *reinterpret_cast<uint16_t*>(dst) = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        } else {
          *reinterpret_cast<float*>(dst) = val;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int b = 0; b < kPer; ++b) {
      const int idx = pass * kPer + b, i = idx / NB, j = idx % NB;
#pragma unroll
      for (int q = 0; q < 32 / kRowsPer; ++q) {
        const int r = pr_row + kRowsPer * q;
        const v4u val = *reinterpret_cast<const v4u*>(region + b * kBlockB +
                                                      (r ^ ((r >> 2) & 1)) * kRowB + 16 * pc);
        if (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mag = max(mag, max(val[e] & 0x7FFFu, (val[e] >> 16) & 0x7FFFu));
        }
        const uint32_t soff = (uint32_t)(((32 * i + kRowsPer * q) * g.ldc + 32 * j) * kEs);
        __builtin_amdgcn_raw_buffer_store_b128(val, out, voff[j], soff, kNontemporal);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next pass overwrites
    __builtin_amdgcn_wave_barrier();
  }
  if (BF16 && g.amax != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off, 64));
    if (lane == 0) atomicMax(g.amax, mag << 16);
  }
}

// K-split tail tiles with the BF16 epilogue.  The two K halves of a tile
// compute partial accumulators P0 and P1; FP32 output adds alpha P0 and
// alpha P1 into a zeroed C, fl(alpha P0 + alpha P1) whatever their order.
// The BF16 output is that sum rounded, so the halves meet in a workspace
// instead: each stores its scaled partial, and thread 0 takes a ticket with
// one acquire-release atomic add on the slot's counter.  The half that draws
// ticket 1 finishes second: the other partial is complete, so it adds it to
// its own (the same commutative sum) and writes the tile; the first half
// returns without writing anything.  No workgroup waits for another.
// Layout: per wave, 16-byte pieces of four consecutive accumulator slots,
// 64 lanes' pieces side by side (1 KiB per wave instruction).
constexpr int64_t kSplitSlotFloats = 4 * kMB * 2 * 16 * 64;   // one K half of a 256 x 256 tile
constexpr int kAgentScope = 16;   // buffer cache policy sc1: coherent across the XCDs

template <int NB>
__device__ __forceinline__ bool bf16_split_exchange(const GemmArgs& g, float16v (&acc)[kMB][NB],
                                                    int part, int64_t slot, int wave,
                                                    float alpha, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  // the slot's two partials; this lane's pieces at voff + 1024 c in each
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      g.ws + 2 * slot * kSplitSlotFloats, (short)0, (int)(2 * kSplitSlotFloats * 4),
      (int)kBufFlags);
  const uint32_t voff = (uint32_t)(wave * (kMB * NB * 4 * 64) + lane) * 16u;
  const uint32_t mine = (uint32_t)(part * kSplitSlotFloats * 4);
  const uint32_t other = (uint32_t)((part ^ 1) * kSplitSlotFloats * 4);
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(v4u, v4f{acc[i][j][4 * q] * alpha, acc[i][j][4 * q + 1] * alpha,
                                        acc[i][j][4 * q + 2] * alpha,
                                        acc[i][j][4 * q + 3] * alpha}),
            ws, voff, mine + (uint32_t)(((i * NB + j) * 4 + q) * 1024), kAgentScope);
  // The partial words move with agent-scope (sc1) stores and loads, which
  // write through and read past the per-XCD caches (the halves usually run
  // on different XCDs); each wave waits until its stores are complete before
  // the barrier.  Thread 0's ticket then orders them formally: every wave's
  // stores happen before it (barrier), it releases them at agent scope and
  // acquires the other half's, and the barrier after it carries that to
  // every wave's loads.  Only thread 0 fences: an agent-scope fence writes
  // back and invalidates this XCD's whole L2, which the workgroups still
  // streaming operands there would pay for.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();     // also: the decoded-A stages are free
  int* ticket = reinterpret_cast<int*>(smem);
  if (threadIdx.x == 0)
    *ticket = (int)__hip_atomic_fetch_add(g.ws_tickets + slot, 1u, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = *ticket == 1;
  __syncthreads();     // the ticket is read before the epilogue reuses the stages
  if (!last) return false;
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f o = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(
                     ws, voff, other + (uint32_t)(((i * NB + j) * 4 + q) * 1024), kAgentScope));
        // (0 + other) + own: the FP32 path's two adds onto a zero, also for
        // two partials of -0 (which it turns into +0)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[i][j][4 * q + k] = (0.0f + o[k]) + acc[i][j][4 * q + k] * alpha;
      }
  return true;
}

// One tile (or half-width tail tile) of the fast path: A rows tm * 256 ..
// +255, B rows b_row0 .. + 64 NB * 4 - 1 (NB blocks of 32 per wave: 2 for
// a whole 256-wide tile, 1 for a half-width one), K part `part`.
template <bool BF16, int NB>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs& g, int64_t tm, int64_t b_row0,
                                              int part, int64_t slot, int wave, uint8_t* smem,
                                              uint8_t* rawA0,
                                              uint8_t* rawA1, uint8_t* rawB0, uint8_t* rawB1,
                                              uint8_t* scA, uint8_t* scB) {
  const int t = threadIdx.x, lane = t & 63;
  const int lrow = lane & 31, lk = lane >> 5;
  const int a_crow[4] = {32 * wave, 32 * wave + 16, 128 + 32 * wave, 128 + 32 * wave + 16};
  // B rows of this wave: 32 NB from 32 NB w (the code loads of a half-width
  // tile repeat their two row ranges; only NB * 2 of them are issued)
  const int bw = 32 * NB * wave;
  const int b_crow[4] = {bw, bw + 16, bw + 32 * (NB - 1), bw + 32 * (NB - 1) + 16};
  // scale slot row 64 w + l holds A row 32 w + l (l < 32) or 128 + 32 w + l - 32,
  // and B row bw + l (whole tile) or bw + l % 32 (half-width, repeated)
  const int a_srow = lane < 32 ? 32 * wave + lane : 128 + 32 * wave + lane - 32;
  const DmaOp va = make_dma(g.a, tm * kTile, a_crow, a_srow);
  const DmaOp vb = make_dma(g.b, b_row0, b_crow, NB == 2 ? bw + lane : bw + (lane & 31));
  // A rows this thread decodes; B rows whose fragments this lane holds; and
  // their scale slot rows (the second row's is 32 further)
  const int ar0 = t >> 1, ar1 = 128 + (t >> 1), ah = t & 1;
  const int br0 = bw + lrow, br1 = NB == 2 ? br0 + 32 : br0;
  const int a_sidx = 64 * wave + (lane >> 1), b_sidx = 64 * wave + lrow;
  // bit positions of the step's two block scales in a scale dword
  const uint32_t apos0 = 16u * ah;   // bit offsets of the first block scale of a K half
  const uint32_t bpos0 = 16u * lk;
  // alpha = s_a s_b, read now so that its latency hides under the prologue's
  // loads instead of following the K loop (uniform: kept in a scalar register)
  float alpha = __uint_as_float(__builtin_amdgcn_readfirstlane(
      __float_as_uint((*g.a.ts) * (*g.b.ts))));

  float16v acc[kMB][NB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = float16v{};

  const int steps = (int)(g.K / kBK), half_steps = (steps + 1) / 2;
  const int s0 = part == 1 ? half_steps : 0;
  const int s1 = part == 0 ? half_steps : steps;
  const int last = s1 - 1;

  // scale group 0 (steps s0 .. s0 + 3), code groups 0 and 1 (steps s0 .. s0 + 3)
  dma_scales(va, scA, wave, s0, last);
  dma_scales(vb, scB, wave, s0, last);
  dma_codes<4>(va, rawA0, a_crow, s0, last);
  dma_codes<2 * NB>(vb, rawB0, b_crow, s0, last);
  dma_codes<4>(va, rawA1, a_crow, s0 + 2, last);
  dma_codes<2 * NB>(vb, rawB1, b_crow, s0 + 2, last);
  // scale group 0 and code group 0 landed (code group 1 may be in flight)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 + 2 * NB));
  __builtin_amdgcn_sched_barrier(0);
  v4u sa[2], sb[2];   // scale dwords of the current 4-step groups
  read_sg(sa, scA, a_sidx);
  read_sg(sb, scB, b_sidx);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slots are read before reloading them
  __builtin_amdgcn_sched_barrier(0);
  dma_scales(va, scA, wave, s0 + 4, last);
  dma_scales(vb, scB, wave, s0 + 4, last);
  RawRegs ra, rb;
  read_raw(ra, rawA0, sa, ar0, ar1, ah, 0, 0);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) store_a(smem, ra, q, p, apos0);
  read_raw(ra, rawA0, sa, ar0, ar1, ah, 1, 1);
  read_raw(rb, rawB0, sb, br0, br1, lk, 0, 0);
  OpsB bcur, bnxt;
  dec_b<NB>(bcur, rb, 0, bpos0);
  __syncthreads();
  OpsA acur, anxt;
  read_a(acur, smem, lrow, lk, 0);

  // Step x (h = (x - s0) % 4) multiplies decoded A stage h % 2 with B(x)
  // (decoded one sub-step ahead from rb) while decoding A(x+1) (ra) into
  // the other stage.  Raw code slot of steps x, x+1 (x even): h / 2.  At the
  // last sub-step: barrier (A(x+1) is complete), then an even step refills
  // its A code slot with steps x+4, x+5 and an odd step its B slot with steps
  // x+3, x+4 (both last read a step earlier), and ra / rb are reloaded with
  // A(x+2) / B(x+1), whose codes were loaded two steps ago.  Scales: the
  // registers sa / sb hold a 4-step group; at h = 2 (A) and h = 3 (B) they
  // move on to the next group and its slot is refilled with the group after.
  // Load order per trip: A codes, B codes, A codes + A scales, B codes + B
  // scales; the counts below leave exactly the loads issued since the ones
  // needed in flight.
  for (int it = s0; it < s1; it += 4) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int x = it + h;
      uint8_t* cur = smem + ((h & 1) ? kStage4 : 0);
      uint8_t* oth = smem + ((h & 1) ? 0 : kStage4);
      const int a2 = ((h + 2) >> 1) & 1, b1 = ((h + 1) >> 1) & 1;   // code slots of A(x+2), B(x+1)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
          read_a(anxt, cur, lrow, lk, s + 1);
          dec_b<NB>(bnxt, rb, s + 1, bpos0);
          if (s == 0) {
            store_a(oth, ra, 0, 0, apos0);
            store_a(oth, ra, 0, 1, apos0);
            store_a(oth, ra, 0, 2, apos0);
          } else if (s == 1) {
            store_a(oth, ra, 0, 3, apos0);
            store_a(oth, ra, 1, 0, apos0);
            store_a(oth, ra, 1, 1, apos0);
          } else {
            store_a(oth, ra, 1, 2, apos0);
            store_a(oth, ra, 1, 3, apos0);
          }
          mfma16<NB>(acc, acur, bcur);
          interleave16();
          acur = anxt;
          bcur = bnxt;
        } else {
          // This wave's own raw data for the next steps first (its code and
          // scale slots are private to it): the load wait and the raw reads,
          // whose latency then passes at the barrier; after it only the
          // shared decoded-A reads remain.  Per trip the loads go A codes (4),
          // B codes (2 NB), A codes + A scales, B codes + B scales; the waits
          // come before this step's loads, so they allow that many fewer in
          // flight.
          if (h == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NB + 2));
          else if (h == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NB));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
          __builtin_amdgcn_sched_barrier(0);
          // a new 4-step scale group first: read_raw takes its scale dwords
          // from these registers (at h = 3 B(x + 1) starts the next group)
          if (h == 2) read_sg(sa, scA, a_sidx);
          if (h == 3) read_sg(sb, scB, b_sidx);
          read_raw(rb, b1 ? rawB1 : rawB0, sb, br0, br1, lk, (h + 1) & 1, (h + 1) & 3);
          read_raw(ra, a2 ? rawA1 : rawA0, sa, ar0, ar1, ah, h & 1, (h + 2) & 3);
          // this wave's decode writes and reads done, then the workgroup
          // barrier; no memory fence, which would also wait for the raw loads
          // in flight
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          read_a(anxt, oth, lrow, lk, 0);
          __builtin_amdgcn_sched_barrier(0);
          if ((h & 1) == 0)
            mfma4_dma<NB, 4>(acc, acur, bcur, va, (h >> 1) ? rawA1 : rawA0, a_crow, x + 4, last);
          else
            mfma4_dma<NB, 2 * NB>(acc, acur, bcur, vb, (h >> 1) ? rawB1 : rawB0, b_crow, x + 3, last);
          dec_b<NB>(bnxt, rb, 0, bpos0);
          mfma_from<NB, 4>(acc, acur, bcur);
          interleave16();
          if (h >= 2) {
            // the scale slot refill after the code loads (the load waits
            // count them in this order); the slot was read before the barrier
            __builtin_amdgcn_sched_barrier(0);
            if (h == 2) dma_scales(va, scA, wave, it + 8, last);
            else dma_scales(vb, scB, wave, it + 8, last);
          }
          acur = anxt;
          bcur = bnxt;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // loads of the groups past the end

  if (BF16 && part >= 0) {
    // a K half of a BF16 tail tile: the workgroup that finishes second writes
    // the tile from both halves' partials, already scaled (alpha 1)
    if (!bf16_split_exchange<NB>(g, acc, part, slot, wave, alpha, smem)) return;
    alpha = 1.0f;
    part = -1;
  }
  if (part < 0 && g.vec_out) {
    __syncthreads();   // every wave is done with the decoded-A stages
    store_c_lds<BF16, NB>(g, acc, tm * kTile, b_row0 + bw, smem, wave, alpha);
  } else {
    store_c<BF16, kMB, NB>(g, acc, tm * kTile, b_row0 + bw, part, alpha);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads4, 1) void k_gemm_dma(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // decoded A, 2 stages
  // raw code slots and scale slots as separate arrays (one LDS object each)
  __shared__ __attribute__((aligned(16))) uint8_t rawA0[kRawBytes], rawA1[kRawBytes];
  __shared__ __attribute__((aligned(16))) uint8_t rawB0[kRawBytes], rawB1[kRawBytes];
  __shared__ __attribute__((aligned(16))) uint8_t scA[kScBytes], scB[kScBytes];
  // wave and tile indices in scalar registers: the buffer descriptors and LDS
  // load bases built from them must be uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tiles_m = (g.M + kTile - 1) / kTile, tiles_n = (g.N + kTile - 1) / kTile;
  int64_t tm, tn;
  int part, nh;
  block_tile(g.full_tiles, tiles_m, tiles_n, g.tail, tm, tn, part, nh);
  tm = __builtin_amdgcn_readfirstlane((int)tm);
  tn = __builtin_amdgcn_readfirstlane((int)tn);
  part = __builtin_amdgcn_readfirstlane(part);
  nh = __builtin_amdgcn_readfirstlane(nh);
  // split slot of a K half (BF16 epilogue): tail tile, and its N half
  const int pieces = g.tail == kTailNK ? 4 : 2;
  const int64_t slot = part < 0 ? 0
                                : ((int64_t)blockIdx.x - g.full_tiles) / pieces *
                                          (g.tail == kTailNK ? 2 : 1) + (nh < 0 ? 0 : nh);
  if (nh < 0)
    gemm_dma_tile<BF16, 2>(g, tm, tn * kTile, part, slot, wave, smem, rawA0, rawA1, rawB0, rawB1,
                           scA, scB);
  else
    gemm_dma_tile<BF16, 1>(g, tm, tn * kTile + 128 * nh, part, slot, wave, smem, rawA0, rawA1,
                           rawB0, rawB1, scA, scB);
}


// Zero the output tiles that split workgroups add into, same tile order as
// the GEMM: 16 workgroups per tile, 16 rows each; with VEC (N and ldc
// multiples of 4, 16-byte aligned base, so a store never straddles N) a
// thread clears 4 columns of 4 rows with 16-byte stores, else one column of
// its 16 rows.
constexpr int kZeroSlabs = kTile / 16;
template <bool VEC>
__global__ __launch_bounds__(256) void k_zero_tiles(float* __restrict__ c, int64_t ldc,
                                                    int64_t M, int64_t N, int64_t tiles_m,
                                                    int64_t tiles_n, int64_t first) {
  int64_t tm, tn;
  grouped(first + blockIdx.x / kZeroSlabs, tiles_m, tiles_n, tm, tn);
  const int64_t row0 = tm * kTile + 16 * (blockIdx.x % kZeroSlabs);
  if (VEC) {
    const int64_t col = tn * kTile + 4 * (threadIdx.x & 63);
    if (col >= N) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t row = row0 + (threadIdx.x >> 6) + 4 * k;
      if (row < M) *reinterpret_cast<v4f*>(&c[row * ldc + col]) = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
  } else {
    const int64_t col = tn * kTile + threadIdx.x;
    if (col >= N) return;
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + r;
      if (row >= M) break;
      c[row * ldc + col] = 0.0f;
    }
  }
}

TilePlan plan_tiles(int64_t M, int64_t N, int64_t steps, bool allow_split, bool allow_narrow) {
  TilePlan p;
  p.tiles_m = (M + kTile - 1) / kTile;
  p.tiles_n = (N + kTile - 1) / kTile;
  const int64_t tiles = p.tiles_m * p.tiles_n;
  // One workgroup per CU is resident (LDS).  A last round that would leave
  // CUs idle is cut into more, shorter pieces: four (half-width x K halves,
  // about 0.3 of a round) when they still fit one round, else two K halves
  // (half a round), else two half-width tiles (about 0.6 of a round).
  const int64_t slots = num_cus();
  p.rem = tiles % slots;
  p.tail = kTailWhole;
  if (tiles > slots && p.rem > 0) {
    if (allow_split && allow_narrow && 4 * p.rem <= slots && steps >= 4) p.tail = kTailNK;
    else if (allow_split && 2 * p.rem <= slots && steps >= 4) p.tail = kTailK;
    else if (allow_narrow && 2 * p.rem <= slots) p.tail = kTailN;
  }
  p.split = (p.tail & kTailK) != 0;
  const int64_t pieces = p.tail == kTailNK ? 4 : 2;
  p.full_tiles = p.tail == kTailWhole ? tiles : tiles - p.rem;
  p.grid = p.tail == kTailWhole ? tiles : p.full_tiles + pieces * p.rem;
  return p;
}

hipError_t zero_split_tiles(const TilePlan& p, float* c, int64_t ldc, int64_t M, int64_t N,
                            hipStream_t s) {
  if (!p.split) return hipSuccess;
  const dim3 grid((unsigned)(p.rem * kZeroSlabs));
  if (N % 4 == 0 && ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0)
    hipLaunchKernelGGL(k_zero_tiles<true>, grid, dim3(256), 0, s, c, ldc, M, N, p.tiles_m,
                       p.tiles_n, p.full_tiles);
  else
    hipLaunchKernelGGL(k_zero_tiles<false>, grid, dim3(256), 0, s, c, ldc, M, N, p.tiles_m,
                       p.tiles_n, p.full_tiles);
  return hipGetLastError();
}

// The BF16 epilogue's K-split workspace: per split slot (a tail tile, or
// one N half of it) two partial buffers, then one ticket word per slot.
static int64_t split_slots(const TilePlan& p) {
  return p.split ? p.rem * (p.tail == kTailNK ? 2 : 1) : 0;
}
static int64_t split_partial_bytes(int64_t slots) {
  return slots * 2 * kSplitSlotFloats * (int64_t)sizeof(float);
}
static int64_t split_ws_bytes(int64_t slots) {
  return slots == 0 ? 0 : split_partial_bytes(slots) + ((slots * 4 + 255) & ~(int64_t)255);
}

int64_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // the plan a fast-path launch with a workspace makes (plan_tiles below)
  return split_ws_bytes(split_slots(plan_tiles(M, N, (K + kBK - 1) / kBK, true, true)));
}

// The BF16 epilogue's start: its amax word (when given) and the n split
// tickets cleared in one launch (a kernel, not a memset: capture-safe).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ amax,
                                                    uint32_t* __restrict__ p, int64_t n) {
  if (amax != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *amax = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

static hipError_t launch_gemm_any(const GemmOperand& a, const GemmOperand& b, int64_t K,
                                  float* c, uint16_t* cb, uint32_t* amax, int64_t ldc,
                                  void* ws, int64_t ws_bytes, hipStream_t s) {
  const bool bf16 = cb != nullptr;
  // 16-byte output stores: 4 FP32 or 8 BF16 values of a row per store
  const uintptr_t cbase = bf16 ? reinterpret_cast<uintptr_t>(cb) : reinterpret_cast<uintptr_t>(c);
  const int vec_out = (ldc % (bf16 ? 8 : 4)) == 0 && (cbase & 15) == 0 &&
                      ldc * kTile * (bf16 ? 2 : 4) < ((int64_t)1 << 31);
  GemmArgs g{a, b, a.rows, b.rows, K, c, cb, amax, ldc, 0, kTailWhole, vec_out};
  const bool ld16 = (a.ld % 16 == 0) && (b.ld % 16 == 0);
  const bool checked = (K % 64) != 0;
  // dword scales: scales contiguous along K, every row's scales 4-byte
  // aligned (K % 64 == 0 makes each row's K/16 bytes a multiple of 4)
  auto sdw_ok = [](const GemmOperand& o) {
    return o.ss_k == 1 && o.ss_row % 4 == 0 && (reinterpret_cast<uintptr_t>(o.scales) & 3) == 0;
  };
  const bool sdw = !checked && ld16 && sdw_ok(a) && sdw_ok(b);
  // fast path: whole 4-step trips in every K range a workgroup takes, scale
  // rows 16-byte aligned (codes are 16-byte aligned, checked by the API)
  const int64_t steps = K / kBK;
  auto sc16 = [](const GemmOperand& o) {   // 4-step scale groups as 16-byte loads
    return o.ss_row % 16 == 0 && (reinterpret_cast<uintptr_t>(o.scales) & 15) == 0;
  };
  const bool dma = sdw && steps % 4 == 0 && sc16(a) && sc16(b);
  // The tail plan: K halves need an FP32 output (two addends onto zero) and,
  // on the fast path, whole 4-step trips per half; half-width tail tiles
  // exist on the fast path only.
  // With a BF16 output the K halves meet in the workspace (bf16_split_exchange),
  // so they need one, and the fast path.
  const bool split_ok = bf16 ? (ws != nullptr && dma && steps % 8 == 0) : (!dma || steps % 8 == 0);
  const TilePlan plan = plan_tiles(g.M, g.N, (K + kBK - 1) / kBK, split_ok, dma);
  g.full_tiles = plan.full_tiles;
  g.tail = plan.tail;
  const dim3 grid((unsigned)plan.grid);
  if (bf16) {
    int64_t slots = 0;
    if (plan.split) {
      slots = split_slots(plan);
      if (split_ws_bytes(slots) > ws_bytes) return hipErrorInvalidValue;
      g.ws = static_cast<float*>(ws);
      g.ws_tickets =
          reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + split_partial_bytes(slots));
    }
    if (amax != nullptr || slots > 0) {
      hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, s, amax, g.ws_tickets, slots);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    const hipError_t e = zero_split_tiles(plan, c, ldc, g.M, g.N, s);
    if (e != hipSuccess) return e;
  }
#define NVFP4_GEMM_LAUNCH_B(C, L, W, B)                                                  \
  do {                                                                                    \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<C, L, W, B>), \
                                       hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                       kLdsBytes);                                       \
    if (e != hipSuccess) return e;                                                        \
    hipLaunchKernelGGL((k_gemm<C, L, W, B>), grid, dim3(kThreads), kLdsBytes, s, g);      \
  } while (0)
#define NVFP4_GEMM_LAUNCH(C, L, W)          \
  do {                                     \
    if (bf16) NVFP4_GEMM_LAUNCH_B(C, L, W, true);  \
    else NVFP4_GEMM_LAUNCH_B(C, L, W, false);      \
  } while (0)
  if (dma) {
    // 64 KiB of dynamic LDS (decoded A) on top of the 72 KiB of raw slots
    const void* fn = bf16 ? reinterpret_cast<const void*>(&k_gemm_dma<true>)
                          : reinterpret_cast<const void*>(&k_gemm_dma<false>);
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStage4);
    if (e != hipSuccess) return e;
    if (bf16) hipLaunchKernelGGL((k_gemm_dma<true>), grid, dim3(kThreads4), 2 * kStage4, s, g);
    else hipLaunchKernelGGL((k_gemm_dma<false>), grid, dim3(kThreads4), 2 * kStage4, s, g);
  } else if (sdw) NVFP4_GEMM_LAUNCH(false, true, true);
  else if (checked) {
    if (ld16) NVFP4_GEMM_LAUNCH(true, true, false);
    else NVFP4_GEMM_LAUNCH(true, false, false);
  } else {
    if (ld16) NVFP4_GEMM_LAUNCH(false, true, false);
    else NVFP4_GEMM_LAUNCH(false, false, false);
  }
#undef NVFP4_GEMM_LAUNCH
#undef NVFP4_GEMM_LAUNCH_B
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, float* c,
                       int64_t ldc, hipStream_t s) {
  return launch_gemm_any(a, b, K, c, nullptr, nullptr, ldc, nullptr, 0, s);
}

hipError_t launch_gemm_bf16(const GemmOperand& a, const GemmOperand& b, int64_t K, uint16_t* c,
                            int64_t ldc, float* amax, void* ws, int64_t ws_bytes, hipStream_t s) {
  return launch_gemm_any(a, b, K, nullptr, c, reinterpret_cast<uint32_t*>(amax), ldc, ws, ws_bytes,
                         s);
}

// The allocation-free BF16 GEMM's workspace: a file-scope device array, one
// per GPU, held for the life of the process.  Its size covers every split
// plan on a 256-CU device (at most 128 slots: 2 x rem <= 256 for K halves,
// 4 x rem <= 256 with N halves).  The host uses its device address (looked
// up once per device), never the symbol itself.
constexpr int64_t kNoAllocSlots = 128;
constexpr int64_t kNoAllocBytes = kNoAllocSlots * 2 * kSplitSlotFloats * 4 + kNoAllocSlots * 4;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

static hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

int64_t gemm_bf16_noalloc_max_bytes() { return kNoAllocBytes; }

hipError_t launch_gemm_bf16_noalloc(const GemmOperand& a, const GemmOperand& b, int64_t K,
                                    uint16_t* c, int64_t ldc, float* amax, hipStream_t s) {
  if (gemm_bf16_workspace_bytes(a.rows, b.rows, K) > kNoAllocBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_gemm_any(a, b, K, nullptr, c, reinterpret_cast<uint32_t*>(amax), ldc, ws,
                         kNoAllocBytes, s);
}

}  // namespace nvfp4
