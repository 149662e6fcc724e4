// nvfp4_quant.hip -- gfx950 kernels for NVFP4 quantization: tensor amax (plain
// and under the 16-point RHT), 1D rowwise, 1D colwise (transpose-quantize,
// optional RHT), 2D 16x16 tiles (optional transposed codes) and dequantize.
//
// Built for HBM bandwidth: 16-byte loads (8 bf16 per lane), lanes of a wave on
// consecutive 16-byte chunks, packed 4-bit stores, no re-reads inside a pass.
// The amax and RTN kernels are bound by HBM; the stochastic-rounding encodes
// by their rounding arithmetic (about 20 VALU per element, plus Philox).
// The tensor scale is re-derived from the device amax by every workgroup, so
// no host round trip separates the amax pass from the encode pass.
//
// Sources: "Pretraining Large Language Models with NVFP4" (summary page,
// format and limitations paragraphs); "NVFP4 Trains with Precision of 16-Bit
// and Speed and Efficiency of 4-Bit" (micro-block scaling, E4M3 scales,
// Hadamard transforms, 2D block quantization, stochastic rounding); news item
// "Soumith Chintala 发布 NVFP4 训练详解文章", section 三 (1D blocks for
// activations and gradients, 2D for weights, RHT on Wgrad inputs).
#include "gemm_tiles.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// amax
// ---------------------------------------------------------------------------
// Zero one or two 32-bit words (the amax accumulators) in one launch.
__global__ void k_zero_u32(uint32_t* p, uint32_t* q) {
  *p = 0u;
  if (q != nullptr) *q = 0u;
}

// Block-wide max of non-negative float bit patterns, then one atomic per
// workgroup.  Non-negative binary32 values order like their bit patterns.
__device__ __forceinline__ void block_max_atomic(uint32_t m, uint32_t* out) {
  __shared__ uint32_t red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = m > o ? m : o;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
    atomicMax(out, r);
  }
}

// |x| of bf16 is its bit pattern with the sign cleared, and non-negative bf16
// patterns order like their values: the amax runs on packed 16-bit integer
// maxima (two elements per 32-bit lane op).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t lo = (a & 0xFFFFu) > (b & 0xFFFFu) ? (a & 0xFFFFu) : (b & 0xFFFFu);
  uint32_t hi = (a >> 16) > (b >> 16) ? (a >> 16) : (b >> 16);
  return lo | (hi << 16);
}

// Each workgroup reads whole 32 KiB chunks (8 loads of 16 bytes per thread,
// the lanes of a wave on consecutive 16-byte pieces); chunks are dealt to the
// workgroups in turn.  On MI355X this runs at 0.72 of the HBM peak, against
// 0.59 for a grid-stride loop whose loads in flight lie a whole grid apart.
constexpr int kAmaxU = 8;
constexpr int64_t kAmaxChunk = (int64_t)kAmaxU * kThreads;  // 16-byte vectors

__device__ __forceinline__ uint32_t amax_acc(uint32_t m, const v4u v) {
  m = pk_max_u16(m, v.x & 0x7FFF7FFFu);
  m = pk_max_u16(m, v.y & 0x7FFF7FFFu);
  m = pk_max_u16(m, v.z & 0x7FFF7FFFu);
  return pk_max_u16(m, v.w & 0x7FFF7FFFu);
}

__global__ __launch_bounds__(kThreads) void k_amax(const v4u* __restrict__ x, int64_t nvec,
                                                     uint32_t* __restrict__ out) {
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kAmaxChunk; c < nvec;
       c += (int64_t)gridDim.x * kAmaxChunk) {
    if (c + kAmaxChunk <= nvec) {
      v4u v[kAmaxU];
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) v[u] = ld_(&x[c + u * kThreads + threadIdx.x]);
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) m = amax_acc(m, v[u]);
    } else {
      for (int64_t i = c + threadIdx.x; i < nvec; i += kThreads) m = amax_acc(m, ld_(&x[i]));
    }
  }
  uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  uint32_t bf = lo > hi ? lo : hi;
  block_max_atomic(bf << 16, out);
}

// amax of the rowwise RHT of x (the transform over every 16 consecutive
// columns of each row), with k_amax's chunked read.  A vector (8 elements) and
// its partner (the other half of the 16-block, vector index ^ 1) sit in
// adjacent lanes: chunks start at even vectors and the vector count is even.
__device__ __forceinline__ float rht_row_amax(const v4u v, uint32_t signs, bool hi) {
  float z[8];
  unpack8_flip(v, hi ? signs >> 8 : signs, z);
  rht16_pair_butterflies<false>(z, hi);   // 4 * the transform
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(z[j]));
  return m;   // 4 * the amax, exactly
}

__global__ __launch_bounds__(kThreads) void k_amax_rht_row(const v4u* __restrict__ x,
                                                             int64_t nvec, uint64_t rht_seed,
                                                             uint32_t* __restrict__ out) {
  const uint32_t signs = rht_sign_bits(rht_seed);
  const bool hi = threadIdx.x & 1;   // vector index parity (chunks start at even vectors)
  float m = 0.0f;
  for (int64_t c = (int64_t)blockIdx.x * kAmaxChunk; c < nvec;
       c += (int64_t)gridDim.x * kAmaxChunk) {
    if (c + kAmaxChunk <= nvec) {
      v4u v[kAmaxU];
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) v[u] = ld_(&x[c + u * kThreads + threadIdx.x]);
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) m = fmaxf(m, rht_row_amax(v[u], signs, hi));
    } else {
      for (int64_t i = c + threadIdx.x; i < nvec; i += kThreads)
        m = fmaxf(m, rht_row_amax(ld_(&x[i]), signs, hi));
    }
  }
  block_max_atomic(__float_as_uint(m * 0.25f), out);
}

// Load a 16-row x 8-column bf16 micro-tile (one 16-byte chunk per row) and
// return column j's 16 values as binary32.
struct Tile16x8 { v4u row[16]; };

__device__ __forceinline__ void tile_load(Tile16x8& t, const uint16_t* __restrict__ x,
                                          int64_t cols, int64_t r0, int64_t c0) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    t.row[j] = ld_(
        reinterpret_cast<const v4u*>(x + (r0 + j) * cols + c0));
}

// The sign of element j is flipped where bit j of signs is set (the RHT's
// sign flips; 0 for none).
__device__ __forceinline__ void tile_column(const Tile16x8& t, int c, float (&v)[16],
                                            uint32_t signs = 0u) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t w = (c >> 1) == 0 ? t.row[j].x : (c >> 1) == 1 ? t.row[j].y
               : (c >> 1) == 2 ? t.row[j].z : t.row[j].w;
    v[j] = (c & 1) ? bf16_hi_flip(w, flip_bit(signs, j)) : bf16_lo_flip(w, flip_bit(signs, j));
  }
}

// amax of RHT(x^T): each work item is 16 consecutive rows x 8 columns.
// PLAIN: also max |x| over the same elements (before the transform) into
// *out_plain, so one read of the tensor gives both statistics.
template <bool PLAIN>
__global__ __launch_bounds__(kThreads) void k_amax_rht(const uint16_t* __restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         uint64_t rht_seed,
                                                         uint32_t* __restrict__ out,
                                                         uint32_t* __restrict__ out_plain) {
  const uint32_t signs = rht_sign_bits(rht_seed);
  const int64_t cg_n = cols / 8, items = (rows / 16) * cg_n;
  float m = 0.0f, p = 0.0f;
  for (int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kThreads) {
    const int64_t rg = it / cg_n, cg = it - rg * cg_n;
    Tile16x8 t;
    tile_load(t, x, cols, rg * 16, cg * 8);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[16];
      tile_column(t, c, v, signs);   // |v| is unaffected by the flips
      if (PLAIN) {
#pragma unroll
        for (int j = 0; j < 16; ++j) p = fmaxf(p, __builtin_fabsf(v[j]));
      }
      rht16_butterflies<false>(v);   // 4 * the transform; the 1/4 is taken on the max
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
    }
  }
  block_max_atomic(__float_as_uint(m * 0.25f), out);
  if (PLAIN) {
    __syncthreads();   // the reduction slots are reused
    block_max_atomic(__float_as_uint(p), out_plain);
  }
}

// ---------------------------------------------------------------------------
// 1D rowwise: blocks of 16 along cols, two lanes per block
// ---------------------------------------------------------------------------
// Each workgroup takes 16 KiB chunks of the input (4 vectors of 8 elements
// per thread, loaded before any is encoded), dealt to the workgroups in turn.
// A vector's partner (i ^ 1, the other half of its 16-block) is always in the
// same wave and in range together with it: chunks start at even vectors and
// the vector count is even (cols % 16 == 0).
constexpr int kRowU = 4;
constexpr int64_t kRowChunk = (int64_t)kRowU * kThreads;

// RHT: each 16-block is first replaced by its 16-point transform (the two
// lanes of the block exchange their halves for the last butterfly stage).
template <bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_row(
    const v4u* __restrict__ x, int64_t nvec, const float* __restrict__ amax,
    uint64_t rht_seed, uint64_t seed, uint32_t stream_id, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ ts_out) {
  __shared__ float rtab[kE4m3Codes];
  static_assert(kThreads >= kE4m3Codes, "one thread per table entry");
  auto load_chunk = [&](v4u (&v)[kRowU], int64_t c) {
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int64_t i = c + u * kThreads + threadIdx.x;
      if (i < nvec) v[u] = ld_(&x[i]);
    }
  };
  // The SR encodes load one chunk ahead (the first one before the table
  // set-up), so that their rounding arithmetic covers the next chunk's
  // loads; the RTN encodes, with little arithmetic per element, run at a
  // higher occupancy without the extra registers.
  constexpr bool kAhead = SR;
  const int64_t stride = (int64_t)gridDim.x * kRowChunk;
  v4u nxt[kRowU];
  if (kAhead) load_chunk(nxt, (int64_t)blockIdx.x * kRowChunk);
  const ScaleCtx sc = scale_ctx(*amax, rtab, threadIdx.x);
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = sc.s_t;
  const uint32_t signs = RHT ? rht_sign_bits(rht_seed) : 0u;
  __syncthreads();
  for (int64_t c = (int64_t)blockIdx.x * kRowChunk; c < nvec; c += stride) {
    v4u vs[kRowU];
    if (kAhead) {
#pragma unroll
      for (int u = 0; u < kRowU; ++u) vs[u] = nxt[u];
      load_chunk(nxt, c + stride);
    } else {
      load_chunk(vs, c);
    }
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int64_t i = c + u * kThreads + threadIdx.x;
      if (i >= nvec) continue;
      const v4u v = vs[u];
      float z[8];
      if (RHT) {
        unpack8_flip(v, (i & 1) ? signs >> 8 : signs, z);
        rht16_pair_butterflies<false>(z, i & 1);   // 4 * the transform
      } else {
        unpack8_flip(v, 0u, z);
      }
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(z[j]));
      m = quad_xor_max<1>(m);
      if (RHT) m *= 0.25f;
      const BlockScale b = block_scale(m, sc);
      const float r = RHT ? quarter_fold(z, b.r, sc) : b.r;
      const uint32_t q = SR ? encode8_sr(z, r, sr_words_g(seed, stream_id, (uint64_t)i))
                      : encode8_rtn(z, r);
      st_(q, &codes[i]);
      if ((i & 1) == 0) scales[i >> 1] = (uint8_t)b.code;
    }
  }
}

// ---------------------------------------------------------------------------
// 1D colwise (transpose-quantize), optional RHT along the rows
// ---------------------------------------------------------------------------
// Workgroup tile: 256 rows (K) x 128 columns.  Thread t owns 16 rows x 8
// columns (cg = t % 16, rg = t / 16); a wave's loads cover 4 rows x 256
// contiguous bytes each.  Codes are staged in LDS as [column][row/2] so the
// stores run along the output's contiguous dimension.
constexpr int kColTileR = 256, kColTileC = 128;

// Tile of the 1-D grid over ceil(rows/256) x ceil(cols/128) workgroup tiles.
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, so
// block b is renumbered so that every XCD owns a contiguous range of tiles,
// taken in bands of 8 tile-rows with the rows fastest.  Neighbouring tiles
// write pieces of the same cache lines (8-byte rowwise scale pieces, 16-byte
// colwise ones, 64-byte rowwise code pieces); this way the pieces meet in
// one L2 while both tiles are resident rather than reaching HBM as separate
// partial-line writes.
// COLS_FIRST: bands of 8 tile-columns, columns fastest instead -- for the
// kernel that also writes the rowwise operand (row-major like its input),
// whose concurrent tiles then write contiguous pieces of the same rows
// (measured: 5% faster there; 11% slower for the plain transpose).
template <bool COLS_FIRST = false>
__device__ __forceinline__ void quant_tile(int64_t rows, int64_t cols, int64_t& r0, int64_t& c0) {
  const int64_t gy = (rows + kColTileR - 1) / kColTileR, gx = (cols + kColTileC - 1) / kColTileC;
  const int64_t n = gx * gy, b = blockIdx.x, per = n / kXcds;
  const int64_t t = b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
  int64_t ty, tx;
  if (COLS_FIRST) grouped(t, gx, gy, tx, ty);
  else grouped(t, gy, gx, ty, tx);
  r0 = ty * kColTileR;
  c0 = tx * kColTileC;
}

static dim3 quant_tile_grid(int64_t rows, int64_t cols) {
  return dim3((unsigned)(((rows + kColTileR - 1) / kColTileR) *
                         ((cols + kColTileC - 1) / kColTileC)));
}

// ROW: the same read also yields the rowwise 1D operand of x (blocks of 16
// along cols: the two lanes holding a row's adjacent 8-column pieces), with
// its own given amax and SR stream -- the tensors the recipe quantizes both
// ways (X, dY) are then read once.
struct RowOut {
  const float* amax;
  uint32_t stream_id;
  uint8_t* codes;    // [rows][cols/2]
  uint8_t* scales;   // [rows][cols/16]
  float* ts_out;
};

template <bool SR, bool RHT, bool ROW>
__global__ __launch_bounds__(kThreads) void k_quant_col(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
    const float* __restrict__ amax, uint64_t rht_seed, uint64_t seed, uint32_t stream_id,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ ts_out,
    RowOut ro) {
  __shared__ v2u lds_codes[kColTileC][kColTileR / 16];   // 8 bytes = 16 codes per block
  __shared__ uint8_t lds_scales[kColTileC][kColTileR / 16];
  __shared__ float rtab[kE4m3Codes], rtab_row[ROW ? kE4m3Codes : 1];
  static_assert(kThreads >= 2 * kE4m3Codes, "threads 0..127 fill rtab, 128..255 rtab_row");
  int64_t r0, c0;
  quant_tile<ROW>(rows, cols, r0, c0);
  const int cg = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int64_t rr = r0 + 16 * rg, cc = c0 + 8 * cg;
  const bool in = rr < rows && cc < cols;
  // the tile's loads go out first: their latency then hides the scale
  // tables' set-up and the sign draw
  Tile16x8 t;
  if (in) tile_load(t, x, cols, rr, cc);
  const ScaleCtx sc = scale_ctx(*amax, rtab, threadIdx.x);
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = sc.s_t;
  ScaleCtx sr_ctx;
  if (ROW) {
    sr_ctx = scale_ctx(*ro.amax, rtab_row, (int)threadIdx.x - 128);
    if (blockIdx.x == 0 && threadIdx.x == 0) *ro.ts_out = sr_ctx.s_t;
  }
  __syncthreads();
  const uint32_t signs = RHT ? rht_sign_bits(rht_seed) : 0u;
  if (in) {
    if (ROW) {
      // rows rr .. rr+15, columns cc .. cc+7: half of a 16-wide block each;
      // the partner lane (cg ^ 1) holds the other half (cols % 16 == 0, so
      // both halves are in range together).  Row i's outputs sit at a
      // uniform offset i * pitch from row rr's.
      uint8_t* const rcodes = ro.codes + rr * (cols / 2) + cc / 2;
      uint8_t* const rscales = ro.scales + rr * (cols / 16) + cc / 16;
      const uint32_t pc = (uint32_t)(cols / 2), ps = (uint32_t)(cols / 16);  // 16 rows < 2^32
      // Philox counter of row rr's 8-element group at column cc (cc is a multiple of 8)
      const uint64_t g_row0 = ((uint64_t)rr * (uint64_t)cols + (uint64_t)cc) >> 3;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const v4u w = t.row[i];
        float z[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                      bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(z[j]));
        m = quad_xor_max<1>(m);
        const BlockScale b = block_scale(m, sr_ctx);
        const uint32_t q = SR ? encode8_sr(z, b.r, sr_words_g(seed, ro.stream_id,
                                                        g_row0 + (uint64_t)i * (uint64_t)(cols >> 3)))
                        : encode8_rtn(z, b.r);
        *reinterpret_cast<uint32_t*>(rcodes + i * pc) = q;
        if ((cg & 1) == 0) rscales[i * ps] = (uint8_t)b.code;
      }
    }
    // output index of (column cc, row rr) over 8: the Philox counter of its
    // 8-element group (rr and rows are multiples of 16)
    const uint64_t g_col0 = ((uint64_t)cc * (uint64_t)rows + (uint64_t)rr) >> 3;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[16];
      tile_column(t, c, v, RHT ? signs : 0u);
      if (RHT) rht16_butterflies<false>(v);   // 4 * the transform
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
      if (RHT) m *= 0.25f;
      const BlockScale b = block_scale(m, sc);
      const float r = RHT ? quarter_fold(v, b.r, sc) : b.r;
      uint32_t q0, q1;
      if (SR) {
        // counters of the column's two 8-element groups (n0 / 8 and n0 / 8 + 1)
        const uint64_t g0 = g_col0 + (uint64_t)c * (uint64_t)(rows >> 3);
        q0 = encode8_sr(v, r, sr_words_g(seed, stream_id, g0));
        q1 = encode8_sr(v + 8, r, sr_words_g(seed, stream_id, g0 + 1));
      } else {
        q0 = encode8_rtn(v, r);
        q1 = encode8_rtn(v + 8, r);
      }
      lds_codes[8 * cg + c][rg] = v2u{q0, q1};
      lds_scales[8 * cg + c][rg] = (uint8_t)b.code;
    }
  }
  __syncthreads();
  // 2048 (column, row-group) pieces per tile; 16 consecutive threads write one
  // column's 128 contiguous code bytes and 16 contiguous scale bytes.
  const int64_t ld_codes = rows / 2, ld_scales = rows / 16;
#pragma unroll
  for (int j = 0; j < (kColTileC * kColTileR / 16) / kThreads; ++j) {
    const int p = threadIdx.x + kThreads * j;
    const int col = p >> 4, g = p & 15;
    const int64_t oc = c0 + col, orow = r0 + 16 * g;
    if (oc < cols && orow < rows) {
      st_(lds_codes[col][g],
                                  reinterpret_cast<v2u*>(codes + oc * ld_codes + orow / 2));
      scales[oc * ld_scales + orow / 16] = lds_scales[col][g];
    }
  }
}

// ---------------------------------------------------------------------------
// 2D: 16x16 blocks
// ---------------------------------------------------------------------------
// Workgroup tile 256 rows x 128 columns, the thread layout of the colwise
// kernel: thread t holds rows 16 (t / 16) .. +15 and columns 8 (t % 16) .. +7,
// so a 16x16 block is the micro-tiles of two adjacent lanes.  Each element is
// encoded once, a row of 8 columns to a dword (the rowwise codes, stored
// directly); the transposed codes are the same nibbles, transposed in
// registers and staged in LDS so that their stores run along the rows of the
// transposed output.

// 8 x 8 transpose of 4-bit entries (in[i] nibble j -> out[j] nibble i): swap
// the off-diagonal 4x4 blocks (16-bit halves), then 2x2 blocks (bytes), then
// single nibbles.
__device__ __forceinline__ void nibble_transpose8(const uint32_t* in, uint32_t* out) {
  uint32_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (in[i] & 0xFFFFu) | (in[i + 4] << 16);
    a[i + 4] = (in[i] >> 16) | (in[i + 4] & 0xFFFF0000u);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = (k & 1) + 4 * (k >> 1);   // 0, 1, 4, 5
    b[i] = (a[i] & 0x00FF00FFu) | ((a[i + 2] & 0x00FF00FFu) << 8);
    b[i + 2] = ((a[i] >> 8) & 0x00FF00FFu) | (a[i + 2] & 0xFF00FF00u);
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    out[i] = (b[i] & 0x0F0F0F0Fu) | ((b[i + 1] & 0x0F0F0F0Fu) << 4);
    out[i + 1] = ((b[i] >> 4) & 0x0F0F0F0Fu) | (b[i + 1] & 0xF0F0F0F0u);
  }
}

template <bool SR>
__global__ __launch_bounds__(kThreads) void k_quant_2d(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
    const float* __restrict__ amax, uint64_t seed, uint32_t stream_id,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ scales_t, float* __restrict__ ts_out) {
  __shared__ v2u lds_codes[kColTileC][kColTileR / 16];   // [column][row group]
  __shared__ float rtab[kE4m3Codes];
  int64_t r0, c0;
  quant_tile(rows, cols, r0, c0);
  const int cg = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int64_t rr = r0 + 16 * rg, cc = c0 + 8 * cg;
  // rows and cols are multiples of 16: a lane pair is in range together
  const bool in = rr < rows && cc < cols;
  Tile16x8 t;   // loaded first: the latency hides the scale table's set-up
  if (in) tile_load(t, x, cols, rr, cc);
  const ScaleCtx sc = scale_ctx(*amax, rtab, threadIdx.x);
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = sc.s_t;
  __syncthreads();
  if (in) {
    // block amax on the bf16 magnitudes (their bit patterns order like the
    // values), two per 32-bit lane op, then the partner lane's half
    uint32_t mp = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mp = pk_max_u16(mp, t.row[i].x & 0x7FFF7FFFu);
      mp = pk_max_u16(mp, t.row[i].y & 0x7FFF7FFFu);
      mp = pk_max_u16(mp, t.row[i].z & 0x7FFF7FFFu);
      mp = pk_max_u16(mp, t.row[i].w & 0x7FFF7FFFu);
    }
    float m = fmaxf(bf16_lo(mp), bf16_hi(mp));
    m = quad_xor_max<1>(m);
    const BlockScale b = block_scale(m, sc);
    uint32_t q[16];
    // row i's codes sit at a uniform offset i * pitch from row rr's
    uint8_t* const rcodes = codes + rr * (cols / 2) + cc / 2;
    const uint32_t pc = (uint32_t)(cols / 2);  // 16 rows of codes span < 2^32 bytes
    // Philox counter of row rr's 8-element group at column cc (cc is a multiple of 8)
    const uint64_t g_row0 = ((uint64_t)rr * (uint64_t)cols + (uint64_t)cc) >> 3;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const v4u w = t.row[i];
      float z[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                    bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
      q[i] = SR ? encode8_sr(z, b.r, sr_words_g(seed, stream_id,
                                                 g_row0 + (uint64_t)i * (uint64_t)(cols >> 3)))
                : encode8_rtn(z, b.r);
      *reinterpret_cast<uint32_t*>(rcodes + i * pc) = q[i];
    }
    if ((cg & 1) == 0) {
      scales[(rr / 16) * (cols / 16) + cc / 16] = (uint8_t)b.code;
      if (scales_t != nullptr) scales_t[(cc / 16) * (rows / 16) + rr / 16] = (uint8_t)b.code;
    }
    if (codes_t != nullptr) {
      uint32_t lo[8], hi[8];
      nibble_transpose8(q, lo);       // rows rr .. rr+7 of each column
      nibble_transpose8(q + 8, hi);   // rows rr+8 .. rr+15
#pragma unroll
      for (int c = 0; c < 8; ++c) lds_codes[8 * cg + c][rg] = v2u{lo[c], hi[c]};
    }
  }
  if (codes_t == nullptr) return;  // uniform across the grid
  __syncthreads();
  // 2048 (column, row-group) pieces per tile; 16 consecutive threads write one
  // column's 128 contiguous code bytes
  const int64_t ld_t = rows / 2;
#pragma unroll
  for (int j = 0; j < (kColTileC * kColTileR / 16) / kThreads; ++j) {
    const int p = threadIdx.x + kThreads * j;
    const int col = p >> 4, g = p & 15;
    const int64_t oc = c0 + col, orow = r0 + 16 * g;
    if (oc < cols && orow < rows)
      st_(lds_codes[col][g], reinterpret_cast<v2u*>(codes_t + oc * ld_t + orow / 2));
  }
}

// ---------------------------------------------------------------------------
// dequantize: out = (E2M1 * E4M3) * s_t
// ---------------------------------------------------------------------------
// Each workgroup iteration takes a piece of one row: kDeqU groups of 4
// elements per thread (one 16-bit code load, one 16-byte store: a wave's
// store covers 1 KiB of the row without gaps); the row index is one uniform
// division per piece.  One group per thread keeps the pieces small, so the
// workgroups in flight write one narrow window of the output (4 KiB pieces:
// 0.49 of HBM peak at 32768 x 8192; 0.44 with a 32-byte run per thread and
// 0.47 with 32 KiB pieces).
constexpr int kDeqU = 1;
__global__ __launch_bounds__(kThreads) void k_dequant(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    int64_t ss_row, int64_t ss_k, int32_t blk_rows, const float* __restrict__ ts,
    int64_t rows, int64_t k, float* __restrict__ out) {
  const float s_t = *ts;
  const int64_t kv = k / 4;                                     // 4-element groups per row
  constexpr int64_t kPiece = (int64_t)kThreads * kDeqU;         // groups per piece
  const int64_t per_row = (kv + kPiece - 1) / kPiece, pieces = rows * per_row;
  for (int64_t p = blockIdx.x; p < pieces; p += gridDim.x) {
    const int64_t r = p / per_row, g0 = (p - r * per_row) * kPiece;
    const uint8_t* const crow = codes + r * ld_codes;
    const uint8_t* const srow = scales + (r / blk_rows) * ss_row;
    uint32_t q[kDeqU];
    uint8_t sc[kDeqU];
#pragma unroll
    for (int u = 0; u < kDeqU; ++u) {
      const int64_t g = g0 + u * kThreads + threadIdx.x;
      if (g < kv) {
        q[u] = *reinterpret_cast<const uint16_t*>(crow + g * 2);
        sc[u] = srow[(g >> 2) * ss_k];                          // 16-element block g / 4
      }
    }
#pragma unroll
    for (int u = 0; u < kDeqU; ++u) {
      const int64_t g = g0 + u * kThreads + threadIdx.x;
      if (g >= kv) continue;
      const float E = e4m3_to_float(sc[u]);
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t c = (q[u] >> (4 * j)) & 0xFu;
        const uint32_t i = c & 7u;
        float mag = i < 4u ? 0.5f * (float)i : (i < 7u ? (float)i - 2.0f : 6.0f);
        float v = (c & 8u) ? -mag : mag;
        o[j] = (v * E) * s_t;
      }
      st_(v4f{o[0], o[1], o[2], o[3]}, reinterpret_cast<v4f*>(out + r * k + g * 4));
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Workgroups for `chunks` equal pieces of work, at most per_cu per CU,
// chosen so that every workgroup takes the same number of pieces (up to one)
// instead of a last trip that only some of them make.
static int balanced_grid(int64_t chunks, int per_cu) {
  const int64_t cap = (int64_t)num_cus() * per_cu;
  if (chunks <= cap) return (int)(chunks < 1 ? 1 : chunks);
  const int64_t trips = (chunks + cap - 1) / cap;
  return (int)((chunks + trips - 1) / trips);
}

// The amax reductions finish with one atomic max per workgroup, all on one
// address and mostly at the end of the launch, where they serialize: two
// workgroups per CU keep the read stream as fast and that tail short.
constexpr int kAmaxPerCu = 2;

static int grid_for(int64_t items, int per_cu) {
  int64_t g = (items + kThreads - 1) / kThreads;
  int64_t cap = (int64_t)num_cus() * per_cu;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_amax(const void* x, int64_t n_elems, float* out, hipStream_t s) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, o, nullptr);
  const int64_t nvec = n_elems / 8;
  const int64_t chunks = (nvec + kAmaxChunk - 1) / kAmaxChunk;
  hipLaunchKernelGGL(k_amax, dim3(balanced_grid(chunks, kAmaxPerCu)), dim3(kThreads), 0, s,
                     reinterpret_cast<const v4u*>(x), nvec, o);
  return hipGetLastError();
}

hipError_t launch_amax_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed,
                           float* out, hipStream_t s, float* out_plain) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  uint32_t* op = reinterpret_cast<uint32_t*>(out_plain);
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, o, op);
  const int64_t items = (rows / 16) * (cols / 8);
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
  const dim3 grid(balanced_grid((items + kThreads - 1) / kThreads, kAmaxPerCu));
  if (op != nullptr)
    hipLaunchKernelGGL(k_amax_rht<true>, grid, dim3(kThreads), 0, s, xh, rows, cols, rht_seed, o,
                       op);
  else
    hipLaunchKernelGGL(k_amax_rht<false>, grid, dim3(kThreads), 0, s, xh, rows, cols, rht_seed, o,
                       nullptr);
  return hipGetLastError();
}

hipError_t launch_amax_rht_row(const void* x, int64_t n_elems, uint64_t rht_seed, float* out,
                               hipStream_t s) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, o, nullptr);
  const int64_t nvec = n_elems / 8;
  const int64_t chunks = (nvec + kAmaxChunk - 1) / kAmaxChunk;
  hipLaunchKernelGGL(k_amax_rht_row, dim3(balanced_grid(chunks, kAmaxPerCu)), dim3(kThreads), 0, s,
                     reinterpret_cast<const v4u*>(x), nvec, rht_seed, o);
  return hipGetLastError();
}

hipError_t launch_quant_row(const void* x, int64_t rows, int64_t cols, const float* amax,
                            bool rht, uint64_t rht_seed, bool sr, uint64_t seed,
                            uint32_t stream_id, uint8_t* codes, uint8_t* scales, float* ts_out,
                            hipStream_t s) {
  const int64_t nvec = rows * cols / 8;
  const int64_t chunks = (nvec + kRowChunk - 1) / kRowChunk;
  // 8 workgroups per compute unit, or more where that would leave a
  // workgroup more than 4 chunks: the extra workgroups queue, and the
  // dispatcher hands them to whichever units finish first, which evens out
  // the units' progress on large tensors (measured: 1D SR encode of a
  // 32768x8192 tensor -10% against 16 chunks per workgroup)
  const int64_t wg = std::min<int64_t>(chunks, std::max<int64_t>((int64_t)num_cus() * 8, (chunks + 3) / 4));
  const dim3 g((unsigned)std::max<int64_t>(wg, 1)), b(kThreads);
  const v4u* xv = reinterpret_cast<const v4u*>(x);
  uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
#define NVFP4_ROW(SRV, RHTV)                                                                  \
  hipLaunchKernelGGL((k_quant_row<SRV, RHTV>), g, b, 0, s, xv, nvec, amax, rht_seed, seed,    \
                     stream_id, cv, scales, ts_out)
  if (sr && rht) NVFP4_ROW(true, true);
  else if (sr) NVFP4_ROW(true, false);
  else if (rht) NVFP4_ROW(false, true);
  else NVFP4_ROW(false, false);
#undef NVFP4_ROW
  return hipGetLastError();
}

hipError_t launch_quant_col(const void* x, int64_t rows, int64_t cols, const float* amax,
                            bool rht, uint64_t rht_seed, bool sr, uint64_t seed,
                            uint32_t stream_id, uint8_t* codes, uint8_t* scales, float* ts_out,
                            hipStream_t s) {
  const dim3 g = quant_tile_grid(rows, cols), b(kThreads);
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
#define NVFP4_COL(SRV, RHTV)                                                                  \
  hipLaunchKernelGGL((k_quant_col<SRV, RHTV, false>), g, b, 0, s, xp, rows, cols, amax,       \
                     rht_seed, seed, stream_id, codes, scales, ts_out, RowOut{})
  if (sr && rht) NVFP4_COL(true, true);
  else if (sr) NVFP4_COL(true, false);
  else if (rht) NVFP4_COL(false, true);
  else NVFP4_COL(false, false);
#undef NVFP4_COL
  return hipGetLastError();
}

hipError_t launch_quant_row_rht(const void* x, int64_t rows, int64_t cols, uint64_t rht_seed,
                               bool sr, uint64_t seed, uint32_t stream_row, uint32_t stream_col,
                               const float* amax_row, const float* amax_rht, uint8_t* codes_row,
                               uint8_t* scales_row, float* ts_row, uint8_t* codes_col,
                               uint8_t* scales_col, float* ts_col, hipStream_t s) {
  const dim3 g = quant_tile_grid(rows, cols), b(kThreads);
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  const RowOut ro{amax_row, stream_row, codes_row, scales_row, ts_row};
  if (sr)
    hipLaunchKernelGGL((k_quant_col<true, true, true>), g, b, 0, s, xp, rows, cols, amax_rht,
                       rht_seed, seed, stream_col, codes_col, scales_col, ts_col, ro);
  else
    hipLaunchKernelGGL((k_quant_col<false, true, true>), g, b, 0, s, xp, rows, cols, amax_rht,
                       rht_seed, seed, stream_col, codes_col, scales_col, ts_col, ro);
  return hipGetLastError();
}

hipError_t launch_quant_2d(const void* x, int64_t rows, int64_t cols, const float* amax, bool sr,
                           uint64_t seed, uint32_t stream_id, uint8_t* codes, uint8_t* codes_t,
                           uint8_t* scales, uint8_t* scales_t, float* ts_out, hipStream_t s) {
  const dim3 g = quant_tile_grid(rows, cols), b(kThreads);
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  if (sr)
    hipLaunchKernelGGL(k_quant_2d<true>, g, b, 0, s, xp, rows, cols, amax, seed, stream_id,
                       codes, codes_t, scales, scales_t, ts_out);
  else
    hipLaunchKernelGGL(k_quant_2d<false>, g, b, 0, s, xp, rows, cols, amax, seed, stream_id,
                       codes, codes_t, scales, scales_t, ts_out);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                          int64_t ss_row, int64_t ss_k, int32_t blk_rows, const float* ts,
                          int64_t rows, int64_t k, float* out, hipStream_t s) {
  const int64_t piece = (int64_t)kThreads * kDeqU;
  const int64_t pieces = rows * ((k / 4 + piece - 1) / piece);
  const int64_t cap = (int64_t)num_cus() * 8;
  const int grid = (int)(pieces < cap ? (pieces < 1 ? 1 : pieces) : cap);
  hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(kThreads), 0, s, codes,
                     ld_codes, scales, ss_row, ss_k, blk_rows, ts, rows, k, out);
  return hipGetLastError();
}

}  // namespace nvfp4
