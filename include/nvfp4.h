/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantize + NVFP4-linear GEMM
 * library (libnvfp4.so).
 *
 * NVFP4 stores a tensor as 4-bit E2M1 elements (values 0, +-0.5, +-1, +-1.5,
 * +-2, +-3, +-4, +-6), one E4M3 scale per 16 consecutive elements, and one
 * FP32 scale for the whole tensor ("Pretraining Large Language Models with
 * NVFP4", summary page, format paragraph; "NVFP4 Trains with Precision of
 * 16-Bit and Speed and Efficiency of 4-Bit", micro-block scaling and E4M3
 * scale-factor sections).  Activations and gradients are scaled in 1D blocks
 * of 16 along the contraction dimension K, weights in 2D 16x16 tiles; the
 * weight-gradient GEMM inputs get a 16-point random Hadamard transform; the
 * gradients are stochastically rounded (news item "Soumith Chintala 发布
 * NVFP4 训练详解文章", section 三; NVIDIA blog, Hadamard, 2D block and
 * stochastic-rounding sections).
 *
 * Quantization of an operand z (K-contiguous, [I][K]) runs in six steps:
 *   1. amax_t = max |z| over the tensor            (a full read of the input)
 *   2. s_t    = amax_t / (6*448)  (1 when amax_t == 0)
 *   3. amax_b = max |z| over each block (1x16, or 16x16 for weights)
 *   4. E_b    = E4M3(amax_b / (6*s_t)), round-to-nearest-even, saturating
 *   5. code   = E2M1(z * (1/(E_b*s_t))), round-to-nearest-even or stochastic
 *               (16 bits of Philox4x32-10 per element: key = seed, counter =
 *               (n/8, stream_id, 0), n = element index in the K-contiguous
 *               output operand)
 *   6. (optional) z = 1/4 * H16 * D * x along K before step 1, D = +-1 signs
 *               from Philox(key = rht_seed, counter = (0,0,0,1)), word 0
 * The GPU output is bit-identical to the CPU reference for every finite
 * input with amax_t >= 2^-100, and for smaller amax_t wherever every non-zero
 * block's element scale 1/(E_b*s_t) is finite (outputs for NaN/Inf inputs
 * are unspecified, and never out of bounds).
 *
 * Conventions (all entry points):
 *  - Every pointer is DEVICE memory owned by the caller; the library never
 *    allocates, frees or synchronises.  `stream` is a hipStream_t (NULL = the
 *    default stream); all work is enqueued on it, in order.
 *  - bf16 inputs are row-major [rows][cols] with 16-byte aligned base
 *    pointers; rows and cols are positive multiples of 16, and cols is at
 *    most 2^28 (16 rows of packed codes then span less than 2^32 bytes).
 *  - Packed codes hold two elements per byte, the even-k element in the low
 *    nibble; code = sign << 3 | magnitude index (0, .5, 1, 1.5, 2, 3, 4, 6).
 *  - Arguments are validated before anything is enqueued; on error nothing
 *    is launched and a negative NVFP4_ERR_* status is returned.  A launch
 *    failure returns NVFP4_ERR_LAUNCH.  nvfp4_last_error() describes the most
 *    recent error of the calling thread.
 *  - amax_io / tensor_scale_out point to one device float each.  With
 *    NVFP4_AMAX_COMPUTE the library computes amax_t into *amax_io; with
 *    NVFP4_AMAX_GIVEN *amax_io must already hold it (e.g. from nvfp4_amax),
 *    which saves the extra full read of the input.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,   /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = -2,  /* a dimension is not a positive multiple of 16, too large, or mismatched */
  NVFP4_ERR_ALIGN = -3,  /* a base pointer or leading dimension is misaligned */
  NVFP4_ERR_ARG = -4,    /* an enum argument is out of range */
  NVFP4_ERR_LAUNCH = -5  /* the HIP runtime refused a launch */
};

enum { NVFP4_AMAX_COMPUTE = 0, NVFP4_AMAX_GIVEN = 1 };

enum {
  NVFP4_ROWWISE = 0, /* blocks run along cols: codes [rows][cols/2], scales [rows][cols/16] */
  NVFP4_COLWISE = 1  /* blocks run along rows: the quantized transpose,
                        codes [cols][rows/2], scales [cols][rows/16] */
};

/* Step 1 alone: *amax_out = max |x| over the bf16 tensor [rows][cols]
 * (NVFP4 format paragraph: the tensor-level FP32 scale needs this full-tensor
 * scan).  rows*cols must be a multiple of 256. */
int nvfp4_amax(const void* x_bf16, int64_t rows, int64_t cols, float* amax_out, void* stream);

/* Step 1 under the transform: *amax_out = max |RHT(x^T)|, the RHT taken over
 * every 16 consecutive rows of each column, signs from rht_seed.  This is
 * the tensor statistic nvfp4_rht_quantize scales by. */
int nvfp4_amax_rht(const void* x_bf16, int64_t rows, int64_t cols, uint64_t rht_seed,
                   float* amax_out, void* stream);

/* Both statistics of one tensor from a single read: *amax_out = max |x| (as
 * nvfp4_amax) and *amax_rht_out = max |RHT(x^T)| (as nvfp4_amax_rht, same
 * seed).  A tensor quantized both plainly and under the transform -- X and dY
 * in the linear-layer recipe, where Fprop / Dgrad take them rowwise and Wgrad
 * takes their RHT transposes ("Pretraining Large Language Models with
 * NVFP4", summary page, recipe paragraph) -- needs both, and each is a full
 * scan of the tensor.  Same shape rules as nvfp4_amax_rht; the two outputs
 * must not alias. */
int nvfp4_amax_both(const void* x_bf16, int64_t rows, int64_t cols, uint64_t rht_seed,
                    float* amax_out, float* amax_rht_out, void* stream);

/* 1D quantization (activations, gradients), round-to-nearest-even.
 * axis NVFP4_ROWWISE: operand = x,   I = rows, K = cols.
 * axis NVFP4_COLWISE: operand = x^T, I = cols, K = rows (Wgrad layout).
 * Outputs: codes [I][K/2], scales_e4m3 [I][K/16], *tensor_scale_out = s_t. */
int nvfp4_quantize1d_rtn(const void* x_bf16, int64_t rows, int64_t cols, int axis,
                         float* amax_io, int amax_mode,
                         uint8_t* codes, uint8_t* scales_e4m3, float* tensor_scale_out,
                         void* stream);

/* As nvfp4_quantize1d_rtn with stochastic rounding: the larger neighbouring
 * E2M1 magnitude is taken with probability (|v|-lo)/(hi-lo) (NVIDIA blog,
 * stochastic-rounding section), decided by 16 bits of
 * Philox4x32-10(key = seed, counter = (n/8, stream_id, 0)). */
int nvfp4_quantize1d_sr(const void* x_bf16, int64_t rows, int64_t cols, int axis,
                        float* amax_io, int amax_mode, uint64_t seed, uint32_t stream_id,
                        uint8_t* codes, uint8_t* scales_e4m3, float* tensor_scale_out,
                        void* stream);

/* 2D quantization (weights): one E4M3 scale per 16x16 tile (NVIDIA blog, 2D
 * block quantization: the forward and backward passes see the same
 * quantized weight).  Operand = w, I = rows, K = cols.
 * Outputs: codes [rows][cols/2]; scales_e4m3 [rows/16][cols/16];
 * codes_t [cols][rows/2] and scales_t_e4m3 [cols/16][rows/16] (each
 * nullable): the same codes and scales transposed, which make the Dgrad
 * operand (w read as [cols][rows]) K-contiguous in both. */
int nvfp4_quantize2d_rtn(const void* w_bf16, int64_t rows, int64_t cols,
                         float* amax_io, int amax_mode,
                         uint8_t* codes, uint8_t* codes_t, uint8_t* scales_e4m3,
                         uint8_t* scales_t_e4m3, float* tensor_scale_out, void* stream);

int nvfp4_quantize2d_sr(const void* w_bf16, int64_t rows, int64_t cols,
                        float* amax_io, int amax_mode, uint64_t seed, uint32_t stream_id,
                        uint8_t* codes, uint8_t* codes_t, uint8_t* scales_e4m3,
                        uint8_t* scales_t_e4m3, float* tensor_scale_out, void* stream);

/* Weight-gradient operand: the quantized transpose of RHT-transformed x
 * (news item, section 三: RHT on the weight-gradient GEMM inputs; summary
 * page, limitations paragraph: only Wgrad, to stay compatible with 2D weight
 * scaling).  x is [rows = K tokens][cols]; the transform runs over every 16
 * consecutive tokens of each column.  Give both Wgrad operands the same
 * rht_seed so the transforms cancel in the product.  use_sr selects
 * stochastic rounding (seed, stream_id) or RTN.  *amax_io is max |RHT(x^T)|.
 * Outputs: codes [cols][rows/2], scales_e4m3 [cols][rows/16]. */
int nvfp4_rht_quantize(const void* x_bf16, int64_t rows, int64_t cols, uint64_t rht_seed,
                       int use_sr, uint64_t sr_seed, uint32_t stream_id,
                       float* amax_io, int amax_mode,
                       uint8_t* codes, uint8_t* scales_e4m3, float* tensor_scale_out,
                       void* stream);

/* The 16-point RHT along either axis ("NVFP4 Trains with Precision of 16-Bit
 * and Speed and Efficiency of 4-Bit", Hadamard-transforms section: the
 * transform can be applied to the linear layers' inputs in the forward and
 * the backward pass; "Pretraining Large Language Models with NVFP4", summary
 * page, limitations paragraph: the recipe itself uses it on Wgrad only, and
 * leaves Fprop / Dgrad with it unvalidated).  Fprop and Dgrad contract over
 * the contiguous dimension of X, W and dY, so their transform runs along the
 * rows of x:
 *   axis NVFP4_ROWWISE: operand = x with every 16 consecutive columns of each
 *     row transformed; I = rows, K = cols; codes [rows][cols/2], scales
 *     [rows][cols/16]; SR element index n = r * cols + k.
 *   axis NVFP4_COLWISE: exactly nvfp4_amax_rht / nvfp4_rht_quantize (the
 *     quantized transpose, transform along the rows).
 * Both GEMM operands of a product must use the same rht_seed so that the
 * transforms cancel.  Other arguments, outputs and validation as in
 * nvfp4_amax_rht and nvfp4_rht_quantize; *amax_io is max |RHT(x)| along the
 * chosen axis. */
int nvfp4_amax_rht1d(const void* x_bf16, int64_t rows, int64_t cols, int axis,
                     uint64_t rht_seed, float* amax_out, void* stream);
int nvfp4_rht_quantize1d(const void* x_bf16, int64_t rows, int64_t cols, int axis,
                         uint64_t rht_seed, int use_sr, uint64_t sr_seed, uint32_t stream_id,
                         float* amax_io, int amax_mode,
                         uint8_t* codes, uint8_t* scales_e4m3, float* tensor_scale_out,
                         void* stream);

/* The two quantizations of one tensor that the recipe needs both of -- the
 * rowwise 1D operand (as nvfp4_quantize1d_*, axis NVFP4_ROWWISE) and the RHT
 * transpose (as nvfp4_rht_quantize) -- from a single read of x.  X (Fprop
 * rowwise, Wgrad under the RHT) and dY (Dgrad rowwise with SR, Wgrad under
 * the RHT with SR) are such tensors ("Pretraining Large Language Models with
 * NVFP4", summary page, recipe paragraph).  Both amaxes are given (e.g. from
 * nvfp4_amax_both); use_sr applies to both outputs, each with its own SR
 * stream id.  Outputs and their validation as in the two single calls; the
 * results are byte-identical to them. */
int nvfp4_quantize_row_rht(const void* x_bf16, int64_t rows, int64_t cols, uint64_t rht_seed,
                           int use_sr, uint64_t sr_seed, uint32_t stream_id_row,
                           uint32_t stream_id_rht, const float* amax_row, const float* amax_rht,
                           uint8_t* codes_row, uint8_t* scales_row, float* tensor_scale_row_out,
                           uint8_t* codes_rht, uint8_t* scales_rht, float* tensor_scale_rht_out,
                           void* stream);

/* A quantized GEMM operand, logically [rows][k], K-contiguous.  The scale of
 * element (r, k) is scales[(r / blk_rows) * ss_row + (k / 16) * ss_k].
 *  1D rowwise operand: blk_rows 1,  ss_row = k/16, ss_k = 1.
 *  2D operand:         blk_rows 16, ss_row = k/16, ss_k = 1.
 *  2D transposed (codes_t of a [R][C] weight, read as [C][R]):
 *                      scales_t with blk_rows 16, ss_row = R/16, ss_k = 1,
 *                      or the untransposed scales with ss_row = 1, ss_k = C/16.
 * Scale codes are finite non-negative E4M3 (0x00..0x7E), as the quantizers
 * write them; other bytes give unspecified (never out-of-bounds) results.
 * The GEMM is fastest when ss_k == 1, ss_row is a multiple of 4, the scales
 * are 4-byte aligned, k is a multiple of 64 and ld_codes of 16. */
typedef struct {
  const uint8_t* codes;      /* [rows][ld_codes] bytes, 16-byte aligned base; ld_codes >= k/2,
                                a multiple of 8 (a multiple of 16 takes the faster path) */
  int64_t ld_codes;
  const uint8_t* scales;     /* E4M3 codes */
  int64_t ss_row, ss_k;
  int32_t blk_rows;          /* 1 or 16 */
  const float* tensor_scale; /* device pointer to s_t */
  int64_t rows, k;
} nvfp4_operand;

/* out[r][c] = (E2M1(code) * E4M3(scale)) * s_t as FP32 [rows][k]: the real
 * value a 4-bit element stands for (blog essay "NVFP4：让大模型从零预训练跑在4位
 * 浮点上", section 2.2: multiply the element by its block scale). */
int nvfp4_dequantize(const nvfp4_operand* q, float* out, void* stream);

/* C[m][n] = s_a * s_b * sum_k A[m,k] * B[n,k] in FP32, A = [M][K], B = [N][K],
 * C row-major with leading dimension ldc >= N (floats, multiple of 4).
 * Fprop  Y  = X W^T : A = rowwise Q(X),  B = 2D Q(W)
 * Dgrad  dX = dY W  : A = rowwise Q(dY), B = 2D Q(W) read through codes_t
 * Wgrad  dW = dY^T X: A = RHT-quantized dY, B = RHT-quantized X (same seed)
 * The decoded E2M1 x E4M3 products are exact in FP16; the contraction runs
 * on the matrix cores with FP32 accumulation (NVIDIA blog: the linear-layer
 * GEMMs are the core compute of pretraining).  M, N, K multiples of 16. */
int nvfp4_gemm(const nvfp4_operand* a, const nvfp4_operand* b, float* c, int64_t ldc,
               void* stream);

/* As nvfp4_gemm with a fused epilogue: C is written as BF16 [M][N] (ldc >= N
 * elements, 2-byte aligned; each entry the FP32 result rounded to nearest,
 * ties to even) and, when amax_out is not NULL, *amax_out receives max |C|
 * over the BF16 values -- the tensor amax the next layer's quantization of C
 * needs, without its separate full read of C (the cost named in "Pretraining
 * Large Language Models with NVFP4", summary page, limitations paragraph).
 * Pass it with NVFP4_AMAX_GIVEN.  Same operands and validation as nvfp4_gemm.
 *
 * workspace: caller-owned device memory, 256-byte aligned, of workspace_bytes
 * >= nvfp4_gemm_bf16_workspace_bytes(M, N, K) bytes, or NULL with 0.  With it
 * the last round's tiles may be cut along K as in the FP32 GEMM: the two
 * halves' FP32 partials meet in the workspace, and every BF16 entry is then
 * exactly the FP32 GEMM's entry rounded (ties to even).  Without it those
 * tiles run as half-width tiles over the whole K (same rounding of their own
 * FP32 sums).  The workspace content on entry does not matter; calls that use
 * one workspace at the same time race.  NVFP4_ERR_ARG: workspace_bytes too
 * small; NVFP4_ERR_ALIGN: workspace not 256-byte aligned. */
int nvfp4_gemm_bf16(const nvfp4_operand* a, const nvfp4_operand* b, uint16_t* c_bf16, int64_t ldc,
                    float* amax_out, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes nvfp4_gemm_bf16 needs for an M x N x K product on the
 * current device (0 when its tiles are never cut along K); a negative
 * NVFP4_ERR_* status for M, N or K not positive. */
int64_t nvfp4_gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* nvfp4_gemm_bf16 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument and no allocation; the K-split partials go to a
 * fixed array of nvfp4_gemm_bf16_noalloc_max_bytes() bytes (64 MiB + 512 B)
 * in each GPU's memory, held by the library until the process ends.  Shapes
 * whose workspace need exceeds it are rejected (NVFP4_ERR_SHAPE; every shape
 * on a 256-CU MI355X fits).  All calls on one GPU share that array: calls
 * that overlap on one GPU race. */
int nvfp4_gemm_bf16_noalloc(const nvfp4_operand* a, const nvfp4_operand* b, uint16_t* c_bf16,
                            int64_t ldc, float* amax_out, void* stream);
int64_t nvfp4_gemm_bf16_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * MXFP4, the format NVFP4 is measured against: 32-element blocks along K, a
 * power-of-two (UE8M0) block scale, no tensor scale ("Pretraining Large
 * Language Models with NVFP4", summary page, format paragraph).  Its scales
 * are what gfx950's scaled FP4 matrix instructions consume, so its GEMM runs
 * on them directly.
 *
 * Scale of a block with largest magnitude amax_b: E = 2^e, e the smallest
 * integer with amax_b <= 6 * 2^e (every block's largest |v| then lies in
 * (3, 6] -- the rounding whose worst case leaves +-4 and +-6 unused, same
 * paragraph), clamped to [-127, 127], stored as the byte e + 127 (an all-zero
 * block gets byte 0).  Element code = E2M1(z * 2^-e), RTN or SR exactly as
 * for NVFP4.  Output bit-identical to the CPU reference for finite inputs.
 * ------------------------------------------------------------------------ */

/* Rowwise MXFP4 quantization of bf16 x [rows][cols] (16-byte aligned; cols a
 * positive multiple of 32).  codes [rows][cols/2] (4-byte aligned),
 * scales_e8m0 [rows][cols/32].  use_sr: 0 = RTN, 1 = SR with
 * Philox4x32-10(key = seed, counter = (n/8, stream_id, 0)), n = r*cols + k. */
int mxfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, int use_sr, uint64_t seed,
                   uint32_t stream_id, uint8_t* codes, uint8_t* scales_e8m0, void* stream);

/* An MXFP4 operand, logically [rows][k], K-contiguous: code of (r, k) in
 * codes[r * ld_codes + k/2] (low nibble = even k), its scale in
 * scales[r * ld_scales + k/32].  The scale array spans rows * ld_scales
 * bytes; scale bytes are 0x00..0xFE as the quantizer writes them. */
typedef struct {
  const uint8_t* codes;
  int64_t ld_codes;    /* >= k/2; GEMM: multiple of 16 and 16-byte aligned codes */
  const uint8_t* scales;
  int64_t ld_scales;   /* >= k/32; the GEMM is fastest with a multiple of 4 */
  int64_t rows, k;     /* rows > 0, k a positive multiple of 32 */
} mxfp4_operand;

/* out[r][k] = E2M1(code) * 2^(scale - 127) as FP32 [rows][k] (exact). */
int mxfp4_dequantize(const mxfp4_operand* q, float* out, void* stream);

/* C[m][n] = sum_k A[m,k] * B[n,k] in FP32 on the scaled FP4 matrix cores
 * (v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 x E2M1, E8M0 scales per 32),
 * A = [M][K], B = [N][K], C row-major with ldc >= N.  Products are exact; the
 * only rounding is the FP32 accumulation. */
int mxfp4_gemm(const mxfp4_operand* a, const mxfp4_operand* b, float* c, int64_t ldc,
               void* stream);

/* ------------------------------------------------------------------------
 * Measurement support (not part of the quantize / GEMM path): the sustained
 * throughput and shader clock of the FP16 matrix cores running the GEMM fast
 * path's MFMA pattern (v_mfma_f32_32x32x16_f16, 8 x 2 independent
 * accumulators per wave, one wave per SIMD, 256 workgroups of 256 threads)
 * from registers, with no loads, decode or LDS -- the ceiling the GEMM's
 * roofline fraction should be read against.  The sustained clock depends on
 * the power the operand bits draw, so `mode` picks the operand data: 0 zeros,
 * 1 values like the GEMM's decoded operands (E2M1 x E4M3 mantissa, random
 * signs), 2 uniform FP16 in [-1, 1).
 *
 * Enqueues on `stream`: fill the operands, a warm-up run, then a run of
 * `iters` loop trips (1 .. 1000000; 16 MFMAs of 2*32*32*16 FLOP per wave per
 * trip; ~200000 runs ~50 ms).  `scratch` is caller-owned device memory of at
 * least nvfp4_probe_scratch_bytes() bytes, 256-byte aligned.  After the
 * stream completes, the last 256 * 4 uint64 of that size hold, per workgroup
 * b, {shader-clock counter at start, at end, 100 MHz real-time counter at
 * start, at end} of the timed run: the clock is d(shader) / d(real-time) *
 * 100 MHz, and the run's duration is (max end - min start) real-time ticks. */
int64_t nvfp4_probe_scratch_bytes(void);
int nvfp4_probe_mfma(int mode, int iters, void* scratch, int64_t scratch_bytes, void* stream);

/* Measurement support: clock stamps.  Enqueues on `stream` one small launch
 * whose 256 workgroups each write 4 uint64 {XCC id, HW_ID register (wave,
 * SIMD, CU, shader-array, engine fields), shader-clock counter, 100 MHz
 * real-time counter} into `stamps` (device memory of at least
 * nvfp4_probe_clock_bytes() bytes, 8-byte aligned, caller-owned).  Stamps
 * taken before and after other work on the same stream give, per compute
 * unit (the shader-clock counters of different CUs are unrelated: pair
 * stamps with equal XCC id and equal HW_ID bits 8..15), d(shader) /
 * d(real-time) * 100 MHz: the average clock that work ran at. */
int64_t nvfp4_probe_clock_bytes(void);
int nvfp4_probe_clock(void* stamps, int64_t stamps_bytes, void* stream);

/* Measurement support: a plain device copy of `bytes` (a positive multiple of
 * 16) from src to dst (device memory, 16-byte aligned, not overlapping),
 * with the read pattern of the amax and rowwise kernels (whole chunks of
 * 8 x 16-byte vectors per thread, non-temporal).  Its bandwidth is the
 * achievable HBM rate of a read + write stream, the reference for the
 * quantizers' bandwidth and for scaling HBM byte counters. */
int nvfp4_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* nvfp4_status_string(int status);

/* Description of the calling thread's most recent error ("" if none). */
const char* nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
