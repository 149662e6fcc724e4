// gemm_tiles.h -- workgroup-tile order shared by the NVFP4 and MXFP4 GEMMs
// (internal to libnvfp4.so): 256 x 256 output tiles, one workgroup per CU,
// XCD-aware renumbering, and the split of a half-empty last round of tiles
// into two K halves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kTile = 256;  // workgroup tile (rows of A and of B)

// Tile order: the grid is 1-D.  Workgroups are dealt round-robin to the 8
// XCDs (each with its own L2), so block b is first renumbered so that every
// XCD owns a contiguous range of tiles; inside that range tiles run in
// groups of kGroupM tile-rows, M fastest, so the workgroups resident on one
// XCD at a time share both A rows and B columns in its L2.
constexpr int kXcds = 8, kGroupM = 8;

// Linear tile index -> (tile row, tile column): groups of kGroupM tile-rows,
// M fastest inside a group.
__device__ __forceinline__ void grouped(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t in = t - group * kGroupM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// How the tiles of a last, partial round of workgroups are cut (whole tiles
// before them run as usual): into two K halves that add into a zeroed
// output, into two half-width (256 x 128) tiles that each write their own
// columns, or both (four pieces).  The half-width cut needs no FP32 addends,
// so it also serves outputs that cannot take them (BF16).
enum TailMode { kTailWhole = 0, kTailK = 1, kTailN = 2, kTailNK = 3 };

// Block -> tile, K part (-1 whole, 0 / 1 halves) and N half (-1 full width,
// 0 / 1).  Blocks below full take whole tiles, renumbered so each XCD owns a
// contiguous range; the blocks after them take the remaining tiles, 2 or 4
// pieces each by the tail mode.
__device__ __forceinline__ void block_tile(int64_t full, int64_t tiles_m, int64_t tiles_n, int tail,
                                           int64_t& tm, int64_t& tn, int& part, int& nh) {
  const int64_t b = blockIdx.x;
  int64_t t;
  part = -1;
  nh = -1;
  if (b < full) {
    const int64_t per = full / kXcds;
    t = b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
  } else {
    const int pieces = tail == kTailNK ? 4 : 2;
    const int64_t q = b - full;
    t = full + q / pieces;
    const int sub = (int)(q % pieces);
    if (tail & kTailK) part = tail == kTailNK ? sub >> 1 : sub;
    if (tail & kTailN) nh = sub & 1;
  }
  grouped(t, tiles_m, tiles_n, tm, tn);
}

// The K-split-only form (tail mode kTailK when the grid goes past full).
__device__ __forceinline__ void block_tile(int64_t full, int64_t tiles_m, int64_t tiles_n,
                                           int64_t& tm, int64_t& tn, int& part) {
  int nh;
  block_tile(full, tiles_m, tiles_n, kTailK, tm, tn, part, nh);
}

// Host-side plan of one launch: tiles_m x tiles_n tiles; grid = full_tiles
// whole tiles plus 2 or 4 workgroups per tail tile.
struct TilePlan {
  int64_t tiles_m, tiles_n, full_tiles, grid, rem;
  int tail;     // TailMode
  bool split;   // tail tiles are cut along K (the output takes two FP32 addends)
};

// allow_split: the output can take two FP32 addends per element;
// allow_narrow: the kernel can run half-width tail tiles.
TilePlan plan_tiles(int64_t M, int64_t N, int64_t steps, bool allow_split = true,
                    bool allow_narrow = false);

// Zero the output tiles the split workgroups add into (no-op without split).
hipError_t zero_split_tiles(const TilePlan& p, float* c, int64_t ldc, int64_t M, int64_t N,
                            hipStream_t s);

}  // namespace nvfp4
