// Internal declarations of the merge kernel, shared with the C ABI (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ada {

// Output tile of one merge workgroup (bf16).  A tile shape is RB row blocks and CT
// column blocks of 16 per wave, with the 4 waves arranged (4 / WGN) x WGN.  Three
// contraction classes use separate shapes: k*r <= kNarrowKR (32 x 256: 512-byte row
// segments of W per tile row), k*r <= kLongKR (64 x 128: half the A_cat columns to
// gather per tile) and longer ones (128 x 128).
#ifndef ADA_NARROW_TILE
#define ADA_NARROW_TILE 1, 8, 2
#endif
#ifndef ADA_SHORT_TILE
#define ADA_SHORT_TILE 2, 4, 2
#endif
#ifndef ADA_LONG_TILE
#define ADA_LONG_TILE 4, 4, 2
#endif
template <int RB, int CT, int WGN>
struct TileShapeT {
  static constexpr int rb = RB, ct = CT, wgn = WGN;
  static constexpr int rows = 16 * RB * (4 / WGN), cols = 16 * CT * WGN;
};
using NarrowTile = TileShapeT<ADA_NARROW_TILE>;
using ShortTile = TileShapeT<ADA_SHORT_TILE>;
using LongTile = TileShapeT<ADA_LONG_TILE>;
constexpr int kNarrowKR = 32;
constexpr int kLongKR = 64;
constexpr int kTileClasses = 3;
// contraction class of a launch whose selections span at most kr_max = k*r terms
__host__ __device__ constexpr int bf16_tile_class(int kr_max) {
  return kr_max <= kNarrowKR ? 0 : kr_max <= kLongKR ? 1 : 2;
}
__host__ __device__ constexpr int bf16_tile_rows(int cls) {
  return cls == 0 ? NarrowTile::rows : cls == 1 ? ShortTile::rows : LongTile::rows;
}
__host__ __device__ constexpr int bf16_tile_cols(int cls) {
  return cls == 0 ? NarrowTile::cols : cls == 1 ? ShortTile::cols : LongTile::cols;
}
constexpr int kTileF32 = 64;    // 64 x 64 for fp32 storage (VALU path)
constexpr int kMaxSlots = 128;  // selected adapters per launch (two selections of <= 64)
constexpr int kMaxKR = 512;     // k * r bound of one launch

// One adapted projection in the device work table.  Tiles of an entry are
// numbered row-major over (row band, column block) starting at tile_base.
struct alignas(16) MergeEntry {
  const void* w;
  void* w_out;
  const void* a;
  const void* b;
  int64_t ld;
  int32_t d_out;
  int32_t d_in;
  int32_t tiles_n;
  int32_t tiles_m;
  int64_t tile_base;
};
static_assert(sizeof(MergeEntry) == 64, "work-table entry is 64 bytes");

// One selection (indices and gates on the device) with its signed coefficient.
struct Selection {
  const int32_t* idx;
  const float* gate;
  int32_t k;
  float coef;  // +scale to fuse, -scale to de-fuse
};

struct MergeParams {
  const MergeEntry* table;  // n_entries + 1 entries (the last one a sentinel)
  const int32_t* lut;       // tile >> lut_shift -> first entry touching that bucket
  int64_t total_tiles;
  int32_t lut_shift;
  int32_t n_entries;
  Selection sel[2];
  int32_t E;
  int32_t r;
  int32_t r_shift;     // log2(r) when r is a power of two, else -1
  int32_t src_is_out;  // 1: read the merged buffer (w_out) instead of w
  int32_t xcd_remap;   // 1: give each XCD a contiguous range of tiles
  int32_t tile_group;  // row bands walked down one column block before moving right
};

hipError_t launch_merge(const MergeParams& p, int dtype, int kr_max, hipStream_t s);

}  // namespace ada
