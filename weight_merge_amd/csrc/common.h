// Internal declarations shared by the HIP sources of libadafuse (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ada {

// Output tile of one merge workgroup.
#ifndef ADA_BF16_ROW_BLOCKS
#define ADA_BF16_ROW_BLOCKS 2
#endif
#ifndef ADA_NT_STORE
#define ADA_NT_STORE 0
#endif
constexpr int kBF16RowBlocks = ADA_BF16_ROW_BLOCKS;  // 16-row MFMA blocks per wave
constexpr int kTileBF16Rows = 32 * kBF16RowBlocks;   // bf16 tile: kTileBF16Rows x kTileBF16Cols
constexpr int kTileBF16Cols = 128;
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
  int32_t src_is_out;  // 1: read the merged buffer (w_out) instead of w
  int32_t xcd_remap;   // 1: give each XCD a contiguous range of tiles
};

hipError_t launch_merge(const MergeParams& p, int dtype, int kr_max, hipStream_t s);

hipError_t launch_pregate(const void* h, const void* router, int d, int E, int k, int dtype,
                          int renorm, int32_t* idx, float* gate, hipStream_t s);

hipError_t launch_gemv(const void* w, int d_out, int d_in, int64_t ld, const void* x, void* y,
                       float* y32, int dtype, hipStream_t s);

hipError_t launch_lora_shrink(const void* a, int E, int r, int d_in, const int32_t* idx, int k,
                              const void* x, float* t, int dtype, hipStream_t s);

hipError_t launch_lora_expand(const void* b, int E, int r, int d_out, const int32_t* idx,
                              const float* gate, int k, float scale, const float* y32,
                              const float* t, void* y, int dtype, hipStream_t s);

}  // namespace ada
