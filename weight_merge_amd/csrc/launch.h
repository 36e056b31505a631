// Internal launch declarations of the pre-gating, decode-GEMV and unmerged-path
// kernels, shared with the C ABI (not installed).
#pragma once

#include "common.h"

namespace ada {

constexpr int kMaxLayerProj = 16;  // projections of one layer launch

hipError_t launch_pregate(const void* h, const void* router, int d, int E, int k, int dtype,
                          int renorm, int32_t* idx, float* gate, hipStream_t s);

hipError_t launch_gemv(const void* w, int d_out, int d_in, int64_t ld, const void* x, void* y,
                       float* y32, int dtype, hipStream_t s);

// Several independent decode GEMVs (at most kMaxLayerProj, passed by value) in one grid:
// row0 is the projection's first row in the stacked rows.
struct GemvLayerProj {
  const void* w;
  const void* x;
  void* y;
  int64_t ld;
  int32_t d_out;
  int32_t d_in;
  int32_t row0;
};
struct GemvLayerParams {
  GemvLayerProj proj[kMaxLayerProj];
  int32_t n;
};
hipError_t launch_gemv_layer(const GemvLayerParams& p, int rows, int dtype, hipStream_t s);

hipError_t launch_lora_shrink(const void* a, int E, int r, int d_in, const int32_t* idx, int k,
                              const void* x, float* t, int dtype, hipStream_t s);

hipError_t launch_lora_expand(const void* b, int E, int r, int d_out, const int32_t* idx,
                              const float* gate, int k, float scale, const float* y32,
                              const float* t, void* y, int dtype, hipStream_t s);

// One layer of the unmerged routed path (at most kMaxLayerProj projections, passed
// by value so the launch needs no device table).
struct LoraLayerProj {
  const void* w;
  const void* a;
  const void* b;
  const void* x;
  void* y;
  int64_t ld;
  int32_t d_out;
  int32_t d_in;
  int32_t dot_row0;  // first row of this projection in the stacked [W; A_sel] grid
  int32_t out_row0;  // first output row of this projection in the expand grid
  int64_t ws_off;    // fp32 workspace: d_out GEMV sums, then k*r shrink sums
};
struct LoraLayerParams {
  LoraLayerProj proj[kMaxLayerProj];
  int32_t n;
  int32_t E;
  int32_t r;
  int32_t k;
  const int32_t* idx;  // [nb][k]
  const float* gate;   // [nb][k]
  float scale;
  float* ws;
  int32_t nb;          // requests of a batch (ada_lora_batch); 1 for ada_lora_layer
};
hipError_t launch_lora_layer(const LoraLayerParams& p, int dot_rows, int out_rows, int dtype, hipStream_t s);

// The allocation-free layer path's device memory: a file-scope array of this many bytes
// per GPU, and its address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
hipError_t static_scratch(void** ptr);

// A batch of requests with a selection each, one group of projections (the unmerged
// path serving mixed selections).  Per projection x is [nb][d_in], y [nb][d_out];
// dot_row0 counts workgroups of the first grid: ceil(d_out / 16) base workgroups (16 W
// rows for every request) then ceil(nb * k*r / 4) shrink workgroups; out_row0 indexes
// the nb * d_out outputs; ws_off is an fp32 block of nb * (d_out + k*r).
constexpr int kMaxBatch = 16;
hipError_t launch_lora_batch(const LoraLayerParams& p, int dot_wgs, int out_rows, int dtype, hipStream_t s);

}  // namespace ada
