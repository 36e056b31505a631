// Decode-step GEMV on the merged backbone, and the kernels of the unmerged,
// per-layer routed baseline.
//
// "AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level Pre-Gating and
// Fused Kernel Optimization", Portuguese summary page, technical summary 2.B:
// after the adapters are fused into the backbone, decoding runs with no routing,
// so each projection of a batch-1 decode step is y = W' x.  That product reads
// every weight once and does 2 flops per weight: bound by HBM bandwidth.
//
// The baseline (technical summary 1 on both pages: conventional dynamic adapters
// route and apply adapters per layer, with several kernel calls per layer) keeps
// the adapters separate: base GEMV (fp32 out), shrink t = A_sel x, expand
// y = RNE(y32 + s * sum_j g_j B_j t_j).
#include "launch.h"

#include <mutex>

namespace ada {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ void dot8(uint4 a, uint4 b, float& acc, uint16_t) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
    acc = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), acc);
  }
}

__device__ __forceinline__ void dot8(uint4 a, uint4 b, float& acc, float) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  f32x2 v = {f, 0.f};
  return uint16_t(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t)) & 0xffffu);
}

__device__ __forceinline__ void store_out(uint16_t* y, int i, float v) { y[i] = to_bf16(v); }
__device__ __forceinline__ void store_out(float* y, int i, float v) { y[i] = v; }

__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}
__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }

// Weight rows stream through once per decode step: nontemporal loads keep them from
// displacing the activations, which every row reuses from the caches.  Measured on
// the 7B decode step (cold weights): 2.49 -> 2.35 ms per token, bit-identical.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Dot product of one row with x by one wave: a lane walks the row with 16-byte loads
// in batches of U vectors, all issued before any is used (U x 64 x 16 bytes in flight
// per wave); the x vectors of the same columns come from L1/L2.  The batch tail is
// branch-free: past the row end a lane re-reads the row's first vector and multiplies
// it by a zero x vector.  One butterfly at the end (every lane gets the sum).
template <typename T, int U>
__device__ __forceinline__ float row_dot(const T* __restrict__ rowp, const T* __restrict__ x, int d_in) {
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int nvec = d_in / VEC;
  const uint4* __restrict__ xv = reinterpret_cast<const uint4*>(x);
  const uint4* __restrict__ wr = reinterpret_cast<const uint4*>(rowp);
  float acc = 0.f;
  for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
    uint4 wv[U], xx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + lane + 64 * u;
      const bool in = v < nvec;
      wv[u] = load_stream(wr + (in ? v : 0));
      const uint4 xr = xv[in ? v : 0];
      xx[u] = in ? xr : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) dot8(wv[u], xx[u], acc, T());
  }
  return wave_sum(acc);
}

constexpr int kGemvBatch = 8;

// Order the LDS accesses of one wave: every write before the fence is complete and
// visible to the wave's other lanes before any access after it, and the compiler
// moves no memory access across it.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One row per wave, four rows per workgroup.
template <typename T>
__global__ void __launch_bounds__(256) gemv_kernel(const T* __restrict__ W, int d_out, int d_in,
                                                   int64_t ld, const T* __restrict__ x,
                                                   T* __restrict__ y, float* __restrict__ y32) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const float s = row_dot<T, kGemvBatch>(W + int64_t(row) * ld, x, d_in);
  if (lane == 0) {
    if (y32)
      y32[row] = s;
    else
      store_out(y, row, s);
  }
}

// Independent GEMVs in one grid (the stacked rows of every projection, one row per
// wave): per projection bit-identical to gemv_kernel, with one launch's ramp and tail
// instead of one per projection.
template <typename T>
__global__ void __launch_bounds__(256) gemv_layer_kernel(GemvLayerParams p) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  int q = 0;
  while (q < p.n - 1 && g >= p.proj[q + 1].row0) ++q;
  const GemvLayerProj& P = p.proj[q];
  const int row = g - P.row0;
  if (row >= P.d_out) return;
  const float s = row_dot<T, kGemvBatch>(static_cast<const T*>(P.w) + int64_t(row) * P.ld,
                                         static_cast<const T*>(P.x), P.d_in);
  if (lane == 0) store_out(static_cast<T*>(P.y), row, s);
}

// t[j*r + rr] = A[idx_j][rr] . x for every slot j < k (0 for an out-of-range index).
template <typename T>
__global__ void __launch_bounds__(256) lora_shrink_kernel(const T* __restrict__ A, int E, int r,
                                                          int d_in, const int32_t* __restrict__ idx,
                                                          int k, const T* __restrict__ x,
                                                          float* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= k * r) return;
  const int j = row / r, rr = row - j * r;
  const int e = idx[j];
  float acc = 0.f;
  if (e >= 0 && e < E) acc = row_dot<T, kGemvBatch>(A + (int64_t(e) * r + rr) * d_in, x, d_in);
  if (lane == 0) t[row] = acc;
}

// Eight consecutive elements of a 16-byte-aligned row as floats.
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = __uint_as_float(w[h] << 16);
    v[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// RNE(y32[i] + sum_j scale * gate[j] * sum_rr B[idx_j][i][rr] t[j*r + rr]) for one row i.
// When r is a multiple of 8 (rows of B and t then start on 16-byte boundaries: B is
// 16-byte aligned and every t block starts at a multiple of 4 floats) the row and t are
// read as 16-byte vectors; the products are summed in the same order either way.
template <typename T>
__device__ __forceinline__ float expand_row(const T* __restrict__ B, int E, int r, int d_out, int i,
                                            const int32_t* __restrict__ idx, const float* __restrict__ gate,
                                            int k, float scale, float y32, const float* __restrict__ t) {
  float acc = y32;
  for (int j = 0; j < k; ++j) {
    const int e = idx[j];
    const float c = scale * gate[j];
    if (e < 0 || e >= E || c == 0.f) continue;
    const T* br = B + (int64_t(e) * d_out + i) * r;
    const float* tj = t + j * r;
    float s = 0.f;
    if ((r & 7) == 0) {
      for (int rr = 0; rr < r; rr += 8) {
        float bv[8], tv[8];
        load8(br + rr, bv);
        load8(tj + rr, tv);
#pragma unroll
        for (int h = 0; h < 8; ++h) s = fmaf(bv[h], tv[h], s);
      }
    } else {
      for (int rr = 0; rr < r; ++rr) s = fmaf(load_elem(br, rr), tj[rr], s);
    }
    acc = fmaf(c, s, acc);
  }
  return acc;
}

template <typename T>
__global__ void __launch_bounds__(256) lora_expand_kernel(const T* __restrict__ B, int E, int r,
                                                          int d_out, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ gate, int k,
                                                          float scale, const float* __restrict__ y32,
                                                          const float* __restrict__ t,
                                                          T* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d_out) return;
  store_out(y, i, expand_row(B, E, r, d_out, i, idx, gate, k, scale, y32[i], t));
}

// ---- one layer of the unmerged routed path in two launches (the projections of a
// layer are independent given their inputs): grid 1 computes every projection's base
// GEMV rows and shrink rows, grid 2 every projection's expand.
template <typename T>
__global__ void __launch_bounds__(256) lora_layer_dot_kernel(LoraLayerParams p) {
  const int lane = threadIdx.x & 63;
  int g = blockIdx.x * 4 + (threadIdx.x >> 6);  // row of the stacked [W_p; A_sel,p] over p
  int q = 0;
  while (q < p.n - 1 && g >= p.proj[q + 1].dot_row0) ++q;
  const LoraLayerProj& P = p.proj[q];
  const int lr = g - P.dot_row0;
  const int kr = p.k * p.r;
  if (lr >= P.d_out + kr) return;
  const T* x = static_cast<const T*>(P.x);
  float* ws = p.ws + P.ws_off;
  if (lr < P.d_out) {
    const float s = row_dot<T, kGemvBatch>(static_cast<const T*>(P.w) + int64_t(lr) * P.ld, x, P.d_in);
    if (lane == 0) ws[lr] = s;
  } else {
    const int sr = lr - P.d_out, j = sr / p.r, rr = sr - j * p.r;
    const int e = p.idx[j];
    float s = 0.f;
    if (e >= 0 && e < p.E)
      s = row_dot<T, kGemvBatch>(static_cast<const T*>(P.a) + (int64_t(e) * p.r + rr) * P.d_in, x, P.d_in);
    if (lane == 0) ws[P.d_out + sr] = s;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) lora_layer_expand_kernel(LoraLayerParams p) {
  const int g = blockIdx.x * 256 + threadIdx.x;  // output row over the concatenated projections
  int q = 0;
  while (q < p.n - 1 && g >= p.proj[q + 1].out_row0) ++q;
  const LoraLayerProj& P = p.proj[q];
  const int i = g - P.out_row0;
  if (i >= P.d_out) return;
  const float* ws = p.ws + P.ws_off;
  store_out(static_cast<T*>(P.y), i,
            expand_row(static_cast<const T*>(P.b), p.E, p.r, P.d_out, i, p.idx, p.gate, p.k, p.scale, ws[i],
                       ws + P.d_out));
}

// ---- a batch of requests, each with its own selection (one group of a layer's
// projections, two launches).  Grid 1, in units of workgroups: per projection,
// ceil(d_out/16) base workgroups, then ceil(nb*k*r / 4) shrink workgroups (one selected
// A row per wave).  A base workgroup computes Y[16 rows][16 requests] = W[rows] X^T on
// MFMA (v_mfma_f32_16x16x32_bf16; fp32: 16x16x4), its 4 waves taking interleaved
// slices of the contraction and adding their partial tiles in a fixed order through
// LDS, so each W row is read from HBM once for the whole batch.  Lane l = 16 q + i of
// a wave supplies W[row i][k .. k+7] (bf16: from the wave's LDS window, filled row by
// row) and X[request i][k .. k+7] (k = k0 + 8 q) and
// receives D[4 q + c][i] = sum_k W[row 4q + c][k] X[request i][k].  Rows past d_out
// and requests past nb re-read row / request 0 and are not stored.
// Grid 2: every request's expand (as ada_lora_layer).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row pitch (bf16 elements) of a wave's staging window in LDS: 128 k plus 8, so the 16
// rows of an MFMA fragment read start 16 bytes apart in the bank space.
constexpr int kBaseLdw = 128 + 8;

// One wave's share of a base tile: contraction steps wave, wave + 4, wave + 8, ...
// bf16: a step is the tile's 16 rows x 128 k.  W is read row by row (each load
// instruction covers 4 rows x 256 contiguous bytes, as the decode GEMV streams W)
// into the wave's own LDS window `stage`, and read back in the MFMA operand layout
// (16 rows x 16 bytes per instruction): loading the operand layout straight from
// HBM touches 16 rows x 64 bytes per instruction, and the 7B decode step with 4 to
// 16 requests ran 10-14% slower that way.  Only
// the wave itself touches its window, and a wave's LDS accesses run in order, so no
// barrier is needed.
template <typename T>
__device__ __forceinline__ f32x4 base_tile_part(const T* __restrict__ W, int64_t ld, int row0, int d_out,
                                                const T* __restrict__ X, int d_in, int nb, int wave,
                                                uint16_t* stage) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, i = lane & 15;
  const T* wrow = W + int64_t(row0 + i < d_out ? row0 + i : 0) * ld;
  const T* xrow = X + int64_t(i < nb ? i : 0) * d_in;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    constexpr int U = 4;  // 32-deep MFMA steps per 128-k window
    // row-by-row loads: instruction u covers tile rows 4u .. 4u+3, lane l reading
    // 16-byte chunk l % 16 of row 4u + l / 16 inside the window
    const T* lrow[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = row0 + 4 * u + (lane >> 4);
      lrow[u] = W + int64_t(r < d_out ? r : 0) * ld;
    }
    for (int k0 = 32 * U * wave; k0 < d_in; k0 += 4 * 32 * U) {
      uint4 wl[U], wv[U], xv[U];
      const int kl = k0 + 8 * (lane & 15);
      const bool inl = kl < d_in;  // d_in is a multiple of 8: whole vectors in or out
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint4 w = load_stream(reinterpret_cast<const uint4*>(lrow[u] + (inl ? kl : 0)));
        wl[u] = inl ? w : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + 32 * u + 8 * q;
        const bool in = k < d_in;
        const uint4 x = *reinterpret_cast<const uint4*>(xrow + (in ? k : 0));
        xv[u] = in ? x : make_uint4(0, 0, 0, 0);
      }
      // the stage window passes W between lanes of this wave: each lane reads what
      // other lanes wrote, which per-lane program order does not order, so the
      // writes are fenced and a wave barrier keeps the compiler from moving the
      // LDS accesses across each other (here, and before the next window's writes)
#pragma unroll
      for (int u = 0; u < U; ++u)
        *reinterpret_cast<uint4*>(stage + (4 * u + (lane >> 4)) * kBaseLdw + 8 * (lane & 15)) = wl[u];
      lds_wave_sync();
#pragma unroll
      for (int u = 0; u < U; ++u) wv[u] = *reinterpret_cast<const uint4*>(stage + i * kBaseLdw + 32 * u + 8 * q);
      lds_wave_sync();
#pragma unroll
      for (int u = 0; u < U; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[u]),
                                                      __builtin_bit_cast(bf16x8_t, xv[u]), acc, 0, 0, 0);
    }
    (void)wrow;
  } else {
    // fp32: lane (q, i) loads 4 consecutive k; MFMA j takes element j of every lane,
    // i.e. k = k0 + 4 q + j (the same permutation of k on both operands)
    for (int k0 = 16 * wave; k0 < d_in; k0 += 4 * 16) {
      const int k = k0 + 4 * q;
      const bool in = k < d_in;  // d_in is a multiple of 8: whole 4-vectors in or out
      const float4 w = *reinterpret_cast<const float4*>(wrow + (in ? k : 0));
      const float4 x = *reinterpret_cast<const float4*>(xrow + (in ? k : 0));
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 wm = in ? w : z, xm = in ? x : z;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wm.x, xm.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wm.y, xm.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wm.z, xm.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wm.w, xm.w, acc, 0, 0, 0);
    }
  }
  return acc;
}

template <typename T>
__global__ void __launch_bounds__(256) lora_batch_dot_kernel(LoraLayerParams p) {
  __shared__ f32x4 part[3][64];
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][16 * kBaseLdw];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = blockIdx.x;  // workgroup index
  int q = 0;
  while (q < p.n - 1 && g >= p.proj[q + 1].dot_row0) ++q;
  const LoraLayerProj& P = p.proj[q];
  const int lw = g - P.dot_row0;
  const int kr = p.k * p.r;
  const int base_wgs = (P.d_out + 15) / 16;
  const T* x = static_cast<const T*>(P.x);
  float* ws = p.ws + P.ws_off;
  if (lw < base_wgs) {
    const int row0 = 16 * lw;
    f32x4 acc = base_tile_part(static_cast<const T*>(P.w), P.ld, row0, P.d_out, x, P.d_in, p.nb, wave,
                               stage[wave]);
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = acc + part[0][lane];
    acc = acc + part[1][lane];
    acc = acc + part[2][lane];
    const int i = lane & 15, qq = lane >> 4;
    if (i < p.nb) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = row0 + 4 * qq + c;
        if (row < P.d_out) ws[int64_t(i) * P.d_out + row] = acc[c];
      }
    }
  } else {
    const int sr = 4 * (lw - base_wgs) + wave;  // request b, slot j, rank rr
    if (sr >= p.nb * kr) return;
    const int b = sr / kr, rem = sr - b * kr, j = rem / p.r, rr = rem - j * p.r;
    const int e = p.idx[b * p.k + j];
    float s = 0.f;
    if (e >= 0 && e < p.E)
      s = row_dot<T, kGemvBatch>(static_cast<const T*>(P.a) + (int64_t(e) * p.r + rr) * P.d_in,
                                 x + int64_t(b) * P.d_in, P.d_in);
    if (lane == 0) ws[int64_t(p.nb) * P.d_out + sr] = s;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) lora_batch_expand_kernel(LoraLayerParams p) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  int q = 0;
  while (q < p.n - 1 && g >= p.proj[q + 1].out_row0) ++q;
  const LoraLayerProj& P = p.proj[q];
  const int o = g - P.out_row0;
  if (o >= p.nb * P.d_out) return;
  const int b = o / P.d_out, i = o - b * P.d_out;
  const int kr = p.k * p.r;
  const float* ws = p.ws + P.ws_off;
  store_out(static_cast<T*>(P.y), o,
            expand_row(static_cast<const T*>(P.b), p.E, p.r, P.d_out, i, p.idx + b * p.k, p.gate + b * p.k, p.k,
                       p.scale, ws[o], ws + int64_t(p.nb) * P.d_out + int64_t(b) * kr));
}

}  // namespace

hipError_t launch_gemv(const void* w, int d_out, int d_in, int64_t ld, const void* x, void* y,
                       float* y32, int dtype, hipStream_t s) {
  const dim3 grid((d_out + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL((gemv_kernel<uint16_t>), grid, block, 0, s, static_cast<const uint16_t*>(w), d_out,
                       d_in, ld, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), y32);
  else
    hipLaunchKernelGGL((gemv_kernel<float>), grid, block, 0, s, static_cast<const float*>(w), d_out, d_in,
                       ld, static_cast<const float*>(x), static_cast<float*>(y), y32);
  return hipGetLastError();
}

hipError_t launch_gemv_layer(const GemvLayerParams& p, int rows, int dtype, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(gemv_layer_kernel<uint16_t>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(gemv_layer_kernel<float>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lora_shrink(const void* a, int E, int r, int d_in, const int32_t* idx, int k,
                              const void* x, float* t, int dtype, hipStream_t s) {
  const dim3 grid((k * r + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(lora_shrink_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(a),
                       E, r, d_in, idx, k, static_cast<const uint16_t*>(x), t);
  else
    hipLaunchKernelGGL(lora_shrink_kernel<float>, grid, block, 0, s, static_cast<const float*>(a), E, r,
                       d_in, idx, k, static_cast<const float*>(x), t);
  return hipGetLastError();
}

hipError_t launch_lora_expand(const void* b, int E, int r, int d_out, const int32_t* idx,
                              const float* gate, int k, float scale, const float* y32,
                              const float* t, void* y, int dtype, hipStream_t s) {
  const dim3 grid((d_out + 255) / 256), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(lora_expand_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(b),
                       E, r, d_out, idx, gate, k, scale, y32, t, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(lora_expand_kernel<float>, grid, block, 0, s, static_cast<const float*>(b), E, r,
                       d_out, idx, gate, k, scale, y32, t, static_cast<float*>(y));
  return hipGetLastError();
}

// ---- device memory for the allocation-free layer path (ada_lora_layer_static): a
// file-scope array, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): it takes each device's address once, with that device current, and uses
// that address.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* addr = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    g_scratch_ptr[dev] = addr;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_lora_layer(const LoraLayerParams& p, int dot_rows, int out_rows, int dtype, hipStream_t s) {
  const dim3 g1((dot_rows + 3) / 4), g2((out_rows + 255) / 256), block(256);
  if (dtype == 1) {
    hipLaunchKernelGGL(lora_layer_dot_kernel<uint16_t>, g1, block, 0, s, p);
    hipLaunchKernelGGL(lora_layer_expand_kernel<uint16_t>, g2, block, 0, s, p);
  } else {
    hipLaunchKernelGGL(lora_layer_dot_kernel<float>, g1, block, 0, s, p);
    hipLaunchKernelGGL(lora_layer_expand_kernel<float>, g2, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_lora_batch(const LoraLayerParams& p, int dot_wgs, int out_rows, int dtype, hipStream_t s) {
  const dim3 g1(dot_wgs), g2((out_rows + 255) / 256), block(256);
  if (dtype == 1) {
    hipLaunchKernelGGL(lora_batch_dot_kernel<uint16_t>, g1, block, 0, s, p);
    hipLaunchKernelGGL(lora_batch_expand_kernel<uint16_t>, g2, block, 0, s, p);
  } else {
    hipLaunchKernelGGL(lora_batch_dot_kernel<float>, g1, block, 0, s, p);
    hipLaunchKernelGGL(lora_batch_expand_kernel<float>, g2, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ada
