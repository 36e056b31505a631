// Token-level pre-gating: router GEMV, top-k and gates in one workgroup.
//
// "AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level Pre-Gating and
// Fused Kernel Optimization", Portuguese summary page, technical summary 2.A, and
// Japanese page, technical overview 2.1: a single light Top-2 router, run once at
// the first layer, picks the LoRA experts for every later layer.  Here:
//   z = R h (fp32 accumulation), the k largest z in descending order with equal
//   scores going to the lower index, and softmax gates over the selected scores
//   (or, with renorm = 0, the full softmax read at the selected experts).
// Each wave reduces whole rows of R with 16-byte loads and a butterfly, so every
// score is summed in the same order whichever wave owns its row.  Wave 0 then holds
// one score per lane (E <= 64) and runs k rounds of a wave-wide argmax on a 64-bit
// key (order-preserving score bits, then the inverted lane index).
#include "launch.h"

namespace ada {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned long long o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key).  -0.0
// and +0.0 are equal scores, so both map to the key of +0.0 (the tie then goes to the
// lower index, as for any other pair of equal scores).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

template <typename T>
__global__ void __launch_bounds__(1024) pregate_kernel(const T* __restrict__ h,
                                                       const T* __restrict__ R, int d, int E,
                                                       int k, int renorm, int32_t* __restrict__ idx_out,
                                                       float* __restrict__ gate_out) {
  __shared__ float z[64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwave = blockDim.x >> 6;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte vector
  const int nvec = d / VEC;
  const uint4* hv = reinterpret_cast<const uint4*>(h);

  for (int e = wave; e < E; e += nwave) {
    const uint4* rv = reinterpret_cast<const uint4*>(R + int64_t(e) * d);
    float acc = 0.f;
    // batches of U vectors per lane, all loads issued before any is used (one round
    // trip per batch instead of one per vector); past the row end a lane re-reads
    // vector 0 and multiplies it by zeros
    constexpr int U = 8;
    for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
      uint4 rr[U], hh[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + lane + 64 * u;
        const bool in = v < nvec;
        rr[u] = rv[in ? v : 0];
        const uint4 hx = hv[in ? v : 0];
        hh[u] = in ? hx : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) dot8(rr[u], hh[u], acc, T());
    }
    acc = wave_sum(acc);
    if (lane == 0) z[e] = acc;
  }
  __syncthreads();
  if (wave != 0) return;

  const bool real = lane < E;
  const float zl = real ? z[lane] : 0.f;
  bool taken = !real;
  int my_e = 0;
  float my_z = 0.f;
  for (int j = 0; j < k; ++j) {
    const unsigned long long key =
        taken ? 0ull : ((static_cast<unsigned long long>(ordered_bits(zl)) << 32) | uint32_t(64 - lane));
    const unsigned long long best = wave_max_u64(key);
    const int e = 64 - int(best & 0xffffffffu);
    const float ze = __shfl(zl, e, 64);
    if (lane == e) taken = true;
    if (lane == j) {
      my_e = e;
      my_z = ze;
    }
  }
  const float zmax = __shfl(my_z, 0, 64);  // the first pick holds the largest score
  float ex;
  if (renorm) {
    ex = lane < k ? expf(my_z - zmax) : 0.f;
  } else {
    ex = real ? expf(zl - zmax) : 0.f;
  }
  const float denom = wave_sum(ex);
  if (lane < k) {
    const float num = renorm ? ex : expf(my_z - zmax);
    idx_out[lane] = my_e;
    gate_out[lane] = num / denom;
  }
}

}  // namespace

hipError_t launch_pregate(const void* h, const void* router, int d, int E, int k, int dtype,
                          int renorm, int32_t* idx, float* gate, hipStream_t s) {
  // one workgroup: up to 16 waves, never more waves than rows
  const int waves = E < 16 ? E : 16;
  const dim3 grid(1), block(64 * waves);
  if (dtype == 1)
    hipLaunchKernelGGL(pregate_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(router), d, E,
                       k, renorm, idx, gate);
  else
    hipLaunchKernelGGL(pregate_kernel<float>, grid, block, 0, s, static_cast<const float*>(h),
                       static_cast<const float*>(router), d, E, k, renorm, idx, gate);
  return hipGetLastError();
}

}  // namespace ada
