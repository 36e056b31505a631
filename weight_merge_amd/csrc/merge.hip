// Fused adapter merge / unmerge / switch: one launch over every registered projection.
//
// What it computes ("AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level
// Pre-Gating and Fused Kernel Optimization", Japanese summary page, technical
// overview 2.2; Portuguese page, technical summary 2.B): the selected adapters' down
// projections A_e (r x d_in) and up projections B_e (d_out x r) are concatenated into
// one rank-(k*r) pair, and
//     dst = RNE(src + B_cat @ A_cat),  B_cat = [c_1 B_{e_1} | ... | c_k B_{e_k}],
//                                      A_cat = [A_{e_1}; ...; A_{e_k}],
// with c_j = +scale * g_j to fuse and -scale * g_j to de-fuse.  The pages split the
// product into GEMM tiles per thread block and hide global-memory latency with a
// prefetch buffer; here one workgroup owns one 64 x 128 output tile of one
// projection, found through a work table, so a single grid covers all layers.
//
// The merge is bound by HBM: every weight is read once and written once, while
// the rank-(k*r) product costs 2*k*r flops per weight.  The layout choices serve
// that stream:
//   * W goes from HBM straight to registers and back, never through LDS.  The
//     MFMA's M index is mapped to W columns and its N index to W rows, so each
//     lane's four accumulator values are four adjacent columns of one row; with
//     a column permutation inside each 64-column strip every lane owns two runs of
//     8 adjacent columns, loaded and stored as 16-byte vectors.
//   * A_cat and B_cat for the tile are gathered into LDS once per K chunk, with the
//     gate and scale folded into B_cat (rounded to bf16), A_cat stored transposed so
//     every MFMA operand fragment is one 16-byte LDS read.
//   * The W loads are issued first, straight after the tile lookup, with every load
//     on the path branch-free and in the global address space, so no wait for the
//     selection or the adapter gathers also waits for the W tile.
//   * Small tiles (64 x 128) keep registers low: four waves per SIMD, so many tiles'
//     W loads are in flight on each CU.
//   * Workgroup ids are remapped so each XCD walks a contiguous range of tiles,
//     keeping a projection's adapter rows and columns in that XCD's L2.
#include "common.h"

namespace ada {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Pointers read from the work table are generic; casting them to the global address
// space lets the compiler emit global_load/global_store, which count only against
// the vector-memory counter (flat accesses also hold the LDS/scalar counter, so every
// LDS wait would wait for the whole W tile).
#define ADA_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const ADA_GLOBAL T* as_global(const void* p) {
  return (const ADA_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ ADA_GLOBAL T* as_global_mut(void* p) {
  return (ADA_GLOBAL T*)(p);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float c) {
  u32x4 o;
  o.x = pack_bf16x2(bf16_lo(v.x) * c, bf16_hi(v.x) * c);
  o.y = pack_bf16x2(bf16_lo(v.y) * c, bf16_hi(v.y) * c);
  o.z = pack_bf16x2(bf16_lo(v.z) * c, bf16_hi(v.z) * c);
  o.w = pack_bf16x2(bf16_lo(v.w) * c, bf16_hi(v.w) * c);
  return o;
}

// Wave 0 gathers the active slots of both selections into LDS, in selection
// order: a slot is active when its index is in range and its coefficient is
// nonzero.  Every workgroup computes the same list.
__device__ __forceinline__ void compact_slots(const MergeParams& p, int* s_exp, float* s_coef,
                                              int* s_n) {
  const int lane = threadIdx.x & 63;
  int n = 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = p.sel[s].k;
    if (k <= 0) continue;
    const bool valid = lane < k;
    const int e = valid ? p.sel[s].idx[lane] : -1;
    const float g = valid ? p.sel[s].gate[lane] : 0.f;
    const float c = p.sel[s].coef * g;
    const bool act = valid && e >= 0 && e < p.E && c != 0.f;
    const unsigned long long m = __ballot(act);
    const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
    if (act) {
      s_exp[pos] = e;
      s_coef[pos] = c;
    }
    n += __popcll(m);
  }
  if (lane == 0) *s_n = n;
}

struct TileRef {
  const void* src;
  void* dst;
  const void* a;
  const void* b;
  int64_t ld;
  int d_out, d_in, row0, col0;
};

// Workgroup -> (projection, tile).  The lookup table maps a bucket of 2^lut_shift
// tiles to the first entry that overlaps it; buckets are no larger than the
// smallest entry, so at most a step or two forward is needed.
__device__ __forceinline__ TileRef find_tile(const MergeParams& p, int tile_rows, int tile_cols) {
  int64_t t = blockIdx.x;
  if (p.xcd_remap) {
    // consecutive workgroups land on consecutive XCDs (round robin over 8);
    // hand XCD x the contiguous range [x*G8/8, (x+1)*G8/8).
    const int64_t G8 = p.total_tiles & ~int64_t(7);
    if (t < G8) t = (t & 7) * (G8 >> 3) + (t >> 3);
  }
  int e = p.lut[t >> p.lut_shift];
  while (t >= p.table[e + 1].tile_base) ++e;
  const MergeEntry* en = p.table + e;
  const int64_t local = t - en->tile_base;
  const int tn = en->tiles_n;
  TileRef r;
  r.src = p.src_is_out ? en->w_out : en->w;
  r.dst = en->w_out;
  r.a = en->a;
  r.b = en->b;
  r.ld = en->ld;
  r.d_out = en->d_out;
  r.d_in = en->d_in;
  r.row0 = int(local / tn) * tile_rows;
  r.col0 = int(local % tn) * tile_cols;
  return r;
}

// ---------------------------------------------------------------- bf16, MFMA path
//
// Workgroup: 4 waves in a 2 x 2 arrangement, each owning a (16 RB) x 64 sub-tile made
// of RB x 4 MFMA blocks of 16 x 16 (v_mfma_f32_16x16x32_bf16); the workgroup tile is
// (32 RB) x 128.  For block (rb, ct) lane l = 16 q + i holds D[4q + c][i] =
// delta[row 16 rb + i][col(ct, 4q + c)], with col(ct, m) = 32 (ct / 2) + 8 (m / 4) +
// 4 (ct % 2) + m % 4 inside the wave's strip: lane (q, i) owns the columns
// 32 h + 8 q + [0, 8) for h = 0, 1.
//
// Order of work inside a workgroup, chosen so HBM never waits on the rest:
//   1. wave 0 loads the selection (k indices and gates, L2-resident);
//   2. every lane issues its W loads (the tile's HBM traffic);
//   3. wave 0 compacts the active slots into LDS (waits for step 1 only);
//   4. the adapter gathers for the first K chunk go to LDS; MFMAs run;
//   5. W + delta is rounded once and stored.
template <int KC, int RB>
__global__ void __launch_bounds__(256) merge_bf16_kernel(MergeParams p) {
  constexpr int BM = 32 * RB, BN = 128;
  constexpr int LDK = KC + 8;  // LDS row pitch in elements (16-byte pad)
  static_assert((BM * KC / 8) % 256 == 0 && (KC * BN / 8) % 256 == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t As[BN * LDK];
  __shared__ int s_exp[kMaxSlots];
  __shared__ float s_coef[kMaxSlots];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int li = lane & 15;
  const int wy = wave >> 1, wx = wave & 1;

  const TileRef T = find_tile(p, BM, BN);
  static_assert(BM == kTileBF16Rows && BN == kTileBF16Cols, "tile matches the work table");
  const ADA_GLOBAL uint16_t* __restrict__ src = as_global<uint16_t>(T.src);
  ADA_GLOBAL uint16_t* __restrict__ dst = as_global_mut<uint16_t>(T.dst);
  const ADA_GLOBAL uint16_t* __restrict__ gA = as_global<uint16_t>(T.a);
  const ADA_GLOBAL uint16_t* __restrict__ gB = as_global<uint16_t>(T.b);

  // 1. selection (wave 0): lane j holds slot j of each selection
  // (branch-free: lanes past k re-read slot 0, which always exists, and are
  // discarded below; exec-masked loads would make the compiler wait for every
  // outstanding load, the W tile included, before the compaction)
  int sel_e[2];
  float sel_g[2];
  if (wave == 0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int j = lane < p.sel[s].k ? lane : 0;
      sel_e[s] = p.sel[s].idx[j];
      sel_g[s] = p.sel[s].gate[j];
    }
  }

  // 2. this lane's W vectors: rows row0 + 16 RB wy + 16 rb + li, columns col0 + 64 wx + 32 h + 8 q
  int64_t woff[RB][2];
  bool ok[RB][2];
  u32x4 wv[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = T.row0 + 16 * RB * wy + 16 * rb + li;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = T.col0 + 64 * wx + 32 * h + 8 * q;
      ok[rb][h] = row < T.d_out && col < T.d_in;
      woff[rb][h] = ok[rb][h] ? int64_t(row) * T.ld + col : 0;  // out of range: re-read W[0][0..8)
      wv[rb][h] = *reinterpret_cast<const ADA_GLOBAL u32x4*>(src + woff[rb][h]);
    }
  }

  // 3. active slots, in selection order: index in range and coefficient nonzero
  if (wave == 0) {
    int n = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float c = p.sel[s].coef * sel_g[s];
      const bool act = lane < p.sel[s].k && sel_e[s] >= 0 && sel_e[s] < p.E && c != 0.f;
      const unsigned long long m = __ballot(act);
      const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
      if (act) {
        s_exp[pos] = sel_e[s];
        s_coef[pos] = c;
      }
      n += __popcll(m);
    }
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const int nslot = s_n;

  if (nslot == 0) {
    // Nothing selected: in place there is nothing to write; out of place, copy.
    if (T.src == T.dst) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (ok[rb][h]) *reinterpret_cast<ADA_GLOBAL u32x4*>(dst + woff[rb][h]) = wv[rb][h];
    return;
  }

  const int r = p.r;
  const int kr = nslot * r;
  const bool rvec = (r & 7) == 0;

  // ---- K-chunk staging: global -> registers, then registers -> LDS.
  constexpr int B_VPT = BM * KC / 8 / 256;  // 16-byte B vectors per thread
  constexpr int A_VPT = KC * BN / 8 / 256;  // 16-byte A vectors per thread
  u32x4 sb[B_VPT];
  float sc[B_VPT];
  u32x4 sa[A_VPT];

  auto stage_load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
      const int v = tid + 256 * i;
      const int row = v / (KC / 8);
      const int kv = v % (KC / 8);
      const int grow = T.row0 + row;
      u32x4 val = (u32x4){0u, 0u, 0u, 0u};
      float c = 0.f;
      if (rvec) {
        // branch-free gather: out-of-range slots/rows re-read an in-range vector and
        // get a zero coefficient
        const int k = k0 + 8 * kv;
        const int j = k / r;
        const int rr = k - j * r;
        const bool in = j < nslot && grow < T.d_out;
        const int js = in ? j : 0;
        const int rs = in ? grow : 0;
        val = *reinterpret_cast<const ADA_GLOBAL u32x4*>(gB + (int64_t(s_exp[js]) * T.d_out + rs) * r + (in ? rr : 0));
        c = in ? s_coef[js] : 0.f;
        sc[i] = c;
      } else {
        // rank not a multiple of 8: gather element by element, coefficient applied here
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int k = k0 + 8 * kv + t;
          const int j = k / r;
          const int rr = k - j * r;
          float x = 0.f;
          if (j < nslot && grow < T.d_out)
            x = __uint_as_float(uint32_t(gB[(int64_t(s_exp[j]) * T.d_out + grow) * r + rr]) << 16) *
                s_coef[j];
          const uint32_t hb = pack_bf16x2(x, 0.f) & 0xffffu;
          w[t >> 1] |= hb << (16 * (t & 1));
        }
        val = (u32x4){w[0], w[1], w[2], w[3]};
        sc[i] = 1.f;
      }
      sb[i] = val;
    }
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
      const int v = tid + 256 * i;
      const int kl = v / (BN / 8);
      const int cv = v % (BN / 8);
      const int k = k0 + kl;
      const int j = k / r;
      const int rr = k - j * r;
      const int gcol = T.col0 + 8 * cv;
      const bool in = j < nslot && gcol < T.d_in;
      const u32x4 val = *reinterpret_cast<const ADA_GLOBAL u32x4*>(
          gA + (int64_t(s_exp[in ? j : 0]) * r + (in ? rr : 0)) * T.d_in + (in ? gcol : 0));
      sa[i] = in ? val : (u32x4){0u, 0u, 0u, 0u};
    }
  };

  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
      const int v = tid + 256 * i;
      const int row = v / (KC / 8);
      const int kv = v % (KC / 8);
      const u32x4 o = rvec ? scale_bf16x8(sb[i], sc[i]) : sb[i];
      *reinterpret_cast<u32x4*>(&Bs[row * LDK + 8 * kv]) = o;
    }
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
      const int v = tid + 256 * i;
      const int kl = v / (BN / 8);
      const int cv = v % (BN / 8);
      const u32x4 x = sa[i];
      uint16_t* col = &As[(8 * cv) * LDK + kl];
      col[0 * LDK] = uint16_t(x.x);
      col[1 * LDK] = uint16_t(x.x >> 16);
      col[2 * LDK] = uint16_t(x.y);
      col[3 * LDK] = uint16_t(x.y >> 16);
      col[4 * LDK] = uint16_t(x.z);
      col[5 * LDK] = uint16_t(x.z >> 16);
      col[6 * LDK] = uint16_t(x.w);
      col[7 * LDK] = uint16_t(x.w >> 16);
    }
  };

  // 4. first K chunk
  stage_load(0);
  stage_store();
  __syncthreads();

  f32x4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rb][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // LDS element offsets of this lane's operand fragments (k offset 8 q included)
  int aoff[4], boff[RB];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int col = 64 * wx + 32 * (ct >> 1) + 8 * (li >> 2) + 4 * (ct & 1) + (li & 3);
    aoff[ct] = col * LDK + 8 * q;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) boff[rb] = (16 * RB * wy + 16 * rb + li) * LDK + 8 * q;

  for (int k0 = 0;;) {
#pragma unroll
    for (int ks = 0; ks < KC / 32; ++ks) {
      bf16x8_t af[4], bfr[RB];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) af[ct] = *reinterpret_cast<const bf16x8_t*>(&As[aoff[ct] + 32 * ks]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bfr[rb] = *reinterpret_cast<const bf16x8_t*>(&Bs[boff[rb] + 32 * ks]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ct], bfr[rb], acc[rb][ct], 0, 0, 0);
    }
    k0 += KC;
    if (k0 >= kr) break;
    __syncthreads();  // every wave is done reading this chunk
    stage_load(k0);
    stage_store();
    __syncthreads();
  }

  // 5. W + delta, one rounding to bf16, 16-byte stores
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!ok[rb][h]) continue;
      const u32x4 w = wv[rb][h];
      const f32x4 d0 = acc[rb][2 * h];
      const f32x4 d1 = acc[rb][2 * h + 1];
      u32x4 o;
      o.x = pack_bf16x2(bf16_lo(w.x) + d0[0], bf16_hi(w.x) + d0[1]);
      o.y = pack_bf16x2(bf16_lo(w.y) + d0[2], bf16_hi(w.y) + d0[3]);
      o.z = pack_bf16x2(bf16_lo(w.z) + d1[0], bf16_hi(w.z) + d1[1]);
      o.w = pack_bf16x2(bf16_lo(w.w) + d1[2], bf16_hi(w.w) + d1[3]);
#if ADA_NT_STORE
      __builtin_nontemporal_store(o, reinterpret_cast<ADA_GLOBAL u32x4*>(dst + woff[rb][h]));
#else
      *reinterpret_cast<ADA_GLOBAL u32x4*>(dst + woff[rb][h]) = o;
#endif
    }
  }
}

// ---------------------------------------------------------------- fp32, VALU path
//
// 64 x 64 tile, each thread a 4 x 4 block; the fp32 product runs on the vector
// ALUs (fp32 storage is used for small stacks only).
template <int KC>
__global__ void __launch_bounds__(256) merge_f32_kernel(MergeParams p) {
  constexpr int BM = kTileF32, BN = kTileF32;
  __shared__ float Bs[BM][KC + 1];
  __shared__ __attribute__((aligned(16))) float As[KC][BN + 4];
  __shared__ int s_exp[kMaxSlots];
  __shared__ float s_coef[kMaxSlots];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const TileRef T = find_tile(p, BM, BN);
  const ADA_GLOBAL float* __restrict__ src = as_global<float>(T.src);
  ADA_GLOBAL float* __restrict__ dst = as_global_mut<float>(T.dst);
  const ADA_GLOBAL float* __restrict__ gA = as_global<float>(T.a);
  const ADA_GLOBAL float* __restrict__ gB = as_global<float>(T.b);

  if ((tid >> 6) == 0) compact_slots(p, s_exp, s_coef, &s_n);
  __syncthreads();
  const int nslot = s_n;
  const int col = T.col0 + 4 * tx;
  const bool colok = col < T.d_in;

  if (nslot == 0) {
    if (T.src == T.dst) return;
    for (int i = 0; i < 4; ++i) {
      const int row = T.row0 + 4 * ty + i;
      if (row < T.d_out && colok)
        *reinterpret_cast<ADA_GLOBAL f32x4*>(dst + int64_t(row) * T.ld + col) =
            *reinterpret_cast<const ADA_GLOBAL f32x4*>(src + int64_t(row) * T.ld + col);
    }
    return;
  }

  const int r = p.r;
  const int kr = nslot * r;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < kr; k0 += KC) {
    for (int e = tid; e < BM * KC; e += 256) {
      const int row = e / KC, kk = e % KC;
      const int k = k0 + kk, j = k / r, rr = k - j * r;
      const int grow = T.row0 + row;
      float v = 0.f;
      if (j < nslot && grow < T.d_out) v = s_coef[j] * gB[(int64_t(s_exp[j]) * T.d_out + grow) * r + rr];
      Bs[row][kk] = v;
    }
    for (int e = tid; e < KC * BN; e += 256) {
      const int kk = e / BN, c = e % BN;
      const int k = k0 + kk, j = k / r, rr = k - j * r;
      const int gcol = T.col0 + c;
      float v = 0.f;
      if (j < nslot && gcol < T.d_in) v = gA[(int64_t(s_exp[j]) * r + rr) * T.d_in + gcol];
      As[kk][c] = v;
    }
    __syncthreads();
    for (int kk = 0; kk < KC; ++kk) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&As[kk][4 * tx]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float b = Bs[4 * ty + i][kk];
        acc[i][0] = fmaf(b, a.x, acc[i][0]);
        acc[i][1] = fmaf(b, a.y, acc[i][1]);
        acc[i][2] = fmaf(b, a.z, acc[i][2]);
        acc[i][3] = fmaf(b, a.w, acc[i][3]);
      }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int row = T.row0 + 4 * ty + i;
    if (row >= T.d_out || !colok) continue;
    const int64_t off = int64_t(row) * T.ld + col;
    const f32x4 w = *reinterpret_cast<const ADA_GLOBAL f32x4*>(src + off);
    f32x4 o;
    o.x = w.x + acc[i][0];
    o.y = w.y + acc[i][1];
    o.z = w.z + acc[i][2];
    o.w = w.w + acc[i][3];
    *reinterpret_cast<ADA_GLOBAL f32x4*>(dst + off) = o;
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int dtype, int kr_max, hipStream_t s) {
  if (p.total_tiles <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.total_tiles)), block(256);
  if (dtype == 1) {
    if (kr_max <= 32)
      hipLaunchKernelGGL((merge_bf16_kernel<32, kBF16RowBlocks>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((merge_bf16_kernel<64, kBF16RowBlocks>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL(merge_f32_kernel<32>, grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ada
