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
// prefetch buffer; here one workgroup owns one output tile of one projection (32 x 256,
// 64 x 128 or 128 x 128 by contraction length), found through a work table, so a
// single grid covers all layers.
//
// The merge is bound by HBM: every weight is read once and written once, while
// the rank-(k*r) product costs 2*k*r flops per weight.  The layout choices serve
// that stream:
//   * W goes from HBM to registers and back in a row-major pattern: each load or
//     store instruction covers whole tile rows (256 or 512 contiguous bytes), with
//     the nontemporal policy (each weight is touched once).  The MFMA's
//     M index is mapped to W columns and its N index to W rows, so each lane's four
//     accumulator values are four adjacent columns of one row; the accumulators
//     reach the W layout through one fp32 pass in LDS.
//   * A_cat and B_cat for the tile are gathered into LDS once per K chunk (double
//     buffered), with the gate and scale folded into B_cat (rounded to bf16).  Both
//     are stored as they lie in memory (16-byte writes); the A operand's transpose
//     happens in the LDS read (ds_read_b64_tr_b16).
//   * The W loads are issued straight after the tile lookup and the selection loads,
//     with every load on the path branch-free and in the global address space, so
//     compacting the selection does not wait for the W tile (the vector-memory
//     counter is in order: the adapter gathers, issued after W, do wait for it, and
//     the K loop starts once both have arrived).
//   * Small tiles keep registers low for short contractions: four waves per SIMD, so
//     many tiles' W loads are in flight on each CU.  At k*r <= 32 the tile is 32 x 256
//     (each tile row a 512-byte run of W; 2.6% faster on the 7B stack than 64 x 128),
//     up to k*r = 64 it is 64 x 128 (half the A_cat columns to gather: the fused
//     switch at k*r = 64 runs 8% slower on 32 x 256).  Long contractions use 128 x 128
//     tiles so each gathered adapter byte serves more weights.  Their latency (one L2
//     round trip per chunk, the W tile's HBM latency) is hidden by other workgroups
//     of the CU rather than inside one: a lean form (one operand buffer, W loaded only
//     for the last chunk, the delta through LDS in halves) fits three workgroups per CU
//     where the double-buffered form fits two, and is 7-13% faster on the 7B stack at
//     every long contraction measured (ranks 8 to 64, k*r 128 to 256).
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

// 16-byte access at a uniform base plus a 32-bit per-lane byte offset: the form the
// compiler maps onto global_load/store with a scalar base and a 32-bit vector offset,
// with no 64-bit address arithmetic per access.  Every W matrix and adapter bank has
// fewer than 2^31 elements, so byte offsets fit in 32 bits.
__device__ __forceinline__ u32x4 load16(const ADA_GLOBAL unsigned char* base, uint32_t off) {
  return *reinterpret_cast<const ADA_GLOBAL u32x4*>(base + off);
}
__device__ __forceinline__ void store16(ADA_GLOBAL unsigned char* base, uint32_t off, u32x4 v) {
  *reinterpret_cast<ADA_GLOBAL u32x4*>(base + off) = v;
}
// The same for the W stream, which a launch touches exactly once: nontemporal loads
// and stores (the adapter gathers, reused by neighbouring tiles through L2, keep the
// default policy).  Measured on the 7B stacks: 2.7% faster at k*r = 256, 3% faster
// for the fused switch, level at k*r = 32; bit-identical.
__device__ __forceinline__ u32x4 load16_stream(const ADA_GLOBAL unsigned char* base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const ADA_GLOBAL u32x4*>(base + off));
}
__device__ __forceinline__ void store16_stream(ADA_GLOBAL unsigned char* base, uint32_t off, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<ADA_GLOBAL u32x4*>(base + off));
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
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

// c * b for two bf16 values b packed in one word, as a pair of bf16 words: hi the
// product rounded to bf16, lo the remainder c*b - hi (formed exactly by the fma, then
// rounded to bf16), so hi + lo carries c*b to about 16 significant bits.
__device__ __forceinline__ void split_bf16x2(uint32_t v, float c, uint32_t& hi, uint32_t& lo) {
  const float b0 = bf16_lo(v), b1 = bf16_hi(v);
  hi = pack_bf16x2(b0 * c, b1 * c);
  lo = pack_bf16x2(fmaf(b0, c, -bf16_lo(hi)), fmaf(b1, c, -bf16_hi(hi)));
}

__device__ __forceinline__ void split_bf16x8(u32x4 v, float c, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
  split_bf16x2(v.x, c, h[0], l[0]);
  split_bf16x2(v.y, c, h[1], l[1]);
  split_bf16x2(v.z, c, h[2], l[2]);
  split_bf16x2(v.w, c, h[3], l[3]);
  hi = (u32x4){h[0], h[1], h[2], h[3]};
  lo = (u32x4){l[0], l[1], l[2], l[3]};
}

// Order the LDS accesses of one wave: writes before it are visible to the wave's other
// lanes after it, and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  // Tile order inside a projection: groups of tile_group row bands, each group walked
  // column block by column block (down the group's bands first).  tile_group = 1 is
  // plain row-major order.  Larger groups let consecutive tiles share an A_cat column
  // slab and keep the group's B_cat rows in L2, which matters when k*r is large.
  int band, cblk;
  {
    const int G = p.tile_group;
    const int tm = en->tiles_m;
    const int grp = int(local / (int64_t(G) * tn));
    const int first = grp * G;
    const int gsize = min(G, tm - first);
    const int within = int(local - int64_t(grp) * G * tn);
    band = first + within % gsize;
    cblk = within / gsize;
  }
  TileRef r;
  r.src = p.src_is_out ? en->w_out : en->w;
  r.dst = en->w_out;
  r.a = en->a;
  r.b = en->b;
  r.ld = en->ld;
  r.d_out = en->d_out;
  r.d_in = en->d_in;
  r.row0 = band * tile_rows;
  r.col0 = cblk * tile_cols;
  return r;
}

// ---------------------------------------------------------------- bf16, MFMA path
//
// Workgroup: 4 waves arranged WGM x WGN (WGM = 4 / WGN); each wave owns a (16 RB) x
// (16 CT) sub-tile made of RB x CT MFMA blocks of 16 x 16 (v_mfma_f32_16x16x32_bf16),
// so the workgroup tile is (16 RB WGM) x (16 CT WGN).  MFMA index m runs over W
// columns and n over W rows: for block (rb, ct), lane l = 16 q + i holds
// D[4q + c][i] = delta[row 16 rb + i][col(ct, 4q + c)] with
// col(ct, m) = 32 (ct / 2) + 8 (m / 4) + 4 (ct % 2) + m % 4 inside the wave's strip,
// so lane (q, i) owns the columns 32 h + 8 q + [0, 8), h = 0 .. CT/2 - 1.
//
// Operands per K chunk of KC, in NBUF LDS buffers (two for short contractions: chunk
// c+1 is stored while chunk c is multiplied; one for a launch whose contraction is a
// single chunk, and for the lean form of long contractions, whose chunk c+1 waits in
// registers until every wave has read chunk c):
//   As[k][col] = A_{e_j}[k - j r][col]               (rows of A_cat, as stored)
//   B_cat rows, in one of two forms that both carry the coefficients c_j = +-s g_j
//   at fp32 accuracy:
//   * split fold (every short contraction, and long ones whose rank is not a
//     multiple of the chunk): c_j B_{e_j} as a pair of bf16 planes,
//       Bh[row][k] = bf16(c_j b),  Bl[row][k] = bf16(c_j b - Bh[row][k]),
//     each multiplied by A_cat on MFMA into the same accumulators, so c_j b enters
//     the product with ~16 significant bits (a single bf16 plane, 8 bits, erred by
//     up to 2^-8 of sum_t |c b_t a_t|, which weights that cancel a large delta feel);
//   * scaled accumulators (long contractions whose chunks each lie in one slot):
//     Bs[row][k] = B_{e_j}[row][k - j r] unscaled, and the slots run in order of
//     increasing |c_j|; before the first chunk of slot j+1 the fp32 accumulators are
//     multiplied by c_j / c_{j+1} (at most 1 in magnitude, so nothing overflows), and
//     the epilogue multiplies the delta by the last slot's c: a Horner form of
//     sum_j c_j (B_{e_j} A_{e_j}) with fp32 roundings only, and no fold work per
//     gathered element.
// A B fragment (8 consecutive k of one row) is one 16-byte LDS read.  An A fragment
// (8 consecutive k of one column) is gathered from the row-major As with two
// ds_read_b64_tr_b16: inside each 16-lane group, lanes 4t..4t+3 point at 16 elements
// of k row t (4 each, in column order col(ct, 4u .. 4u+3) for lane 4t+u) and lane c
// receives element c of rows t = 0..3, i.e. 4 consecutive k of column col(ct, c).
//
// Order of work inside a workgroup, chosen so HBM never waits on the rest:
//   1. wave 0 loads the selection (k indices and gates, L2-resident);
//   2. every lane issues its W loads (the tile's HBM traffic; the lean form issues them
//      at step 4's last chunk instead, to keep its registers for more workgroups);
//   3. wave 0 compacts the active slots into LDS (waits for step 1 only);
//   4. K chunks: gather chunk c+1 into registers while the MFMAs consume chunk c;
//   5. W + delta is rounded once and stored.
//
// RMODE fixes how the contraction index k maps to (slot j, rank rr) and how B is
// gathered, so the K loop has no runtime branches:
//   0: r a power of two and a multiple of 8 (shifts; 16-byte B vectors)
//   1: r a multiple of 8 (division; 16-byte B vectors)
//   2: any other r (division; B element by element)
//   3: r a power of two and a multiple of KC: every chunk lies inside one slot, so the
//      slot, its coefficient and its base addresses are uniform per chunk
// LONG marks the long-contraction instantiations (k*r > 64: 128 x 128 tiles): they ask
// for two waves per SIMD (three or four in the lean form, NBUF = 1) and defer the gather masks
// (step 4); with RMODE 3 they use the scaled accumulators, otherwise the split fold.
#ifndef ADA_WAVES_PER_EU
#define ADA_WAVES_PER_EU 1
#endif
template <int KC, int RB, int CT, int WGN, int RMODE, bool LONG, int NBUF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LONG ? (NBUF == 1 ? (KC == 32 && RMODE == 3 ? 4 : 3) : 2) : ADA_WAVES_PER_EU, 8)))
merge_bf16_kernel(MergeParams p) {
  constexpr int WGM = 4 / WGN;
  constexpr int BM = 16 * RB * WGM, BN = 16 * CT * WGN;
  constexpr bool kAccScale = LONG && RMODE == 3;  // coefficients on the fp32 accumulators
  // lean form of a long contraction (one operand buffer): W is loaded for the last
  // chunk and the delta passes through LDS in two halves, so a workgroup takes 35-40 KB
  // and <= 168 VGPRs and three share a CU (four at 32-deep chunks on scaled
  // accumulators, which fit 128 VGPRs: 5-7% faster than three at rank 32)
  constexpr bool kLean = LONG && NBUF == 1;
  static_assert(!LONG || kLean, "long contractions run in the lean form");
  constexpr bool kSplit = !kAccScale;             // coefficients folded into B as a bf16 pair
  constexpr int NPL = kSplit ? 2 : 1;             // B planes per buffer
  constexpr int LDB = KC + 8;   // B plane row pitch (elements)
  // As row pitch: BN + 32 elements is 16 (mod 64) banks, so the 16 lanes of a
  // transposed read (4 k rows x 4 column chunks) touch 16 disjoint bank pairs; the
  // short-contraction tiles read A once per tile and keep the smaller pitch, whose
  // LDS footprint stays under the delta tile's
  constexpr int LDA = BN + (LONG ? 32 : 8);
  constexpr int NBV = BM * KC / 8;  // 16-byte B vectors per chunk
  constexpr int NAV = KC * BN / 8;  // 16-byte A vectors per chunk
  constexpr int B_VPT = (NBV + 255) / 256;
  constexpr int A_VPT = (NAV + 255) / 256;
  static_assert(WGM * WGN == 4 && CT % 2 == 0 && NBV % 64 == 0 && NAV % 64 == 0, "tile shape");
  static_assert(NBUF == 1 || NBUF == 2, "one or two operand buffers");
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;

  // LDS: the operand chunk buffers, and (after the last MFMA) the fp32 delta tile in
  // the same bytes
  constexpr int LDD = BN + 4;  // delta row pitch (floats): 16 rows of a 16-byte column write hit 64 banks
  constexpr int BPLANE = BM * LDB;
  constexpr int STAGE_BYTES = NBUF * (NPL * BPLANE + KC * LDA) * 2;
  constexpr int DELTA_BYTES = (kLean ? BM / 2 : BM) * LDD * 4;
  constexpr int SMEM = STAGE_BYTES > DELTA_BYTES ? STAGE_BYTES : DELTA_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  uint16_t (*Bs)[NPL * BPLANE] = reinterpret_cast<uint16_t (*)[NPL * BPLANE]>(smem);
  uint16_t (*As)[KC * LDA] = reinterpret_cast<uint16_t (*)[KC * LDA]>(smem + NBUF * NPL * BPLANE * 2);
  float* Ds = reinterpret_cast<float*>(smem);
  __shared__ int s_exp[kMaxSlots];
  __shared__ float s_coef[kMaxSlots];
  __shared__ float s_ratio[kAccScale ? kMaxSlots : 1];  // c_j / c_{j+1} in slot order
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int li = lane & 15;
  const int wy = wave / WGN, wx = wave % WGN;

  const TileRef T = find_tile(p, BM, BN);
  const ADA_GLOBAL unsigned char* __restrict__ src = as_global<unsigned char>(T.src);
  ADA_GLOBAL unsigned char* __restrict__ dst = as_global_mut<unsigned char>(T.dst);
  const ADA_GLOBAL unsigned char* __restrict__ gA = as_global<unsigned char>(T.a);
  const ADA_GLOBAL unsigned char* __restrict__ gB = as_global<unsigned char>(T.b);
  const ADA_GLOBAL uint16_t* __restrict__ gB16 = as_global<uint16_t>(T.b);

  // 1. selection (wave 0): lane j holds slot j of each selection (branch-free: lanes
  // past k re-read slot 0, which always exists, and are discarded below; exec-masked
  // loads would make the compiler wait for every outstanding load, the W tile
  // included, before the compaction)
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

  // 2. this thread's W vectors, row-major over the tile: vector v = tid + 256 u holds
  //    row v / (BN/8), columns 8 (v % (BN/8)) .. + 7, so one load instruction covers
  //    whole 256-byte row segments (the MFMA layout would give 16 rows x 64 bytes,
  //    which streams about 20% slower)
  constexpr int NV = BM * BN / 8 / 256;
  static_assert(NV * 2048 == BM * BN, "W split");
  //    Vector u's row is row_t + u (256 / (BN/8)) and its column col_t for every u, so
  //    the byte offsets are recomputed from these two where they are used rather than
  //    held in eight registers across the K loop (15 fewer VGPRs for 128 x 128 tiles;
  //    0.8% faster at k*r = 32, bit-identical).
  static_assert(256 % (BN / 8) == 0, "W rows per vector step");
  constexpr int kRowStep = 256 / (BN / 8);
  const int row_t = T.row0 + tid / (BN / 8);
  const int col_t = T.col0 + 8 * (tid % (BN / 8));
  const uint32_t woff0 = 2u * (uint32_t(row_t) * uint32_t(T.ld) + uint32_t(col_t));
  const uint32_t wstep = 2u * uint32_t(kRowStep) * uint32_t(T.ld);
  auto w_ok = [&](int u) { return row_t + kRowStep * u < T.d_out && col_t < T.d_in; };
  auto w_off = [&](int u) { return w_ok(u) ? woff0 + uint32_t(u) * wstep : 0u; };  // out of range: W[0][0..8)
  u32x4 wv[NV];
  if constexpr (!kLean) {
#pragma unroll
    for (int u = 0; u < NV; ++u) wv[u] = load16_stream(src, w_off(u));
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
    if constexpr (kAccScale) {
      // Scaled accumulators: order the slots by increasing |c| (equal magnitudes keep
      // their order) and record the ratio of each slot's coefficient to the next one's.
      // Every chunk here lies inside one slot of r >= KC terms, and one launch spans at
      // most kMaxKR terms, so there are at most kMaxKR / KC <= 64 slots: one per lane.
      // The magnitudes are compared as the integers of their bits, a total order (NaN
      // above infinity), so the ranks are a permutation whatever the gates hold.
      lds_wave_sync();
      const bool mine = lane < n;
      const int e_l = mine ? s_exp[lane] : 0;
      const float c_l = mine ? s_coef[lane] : 0.f;
      const uint32_t a_l = __float_as_uint(c_l) & 0x7fffffffu;
      int rank = 0;
      for (int i = 0; i < n; ++i) {
        const uint32_t a_i = __float_as_uint(s_coef[i]) & 0x7fffffffu;
        rank += (a_i < a_l || (a_i == a_l && i < lane)) ? 1 : 0;
      }
      lds_wave_sync();
      if (mine) {
        s_exp[rank] = e_l;
        s_coef[rank] = c_l;
      }
      lds_wave_sync();
      if (lane + 1 < n) s_ratio[lane] = s_coef[lane] / s_coef[lane + 1];
    }
  }
  __syncthreads();
  const int nslot = s_n;

  if (nslot == 0) {
    // Nothing selected: in place there is nothing to write; out of place, copy.
    if (T.src == T.dst) return;
    if constexpr (kLean) {
#pragma unroll
      for (int u = 0; u < NV; ++u) wv[u] = load16_stream(src, w_off(u));
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (w_ok(u)) store16_stream(dst, w_off(u), wv[u]);
    return;
  }

  const int r = p.r;
  const int r_shift = p.r_shift;
  const int kr = nslot * r;
  const int nchunks = (kr + KC - 1) / KC;
  constexpr bool rvec = RMODE != 2;
  // contraction index k -> (slot j, rank rr)
  auto split = [&](int k, int& j, int& rr) {
    if constexpr (RMODE == 0) {
      j = k >> r_shift;
      rr = k & (r - 1);
    } else {
      j = k / r;
      rr = k - j * r;
    }
  };

  // ---- K-chunk gathers: global -> registers (stage_load), registers -> LDS (stage_store).
  // Branch-free: out-of-range slots, rows or columns re-read an in-range vector, which
  // is replaced by zeros when stored to LDS (RMODE 3 has no out-of-range slots and
  // keeps the re-read rows and columns: they only reach outputs that are not stored).
  // Vector v of a chunk: B row v / (KC/8), k 8 (v % (KC/8));
  // A k row v / (BN/8), columns 8 (v % (BN/8)).  Threads past the vector count (whole
  // waves, as the counts are multiples of 64) skip.
  u32x4 sb[B_VPT];
  u32x4 sbl[B_VPT];  // RMODE 2: the lo plane, split at the load
  float sc[B_VPT];
  u32x4 sa[A_VPT];
  // Long contractions apply the in-range masks in stage_store: applied at the load,
  // the AND makes the wave wait for the prefetched chunk before the MFMAs on the
  // current one.  Short ones (at most one prefetch) mask at the load, which keeps
  // their registers lower.
  constexpr bool kDefer = LONG;
  uint32_t sbm[B_VPT], sam[A_VPT];

  // RMODE 3: per-thread parts of the gather offsets, fixed across chunks
  uint32_t b_off3[B_VPT], a_off3[A_VPT];
  if constexpr (RMODE == 3) {
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
      const int v = tid + 256 * i;
      const int grow = T.row0 + v / (KC / 8);
      b_off3[i] = 2u * (uint32_t(grow < T.d_out ? grow : 0) * uint32_t(r) + 8u * uint32_t(v % (KC / 8)));
    }
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
      const int v = tid + 256 * i;
      const int gcol = T.col0 + 8 * (v % (BN / 8));
      a_off3[i] = 2u * (uint32_t(v / (BN / 8)) * uint32_t(T.d_in) + uint32_t(gcol < T.d_in ? gcol : 0));
    }
  }

  auto stage_load = [&](int k0) {
    if constexpr (RMODE == 3) {
      const int j = k0 >> r_shift;  // < nslot: the chunks tile the contraction exactly
      const int rr0 = k0 & (r - 1);
      const int e = __builtin_amdgcn_readfirstlane(s_exp[j]);
      const float c = kSplit ? s_coef[j] : 1.f;
      const ADA_GLOBAL unsigned char* bj = gB + 2u * (uint32_t(e) * uint32_t(T.d_out) * uint32_t(r) + uint32_t(rr0));
      const ADA_GLOBAL unsigned char* aj = gA + 2u * ((uint32_t(e) * uint32_t(r) + uint32_t(rr0)) * uint32_t(T.d_in));
#pragma unroll
      for (int i = 0; i < B_VPT; ++i) {
        if (NBV % 256 != 0 && tid + 256 * i >= NBV) break;
        const u32x4 val = load16(bj, b_off3[i]);
        sb[i] = val;
        sc[i] = c;
      }
#pragma unroll
      for (int i = 0; i < A_VPT; ++i) {
        if (NAV % 256 != 0 && tid + 256 * i >= NAV) break;
        const u32x4 val = load16(aj, a_off3[i]);
        sa[i] = val;
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
      const int v = tid + 256 * i;
      if (NBV % 256 != 0 && v >= NBV) break;
      const int row = v / (KC / 8);
      const int kv = v % (KC / 8);
      const int grow = T.row0 + row;
      if constexpr (rvec) {
        int j, rr;
        split(k0 + 8 * kv, j, rr);
        const bool in = j < nslot && grow < T.d_out;
        const int js = in ? j : 0;
        const u32x4 val = load16(
            gB, 2u * ((uint32_t(s_exp[js]) * uint32_t(T.d_out) + uint32_t(in ? grow : 0)) * uint32_t(r) +
                      uint32_t(in ? rr : 0)));
        // a mask, not a select: a select of a load lets the compiler sink the load into
        // an exec-masked block of its own
        sbm[i] = 0u - uint32_t(in);
        sb[i] = kDefer ? val : (val & (u32x4)sbm[i]);
        sc[i] = s_coef[js];
      } else {
        // rank not a multiple of 8: element by element, the coefficient applied and
        // the product split into its two bf16 planes here
        uint32_t wh[4] = {0, 0, 0, 0}, wl[4] = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          int j, rr;
          split(k0 + 8 * kv + t, j, rr);
          float b = 0.f, c = 0.f;
          if (j < nslot && grow < T.d_out) {
            b = __uint_as_float(uint32_t(gB16[(int64_t(s_exp[j]) * T.d_out + grow) * r + rr]) << 16);
            c = s_coef[j];
          }
          const uint32_t hb = pack_bf16x2(b * c, 0.f) & 0xffffu;
          const uint32_t lb = pack_bf16x2(fmaf(b, c, -bf16_lo(hb)), 0.f) & 0xffffu;
          wh[t >> 1] |= hb << (16 * (t & 1));
          wl[t >> 1] |= lb << (16 * (t & 1));
        }
        sb[i] = (u32x4){wh[0], wh[1], wh[2], wh[3]};
        sbl[i] = (u32x4){wl[0], wl[1], wl[2], wl[3]};
        sbm[i] = ~0u;
        sc[i] = 1.f;
      }
    }
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
      const int v = tid + 256 * i;
      if (NAV % 256 != 0 && v >= NAV) break;
      const int kl = v / (BN / 8);
      const int cv = v % (BN / 8);
      int j, rr;
      split(k0 + kl, j, rr);
      const int gcol = T.col0 + 8 * cv;
      const bool in = j < nslot && gcol < T.d_in;
      const u32x4 val = load16(
          gA, 2u * ((uint32_t(s_exp[in ? j : 0]) * uint32_t(r) + uint32_t(in ? rr : 0)) * uint32_t(T.d_in) +
                    uint32_t(in ? gcol : 0)));
      sam[i] = 0u - uint32_t(in);
      sa[i] = kDefer ? val : (val & (u32x4)sam[i]);
    }
  };

  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
      const int v = tid + 256 * i;
      if (NBV % 256 != 0 && v >= NBV) break;
      const int row = v / (KC / 8);
      const int kv = v % (KC / 8);
      // (RMODE 3 has nothing to mask: an out-of-range row or column re-read row 0 or
      // column 0, whose products reach only output rows or columns never stored;
      // short tiles were masked at the load)
      const u32x4 v8 = (RMODE == 3 || !kDefer) ? sb[i] : (sb[i] & (u32x4)sbm[i]);
      u32x4* bh = reinterpret_cast<u32x4*>(&Bs[buf][row * LDB + 8 * kv]);
      if constexpr (kAccScale) {
        *bh = v8;
      } else if constexpr (rvec) {
        u32x4 hi, lo;
        split_bf16x8(v8, sc[i], hi, lo);
        bh[0] = hi;
        *reinterpret_cast<u32x4*>(&Bs[buf][BPLANE + row * LDB + 8 * kv]) = lo;
      } else {
        bh[0] = v8;
        *reinterpret_cast<u32x4*>(&Bs[buf][BPLANE + row * LDB + 8 * kv]) = sbl[i];
      }
    }
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
      const int v = tid + 256 * i;
      if (NAV % 256 != 0 && v >= NAV) break;
      const int kl = v / (BN / 8);
      const int cv = v % (BN / 8);
      *reinterpret_cast<u32x4*>(&As[buf][kl * LDA + 8 * cv]) =
          (RMODE == 3 || !kDefer) ? sa[i] : (sa[i] & (u32x4)sam[i]);
    }
  };

  // LDS element offsets of this lane's fragments inside a chunk buffer
  //   B: row 16 RB wy + 16 rb + li, k 8 q (+ 32 ks)
  //   A (transposed read): k row 8 q + (li / 4) (+ 4 for the upper half, + 32 ks),
  //      columns 16 CT wx + 32 (ct / 2) + 4 (ct % 2) + 8 (li % 4) .. + 3
  int boff[RB], aoff[CT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) boff[rb] = (16 * RB * wy + 16 * rb + li) * LDB + 8 * q;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    aoff[ct] = (8 * q + (li >> 2)) * LDA + 16 * CT * wx + 32 * (ct >> 1) + 4 * (ct & 1) + 8 * (li & 3);

  f32x4 acc[RB][CT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rb][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // 4. chunk 0, then the pipelined K loop (one barrier per chunk: chunk c+1 is
  // written to the other buffer, which every wave finished reading at the previous
  // barrier).  With the split fold every B fragment is multiplied twice, hi plane
  // first for all blocks, then the lo plane, so dependent MFMAs are RB*CT apart.
  auto mfma_chunk = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KC / 32; ++ks) {
      bf16x8_t af[CT], bfr[RB];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)((lds_u16*)As[buf] + aoff[ct] + 32 * ks * LDA));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)((lds_u16*)As[buf] + aoff[ct] + (32 * ks + 4) * LDA));
        const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        af[ct] = __builtin_bit_cast(bf16x8_t, both);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        bfr[rb] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][boff[rb] + 32 * ks]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ct], bfr[rb], acc[rb][ct], 0, 0, 0);
      if constexpr (kSplit) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          bfr[rb] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][BPLANE + boff[rb] + 32 * ks]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ct], bfr[rb], acc[rb][ct], 0, 0, 0);
      }
    }
  };
  // Scaled accumulators: entering chunk c + 1, which starts slot j + 1 when
  // (c + 1) KC is a multiple of r, multiply by c_j / c_{j+1}.
  auto rescale = [&](int c) {
    if constexpr (kAccScale) {
      const int k1 = (c + 1) * KC;
      if ((k1 & (r - 1)) == 0) {
        const float rho = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_ratio[(k1 >> r_shift) - 1])));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            acc[rb][ct][0] *= rho;
            acc[rb][ct][1] *= rho;
            acc[rb][ct][2] *= rho;
            acc[rb][ct][3] *= rho;
          }
      }
    }
  };
  stage_load(0);
  stage_store(0);
  __syncthreads();
  if constexpr (kLean) {
    // 4'. one operand buffer: chunk c+1 waits in registers until every wave has read
    // chunk c (a second barrier per chunk, for half the operand LDS).  The last chunk
    // is peeled off the loop, so every gather issued in the loop body is consumed in
    // the same body (a load that could still be pending at the loop exit would make the
    // compiler wait on it in the epilogue, and with it on the epilogue's stores), and
    // the gathers are pinned ahead of the MFMAs (the scheduler would sink them to the
    // end of the chunk to shorten their live ranges).
    for (int c = 0; c + 1 < nchunks; ++c) {
      stage_load((c + 1) * KC);
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk(0);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      stage_store(0);
      rescale(c);
      __syncthreads();
    }
    // W for the epilogue goes out now, into the registers the operand staging no
    // longer needs; its HBM latency overlaps the last chunk here and the other
    // workgroups of the CU.  Its offsets, and the delta's, are recomputed from a
    // thread index the compiler cannot see through (the empty asm): hoisted to the
    // kernel's start they would stay live across the K loop and spill.
    int tid_l = tid;
    asm volatile("" : "+v"(tid_l));
    const int row_l = T.row0 + tid_l / (BN / 8);
    const int col_l = T.col0 + 8 * (tid_l % (BN / 8));
    const uint32_t woff_l = 2u * (uint32_t(row_l) * uint32_t(T.ld) + uint32_t(col_l));
    auto wl_ok = [&](int u) { return row_l + kRowStep * u < T.d_out && col_l < T.d_in; };
    auto wl_off = [&](int u) { return wl_ok(u) ? woff_l + uint32_t(u) * wstep : 0u; };
#pragma unroll
    for (int u = 0; u < NV; ++u) wv[u] = load16_stream(src, wl_off(u));
    __builtin_amdgcn_sched_barrier(0);
    mfma_chunk(0);

    // 5'. the delta in two halves of BM / 2 rows (WGM = 2 row groups of waves): the
    // waves of group h write theirs, then every thread finishes its W vectors of those
    // rows (vectors u < NV / 2 lie in the first half)
    static_assert(WGM == 2 && NV % 2 == 0 && (NV / 2) * kRowStep == BM / 2, "two row halves");
    const float cl = kAccScale ? s_coef[nslot - 1] : 1.f;
    const int q_l = (tid_l & 63) >> 4, li_l = tid_l & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // every wave is done reading the operand chunk, then the first half
      if (wy == h) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int row = 16 * RB * wy + 16 * rb + li_l - h * (BM / 2);
            const int col = 16 * CT * wx + 32 * (ct >> 1) + 8 * q_l + 4 * (ct & 1);
            *reinterpret_cast<f32x4*>(&Ds[row * LDD + col]) = acc[rb][ct];
          }
      }
      __syncthreads();
#pragma unroll
      for (int u = h * (NV / 2); u < (h + 1) * (NV / 2); ++u) {
        if (!wl_ok(u)) continue;
        const int v = tid_l + 256 * u;
        const float* d = &Ds[(v / (BN / 8) - h * (BM / 2)) * LDD + 8 * (v % (BN / 8))];
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(d);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(d + 4);
        const u32x4 w = wv[u];
        u32x4 o;
        if constexpr (kAccScale) {
          o.x = pack_bf16x2(fmaf(d0[0], cl, bf16_lo(w.x)), fmaf(d0[1], cl, bf16_hi(w.x)));
          o.y = pack_bf16x2(fmaf(d0[2], cl, bf16_lo(w.y)), fmaf(d0[3], cl, bf16_hi(w.y)));
          o.z = pack_bf16x2(fmaf(d1[0], cl, bf16_lo(w.z)), fmaf(d1[1], cl, bf16_hi(w.z)));
          o.w = pack_bf16x2(fmaf(d1[2], cl, bf16_lo(w.w)), fmaf(d1[3], cl, bf16_hi(w.w)));
        } else {
          o.x = pack_bf16x2(bf16_lo(w.x) + d0[0], bf16_hi(w.x) + d0[1]);
          o.y = pack_bf16x2(bf16_lo(w.y) + d0[2], bf16_hi(w.y) + d0[3]);
          o.z = pack_bf16x2(bf16_lo(w.z) + d1[0], bf16_hi(w.z) + d1[1]);
          o.w = pack_bf16x2(bf16_lo(w.w) + d1[2], bf16_hi(w.w) + d1[3]);
        }
        store16_stream(dst, wl_off(u), o);
      }
    }
    return;
  }
  if constexpr (NBUF == 1) {
    // the launch's contraction fits one chunk (the host picks this form only then)
    mfma_chunk(0);
  } else {
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < nchunks;
      if (more) stage_load((c + 1) * KC);
      mfma_chunk(buf);
      if (more) {
        stage_store(buf ^ 1);
        __syncthreads();
      }
    }
  }

  // 5. delta through LDS into the row-major layout of the W vectors: lane (q, i) of
  //    block (rb, ct) holds 4 adjacent columns of one row (a 16-byte write); then
  //    W + delta is rounded once and stored (short contractions: the split fold has
  //    already applied the coefficients)
  __syncthreads();  // every wave is done reading the operand chunks the delta overwrites
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int row = 16 * RB * wy + 16 * rb + li;
      const int col = 16 * CT * wx + 32 * (ct >> 1) + 8 * q + 4 * (ct & 1);
      *reinterpret_cast<f32x4*>(&Ds[row * LDD + col]) = acc[rb][ct];
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (!w_ok(u)) continue;
    const int v = tid + 256 * u;
    const float* d = &Ds[(v / (BN / 8)) * LDD + 8 * (v % (BN / 8))];
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(d);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(d + 4);
    const u32x4 w = wv[u];
    u32x4 o;
    o.x = pack_bf16x2(bf16_lo(w.x) + d0[0], bf16_hi(w.x) + d0[1]);
    o.y = pack_bf16x2(bf16_lo(w.y) + d0[2], bf16_hi(w.y) + d0[3]);
    o.z = pack_bf16x2(bf16_lo(w.z) + d1[0], bf16_hi(w.z) + d1[1]);
    o.w = pack_bf16x2(bf16_lo(w.w) + d1[2], bf16_hi(w.w) + d1[3]);
    store16_stream(dst, w_off(u), o);
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

template <int KC, class S, bool LONG, int NBUF>
void launch_bf16(const MergeParams& p, dim3 grid, dim3 block, hipStream_t s) {
  if (p.r_shift >= 0 && p.r % KC == 0)
    hipLaunchKernelGGL((merge_bf16_kernel<KC, S::rb, S::ct, S::wgn, 3, LONG, NBUF>), grid, block, 0, s, p);
  else if (p.r_shift >= 0 && (p.r & 7) == 0)
    hipLaunchKernelGGL((merge_bf16_kernel<KC, S::rb, S::ct, S::wgn, 0, LONG, NBUF>), grid, block, 0, s, p);
  else if ((p.r & 7) == 0)
    hipLaunchKernelGGL((merge_bf16_kernel<KC, S::rb, S::ct, S::wgn, 1, LONG, NBUF>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((merge_bf16_kernel<KC, S::rb, S::ct, S::wgn, 2, LONG, NBUF>), grid, block, 0, s, p);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int dtype, int kr_max, hipStream_t s) {
  if (p.total_tiles <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.total_tiles)), block(256);
  if (dtype == 1) {
    // the caller built p's work table for the tile class of kr_max
    // short contractions loop over 32-deep chunks (a 64-deep chunk costs a wave per
    // SIMD in registers: the fused switch at k*r = 64 ran 30% slower with it)
    // k*r <= 32 is a single chunk (one operand buffer); long contractions run in the lean
    // form (one operand buffer, three workgroups per CU): 64-deep chunks, one slot each,
    // on scaled accumulators when the rank is a power-of-two multiple of 64, else
    // 32-deep chunks (scaled accumulators again at rank 32; otherwise the split fold)
    switch (bf16_tile_class(kr_max)) {
      case 0: launch_bf16<32, NarrowTile, false, 1>(p, grid, block, s); break;
      case 1: launch_bf16<32, ShortTile, false, 2>(p, grid, block, s); break;
      default:
        if (p.r_shift >= 0 && p.r % 64 == 0)
          hipLaunchKernelGGL((merge_bf16_kernel<64, LongTile::rb, LongTile::ct, LongTile::wgn, 3, true, 1>), grid,
                             block, 0, s, p);
        else
          launch_bf16<32, LongTile, true, 1>(p, grid, block, s);
        break;
    }
  } else {
    hipLaunchKernelGGL(merge_f32_kernel<32>, grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ada
