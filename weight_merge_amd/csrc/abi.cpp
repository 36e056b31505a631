// C ABI of libadafuse: argument checks (host only, before any HIP call), the
// per-model work table, and kernel launches.  The operations themselves are
// documented in include/adafuse.h and in the kernel sources.
#include "adafuse.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "launch.h"

#ifndef ADA_LONG_TILE_GROUP
#define ADA_LONG_TILE_GROUP 8
#endif

namespace {

constexpr uint64_t kModelMagic = 0x6164614675736521ull;
constexpr int64_t kMaxDim = int64_t(1) << 22;     // rows or columns of one projection
constexpr int64_t kMaxTiles = (int64_t(1) << 24) - 1;  // one grid: tiles * 256 threads < 2^32
constexpr int64_t kMaxElems = int64_t(1) << 31;        // per W matrix and per adapter bank

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dim_ok(int64_t d) { return d > 0 && d % 8 == 0 && d <= kMaxDim; }
bool dtype_ok(int32_t dt) { return dt == ADA_F32 || dt == ADA_BF16; }

}  // namespace

// One tile decomposition of the registered projections: the work table (one entry
// per projection plus a sentinel) and the tile -> entry lookup buckets.
struct TileTable {
  const ada::MergeEntry* entries;
  const int32_t* lut;
  int64_t total_tiles;
  int32_t lut_shift;
  int32_t tile_rows;
};

struct ada_model_s {
  uint64_t magic;
  int32_t dtype;
  int32_t E;
  int32_t r;
  int32_t n_proj;
  int32_t device;
  void* dev;          // one allocation holding every table
  std::vector<unsigned char> host;  // the tables' host image, the source of the asynchronous upload
  hipEvent_t uploaded;              // recorded on the creation stream after the upload
  TileTable tab[ada::kTileClasses];  // bf16: one per contraction class (32 x 256, 64 x 128, 128 x 128); fp32: all 64 x 64
};

namespace {

bool model_ok(const ada_model_s* m) { return m != nullptr && m->magic == kModelMagic; }

int launch_merge_common(ada_model m, const ada::Selection& s0, const ada::Selection& s1,
                        int src_is_out, int kr_max, void* stream) {
  // the work table lives on the device that was current at ada_model_create
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return ADA_EHIP;
  if (device != m->device) return ADA_EINVAL;
  const int cls = m->dtype == ADA_BF16 ? ada::bf16_tile_class(kr_max) : 0;
  const TileTable& t = m->tab[cls];
  ada::MergeParams p{};
  p.table = t.entries;
  p.lut = t.lut;
  p.total_tiles = t.total_tiles;
  p.lut_shift = t.lut_shift;
  p.n_entries = m->n_proj;
  p.sel[0] = s0;
  p.sel[1] = s1;
  p.E = m->E;
  p.r = m->r;
  p.r_shift = (m->r & (m->r - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(m->r)) : -1;
  p.src_is_out = src_is_out;
  p.xcd_remap = 1;
  // row bands walked in groups down each column block, so consecutive tiles share A_cat
  // columns and B_cat rows in L2: a gain once k*r > 32 (the 7B fused switch at k*r = 64
  // runs 2.5% faster), a small loss on 32 x 256 tiles, which walk plain row-major order
  p.tile_group = cls == 0 ? 1 : ADA_LONG_TILE_GROUP;
  const hipError_t e = ada::launch_merge(p, m->dtype, kr_max, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

// Host image of one tile decomposition.
struct HostTable {
  std::vector<ada::MergeEntry> ent;
  std::vector<int32_t> lut;
  int64_t total = 0;
  int32_t shift = 0;
  int32_t tile_rows = 0;
};

int build_table(const ada_proj* projs, int32_t n_proj, int tile_r, int tile_c, HostTable& h) {
  h.tile_rows = tile_r;
  h.ent.assign(static_cast<size_t>(n_proj) + 1, ada::MergeEntry{});
  int64_t min_tiles = INT64_MAX;
  for (int32_t i = 0; i < n_proj; ++i) {
    const ada_proj& p = projs[i];
    const int64_t tm = (p.d_out + tile_r - 1) / tile_r, tn = (p.d_in + tile_c - 1) / tile_c;
    ada::MergeEntry& e = h.ent[i];
    e.w = p.w;
    e.w_out = p.w_out != nullptr ? p.w_out : p.w;
    e.a = p.a;
    e.b = p.b;
    e.ld = p.ld_w;
    e.d_out = p.d_out;
    e.d_in = p.d_in;
    e.tiles_n = static_cast<int32_t>(tn);
    e.tiles_m = static_cast<int32_t>(tm);
    e.tile_base = h.total;
    h.total += tm * tn;
    min_tiles = std::min(min_tiles, tm * tn);
    if (h.total > kMaxTiles) return ADA_ESHAPE;
  }
  h.ent[n_proj].tile_base = h.total;  // sentinel
  // bucket size 2^shift <= smallest entry, so a bucket overlaps at most two entries
  while ((int64_t(2) << h.shift) <= min_tiles && h.shift < 30) ++h.shift;
  const int64_t n_buckets = ((h.total - 1) >> h.shift) + 1;
  h.lut.resize(static_cast<size_t>(n_buckets));
  int32_t i = 0;
  for (int64_t b = 0; b < n_buckets; ++b) {
    const int64_t t = b << h.shift;
    while (t >= h.ent[i + 1].tile_base) ++i;
    h.lut[b] = i;
  }
  return ADA_OK;
}

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

int check_selection(const ada_model_s* m, const int32_t* idx, const float* gate, int32_t k) {
  if (idx == nullptr || gate == nullptr) return ADA_EINVAL;
  if (!aligned4(idx) || !aligned4(gate)) return ADA_EALIGN;
  if (k < 1 || k > m->E) return ADA_ESHAPE;
  return ADA_OK;
}

// Checks and launch parameters of one layer of the unmerged routed path (everything but
// the fp32 intermediates' address); ws_bytes is the space those intermediates need.
int prepare_lora_layer(const ada_lora_proj* projs, int32_t n_proj, int32_t E, int32_t r, const int32_t* idx,
                       const float* gate, int32_t k, float scale, int32_t dtype, ada::LoraLayerParams& p,
                       int64_t& dot_rows, int64_t& out_rows, int64_t& ws_bytes) {
  if (projs == nullptr || idx == nullptr || gate == nullptr) return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (!aligned4(idx) || !aligned4(gate)) return ADA_EALIGN;
  if (n_proj < 1 || n_proj > ada::kMaxLayerProj) return ADA_ESHAPE;
  if (E < 1 || E > 64 || r < 1 || k < 1 || k > E || int64_t(k) * r > ada::kMaxKR) return ADA_ESHAPE;
  const int esz = dtype == ADA_BF16 ? 2 : 4;
  int64_t ws = 0;
  dot_rows = out_rows = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    const ada_lora_proj& q = projs[i];
    if (q.w == nullptr || q.a == nullptr || q.b == nullptr || q.x == nullptr || q.y == nullptr) return ADA_EINVAL;
    if (!aligned16(q.w) || !aligned16(q.a) || !aligned16(q.b) || !aligned16(q.x) || !aligned16(q.y))
      return ADA_EALIGN;
    if (!dim_ok(q.d_out) || !dim_ok(q.d_in) || q.ld_w < q.d_in || q.ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
    if ((q.ld_w * esz) % 16 != 0) return ADA_EALIGN;
    ada::LoraLayerProj& P = p.proj[i];
    P.w = q.w;
    P.a = q.a;
    P.b = q.b;
    P.x = q.x;
    P.y = q.y;
    P.ld = q.ld_w;
    P.d_out = q.d_out;
    P.d_in = q.d_in;
    P.dot_row0 = static_cast<int32_t>(dot_rows);
    P.out_row0 = static_cast<int32_t>(out_rows);
    P.ws_off = ws;
    dot_rows += q.d_out + int64_t(k) * r;
    out_rows += q.d_out;
    ws = (ws + q.d_out + int64_t(k) * r + 3) & ~int64_t(3);  // keep every block 16-byte aligned
  }
  if (dot_rows >= (int64_t(1) << 30)) return ADA_ESHAPE;
  p.n = n_proj;
  p.E = E;
  p.r = r;
  p.k = k;
  p.idx = idx;
  p.gate = gate;
  p.scale = scale;
  p.nb = 1;
  ws_bytes = ws * 4;
  return ADA_OK;
}

}  // namespace

extern "C" {

const char* ada_status_string(int status) {
  switch (status) {
    case ADA_OK: return "ok";
    case ADA_EINVAL: return "invalid argument (null pointer, bad handle or flag)";
    case ADA_ESHAPE: return "unsupported size (dimensions must be positive multiples of 8; 1<=k<=E<=64; k*r<=512)";
    case ADA_EDTYPE: return "unsupported or mismatched dtype";
    case ADA_EALIGN: return "pointer or row stride not 16-byte aligned";
    case ADA_EHIP: return "HIP runtime call or kernel launch failed";
    case ADA_ENOMEM: return "device allocation of the work table failed";
    default: return "unknown status";
  }
}

int ada_model_create(const ada_proj* projs, int32_t n_proj, int32_t E, int32_t r, int32_t dtype,
                     void* stream, ada_model* out) {
  if (out == nullptr || projs == nullptr) return ADA_EINVAL;
  *out = nullptr;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (n_proj < 1 || n_proj > (1 << 20)) return ADA_ESHAPE;
  if (E < 1 || E > 64 || r < 1 || r > ada::kMaxKR) return ADA_ESHAPE;
  const int esz = dtype == ADA_BF16 ? 2 : 4;
  for (int32_t i = 0; i < n_proj; ++i) {
    const ada_proj& p = projs[i];
    if (p.w == nullptr || p.a == nullptr || p.b == nullptr) return ADA_EINVAL;
    if (!aligned16(p.w) || !aligned16(p.a) || !aligned16(p.b) ||
        (p.w_out != nullptr && !aligned16(p.w_out)))
      return ADA_EALIGN;
    if (!dim_ok(p.d_out) || !dim_ok(p.d_in)) return ADA_ESHAPE;
    if (p.ld_w < p.d_in || p.ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
    if ((p.ld_w * esz) % 16 != 0) return ADA_EALIGN;
    // the merge kernels address W and the adapter banks with 32-bit element offsets
    if (int64_t(p.d_out) * p.ld_w >= kMaxElems || int64_t(E) * r * p.d_in >= kMaxElems ||
        int64_t(E) * r * p.d_out >= kMaxElems)
      return ADA_ESHAPE;
  }
  HostTable ht[ada::kTileClasses];
  for (int t = 0; t < ada::kTileClasses; ++t) {
    const int tile_r = dtype == ADA_BF16 ? ada::bf16_tile_rows(t) : ada::kTileF32;
    const int tile_c = dtype == ADA_BF16 ? ada::bf16_tile_cols(t) : ada::kTileF32;
    if (int st = build_table(projs, n_proj, tile_r, tile_c, ht[t]); st != ADA_OK) return st;
  }

  size_t off[2 * ada::kTileClasses], bytes = 0;
  for (int t = 0; t < ada::kTileClasses; ++t) {
    off[2 * t] = bytes;
    bytes = align16(bytes + ht[t].ent.size() * sizeof(ada::MergeEntry));
    off[2 * t + 1] = bytes;
    bytes = align16(bytes + ht[t].lut.size() * sizeof(int32_t));
  }
  std::vector<unsigned char> host(bytes, 0);
  for (int t = 0; t < ada::kTileClasses; ++t) {
    std::copy_n(reinterpret_cast<const unsigned char*>(ht[t].ent.data()),
                ht[t].ent.size() * sizeof(ada::MergeEntry), host.data() + off[2 * t]);
    std::copy_n(reinterpret_cast<const unsigned char*>(ht[t].lut.data()), ht[t].lut.size() * sizeof(int32_t),
                host.data() + off[2 * t + 1]);
  }
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return ADA_EHIP;
  ada_model_s* m = new (std::nothrow) ada_model_s{};
  if (m == nullptr) return ADA_ENOMEM;
  m->host = std::move(host);
  void* dev = nullptr;
  if (hipMalloc(&dev, bytes) != hipSuccess) {
    delete m;
    return ADA_ENOMEM;
  }
  // the upload is ordered on the caller's stream; the host image it reads lives in the
  // model until destroy, which first waits for this event
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipEventCreateWithFlags(&m->uploaded, hipEventDisableTiming) != hipSuccess) {
    (void)hipFree(dev);
    delete m;
    return ADA_EHIP;
  }
  if (hipMemcpyAsync(dev, m->host.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(m->uploaded, s) != hipSuccess) {
    (void)hipStreamSynchronize(s);
    (void)hipEventDestroy(m->uploaded);
    (void)hipFree(dev);
    delete m;
    return ADA_EHIP;
  }
  m->magic = kModelMagic;
  m->dtype = dtype;
  m->E = E;
  m->r = r;
  m->n_proj = n_proj;
  m->device = device;
  m->dev = dev;
  for (int t = 0; t < ada::kTileClasses; ++t) {
    unsigned char* base = static_cast<unsigned char*>(dev);
    m->tab[t].entries = reinterpret_cast<const ada::MergeEntry*>(base + off[2 * t]);
    m->tab[t].lut = reinterpret_cast<const int32_t*>(base + off[2 * t + 1]);
    m->tab[t].total_tiles = ht[t].total;
    m->tab[t].lut_shift = ht[t].shift;
    m->tab[t].tile_rows = ht[t].tile_rows;
  }
  *out = m;
  return ADA_OK;
}

void ada_model_destroy(ada_model m) {
  if (!model_ok(m)) return;
  m->magic = 0;
  (void)hipEventSynchronize(m->uploaded);  // the upload reads m->host
  (void)hipEventDestroy(m->uploaded);
  (void)hipFree(m->dev);
  delete m;
}

int64_t ada_model_tiles(ada_model m) {
  if (!model_ok(m)) return ADA_EINVAL;
  return m->tab[0].total_tiles;
}

int64_t ada_model_device_bytes(ada_model m) {
  if (!model_ok(m)) return ADA_EINVAL;
  return static_cast<int64_t>(m->host.size());
}

int ada_pregate(const void* h, const void* router, int32_t d, int32_t E, int32_t k, int32_t dtype,
                int32_t renorm, int32_t* idx_out, float* gate_out, void* stream) {
  if (h == nullptr || router == nullptr || idx_out == nullptr || gate_out == nullptr) return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (renorm != 0 && renorm != 1) return ADA_EINVAL;
  if (!aligned16(h) || !aligned16(router) || !aligned4(idx_out) || !aligned4(gate_out)) return ADA_EALIGN;
  if (!dim_ok(d) || E < 1 || E > 64 || k < 1 || k > E) return ADA_ESHAPE;
  const hipError_t e = ada::launch_pregate(h, router, d, E, k, dtype, renorm, idx_out, gate_out,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

int ada_merge(ada_model m, const int32_t* idx, const float* gate, int32_t k, float scale,
              void* stream) {
  if (!model_ok(m)) return ADA_EINVAL;
  if (int s = check_selection(m, idx, gate, k); s != ADA_OK) return s;
  if (int64_t(k) * m->r > ada::kMaxKR) return ADA_ESHAPE;
  const ada::Selection s0{idx, gate, k, scale};
  const ada::Selection s1{idx, gate, 0, 0.f};  // empty; pointers valid for branch-free reads
  return launch_merge_common(m, s0, s1, 0, k * m->r, stream);
}

int ada_unmerge(ada_model m, const int32_t* idx, const float* gate, int32_t k, float scale,
                void* stream) {
  if (!model_ok(m)) return ADA_EINVAL;
  if (int s = check_selection(m, idx, gate, k); s != ADA_OK) return s;
  if (int64_t(k) * m->r > ada::kMaxKR) return ADA_ESHAPE;
  const ada::Selection s0{idx, gate, k, -scale};
  const ada::Selection s1{idx, gate, 0, 0.f};  // empty; pointers valid for branch-free reads
  return launch_merge_common(m, s0, s1, 1, k * m->r, stream);
}

int ada_switch(ada_model m, const int32_t* idx_prev, const float* gate_prev, int32_t k_prev,
               const int32_t* idx_cur, const float* gate_cur, int32_t k_cur, float scale,
               void* stream) {
  if (!model_ok(m)) return ADA_EINVAL;
  if (int s = check_selection(m, idx_prev, gate_prev, k_prev); s != ADA_OK) return s;
  if (int s = check_selection(m, idx_cur, gate_cur, k_cur); s != ADA_OK) return s;
  if (int64_t(k_prev + k_cur) * m->r > ada::kMaxKR) return ADA_ESHAPE;
  const ada::Selection s0{idx_prev, gate_prev, k_prev, -scale};
  const ada::Selection s1{idx_cur, gate_cur, k_cur, scale};
  return launch_merge_common(m, s0, s1, 1, (k_prev + k_cur) * m->r, stream);
}

int ada_decode_gemv(const void* w, int32_t d_out, int32_t d_in, int64_t ld_w, const void* x,
                    void* y, int32_t dtype, void* stream) {
  if (w == nullptr || x == nullptr || y == nullptr) return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return ADA_EALIGN;
  if (!dim_ok(d_out) || !dim_ok(d_in) || ld_w < d_in || ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
  if ((ld_w * (dtype == ADA_BF16 ? 2 : 4)) % 16 != 0) return ADA_EALIGN;
  const hipError_t e = ada::launch_gemv(w, d_out, d_in, ld_w, x, y, nullptr, dtype,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

int ada_decode_gemv_layer(const ada_gemv_proj* projs, int32_t n_proj, int32_t dtype, void* stream) {
  if (projs == nullptr) return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (n_proj < 1 || n_proj > ada::kMaxLayerProj) return ADA_ESHAPE;
  const int esz = dtype == ADA_BF16 ? 2 : 4;
  ada::GemvLayerParams p{};
  int64_t rows = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    const ada_gemv_proj& q = projs[i];
    if (q.w == nullptr || q.x == nullptr || q.y == nullptr) return ADA_EINVAL;
    if (!aligned16(q.w) || !aligned16(q.x) || !aligned16(q.y)) return ADA_EALIGN;
    if (!dim_ok(q.d_out) || !dim_ok(q.d_in) || q.ld_w < q.d_in || q.ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
    if ((q.ld_w * esz) % 16 != 0) return ADA_EALIGN;
    ada::GemvLayerProj& P = p.proj[i];
    P.w = q.w;
    P.x = q.x;
    P.y = q.y;
    P.ld = q.ld_w;
    P.d_out = q.d_out;
    P.d_in = q.d_in;
    P.row0 = static_cast<int32_t>(rows);
    rows += q.d_out;
  }
  if (rows >= (int64_t(1) << 30)) return ADA_ESHAPE;
  p.n = n_proj;
  const hipError_t e = ada::launch_gemv_layer(p, static_cast<int>(rows), dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

int ada_lora_apply(const void* w, int32_t d_out, int32_t d_in, int64_t ld_w, const void* a,
                   const void* b, int32_t E, int32_t r, const int32_t* idx, const float* gate,
                   int32_t k, float scale, const void* x, void* y, void* workspace,
                   int64_t workspace_bytes, int32_t dtype, void* stream) {
  if (w == nullptr || a == nullptr || b == nullptr || idx == nullptr || gate == nullptr ||
      x == nullptr || y == nullptr || workspace == nullptr)
    return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (!aligned16(w) || !aligned16(a) || !aligned16(b) || !aligned16(x) || !aligned16(y) ||
      !aligned16(workspace) || !aligned4(idx) || !aligned4(gate))
    return ADA_EALIGN;
  if (!dim_ok(d_out) || !dim_ok(d_in) || ld_w < d_in || ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
  if ((ld_w * (dtype == ADA_BF16 ? 2 : 4)) % 16 != 0) return ADA_EALIGN;
  if (E < 1 || E > 64 || r < 1 || k < 1 || k > E || int64_t(k) * r > ada::kMaxKR) return ADA_ESHAPE;
  if (workspace_bytes < (int64_t(d_out) + int64_t(k) * r) * 4) return ADA_ESHAPE;
  float* y32 = static_cast<float*>(workspace);
  float* t = y32 + d_out;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (ada::launch_gemv(w, d_out, d_in, ld_w, x, nullptr, y32, dtype, s) != hipSuccess) return ADA_EHIP;
  if (ada::launch_lora_shrink(a, E, r, d_in, idx, k, x, t, dtype, s) != hipSuccess) return ADA_EHIP;
  if (ada::launch_lora_expand(b, E, r, d_out, idx, gate, k, scale, y32, t, y, dtype, s) != hipSuccess)
    return ADA_EHIP;
  return ADA_OK;
}

int ada_lora_layer(const ada_lora_proj* projs, int32_t n_proj, int32_t E, int32_t r, const int32_t* idx,
                   const float* gate, int32_t k, float scale, void* workspace, int64_t workspace_bytes,
                   int32_t dtype, void* stream) {
  if (workspace == nullptr) return ADA_EINVAL;
  if (!aligned16(workspace)) return ADA_EALIGN;
  ada::LoraLayerParams p{};
  int64_t dot_rows = 0, out_rows = 0, ws_bytes = 0;
  if (int st = prepare_lora_layer(projs, n_proj, E, r, idx, gate, k, scale, dtype, p, dot_rows, out_rows, ws_bytes);
      st != ADA_OK)
    return st;
  if (workspace_bytes < ws_bytes) return ADA_ESHAPE;
  p.ws = static_cast<float*>(workspace);
  const hipError_t e = ada::launch_lora_layer(p, static_cast<int>(dot_rows), static_cast<int>(out_rows), dtype,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

int ada_lora_layer_static(const ada_lora_proj* projs, int32_t n_proj, int32_t E, int32_t r, const int32_t* idx,
                          const float* gate, int32_t k, float scale, int32_t dtype, void* stream) {
  ada::LoraLayerParams p{};
  int64_t dot_rows = 0, out_rows = 0, ws_bytes = 0;
  if (int st = prepare_lora_layer(projs, n_proj, E, r, idx, gate, k, scale, dtype, p, dot_rows, out_rows, ws_bytes);
      st != ADA_OK)
    return st;
  if (ws_bytes > static_cast<int64_t>(ada::kStaticScratchBytes)) return ADA_ESHAPE;
  void* scratch = nullptr;  // this device's copy of the library's static array (no allocation)
  if (ada::static_scratch(&scratch) != hipSuccess) return ADA_EHIP;
  p.ws = static_cast<float*>(scratch);
  const hipError_t e = ada::launch_lora_layer(p, static_cast<int>(dot_rows), static_cast<int>(out_rows), dtype,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

int ada_lora_batch(const ada_lora_proj* projs, int32_t n_proj, int32_t nb, int32_t E, int32_t r,
                   const int32_t* idx, const float* gate, int32_t k, float scale, void* workspace,
                   int64_t workspace_bytes, int32_t dtype, void* stream) {
  if (projs == nullptr || idx == nullptr || gate == nullptr || workspace == nullptr) return ADA_EINVAL;
  if (!dtype_ok(dtype)) return ADA_EDTYPE;
  if (!aligned4(idx) || !aligned4(gate) || !aligned16(workspace)) return ADA_EALIGN;
  if (n_proj < 1 || n_proj > ada::kMaxLayerProj || nb < 1 || nb > ada::kMaxBatch) return ADA_ESHAPE;
  if (E < 1 || E > 64 || r < 1 || k < 1 || k > E || int64_t(k) * r > ada::kMaxKR) return ADA_ESHAPE;
  const int esz = dtype == ADA_BF16 ? 2 : 4;
  const int64_t kr = int64_t(k) * r;
  ada::LoraLayerParams p{};
  int64_t dot_rows = 0, out_rows = 0, ws = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    const ada_lora_proj& q = projs[i];
    if (q.w == nullptr || q.a == nullptr || q.b == nullptr || q.x == nullptr || q.y == nullptr) return ADA_EINVAL;
    if (!aligned16(q.w) || !aligned16(q.a) || !aligned16(q.b) || !aligned16(q.x) || !aligned16(q.y))
      return ADA_EALIGN;
    if (!dim_ok(q.d_out) || !dim_ok(q.d_in) || q.ld_w < q.d_in || q.ld_w > (int64_t(1) << 40)) return ADA_ESHAPE;
    if ((q.ld_w * esz) % 16 != 0) return ADA_EALIGN;
    ada::LoraLayerProj& P = p.proj[i];
    P.w = q.w;
    P.a = q.a;
    P.b = q.b;
    P.x = q.x;
    P.y = q.y;
    P.ld = q.ld_w;
    P.d_out = q.d_out;
    P.d_in = q.d_in;
    P.dot_row0 = static_cast<int32_t>(dot_rows);
    P.out_row0 = static_cast<int32_t>(out_rows);
    P.ws_off = ws;
    dot_rows += (q.d_out + 15) / 16 + (nb * kr + 3) / 4;  // workgroups: 16 W rows each, then 4 shrink rows each
    out_rows += int64_t(nb) * q.d_out;
    ws = (ws + nb * (q.d_out + kr) + 3) & ~int64_t(3);  // keep every block 16-byte aligned
  }
  if (dot_rows >= (int64_t(1) << 30) || out_rows >= (int64_t(1) << 30)) return ADA_ESHAPE;
  if (workspace_bytes < ws * 4) return ADA_ESHAPE;
  p.n = n_proj;
  p.E = E;
  p.r = r;
  p.k = k;
  p.idx = idx;
  p.gate = gate;
  p.scale = scale;
  p.ws = static_cast<float*>(workspace);
  p.nb = nb;
  const hipError_t e = ada::launch_lora_batch(p, static_cast<int>(dot_rows), static_cast<int>(out_rows), dtype,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : ADA_EHIP;
}

}  // extern "C"
