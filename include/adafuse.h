/*
 * adafuse.h -- C ABI of the AdaFuse pre-gating and fused adapter-merge library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (both summary pages of "AdaFuse: Accelerating Dynamic Adapter
 * Inference via Token-Level Pre-Gating and Fused Kernel Optimization", cited here
 * as [pt] for the Portuguese page and [ja] for the Japanese page):
 *   - a single light router runs once on the leading token and picks the top-k
 *     LoRA experts for every later layer ([pt] technical summary 2.A; [ja] 2.1);
 *   - the picked adapters are fused into the backbone weights before decoding, in
 *     one kernel call covering every layer ([pt] 2.B; [ja] 2.2), by concatenating
 *     their down and up projections ([ja] 2.2);
 *   - the fusion is undone, or switched to another selection, in one pass as well
 *     ([pt] 2.B).
 * Merged weights: W' = W + s * sum_j g_j * B_{e_j} A_{e_j}.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer unless stated otherwise, 16-byte
 *     aligned, row-major, owned by the caller.  The library never allocates or
 *     frees caller memory, and the hot calls (pregate, merge, unmerge, switch,
 *     decode_gemv, decode_gemv_layer, lora_apply, lora_layer, lora_batch) allocate
 *     nothing at all.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     calls are asynchronous on that stream and return once the work is enqueued.
 *   - Return value: ADA_OK (0) or a negative ada_status.  All argument checks run
 *     on the host before any HIP call, so a rejected call has no effect.  A fault
 *     inside a kernel surfaces at the caller's next synchronisation of the stream.
 *   - dtype: ADA_F32 (fp32 storage) or ADA_BF16 (bf16 storage).  Gates are fp32
 *     and every reduction accumulates in fp32; results are rounded to the storage
 *     type once, to nearest-even.
 *   - Dimensions d, d_in, d_out and row strides are counts of elements and must be
 *     multiples of 8; 1 <= k <= E <= 64; k*r <= 512.
 *   - LoRA layout: A (down) is [E][r][d_in], B (up) is [E][d_out][r], contiguous;
 *     W is [d_out][ld_w] with ld_w >= d_in.
 */
#ifndef ADAFUSE_H
#define ADAFUSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ADA_OK = 0,
  ADA_EINVAL = -1,  /* null pointer, null or destroyed handle, bad flag value    */
  ADA_ESHAPE = -2,  /* a size outside the supported range, or not a multiple of 8 */
  ADA_EDTYPE = -3,  /* unknown dtype, or a dtype other than the model's           */
  ADA_EALIGN = -4,  /* a pointer or row stride not 16-byte aligned                */
  ADA_EHIP = -5,    /* a HIP runtime call or kernel launch failed                 */
  ADA_ENOMEM = -6   /* the model's work table could not be allocated              */
} ada_status;

typedef enum { ADA_F32 = 0, ADA_BF16 = 1 } ada_dtype;

/* One adapted projection: base weights and its bank of E LoRA adapters. */
typedef struct {
  void* w;          /* [d_out][ld_w] base weights                                */
  void* w_out;      /* NULL or == w: merge in place; else [d_out][ld_w] output,    */
                    /* written by merge, and the buffer unmerge/switch act on     */
  const void* a;    /* [E][r][d_in] down projections                              */
  const void* b;    /* [E][d_out][r] up projections                               */
  int32_t d_out;
  int32_t d_in;
  int64_t ld_w;     /* row stride of w and w_out, elements                        */
} ada_proj;

typedef struct ada_model_s* ada_model;

/*
 * Register a stack of adapted projections (every layer and projection of a
 * model, in any order).  Builds the per-projection work table the one-launch
 * merge walks ([ja] 2.2: the large product is split into GEMM tiles assigned to
 * thread blocks) and uploads it to the current device; this is the only call that
 * allocates (one device allocation for one table per contraction class, three in
 * all: ~64 bytes per projection each plus a small tile index, and the tables' host
 * image, kept until destroy).
 * n_proj >= 1; all projections share E, r and dtype.  On success *out owns the
 * table until ada_model_destroy.  ada_merge, ada_unmerge and ada_switch return
 * ADA_EINVAL when another device is current than at creation.  The registered pointers must stay valid, and
 * may not be registered twice in one model.  An out-of-place w_out must not overlap
 * any registered w, w_out, a or b (the launch reads and writes all tiles at once).
 * Ordering: the table is copied to the device asynchronously on `stream` (a
 * hipStream_t as void*, NULL = the default stream).  Merges enqueued on that stream
 * after this call see it; a merge on another stream must be ordered after `stream`
 * by the caller (for instance by synchronizing `stream` once).  Argument checks run
 * before any HIP call; on an error nothing is allocated and *out is NULL.
 */
int ada_model_create(const ada_proj* projs, int32_t n_proj, int32_t E, int32_t r,
                     int32_t dtype, void* stream, ada_model* out);

/* Free the model's work table (waiting first for its upload).  NULL is ignored.
 * Call after the model's last enqueued merge has completed. */
void ada_model_destroy(ada_model m);

/* Number of output tiles one merge launch of this model covers at k*r <= 32
 * (32 x 256 tiles for bf16, 64 x 64 for fp32; for measurement); negative status on
 * a bad handle. */
int64_t ada_model_tiles(ada_model m);

/* Device bytes the model owns (its work tables), for footprint reports; negative
 * status on a bad handle. */
int64_t ada_model_device_bytes(ada_model m);

/*
 * Token-level pre-gating ([pt] 2.A; [ja] 2.1).  z = R h (fp32 accumulation);
 * idx_out[0..k) = the k largest z in descending order, equal z lower index first;
 * gate_out[j] = exp(z[idx_j] - z[idx_0]) / sum_i exp(z[idx_i] - z[idx_0]) when
 * renorm = 1 (softmax over the selected logits), or the full softmax over all E
 * logits read at idx_j when renorm = 0.  One workgroup; results stay on the
 * device (idx_out, gate_out are device pointers) for the merge to read.
 *   h: [d] hidden state of the leading token; router: [E][d]; dtype of both.
 *   NaN logits give an unspecified (but in-range) selection.
 */
int ada_pregate(const void* h, const void* router, int32_t d, int32_t E, int32_t k,
                int32_t dtype, int32_t renorm, int32_t* idx_out, float* gate_out,
                void* stream);

/*
 * Fused merge of the selected adapters into every registered projection in ONE
 * kernel launch ([pt] 2.B; [ja] 2.2):
 *   w_out (or w in place) = RNE(w + sum_j scale*gate[j] * B[idx[j]] @ A[idx[j]]).
 * Each coefficient scale*gate[j] is applied at fp32 accuracy and products are
 * summed in fp32, so the result is the exact merge rounded once to the storage type
 * (to within fp32 accumulation).  idx, gate: device arrays of k entries (as written
 * by ada_pregate).  Slots whose gate is 0 are skipped; if every gate is 0 an
 * in-place merge writes nothing and an out-of-place merge copies w.  Indices outside
 * [0, E) are skipped.  The caller keeps (idx, gate, scale) to unmerge.  On an
 * out-of-place model every call reads the untouched w, so calling it again with a
 * new selection is a drift-free switch.  Overlapping calls on one model's weights
 * race.  k*r <= 512.
 */
int ada_merge(ada_model m, const int32_t* idx, const float* gate, int32_t k,
              float scale, void* stream);

/*
 * De-fuse ([pt] 2.B): buffer = RNE(buffer - sum_j scale*gate[j] * B[idx[j]] @ A[idx[j]])
 * on the merged buffer (w in place, or w_out for an out-of-place model), in one
 * launch.  In bf16 this returns W to within rounding, not bit-exactly; repeated
 * merge/unmerge cycles drift, so long-running callers restore from a pristine
 * copy (or use an out-of-place model and simply merge again).
 */
int ada_unmerge(ada_model m, const int32_t* idx, const float* gate, int32_t k,
                float scale, void* stream);

/*
 * Fused switch between selections ([pt] 2.B: undo the previous token's fusion and
 * apply the current one in one pass): buffer = RNE(buffer - delta(prev) + delta(cur)),
 * one read and one write of every weight.  (k_prev + k_cur) * r <= 512.
 * Drift: every switch rounds the buffer to bf16 again, so a chain of switches moves
 * away from W + delta(cur).  From a fresh merge one switch stays within the stated
 * tolerance (8e-3 |ref| + 1e-4); measured on a 512 x 4096 projection (rank 16, top-2),
 * 0.001% of weights are outside it after 2 switches, 1% after 8 and 11% after 31.
 * Per-token switching without drift: register the model out of place (w_out != w)
 * and call ada_merge for each new selection, which reads the untouched w and writes
 * w_out (the same one read and one write per weight).  In-place models that switch
 * must restore w from pristine weights before the second switch.
 */
int ada_switch(ada_model m, const int32_t* idx_prev, const float* gate_prev, int32_t k_prev,
               const int32_t* idx_cur, const float* gate_cur, int32_t k_cur, float scale,
               void* stream);

/*
 * Decode-step projection on the merged backbone ([pt] 2.B: after fusion, decoding
 * runs with no routing): y[d_out] = RNE(w @ x), fp32 accumulation.
 *   w: [d_out][ld_w]; x: [d_in]; y: [d_out]; all of `dtype`.
 */
int ada_decode_gemv(const void* w, int32_t d_out, int32_t d_in, int64_t ld_w,
                    const void* x, void* y, int32_t dtype, void* stream);

/* One decode GEMV for ada_decode_gemv_layer. */
typedef struct {
  const void* w;    /* [d_out][ld_w] weights                         */
  const void* x;    /* [d_in] input                                   */
  void* y;          /* [d_out] output                                 */
  int32_t d_out;
  int32_t d_in;
  int64_t ld_w;
} ada_gemv_proj;

/*
 * Up to 16 independent decode GEMVs (for instance the q, k and v projections of a
 * layer, which read the same hidden state) in ONE launch: y_p = RNE(w_p @ x_p) for
 * every p, each bit-identical to ada_decode_gemv on the same operands.  Fewer launches
 * per decode step leave less launch ramp and tail, which the small projections of a
 * batch-1 step are bound by.
 */
int ada_decode_gemv_layer(const ada_gemv_proj* projs, int32_t n_proj, int32_t dtype, void* stream);

/*
 * One projection of the conventional, unmerged dynamic-adapter layer the pages
 * compare against ([pt] technical summary 1; [ja] 1): y = RNE(w @ x + scale *
 * sum_j gate[j] * B[idx[j]] (A[idx[j]] x)), computed as separate base-GEMV, shrink
 * and expand kernels (three launches).  `workspace` is a caller-owned device
 * buffer of at least (d_out + k*r) * 4 bytes for the fp32 intermediates.
 */
int ada_lora_apply(const void* w, int32_t d_out, int32_t d_in, int64_t ld_w,
                   const void* a, const void* b, int32_t E, int32_t r,
                   const int32_t* idx, const float* gate, int32_t k, float scale,
                   const void* x, void* y, void* workspace, int64_t workspace_bytes,
                   int32_t dtype, void* stream);

/* One projection of a layer for ada_lora_layer. */
typedef struct {
  const void* w;    /* [d_out][ld_w] base weights                   */
  const void* a;    /* [E][r][d_in] down projections                */
  const void* b;    /* [E][d_out][r] up projections                 */
  const void* x;    /* [d_in] input                                  */
  void* y;          /* [d_out] output                                */
  int32_t d_out;
  int32_t d_in;
  int64_t ld_w;
} ada_lora_proj;

/*
 * One layer of the unmerged, routed path for up to 16 projections in two launches
 * (the same arithmetic as ada_lora_apply per projection, bit for bit): one grid
 * computes every projection's base-GEMV rows and shrink rows A[idx_j] x, one grid
 * every expand.  This is the strongest unmerged comparator for the merged path
 * ([pt] technical summary 1: several kernel calls per layer in the conventional
 * design).  All projections share E, r, the selection and the dtype.  `workspace`:
 * caller-owned device memory of at least 4 * sum_p roundup4(d_out_p + k*r) bytes
 * (one fp32 block per projection, each starting 16-byte aligned).
 */
int ada_lora_layer(const ada_lora_proj* projs, int32_t n_proj, int32_t E, int32_t r,
                   const int32_t* idx, const float* gate, int32_t k, float scale,
                   void* workspace, int64_t workspace_bytes, int32_t dtype, void* stream);

/*
 * ada_lora_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the fp32 intermediates live in a static device array inside the
 * library, 4 MiB per GPU, which each GPU the library runs on holds until the process
 * ends.  The call allocates nothing; it returns ADA_ESHAPE (before any HIP call) when
 * the layer needs more than 4 MiB of intermediates (4 * sum_p roundup4(d_out_p + k*r)
 * bytes > 4 MiB), and otherwise computes exactly what ada_lora_layer computes.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (other streams, other host threads) race, so order them.  The array's contents are
 * left from the last call; every element a call reads it has written first.
 */
int ada_lora_layer_static(const ada_lora_proj* projs, int32_t n_proj, int32_t E, int32_t r,
                          const int32_t* idx, const float* gate, int32_t k, float scale,
                          int32_t dtype, void* stream);

/*
 * A batch of nb requests (1 <= nb <= 16), each with its OWN selection, through one
 * layer of the unmerged routed path, in two launches.  The pages treat batch-1
 * requests with one selection each; a merged backbone can hold only one selection,
 * so requests with different selections are served unmerged:
 *   y_b = RNE(w @ x_b + scale * sum_j gate[b][j] * B[idx[b][j]] (A[idx[b][j]] x_b)).
 * Every W row is read once for the whole batch (the base product runs on MFMA, 16
 * rows by 16 requests per workgroup).  Per projection, x is [nb][d_in] and y is
 * [nb][d_out] (rows contiguous); idx and gate are device arrays [nb][k].  Request
 * b's result equals ada_lora_layer on (x_b, idx[b], gate[b]) up to the order of the
 * base product's fp32 sums.  `workspace`: caller-owned device memory of at least
 * 4 * sum_p roundup4(nb * (d_out_p + k*r)) bytes.
 */
int ada_lora_batch(const ada_lora_proj* projs, int32_t n_proj, int32_t nb, int32_t E, int32_t r,
                   const int32_t* idx, const float* gate, int32_t k, float scale,
                   void* workspace, int64_t workspace_bytes, int32_t dtype, void* stream);

/* Static text for a status code (never NULL). */
const char* ada_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ADAFUSE_H */
