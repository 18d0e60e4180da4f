// Internal declarations of libgnn (not installed).  Device helpers shared by
// the kernels, the plan object, and the host-side error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "gnn.h"

namespace gnn {

// ---------------------------------------------------------------------------
// Host-side error handling
// ---------------------------------------------------------------------------

void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

#define GNN_HIP(call)                                                              \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      return ::gnn::fail(e_ == hipErrorOutOfMemory ? GNN_ERR_OUT_OF_MEMORY         \
                                                    : GNN_ERR_DEVICE,              \
                         std::string(#call) + ": " + hipGetErrorString(e_));       \
    }                                                                              \
  } while (0)

#define GNN_LAUNCH_CHECK(what)                                                     \
  do {                                                                             \
    hipError_t e_ = hipGetLastError();                                             \
    if (e_ != hipSuccess)                                                          \
      return ::gnn::fail(GNN_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define GNN_TRY(expr)            \
  do {                           \
    int s_ = (expr);             \
    if (s_ != GNN_OK) return s_; \
  } while (0)

// Every device allocation of the library goes through these two calls.
// GNN_FAIL_ALLOC=k (or k:tag; a new value restarts the count) in the
// environment makes the k-th allocation after the variable took its value fail with GNN_ERR_OUT_OF_MEMORY before any
// HIP call, so that the error paths can be exercised.
int dev_malloc(void** p, size_t bytes);
int dev_malloc_async(void** p, size_t bytes, hipStream_t s);
// Stream-ordered release of a dev_malloc_async block: kept in the library's
// per-device, per-stream cache for the next request on `s` (other pointers go
// to hipFreeAsync).  release_cached_memory hands the current device's cached
// blocks back to the runtime.
int dev_free_async(void* p, hipStream_t s);
int release_cached_memory();

// Stream-ordered temporaries of one call: taken on `s`, and all freed on `s`
// when the object goes out of scope, early error returns included.
struct StreamTemps {
  hipStream_t s;
  void* p[24] = {};
  int n = 0;
  explicit StreamTemps(hipStream_t st) : s(st) {}
  StreamTemps(const StreamTemps&) = delete;
  StreamTemps& operator=(const StreamTemps&) = delete;
  template <typename T>
  int get(T** out, size_t bytes) {
    if (n >= (int)(sizeof(p) / sizeof(p[0]))) return fail(GNN_ERR_DEVICE, "too many temporaries");
    void* q = nullptr;
    int rc = dev_malloc_async(&q, bytes, s);
    if (rc != GNN_OK) return rc;
    p[n++] = q;
    *out = static_cast<T*>(q);
    return GNN_OK;
  }
  // free everything now, reporting a failed free
  int release() {
    int first = GNN_OK;
    for (int k = 0; k < n; ++k) {
      const int rc = dev_free_async(p[k], s);
      if (rc != GNN_OK && first == GNN_OK) first = rc;
    }
    n = 0;
    return first;
  }
  ~StreamTemps() {
    for (int k = 0; k < n; ++k) (void)dev_free_async(p[k], s);
  }
};

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------

struct WsbLayout {
  int32_t n_windows = 0;
  int64_t n_blocks = 0;     // 16x8 blocks
  int64_t n_tiles = 0;      // dense 16x16 tiles routed to MFMA
  int64_t n_resid = 0;      // residual CSR edges
  int32_t* win_ptr = nullptr;     // [n_windows + 1] block offsets
  int32_t* blk_col = nullptr;     // [n_blocks * 8]
  uint64_t* blk_bits = nullptr;   // [n_blocks * 2]
  int32_t* tile_ptr = nullptr;    // [n_windows + 1] dense-tile offsets
  int32_t* tile_blk = nullptr;    // [n_tiles] first 16x8 block of each dense tile
  int32_t* res_ptr = nullptr;     // [n_rows + 1] residual CSR
  int32_t* res_col = nullptr;     // [n_resid]
};

}  // namespace gnn

struct gnn_plan {
  int32_t n_rows = 0, n_cols = 0;
  int64_t nnz = 0;
  const int32_t* row_ptr = nullptr;
  const int32_t* col_idx = nullptr;
  gnn_plan_opts opts{};
  hipStream_t stream = nullptr;
  // a transient plan: all its memory is allocated and freed stream-ordered on
  // `stream`, and it was built without reading anything back to the host
  bool async_mem = false;

  // structure fingerprint: kFingerprint evenly spaced entries of row_ptr
  // (first and last included) and of col_idx, sampled when the plan was
  // built (host copy) and re-sampled into fp_dev by plan_verify
  static constexpr int kFingerprint = 64;
  int32_t fp_host[2 * kFingerprint] = {};
  int32_t* fp_dev = nullptr;

  // degrees
  int32_t* deg_out = nullptr;  // [n_cols]; NULL until counted (transient plans: on first use)

  // degree bins (appendix D.1: light / heavy split by a degree quantile)
  int32_t light_max = 32;
  int32_t heavy_thr = 0;     // rows above are split into chunks (INT32_MAX: never)
  int32_t chunk_edges = 512;
  int64_t n_light = 0, n_medium = 0, n_heavy = 0;
  // items: the chunks of split rows first, then one per medium row (those
  // longer than att_item_thr first); the index of a chunk item is also its
  // partial slot in the workspace
  int4* items = nullptr;     // [n_items] (row, e_begin, e_end, multi index or -1)
  int64_t n_items = 0;       // (upper bounds when item_count is set)
  int64_t n_slots = 0;       // chunk items of split rows
  int32_t att_item_thr = 0;  // medium rows longer than this come before the others
  int64_t n_att_items = 0;   // chunks and those rows: the items an attention call with
                             // a one-slot bound of att_item_thr runs (a bound as n_items)
  int32_t* item_count = nullptr;   // device, plans built without a host read-back: the item count
  int32_t* multi_count = nullptr;  // device, same plans: the split-row count (item_count + 1)
  int4* multi = nullptr;     // [n_multi] (row, first chunk item, chunk count, 0)
  int64_t n_multi = 0;
  int32_t max_items_per_row = 0;

  // rows of at most att_lmax edges, longest first (built on the first
  // attention call): one slot per row, equal lengths side by side
  int32_t* att_rows = nullptr;   // [n_rows]
  int32_t* att_woff = nullptr;   // [windows + 1] listed rows before each window of rows
  int32_t* att_count = nullptr;  // device: number of listed rows (att_woff's last entry)
  int32_t att_lmax = -1;

  // the transpose A^T (built on the first backward call): its CSR arrays,
  // the position in A of each of its entries, and a plan over it
  gnn_plan* tplan = nullptr;
  int32_t* t_row_ptr = nullptr;  // [n_cols + 1]
  int32_t* t_col = nullptr;      // [nnz] rows of A
  int32_t* t_edge = nullptr;     // [nnz]
  float* t_val = nullptr;        // [nnz] edge values in transposed order (per call)
  float* delta = nullptr;        // attention backward: [n_rows, H] <O, dO> per (row, head)
  size_t delta_cap = 0;
  uint16_t* dob = nullptr;       // block-sparse attention backward: dO in bf16, [n_rows, H, D]
  size_t dob_cap = 0;

  // workspace (partials / packed words); grows on demand
  void* ws = nullptr;
  size_t ws_bytes = 0;

  gnn::WsbLayout wsb;
  bool has_wsb = false;

  // every device allocation of the plan
  void* allocs[32] = {};
  int n_allocs = 0;
};

namespace gnn {

int plan_alloc(gnn_plan* p, void** ptr, size_t bytes);
int plan_workspace(gnn_plan* p, size_t bytes, void** out);
// a plan-owned buffer that grows on demand (freed with the plan)
int plan_grow(gnn_plan* p, void** buf, size_t* cap, size_t bytes);
int plan_build(const gnn_csr* csr, const gnn_plan_opts* opts, hipStream_t s, gnn_plan* p);
// The transient plan of a call made without one: one work item per row
// longer than the light bound (no split rows), built on `s` with
// stream-ordered memory and no host synchronisation; its item count stays on
// the device (item_count), n_items holds an upper bound for grid sizes.  Its
// out-degrees are counted on first use (plan_deg_out).
// Plan without a host read-back (calls given no plan): rows longer than
// light_max are items, rows longer than one chunk are split, and the counts
// stay on the device.
int plan_build_async(const gnn_csr* csr, hipStream_t s, gnn_plan* p, int32_t light_max);
// Attention kernels give one slot to each row up to this many entries; the
// plans they build without a read-back take it as their light bound (their
// shorter items would run on the slot path anyway).
constexpr int32_t kAttSlotRows = 128;
// deg_out[j] = entries with column j (columns outside [0, n_cols) are not
// counted); enqueued on `s`, temporaries stream-ordered.
int count_out_degrees(const int32_t* col_idx, int64_t nnz, int32_t n_cols, int32_t* deg_out, hipStream_t s);
// The plan's out-degrees, counted now if the plan does not hold them yet.
int plan_deg_out(gnn_plan* p, hipStream_t s);
int plan_build_wsb(gnn_plan* p, hipStream_t s);
int plan_att_rows(gnn_plan* p, int32_t lmax, hipStream_t s);
int plan_transpose(gnn_plan* p, hipStream_t s);
int plan_transpose_wsb(gnn_plan* p, hipStream_t s);
int check_plan(const gnn_plan* p, const gnn_csr* csr);
// Enqueue the fingerprint samples of the plan's CSR into p->fp_dev.
int plan_sample_fingerprint(gnn_plan* p, hipStream_t s);
// Re-sample the fingerprint and compare it with the one taken at build time
// (synchronises `s`; allocates nothing): PLAN_MISMATCH if they differ.
int plan_verify(gnn_plan* p, hipStream_t s);

// Launchers (host).  All validate nothing: the entry points did.
int launch_aggregate(gnn_plan* p, const void* X, gnn_dtype xt, int32_t F, int64_t ldx, float* Y,
                     int64_t ldy, int mode, gnn_norm norm, const float* edge_val, int32_t* arg,
                     hipStream_t s);
int launch_reduce_multi(gnn_plan* p, const void* X, gnn_dtype xt, int32_t F, int64_t ldx,
                        float* Ysum, float* Ymean, float* Ymax, int32_t* argmax, float* Ymin,
                        int32_t* argmin, int64_t ldy, hipStream_t s, void* ws = nullptr);
// Workspace bytes launch_reduce_multi needs for the plan's split rows at
// width F (0 without split rows); `ws` above, when given, must hold them.
size_t reduce_multi_ws_bytes(const gnn_plan* pl, int32_t F);
int launch_gatv2(gnn_plan* p, const void* xl, const void* xr, gnn_dtype xt, const float* att,
                 int32_t H, int32_t D, float slope, float* out, float* lse, hipStream_t s);
int launch_gt_csr(gnn_plan* p, const void* q, const void* k, const void* v, gnn_dtype xt, int32_t H,
                  int32_t D, float scale, float* out, float* lse, hipStream_t s);
// GNN_OK if the fused CSR attention kernels have a lane mapping for heads
// of D elements of `xt` (gt: Graph Transformer, else GATv2).
int attention_mapping_supported(int gt, gnn_dtype xt, int32_t H, int32_t D);
int launch_gt_block16(gnn_plan* p, const void* q, const void* k, const void* v, int32_t H,
                      int32_t D, float scale, float* out, float* lse, hipStream_t s);
int launch_project(const void* X, int32_t n, int32_t f_in, int64_t ldx, int32_t n_mat, const void* const* W,
                   int32_t f_out, void* const* Y, hipStream_t s);
int launch_reorder(const gnn_csr* csr, gnn_reorder_kind kind, int32_t* perm, int32_t* rp_out,
                   int32_t* ci_out, hipStream_t s);
int launch_permute_rows(const int32_t* perm, int32_t n, const void* X, int elem_bytes, int32_t F,
                        int64_t ldx, void* Xout, int64_t ldo, hipStream_t s);
int launch_copy(const void* src, void* dst, int64_t n, hipStream_t s);

// Device-wide exclusive scan of int32 counts into int32 offsets (out has n+1
// entries, out[n] = total).  Scratch: scan_scratch_bytes(n) bytes at
// `scratch`, or (NULL) allocated and freed stream-ordered.
size_t scan_scratch_bytes(int64_t n);
int exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, hipStream_t s, void* scratch = nullptr);

// Stable LSD radix sort of 64-bit keys by bits [begin_bit, end_bit); result
// in `keys`, `tmp` is scratch of n keys.  Further scratch:
// radix_scratch_bytes(n) bytes at `scratch`, or (NULL) allocated.
size_t radix_scratch_bytes(int64_t n);
int radix_sort_u64(uint64_t* keys, uint64_t* tmp, int64_t n, int begin_bit, int end_bit,
                   hipStream_t s, void* scratch = nullptr);

// Bump allocator over one device block: every temporary of a call carved
// from a single allocation (256-byte aligned pieces).
struct Arena {
  char* base = nullptr;
  size_t cap = 0, off = 0;
  static size_t round(size_t b) { return (b + 255) & ~(size_t)255; }
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base + off);
    off += round(count * sizeof(T));
    return p;
  }
};

// dot-aggr micro-benchmark (dot_aggr.hip): map 0 = feature-parallel,
// 1 = neighbour-parallel; vec = 16-byte loads per lane
int launch_dot_aggr(gnn_plan* p, const float* X, int32_t D, int64_t ldx, int map, bool vec, float* y,
                    hipStream_t s);

int launch_spmm_block16(gnn_plan* p, const void* X, gnn_dtype xt, int32_t F, int64_t ldx, float* Y, int64_t ldy,
                        gnn_norm norm, hipStream_t s);

// Backward launchers (transposed walks; see transpose.hip, attention_bwd.hip)
int launch_spmm_backward(gnn_plan* p, const float* dY, int32_t F, int64_t ldy, float* dX, int64_t ldx,
                         gnn_norm norm, const float* edge_val, hipStream_t s);
int launch_reduce_backward(gnn_plan* p, int op, const float* dY, int32_t F, int64_t ldy,
                           const int32_t* arg, float* dX, int64_t ldx, hipStream_t s);
int launch_gt_backward(gnn_plan* p, const void* q, const void* k, const void* v, gnn_dtype xt, int32_t H,
                       int32_t D, float scale, const float* out, const float* lse, const float* dout,
                       float* dq, float* dk, float* dv, hipStream_t s);
int launch_gt_backward_block16(gnn_plan* p, const void* q, const void* k, const void* v, int32_t H, int32_t D,
                               float scale, const float* out, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, hipStream_t s);
int launch_gatv2_backward(gnn_plan* p, const void* xl, const void* xr, gnn_dtype xt, const float* att,
                          int32_t H, int32_t D, float slope, const float* out, const float* lse,
                          const float* dout, float* dxl, float* dxr, float* datt, hipStream_t s);

// Aggregation modes for launch_aggregate
enum AggMode { AGG_SUM = 0, AGG_MEAN = 1, AGG_MAX = 2, AGG_MIN = 3, AGG_SPMM = 4 };

}  // namespace gnn

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

namespace gnn {
namespace dev {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Order-preserving map of IEEE-754 float bits to uint32 (appendix D.1):
// negative values have every bit inverted, non-negative values get the sign
// bit set; unsigned order then equals float order with -0.0 < +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  // negative: every bit flipped; otherwise the sign bit set (an arithmetic
  // shift, an or and an xor, no compare)
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  // sign bit set: clear it; otherwise flip every bit
  return __uint_as_float(k ^ (~(uint32_t)((int32_t)k >> 31) | 0x80000000u));
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X; this
// maps the hardware workgroup id to a logical one so that each XCD receives
// runs of `run` consecutive logical ids (neighbouring rows share one L2),
// the runs of the 8 XCDs interleaved so that all XCDs sweep the row range
// together.  run = 0: one run per XCD (each XCD a contiguous eighth).  Ids
// past the last whole group of 8 runs keep the hardware order.  One run per
// XCD loads one XCD with all the heavy rows of a degree-sorted graph; runs
// of 128 workgroups keep the locality and spread every part of the row range
// over all eight XCDs.
#ifndef GNN_XCD_RUN
#define GNN_XCD_RUN 128
#endif
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t NX = 8;
  const uint32_t run = GNN_XCD_RUN > 0 ? (uint32_t)GNN_XCD_RUN : (nblocks / NX > 0 ? nblocks / NX : 1);
  const uint32_t full = nblocks / (NX * run) * (NX * run);
  if (bid >= full) return bid;
  const uint32_t x = bid % NX, k = bid / NX;
  return ((k / run) * NX + x) * run + k % run;
}

}  // namespace dev
}  // namespace gnn
