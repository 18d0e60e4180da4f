// C ABI of libgnn: host-side validation, plans, dispatch to the launchers.
// Declarations and the contract of every entry point are in include/gnn.h.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>

#include "gnn_internal.h"

static __device__ __align__(256) unsigned char scratch[GNN_NOALLOC_SCRATCH_BYTES];

namespace gnn {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

namespace {

int check_csr(const gnn_csr* c, bool need_square) {
  if (!c) return fail(GNN_ERR_INVALID_VALUE, "csr is NULL");
  if (c->n_rows < 0 || c->n_cols < 0 || c->nnz < 0)
    return fail(GNN_ERR_INVALID_VALUE, "negative CSR size");
  if (c->nnz >= 2147483648LL) return fail(GNN_ERR_SIZE_OVERFLOW, "nnz must be < 2^31");
  if (!c->row_ptr) return fail(GNN_ERR_INVALID_VALUE, "row_ptr is NULL");
  if (c->nnz > 0 && !c->col_idx) return fail(GNN_ERR_INVALID_VALUE, "col_idx is NULL");
  if (c->nnz > 0 && c->n_cols == 0) return fail(GNN_ERR_INVALID_VALUE, "edges but n_cols == 0");
  if (need_square && c->n_rows != c->n_cols)
    return fail(GNN_ERR_INVALID_VALUE, "operation needs a square CSR (n_rows == n_cols)");
  return GNN_OK;
}

int check_dtype(gnn_dtype t) {
  if (t != GNN_F32 && t != GNN_BF16) return fail(GNN_ERR_INVALID_VALUE, "unknown dtype");
  return GNN_OK;
}

bool debug_validation() {
  const char* env = getenv("GNN_DEBUG_VALIDATE");
  return env && strcmp(env, "1") == 0;
}

int debug_validate(const gnn_csr* c, hipStream_t s);

// A plan given by the caller must be bound to this CSR (with
// GNN_DEBUG_VALIDATE=1 also by its sampled contents); otherwise build a
// transient one (synchronises the stream) that the caller of this helper frees.
// transient_light: the light bound of a plan built here without a read-back
int get_plan(const gnn_csr* csr, gnn_plan* given, hipStream_t s, gnn_plan** use, bool* transient,
             bool need_wsb = false, int32_t transient_light = 32) {
  *transient = false;
  if (given) {
    GNN_TRY(check_plan(given, csr));
    if (debug_validation()) GNN_TRY(plan_verify(given, s));
    if (need_wsb && !given->has_wsb)
      return fail(GNN_ERR_INVALID_VALUE, "plan was built without build_wsb");
    *use = given;
    return GNN_OK;
  }
  gnn_plan* p = nullptr;
  if (need_wsb) {
    // the WSB layout is sized from counts read back to the host
    gnn_plan_opts o{};
    o.build_wsb = 1;
    GNN_TRY(gnn_plan_create(csr, &o, s, &p));
  } else {
    GNN_TRY(debug_validate(csr, s));
    p = new (std::nothrow) gnn_plan();
    if (!p) return fail(GNN_ERR_OUT_OF_MEMORY, "host allocation failed");
    const int rc = plan_build_async(csr, s, p, transient_light);
    if (rc != GNN_OK) {
      std::string keep = g_last_error;
      gnn_plan_destroy(p);
      g_last_error = keep;
      return rc;
    }
  }
  *use = p;
  *transient = true;
  return GNN_OK;
}

struct PlanGuard {
  gnn_plan* p;
  bool own;
  ~PlanGuard() {
    if (own && p) gnn_plan_destroy(p);
  }
};

// The checks of the CSR contents that host validation leaves out, O(n + nnz):
// bad[0] row_ptr decreases somewhere, bad[1] row_ptr[0] != 0 or row_ptr[n] !=
// nnz, bad[2] a column outside [0, n_cols).  Reads the two arrays only within
// their stated sizes and never indexes by their values.
__global__ void k_check_csr(const int32_t* rp, const int32_t* ci, int32_t n, int64_t nnz, int32_t n_cols,
                            int* bad) {
  const int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = i0; r < n; r += stride)
    if (rp[r] > rp[r + 1]) bad[0] = 1;
  if (i0 == 0 && (rp[0] != 0 || (int64_t)rp[n] != nnz)) bad[1] = 1;
  for (int64_t e = i0; e < nnz; e += stride) {
    const int32_t c = ci[e];
    if (c < 0 || c >= n_cols) bad[2] = 1;
  }
}

// With GNN_DEBUG_VALIDATE=1 in the environment, run k_check_csr before
// anything reads the CSR (synchronises the stream; allocates).
int debug_validate(const gnn_csr* c, hipStream_t s) {
  if (!debug_validation()) return GNN_OK;
  int* d = nullptr;
  GNN_TRY(dev_malloc((void**)&d, 3 * sizeof(int)));
  int h[3] = {0, 0, 0};
  hipError_t e = hipMemcpy(d, h, sizeof(h), hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    const int64_t work = std::max<int64_t>(c->n_rows, c->nnz);
    const unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>((work + 255) / 256, 1), 4096);
    hipLaunchKernelGGL(k_check_csr, dim3(blocks), dim3(256), 0, s, c->row_ptr, c->col_idx, c->n_rows, c->nnz,
                       c->n_cols, d);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
  const hipError_t ef = hipFree(d);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return fail(GNN_ERR_DEVICE, std::string("CSR check: ") + hipGetErrorString(e));
  if (h[1]) return fail(GNN_ERR_INVALID_VALUE, "CSR check: row_ptr[0] != 0 or row_ptr[n_rows] != nnz");
  if (h[0]) return fail(GNN_ERR_INVALID_VALUE, "CSR check: row_ptr decreases");
  if (h[2]) return fail(GNN_ERR_INVALID_VALUE, "CSR check: a column index outside [0, n_cols)");
  return GNN_OK;
}

// Scratch memory of gnn_reduce_multi_noalloc (the array `scratch`, file
// scope): every GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (in host code it
// is a host-side stand-in, not a device address): scratch_address() looks up
// the device address once per device with hipGetSymbolAddress and keeps it.
constexpr size_t kNoallocScratchBytes = (size_t)GNN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the device that `s` belongs to, which must
// be the calling thread's current device.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  GNN_HIP(hipGetDevice(&dev));
  if (s) {
    hipDevice_t sdev = -1;
    GNN_HIP(hipStreamGetDevice(s, &sdev));
    if ((int)sdev != dev)
      return fail(GNN_ERR_INVALID_VALUE, "the stream belongs to another device than the current one");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(GNN_ERR_DEVICE, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a)
      return fail(GNN_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_addr[dev] = a;
  }
  *out = g_scratch_addr[dev];
  return GNN_OK;
}

}  // namespace

int check_plan(const gnn_plan* p, const gnn_csr* csr) {
  if (p->n_rows != csr->n_rows || p->n_cols != csr->n_cols || p->nnz != csr->nnz ||
      p->row_ptr != csr->row_ptr || p->col_idx != csr->col_idx)
    return fail(GNN_ERR_PLAN_MISMATCH, "plan was built for another CSR");
  return GNN_OK;
}

}  // namespace gnn

using namespace gnn;

extern "C" {

const char* gnn_status_string(int status) {
  switch (status) {
    case GNN_OK: return "GNN_OK";
    case GNN_ERR_INVALID_VALUE: return "GNN_ERR_INVALID_VALUE";
    case GNN_ERR_UNSUPPORTED: return "GNN_ERR_UNSUPPORTED";
    case GNN_ERR_OUT_OF_MEMORY: return "GNN_ERR_OUT_OF_MEMORY";
    case GNN_ERR_DEVICE: return "GNN_ERR_DEVICE";
    case GNN_ERR_SIZE_OVERFLOW: return "GNN_ERR_SIZE_OVERFLOW";
    case GNN_ERR_PLAN_MISMATCH: return "GNN_ERR_PLAN_MISMATCH";
    default: return "GNN_ERR_UNKNOWN";
  }
}

const char* gnn_last_error(void) { return g_last_error.c_str(); }

int gnn_plan_create(const gnn_csr* csr, const gnn_plan_opts* opts, void* stream, gnn_plan** out) {
  if (!out) return fail(GNN_ERR_INVALID_VALUE, "out is NULL");
  *out = nullptr;
  GNN_TRY(check_csr(csr, false));
  if (opts) {
    if (opts->light_max_deg < 0 || opts->chunk_edges < 0 || opts->wsb_min_nnz < 0 || opts->att_slot_max < 0 ||
        opts->heavy_quantile > 1.0f)
      return fail(GNN_ERR_INVALID_VALUE, "invalid plan options");
    if (opts->build_wsb && csr->n_rows != csr->n_cols)
      return fail(GNN_ERR_INVALID_VALUE, "WSB tiles need a square CSR");
  }
  GNN_TRY(debug_validate(csr, (hipStream_t)stream));
  gnn_plan* p = new (std::nothrow) gnn_plan();
  if (!p) return fail(GNN_ERR_OUT_OF_MEMORY, "host allocation failed");
  int rc = plan_build(csr, opts, (hipStream_t)stream, p);
  if (rc != GNN_OK) {
    std::string keep = g_last_error;
    gnn_plan_destroy(p);
    g_last_error = keep;
    return rc;
  }
  *out = p;
  return GNN_OK;
}

int gnn_plan_destroy(gnn_plan* p) {
  if (!p) return GNN_OK;
  int rc = GNN_OK;
  if (p->tplan) {
    rc = gnn_plan_destroy(p->tplan);  // its CSR arrays belong to p and are freed below
    p->tplan = nullptr;
  }
  if (p->async_mem) {
    // a transient plan: everything is freed in stream order, no wait
    auto release = [&rc, p](void* ptr) {
      if (ptr && dev_free_async(ptr, p->stream) != GNN_OK) rc = GNN_ERR_DEVICE;
    };
    for (int k = 0; k < p->n_allocs; ++k) release(p->allocs[k]);
    release(p->ws);
    release(p->delta);
    release(p->dob);
    delete p;
    return rc;
  }
  if (p->n_allocs > 0 || p->ws) {
    if (hipStreamSynchronize(p->stream) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "plan stream sync failed");
  }
  auto release = [&rc](void* ptr) {
    if (ptr && hipFree(ptr) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "hipFree of a plan buffer failed");
  };
  for (int k = 0; k < p->n_allocs; ++k) release(p->allocs[k]);
  release(p->ws);
  release(p->delta);
  release(p->dob);
  delete p;
  return rc;
}

int gnn_plan_verify(gnn_plan* plan, const gnn_csr* csr, void* stream) {
  if (!plan) return fail(GNN_ERR_INVALID_VALUE, "plan is NULL");
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_plan(plan, csr));
  return plan_verify(plan, (hipStream_t)stream);
}

int gnn_plan_stats(const gnn_plan* p, int64_t* c, int32_t n) {
  if (!p || !c || n < 9) return fail(GNN_ERR_INVALID_VALUE, "plan_stats: null or n < 9");
  c[0] = p->n_light;
  c[1] = p->n_medium;
  c[2] = p->n_heavy;
  c[3] = p->n_items;
  c[4] = p->heavy_thr;
  c[5] = p->has_wsb ? p->wsb.n_windows : 0;
  c[6] = p->has_wsb ? p->wsb.n_blocks : 0;
  c[7] = p->has_wsb ? p->wsb.n_tiles : 0;
  c[8] = p->has_wsb ? p->wsb.n_resid : 0;
  for (int32_t k = 9; k < n; ++k) c[k] = 0;
  return GNN_OK;
}

int gnn_plan_wsb_export(const gnn_plan* p, int32_t* win_ptr, int32_t* blk_col, uint64_t* blk_bits,
                        void* stream) {
  if (!p || !win_ptr || !blk_col || !blk_bits) return fail(GNN_ERR_INVALID_VALUE, "wsb_export: NULL");
  if (!p->has_wsb) return fail(GNN_ERR_INVALID_VALUE, "plan has no WSB tiles");
  hipStream_t s = (hipStream_t)stream;
  GNN_HIP(hipMemcpyAsync(win_ptr, p->wsb.win_ptr, ((size_t)p->wsb.n_windows + 1) * 4,
                         hipMemcpyDeviceToDevice, s));
  if (p->wsb.n_blocks > 0) {
    GNN_HIP(hipMemcpyAsync(blk_col, p->wsb.blk_col, (size_t)p->wsb.n_blocks * 32,
                           hipMemcpyDeviceToDevice, s));
    GNN_HIP(hipMemcpyAsync(blk_bits, p->wsb.blk_bits, (size_t)p->wsb.n_blocks * 16,
                           hipMemcpyDeviceToDevice, s));
  }
  return GNN_OK;
}

int gnn_spmm(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx, float* Y,
             int64_t ldy, gnn_norm norm, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (norm < GNN_NORM_NONE || norm > GNN_NORM_BOTH) return fail(GNN_ERR_INVALID_VALUE, "unknown norm");
  if (F <= 0 || ldx < F || ldy < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldx >= F, ldy >= F");
  if (!Y || (!X && csr->n_cols > 0)) return fail(GNN_ERR_INVALID_VALUE, "X or Y is NULL");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  return launch_aggregate(p, X, xtype, F, ldx, Y, ldy, AGG_SPMM, norm, csr->edge_val, nullptr, s);
}

int gnn_spmm_block16(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx, float* Y,
                     int64_t ldy, gnn_norm norm, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, true));
  GNN_TRY(check_dtype(xtype));
  if (norm < GNN_NORM_NONE || norm > GNN_NORM_BOTH) return fail(GNN_ERR_INVALID_VALUE, "unknown norm");
  if (F <= 0 || ldx < F || ldy < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldx >= F, ldy >= F");
  if (!Y || (!X && csr->n_cols > 0)) return fail(GNN_ERR_INVALID_VALUE, "X or Y is NULL");
  if (csr->edge_val) return fail(GNN_ERR_UNSUPPORTED, "the block-sparse SpMM takes no edge values");
  const int64_t epc = xtype == GNN_BF16 ? 8 : 4;  // elements per 16-byte chunk
  if (F % epc != 0 || ldx % epc != 0 || ldy % 4 != 0 || ((uintptr_t)X | (uintptr_t)Y) % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "block-sparse SpMM needs 16-byte rows: F and ldx multiples of 16 bytes, "
                                     "ldy a multiple of 4, X and Y 16-byte aligned");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, true));
  PlanGuard g{p, tr};
  return launch_spmm_block16(p, X, xtype, F, ldx, Y, ldy, norm, s);
}

int gnn_reduce(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
               gnn_reduce_op op, float* Y, int64_t ldy, int32_t* arg, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (op < GNN_SUM || op > GNN_MIN) return fail(GNN_ERR_INVALID_VALUE, "unknown reduce op");
  if (F <= 0 || ldx < F || ldy < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldx >= F, ldy >= F");
  if (!Y || (!X && csr->n_cols > 0)) return fail(GNN_ERR_INVALID_VALUE, "X or Y is NULL");
  if (arg && (op == GNN_SUM || op == GNN_MEAN))
    return fail(GNN_ERR_INVALID_VALUE, "arg is only defined for MAX / MIN");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  int mode = op == GNN_SUM ? AGG_SUM : op == GNN_MEAN ? AGG_MEAN : op == GNN_MAX ? AGG_MAX : AGG_MIN;
  return launch_aggregate(p, X, xtype, F, ldx, Y, ldy, mode, GNN_NORM_NONE, nullptr, arg, s);
}

int gnn_reduce_multi(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
                     float* Y_sum, float* Y_mean, float* Y_max, int32_t* arg_max, float* Y_min,
                     int32_t* arg_min, int64_t ldy, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (F <= 0 || ldx < F || ldy < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldx >= F, ldy >= F");
  if (!Y_sum && !Y_mean && !Y_max && !Y_min) return fail(GNN_ERR_INVALID_VALUE, "no output requested");
  if ((arg_max && !Y_max) || (arg_min && !Y_min))
    return fail(GNN_ERR_INVALID_VALUE, "an index output needs its value output");
  if (!X && csr->n_cols > 0) return fail(GNN_ERR_INVALID_VALUE, "X is NULL");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  return launch_reduce_multi(p, X, xtype, F, ldx, Y_sum, Y_mean, Y_max, arg_max, Y_min, arg_min, ldy, s);
}

int gnn_reduce_multi_noalloc(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
                             float* Y_sum, float* Y_mean, float* Y_max, int32_t* arg_max, float* Y_min,
                             int32_t* arg_min, int64_t ldy, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (F <= 0 || ldx < F || ldy < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldx >= F, ldy >= F");
  if (!Y_sum && !Y_mean && !Y_max && !Y_min) return fail(GNN_ERR_INVALID_VALUE, "no output requested");
  if ((arg_max && !Y_max) || (arg_min && !Y_min))
    return fail(GNN_ERR_INVALID_VALUE, "an index output needs its value output");
  if (!X && csr->n_cols > 0) return fail(GNN_ERR_INVALID_VALUE, "X is NULL");
  if (!plan) return fail(GNN_ERR_INVALID_VALUE, "the allocation-free call needs a plan built beforehand");
  GNN_TRY(check_plan(plan, csr));
  if (csr->n_rows == 0) return GNN_OK;
  const size_t need = reduce_multi_ws_bytes(plan, F);
  if (need > kNoallocScratchBytes)
    return fail(GNN_ERR_SIZE_OVERFLOW, "the plan's split rows need " + std::to_string(need) +
                                           " bytes of scratch at this F; the allocation-free call holds at most " +
                                           std::to_string(kNoallocScratchBytes));
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (need > 0) GNN_TRY(scratch_address(s, &ws));
  return launch_reduce_multi(plan, X, xtype, F, ldx, Y_sum, Y_mean, Y_max, arg_max, Y_min, arg_min, ldy, s,
                             ws);
}

int gnn_gatv2_fused(const gnn_csr* csr, const void* xl, const void* xr, gnn_dtype xtype,
                    const float* att, int32_t H, int32_t D, float neg_slope, float* out, float* lse,
                    gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (H <= 0 || D <= 0) return fail(GNN_ERR_INVALID_VALUE, "need H > 0 and D > 0");
  if (!xl || !att || !out || (!xr && csr->n_cols > 0))
    return fail(GNN_ERR_INVALID_VALUE, "xl, xr, att or out is NULL");
  if ((int64_t)H * D >= ((int64_t)1 << 28)) return fail(GNN_ERR_SIZE_OVERFLOW, "H * D too large");
  GNN_TRY(attention_mapping_supported(0, xtype, H, D));
  if (((uintptr_t)xl | (uintptr_t)xr | (uintptr_t)out) % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "xl, xr and out must be 16-byte aligned");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, false, kAttSlotRows));
  PlanGuard g{p, tr};
  return launch_gatv2(p, xl, xr, xtype, att, H, D, neg_slope, out, lse, s);
}

int gnn_gt_fused(const gnn_csr* csr, const void* q, const void* k, const void* v, gnn_dtype xtype,
                 int32_t H, int32_t D, float scale, gnn_gt_mode mode, float* out, float* lse,
                 gnn_plan* plan, void* stream) {
  if (mode != GNN_GT_CSR && mode != GNN_GT_BLOCK16 && mode != GNN_GT_AUTO)
    return fail(GNN_ERR_INVALID_VALUE, "unknown GT mode");
  if (mode == GNN_GT_AUTO) {
    bool fits = xtype == GNN_BF16 && (D == 32 || D == 64 || D == 128 || D == 256) && csr &&
                csr->n_rows == csr->n_cols && H > 0 && (int64_t)H * D < ((int64_t)1 << 28);
    mode = GNN_GT_CSR;
    if (fits && plan && plan->has_wsb && check_plan(plan, csr) == GNN_OK) {
      const int64_t dense = plan->nnz - plan->wsb.n_resid;
      if (plan->wsb.n_tiles > 0 && 2 * dense >= plan->nnz && dense >= 32 * plan->wsb.n_tiles)
        mode = GNN_GT_BLOCK16;
    }
  }
  GNN_TRY(check_csr(csr, mode == GNN_GT_BLOCK16));
  GNN_TRY(check_dtype(xtype));
  if (H <= 0 || D <= 0) return fail(GNN_ERR_INVALID_VALUE, "need H > 0 and D > 0");
  if (!q || !out || ((!k || !v) && csr->n_cols > 0))
    return fail(GNN_ERR_INVALID_VALUE, "q, k, v or out is NULL");
  if ((int64_t)H * D >= ((int64_t)1 << 28)) return fail(GNN_ERR_SIZE_OVERFLOW, "H * D too large");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  if (mode == GNN_GT_BLOCK16 && (xtype != GNN_BF16 || (D != 32 && D != 64 && D != 128 && D != 256)))
    return fail(GNN_ERR_UNSUPPORTED, "BLOCK16 needs bf16 and D in {32, 64, 128, 256}");
  GNN_TRY(attention_mapping_supported(1, xtype, H, D));
  if (csr->n_rows == 0) return GNN_OK;
  float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)D);
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, mode == GNN_GT_BLOCK16, kAttSlotRows));
  PlanGuard g{p, tr};
  if (mode == GNN_GT_BLOCK16) return launch_gt_block16(p, q, k, v, H, D, sc, out, lse, s);
  return launch_gt_csr(p, q, k, v, xtype, H, D, sc, out, lse, s);
}

int gnn_project(const void* X, int32_t n, int32_t f_in, int64_t ldx, int32_t n_mat, const void* const* W,
                int32_t f_out, void* const* Y, void* stream) {
  if (n < 0 || f_in <= 0 || f_out <= 0) return fail(GNN_ERR_INVALID_VALUE, "need n >= 0, f_in > 0, f_out > 0");
  if (n_mat < 1 || n_mat > 3) return fail(GNN_ERR_INVALID_VALUE, "n_mat must be 1, 2 or 3");
  if (ldx < f_in) return fail(GNN_ERR_INVALID_VALUE, "need ldx >= f_in");
  if (!W || !Y) return fail(GNN_ERR_INVALID_VALUE, "W or Y is NULL");
  if (f_in % 32 != 0 || f_in > 512 || f_out % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "projection needs f_in a multiple of 32 up to 512 and f_out a multiple of 16");
  if (ldx % 8 != 0 || (uintptr_t)X % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "X must be 16-byte aligned with ldx a multiple of 8");
  for (int m = 0; m < n_mat; ++m) {
    if (!W[m] || !Y[m]) return fail(GNN_ERR_INVALID_VALUE, "a weight or output pointer is NULL");
    if (((uintptr_t)W[m] | (uintptr_t)Y[m]) % 16 != 0)
      return fail(GNN_ERR_UNSUPPORTED, "weights and outputs must be 16-byte aligned");
  }
  if ((int64_t)n * f_out >= ((int64_t)1 << 40)) return fail(GNN_ERR_SIZE_OVERFLOW, "output too large");
  if (n == 0) return GNN_OK;
  if (!X) return fail(GNN_ERR_INVALID_VALUE, "X is NULL");
  return launch_project(X, n, f_in, ldx, n_mat, W, f_out, Y, (hipStream_t)stream);
}

int gnn_spmm_backward(const gnn_csr* csr, const float* dY, int32_t F, int64_t ldy, float* dX, int64_t ldx,
                      gnn_norm norm, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  if (norm < GNN_NORM_NONE || norm > GNN_NORM_BOTH) return fail(GNN_ERR_INVALID_VALUE, "unknown norm");
  if (F <= 0 || ldy < F || ldx < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldy >= F, ldx >= F");
  if ((!dY && csr->n_rows > 0) || (!dX && csr->n_cols > 0)) return fail(GNN_ERR_INVALID_VALUE, "dY or dX is NULL");
  if (csr->n_cols == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  return launch_spmm_backward(p, dY, F, ldy, dX, ldx, norm, csr->edge_val, s);
}

int gnn_reduce_backward(const gnn_csr* csr, gnn_reduce_op op, const float* dY, int32_t F, int64_t ldy,
                        const int32_t* arg, float* dX, int64_t ldx, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  if (op < GNN_SUM || op > GNN_MIN) return fail(GNN_ERR_INVALID_VALUE, "unknown reduce op");
  if (F <= 0 || ldy < F || ldx < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0, ldy >= F, ldx >= F");
  if ((!dY && csr->n_rows > 0) || (!dX && csr->n_cols > 0)) return fail(GNN_ERR_INVALID_VALUE, "dY or dX is NULL");
  if ((op == GNN_MAX || op == GNN_MIN) && !arg && csr->n_rows > 0)
    return fail(GNN_ERR_INVALID_VALUE, "MAX / MIN backward needs the forward's arg");
  if (csr->n_cols == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  return launch_reduce_backward(p, op, dY, F, ldy, arg, dX, ldx, s);
}

int gnn_gatv2_backward(const gnn_csr* csr, const void* xl, const void* xr, gnn_dtype xtype, const float* att,
                       int32_t H, int32_t D, float neg_slope, const float* out, const float* lse,
                       const float* dout, float* dxl, float* dxr, float* datt, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (H <= 0 || D <= 0) return fail(GNN_ERR_INVALID_VALUE, "need H > 0 and D > 0");
  if (!att || !datt || ((!xl || !out || !lse || !dout || !dxl) && csr->n_rows > 0) ||
      ((!xr || !dxr) && csr->n_cols > 0))
    return fail(GNN_ERR_INVALID_VALUE, "a required tensor is NULL");
  const int64_t esz = xtype == GNN_BF16 ? 2 : 4;
  if ((int64_t)H * D >= ((int64_t)1 << 28)) return fail(GNN_ERR_SIZE_OVERFLOW, "H * D too large");
  if ((D * esz) % 16 != 0 || D * esz > 1024)
    return fail(GNN_ERR_UNSUPPORTED, "GATv2 backward needs D * element size a multiple of 16 bytes, at most 1 KB");
  if (((uintptr_t)xl | (uintptr_t)xr | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dxl | (uintptr_t)dxr) % 16)
    return fail(GNN_ERR_UNSUPPORTED, "row tensors must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, false, kAttSlotRows));
  PlanGuard g{p, tr};
  return launch_gatv2_backward(p, xl, xr, xtype, att, H, D, neg_slope, out, lse, dout, dxl, dxr, datt, s);
}

int gnn_gt_backward(const gnn_csr* csr, const void* q, const void* k, const void* v, gnn_dtype xtype, int32_t H,
                    int32_t D, float scale, const float* out, const float* lse, const float* dout, float* dq,
                    float* dk, float* dv, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, false));
  GNN_TRY(check_dtype(xtype));
  if (H <= 0 || D <= 0) return fail(GNN_ERR_INVALID_VALUE, "need H > 0 and D > 0");
  if (((!q || !out || !lse || !dout || !dq) && csr->n_rows > 0) || ((!k || !v || !dk || !dv) && csr->n_cols > 0))
    return fail(GNN_ERR_INVALID_VALUE, "a required tensor is NULL");
  const int64_t esz = xtype == GNN_BF16 ? 2 : 4;
  if ((int64_t)H * D >= ((int64_t)1 << 28)) return fail(GNN_ERR_SIZE_OVERFLOW, "H * D too large");
  if ((D * esz) % 16 != 0 || D * esz > 1024)
    return fail(GNN_ERR_UNSUPPORTED, "GT backward needs D * element size a multiple of 16 bytes, at most 1 KB");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) % 16)
    return fail(GNN_ERR_UNSUPPORTED, "row tensors must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, false, kAttSlotRows));
  PlanGuard g{p, tr};
  return launch_gt_backward(p, q, k, v, xtype, H, D, scale, out, lse, dout, dq, dk, dv, s);
}

int gnn_gt_backward_block16(const gnn_csr* csr, const void* q, const void* k, const void* v, int32_t H,
                            int32_t D, float scale, const float* out, const float* lse, const float* dout,
                            float* dq, float* dk, float* dv, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, true));
  if (H <= 0 || D <= 0) return fail(GNN_ERR_INVALID_VALUE, "need H > 0 and D > 0");
  if ((!q || !out || !lse || !dout || !dq || !k || !v || !dk || !dv) && csr->n_rows > 0)
    return fail(GNN_ERR_INVALID_VALUE, "a required tensor is NULL");
  if (D != 32 && D != 64 && D != 128)
    return fail(GNN_ERR_UNSUPPORTED, "block-sparse GT backward needs bf16 and D in {32, 64, 128}");
  if ((int64_t)H * D * 2 > 2048) return fail(GNN_ERR_UNSUPPORTED, "H*D*2 must be at most 2048 bytes");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) % 16)
    return fail(GNN_ERR_UNSUPPORTED, "row tensors must be 16-byte aligned");
  if (csr->n_rows == 0) return GNN_OK;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)D);
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr, true));
  PlanGuard g{p, tr};
  return launch_gt_backward_block16(p, q, k, v, H, D, sc, out, lse, dout, dq, dk, dv, s);
}

int gnn_reorder(const gnn_csr* csr, gnn_reorder_kind kind, int32_t* perm, int32_t* row_ptr_out,
                int32_t* col_idx_out, void* stream) {
  GNN_TRY(check_csr(csr, true));
  if (kind != GNN_REORDER_DEGREE && kind != GNN_REORDER_RCM)
    return fail(GNN_ERR_INVALID_VALUE, "unknown reorder kind");
  if (!perm) return fail(GNN_ERR_INVALID_VALUE, "perm is NULL");
  if ((row_ptr_out == nullptr) != (col_idx_out == nullptr))
    return fail(GNN_ERR_INVALID_VALUE, "give both row_ptr_out and col_idx_out, or neither");
  if (csr->n_rows == 0) return GNN_OK;
  GNN_TRY(debug_validate(csr, (hipStream_t)stream));
  return launch_reorder(csr, kind, perm, row_ptr_out, col_idx_out, (hipStream_t)stream);
}

int gnn_permute_rows(const int32_t* perm, int32_t n, const void* X, gnn_dtype xtype, int32_t F,
                     int64_t ldx, void* Xout, int64_t ldo, void* stream) {
  GNN_TRY(check_dtype(xtype));
  if (n < 0 || F <= 0 || ldx < F || ldo < F) return fail(GNN_ERR_INVALID_VALUE, "bad sizes");
  if (n == 0) return GNN_OK;
  if (!perm || !X || !Xout) return fail(GNN_ERR_INVALID_VALUE, "NULL pointer");
  return launch_permute_rows(perm, n, X, xtype == GNN_BF16 ? 2 : 4, F, ldx, Xout, ldo,
                             (hipStream_t)stream);
}

int gnn_dot_aggr(const gnn_csr* csr, const float* X, int32_t D, int64_t ldx, gnn_dot_map map,
                 gnn_dot_load load, float* y, gnn_plan* plan, void* stream) {
  GNN_TRY(check_csr(csr, true));
  if (map != GNN_DOT_FEATURE && map != GNN_DOT_NEIGHBOR) return fail(GNN_ERR_INVALID_VALUE, "unknown dot-aggr map");
  if (load != GNN_LOAD_SCALAR && load != GNN_LOAD_VEC16) return fail(GNN_ERR_INVALID_VALUE, "unknown load width");
  if (D <= 0 || ldx < D) return fail(GNN_ERR_INVALID_VALUE, "need D > 0 and ldx >= D");
  if (D > 1024) return fail(GNN_ERR_UNSUPPORTED, "dot-aggr supports D <= 1024");
  if (csr->edge_val) return fail(GNN_ERR_INVALID_VALUE, "dot-aggr takes no edge values");
  if (csr->n_rows > 0 && (!X || !y)) return fail(GNN_ERR_INVALID_VALUE, "X or y is NULL");
  if (load == GNN_LOAD_VEC16 && (D % 4 != 0 || ldx % 4 != 0 || (uintptr_t)X % 16 != 0))
    return fail(GNN_ERR_INVALID_VALUE, "16-byte loads need D and ldx multiples of 4 and X 16-byte aligned");
  if (csr->n_rows == 0) return GNN_OK;
  hipStream_t s = (hipStream_t)stream;
  gnn_plan* p = nullptr;
  bool tr = false;
  GNN_TRY(get_plan(csr, plan, s, &p, &tr));
  PlanGuard g{p, tr};
  return launch_dot_aggr(p, X, D, ldx, map == GNN_DOT_NEIGHBOR ? 1 : 0, load == GNN_LOAD_VEC16, y, s);
}

int gnn_release_cached_memory(void) { return release_cached_memory(); }

int gnn_copy_bytes(const void* src, void* dst, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!src || !dst))) return fail(GNN_ERR_INVALID_VALUE, "bad copy arguments");
  if (n == 0) return GNN_OK;
  return launch_copy(src, dst, n, (hipStream_t)stream);
}

}  // extern "C"
