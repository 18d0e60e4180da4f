// The transpose of a plan's CSR, and the backward passes that walk it:
// SpMM (dX = A_norm^T dY) and the reductions (sum / mean through the
// transpose; max / min by scattering each gradient element to the source the
// forward selected).
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations": the SpMM and reduction appendix (the forward Y = A X and
// its adjoint; the reduction backward as a sparse scatter-add into the stored
// argmin / argmax with atomic adds) and the attention appendix, whose
// backward walks the transposed CSR.
//
// The transpose is built once per plan: the entries of A are radix-sorted by
// (column, position), so within a transposed row they keep their order in A,
// and a full plan (bins, items) is built over it; the aggregation kernels then
// run on it unchanged.  Results are deterministic except for max / min, whose
// scatter adds through atomics (the order of additions into one element may
// vary between runs when several rows selected the same source).
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

// ends[e] = number of rows of A ending at entry position e (e < nnz), so the
// row of entry e is the number of rows ending at or before e.
__global__ void k_row_ends(const int32_t* row_ptr, int32_t n, int64_t nnz, int32_t* ends) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t e = row_ptr[i + 1];
  if (e < nnz) atomicAdd(&ends[e], 1);
}

__global__ void k_t_keys(const int32_t* col_idx, int64_t nnz, uint64_t* keys) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < nnz) keys[e] = ((uint64_t)(uint32_t)col_idx[e] << 32) | (uint64_t)e;
}

// entry t of A^T: its position in A and its column in A^T (the row in A,
// = the exclusive scan of `ends` at e + 1)
__global__ void k_t_fill(const uint64_t* keys, int64_t nnz, const int32_t* rows_excl, int32_t* t_col,
                         int32_t* t_edge) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nnz) return;
  const int32_t e = (int32_t)(uint32_t)keys[t];
  t_edge[t] = e;
  t_col[t] = rows_excl[e + 1];
}

__global__ void k_gather_f32(const float* src, const int32_t* idx, int64_t n, float* dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) dst[t] = src[idx[t]];
}

__global__ void k_zero_rows(float* X, int32_t n, int32_t F, int64_t ld) {
  const int64_t total = (int64_t)n * F;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / F, f = t - r * F;
    X[r * ld + f] = 0.0f;
  }
}

// dX[arg[i, f], f] += dY[i, f]; arg -1 (empty row) passes nothing, and
// indices outside [0, n_cols) are ignored rather than written.
__global__ void k_scatter_arg(const float* dY, int64_t ldy, const int32_t* arg, int32_t F, int32_t n_rows,
                              int32_t n_cols, float* dX, int64_t ldx) {
  const int64_t total = (int64_t)n_rows * F;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / F, f = t - i * F;
    const int32_t j = arg[t];
    if (j >= 0 && j < n_cols) atomicAdd(dX + (int64_t)j * ldx + f, dY[i * ldy + f]);
  }
}

unsigned grid_for(int64_t n, int64_t cap = 1 << 20) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, cap));
}

}  // namespace

int plan_transpose(gnn_plan* p, hipStream_t s) {
  if (p->tplan) return GNN_OK;
  const int32_t n = p->n_rows, nc = p->n_cols;
  const int64_t m = p->nnz;
  // (kept across a failed attempt, so that a retry reuses them)
  if (!p->t_row_ptr) GNN_TRY(plan_alloc(p, (void**)&p->t_row_ptr, ((size_t)nc + 1) * 4));
  if (!p->t_col) GNN_TRY(plan_alloc(p, (void**)&p->t_col, (size_t)std::max<int64_t>(m, 1) * 4));
  if (!p->t_edge) GNN_TRY(plan_alloc(p, (void**)&p->t_edge, (size_t)std::max<int64_t>(m, 1) * 4));
  // row pointers of A^T: the exclusive scan of the out-degrees
  GNN_TRY(plan_deg_out(p, s));
  GNN_TRY(exclusive_scan_i32(p->deg_out, p->t_row_ptr, nc, s));
  if (m > 0) {
    int32_t *ends = nullptr, *rows = nullptr;
    uint64_t *keys = nullptr, *tmp = nullptr;
    StreamTemps tt(s);
    GNN_TRY(tt.get(&ends, ((size_t)m + 1) * 4));
    GNN_TRY(tt.get(&rows, ((size_t)m + 1) * 4));
    GNN_TRY(tt.get(&keys, (size_t)m * 8));
    GNN_TRY(tt.get(&tmp, (size_t)m * 8));
    GNN_HIP(hipMemsetAsync(ends, 0, ((size_t)m + 1) * 4, s));
    hipLaunchKernelGGL(k_row_ends, dim3(grid_for(n)), dim3(256), 0, s, p->row_ptr, n, m, ends);
    GNN_LAUNCH_CHECK("transpose: row ends");
    int rc = exclusive_scan_i32(ends, rows, m, s);
    if (rc == GNN_OK) {
      hipLaunchKernelGGL(k_t_keys, dim3(grid_for(m, 1ll << 31)), dim3(256), 0, s, p->col_idx, m, keys);
      int cbits = 1;
      while (((int64_t)(nc > 0 ? nc - 1 : 0) >> cbits) != 0) ++cbits;
      rc = radix_sort_u64(keys, tmp, m, 32, 32 + cbits, s);
    }
    if (rc == GNN_OK) {
      hipLaunchKernelGGL(k_t_fill, dim3(grid_for(m, 1ll << 31)), dim3(256), 0, s, keys, m, rows, p->t_col,
                         p->t_edge);
      if (hipGetLastError() != hipSuccess) rc = fail(GNN_ERR_DEVICE, "transpose: fill launch failed");
    }
    if (rc != GNN_OK) return rc;
    GNN_TRY(tt.release());
  }
  gnn_csr t{};
  t.n_rows = nc;
  t.n_cols = n;
  t.nnz = m;
  t.row_ptr = p->t_row_ptr;
  t.col_idx = p->t_col;
  gnn_plan_opts o = p->opts;
  o.build_wsb = 0;
  gnn_plan* tp = new (std::nothrow) gnn_plan();
  if (!tp) return fail(GNN_ERR_OUT_OF_MEMORY, "host allocation failed");
  // a transient plan's transpose is transient too: built without a host wait
  const int rc = p->async_mem ? plan_build_async(&t, s, tp, p->light_max) : plan_build(&t, &o, s, tp);
  if (rc != GNN_OK) {
    for (int k = 0; k < tp->n_allocs; ++k)
      (void)(tp->async_mem ? dev_free_async(tp->allocs[k], s) : (int)hipFree(tp->allocs[k]));
    if (tp->ws) (void)(tp->async_mem ? dev_free_async(tp->ws, s) : (int)hipFree(tp->ws));
    delete tp;
    return rc;
  }
  p->tplan = tp;
  return GNN_OK;
}

// The block-sparse layout of A^T (windows of 16 source columns), built on the
// first block-sparse backward call with the plan's density threshold.
int plan_transpose_wsb(gnn_plan* p, hipStream_t s) {
  GNN_TRY(plan_transpose(p, s));
  if (p->tplan->has_wsb) return GNN_OK;
  p->tplan->opts.wsb_min_nnz = p->opts.wsb_min_nnz;
  return plan_build_wsb(p->tplan, s);
}

int launch_spmm_backward(gnn_plan* p, const float* dY, int32_t F, int64_t ldy, float* dX, int64_t ldx,
                         gnn_norm norm, const float* edge_val, hipStream_t s) {
  GNN_TRY(plan_transpose(p, s));
  const float* ev = nullptr;
  if (edge_val && p->nnz > 0) {
    if (!p->t_val) GNN_TRY(plan_alloc(p, (void**)&p->t_val, (size_t)p->nnz * 4));
    hipLaunchKernelGGL(k_gather_f32, dim3(grid_for(p->nnz, 1ll << 31)), dim3(256), 0, s, edge_val,
                       p->t_edge, p->nnz, p->t_val);
    GNN_LAUNCH_CHECK("transpose: edge values");
    ev = p->t_val;
  }
  // weights of A^T: 1 / deg_in(i) of the entry's source in A^T is RIGHT
  // there, 1 / deg_out(j) of its destination is LEFT there
  const gnn_norm tn = norm == GNN_NORM_LEFT ? GNN_NORM_RIGHT : (norm == GNN_NORM_RIGHT ? GNN_NORM_LEFT : norm);
  return launch_aggregate(p->tplan, dY, GNN_F32, F, ldy, dX, ldx, AGG_SPMM, tn, ev, nullptr, s);
}

int launch_reduce_backward(gnn_plan* p, int op, const float* dY, int32_t F, int64_t ldy, const int32_t* arg,
                           float* dX, int64_t ldx, hipStream_t s) {
  if (op == GNN_SUM) return launch_spmm_backward(p, dY, F, ldy, dX, ldx, GNN_NORM_NONE, nullptr, s);
  if (op == GNN_MEAN) return launch_spmm_backward(p, dY, F, ldy, dX, ldx, GNN_NORM_LEFT, nullptr, s);
  if (p->n_cols > 0) {
    hipLaunchKernelGGL(k_zero_rows, dim3(grid_for((int64_t)p->n_cols * F, 16384)), dim3(256), 0, s, dX,
                       p->n_cols, F, ldx);
    GNN_LAUNCH_CHECK("reduce backward: zero");
  }
  if (p->n_rows > 0) {
    hipLaunchKernelGGL(k_scatter_arg, dim3(grid_for((int64_t)p->n_rows * F, 65536)), dim3(256), 0, s, dY,
                       ldy, arg, F, p->n_rows, p->n_cols, dX, ldx);
    GNN_LAUNCH_CHECK("reduce backward: scatter");
  }
  return GNN_OK;
}

}  // namespace gnn
