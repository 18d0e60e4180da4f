// Measured choice of a plan's degree-binning knobs (gnn_plan_autotune).
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.1: the heavy-row threshold (a degree quantile)
// and the chunk size of split rows are autotuning parameters of the
// degree-aware reductions.  The candidates here are a small grid around the
// measured defaults; each is timed on the caller's graph and features through
// the library's own entry points.
#include <cfloat>
#include <vector>

#include "gnn_internal.h"

namespace gnn {
namespace {

struct Buffers {
  std::vector<void*> ptrs;
  ~Buffers() {
    for (void* q : ptrs) (void)hipFree(q);
  }
  int get(void** out, size_t bytes) {
    GNN_TRY(dev_malloc(out, std::max<size_t>(bytes, 16)));
    ptrs.push_back(*out);
    return GNN_OK;
  }
};

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

}  // namespace
}  // namespace gnn

using namespace gnn;

extern "C" int gnn_plan_autotune(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
                                 gnn_tune_op op, int32_t reps, gnn_plan_opts* best, float* best_ms,
                                 float* default_ms, void* stream) {
  if (!csr) return fail(GNN_ERR_INVALID_VALUE, "csr is NULL");
  if (!best || !best_ms) return fail(GNN_ERR_INVALID_VALUE, "best or best_ms is NULL");
  if (op != GNN_TUNE_SPMM && op != GNN_TUNE_SUM && op != GNN_TUNE_MULTI)
    return fail(GNN_ERR_INVALID_VALUE, "unknown autotune operation");
  if (reps < 1 || reps > 1000) return fail(GNN_ERR_INVALID_VALUE, "reps must be in [1, 1000]");
  if (xtype != GNN_F32 && xtype != GNN_BF16) return fail(GNN_ERR_INVALID_VALUE, "unknown dtype");
  if (F <= 0 || ldx < F) return fail(GNN_ERR_INVALID_VALUE, "need F > 0 and ldx >= F");
  if (!X && csr->n_cols > 0) return fail(GNN_ERR_INVALID_VALUE, "X is NULL");
  if (csr->n_rows < 0 || csr->nnz < 0) return fail(GNN_ERR_INVALID_VALUE, "negative CSR size");
  hipStream_t s = (hipStream_t)stream;

  // outputs of the timed operation, [n_rows, F]
  const size_t out_bytes = (size_t)std::max(csr->n_rows, 1) * (size_t)F * 4;
  Buffers buf;
  float* y[4] = {};
  int32_t* arg[2] = {};
  const int n_val = op == GNN_TUNE_MULTI ? 4 : 1;
  for (int i = 0; i < n_val; ++i) GNN_TRY(buf.get((void**)&y[i], out_bytes));
  if (op == GNN_TUNE_MULTI)
    for (int i = 0; i < 2; ++i) GNN_TRY(buf.get((void**)&arg[i], out_bytes));
  Events ev;
  GNN_HIP(hipEventCreate(&ev.a));
  GNN_HIP(hipEventCreate(&ev.b));

  auto run = [&](gnn_plan* plan) -> int {
    if (op == GNN_TUNE_SPMM) return gnn_spmm(csr, X, xtype, F, ldx, y[0], F, GNN_NORM_NONE, plan, stream);
    if (op == GNN_TUNE_SUM) return gnn_reduce(csr, X, xtype, F, ldx, GNN_SUM, y[0], F, nullptr, plan, stream);
    return gnn_reduce_multi(csr, X, xtype, F, ldx, y[0], y[1], y[2], arg[0], y[3], arg[1], F, plan, stream);
  };

  const float gammas[3] = {0.99f, 0.999f, -1.0f};
  const int32_t lights[2] = {16, 32};
  const int32_t chunks[2] = {256, 1024};
  float t_best = FLT_MAX, t_default = -1.0f;
  gnn_plan_opts o_best{};
  for (float gm : gammas)
    for (int32_t lt : lights)
      for (int32_t ch : chunks) {
        gnn_plan_opts o{};
        o.heavy_quantile = gm;
        o.light_max_deg = lt;
        o.chunk_edges = ch;
        gnn_plan* plan = nullptr;
        GNN_TRY(gnn_plan_create(csr, &o, stream, &plan));
        int rc = run(plan);  // untimed
        if (rc == GNN_OK && hipEventRecord(ev.a, s) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event record");
        for (int r = 0; rc == GNN_OK && r < reps; ++r) rc = run(plan);
        if (rc == GNN_OK && hipEventRecord(ev.b, s) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event record");
        if (rc == GNN_OK && hipEventSynchronize(ev.b) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event sync");
        float ms = 0.0f;
        if (rc == GNN_OK && hipEventElapsedTime(&ms, ev.a, ev.b) != hipSuccess)
          rc = fail(GNN_ERR_DEVICE, "event time");
        const int rd = gnn_plan_destroy(plan);
        if (rc != GNN_OK) return rc;
        if (rd != GNN_OK) return rd;
        ms /= (float)reps;
        if (gm == 0.99f && lt == 32 && ch == 1024) t_default = ms;
        if (ms < t_best) {
          t_best = ms;
          o_best = o;
        }
      }
  *best = o_best;
  *best_ms = t_best;
  if (default_ms) *default_ms = t_default;
  GNN_HIP(hipStreamSynchronize(s));
  return GNN_OK;
}
