// Measured choice of a plan's knobs (gnn_plan_autotune for the aggregations,
// gnn_plan_autotune_attention for the fused attention layers).
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.1: the heavy-row threshold (a degree quantile)
// and the chunk size of split rows are autotuning parameters of the
// degree-aware kernels; appendix D.3 and section 5 choose between the CSR and
// the block-sparse (WSB) attention by the graph's local density.  The
// candidates here are small grids around the measured defaults; each is timed
// on the caller's graph and inputs through the library's own entry points.
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

extern "C" int gnn_plan_autotune_attention(const gnn_csr* csr, gnn_tune_att_op op, const void* q, const void* k,
                                           const void* v, gnn_dtype xtype, const float* att, int32_t H, int32_t D,
                                           int32_t reps, gnn_plan_opts* best, gnn_gt_mode* best_mode,
                                           float* best_ms, float* default_ms, void* stream) {
  if (!csr) return fail(GNN_ERR_INVALID_VALUE, "csr is NULL");
  if (!best || !best_ms || !best_mode) return fail(GNN_ERR_INVALID_VALUE, "best, best_mode or best_ms is NULL");
  if (op != GNN_TUNE_GATV2 && op != GNN_TUNE_GT) return fail(GNN_ERR_INVALID_VALUE, "unknown attention operation");
  if (reps < 1 || reps > 1000) return fail(GNN_ERR_INVALID_VALUE, "reps must be in [1, 1000]");
  if (xtype != GNN_F32 && xtype != GNN_BF16) return fail(GNN_ERR_INVALID_VALUE, "unknown dtype");
  if (H <= 0 || D <= 0 || (int64_t)H * D >= ((int64_t)1 << 28)) return fail(GNN_ERR_INVALID_VALUE, "bad H or D");
  if (csr->n_rows < 0 || csr->nnz < 0) return fail(GNN_ERR_INVALID_VALUE, "negative CSR size");
  if (op == GNN_TUNE_GATV2 && !att) return fail(GNN_ERR_INVALID_VALUE, "att is NULL");
  if (csr->n_rows > 0 && (!q || !k || (op == GNN_TUNE_GT && !v)))
    return fail(GNN_ERR_INVALID_VALUE, "an input is NULL");
  GNN_TRY(attention_mapping_supported(op == GNN_TUNE_GT ? 1 : 0, xtype, H, D));
  hipStream_t s = (hipStream_t)stream;

  // outputs of the timed operation
  Buffers buf;
  float* out = nullptr;
  float* lse = nullptr;
  GNN_TRY(buf.get((void**)&out, (size_t)std::max(csr->n_rows, 1) * H * D * 4));
  GNN_TRY(buf.get((void**)&lse, (size_t)std::max(csr->n_rows, 1) * H * 4));
  Events ev;
  GNN_HIP(hipEventCreate(&ev.a));
  GNN_HIP(hipEventCreate(&ev.b));

  auto run = [&](gnn_plan* plan, gnn_gt_mode mode) -> int {
    if (op == GNN_TUNE_GATV2) return gnn_gatv2_fused(csr, q, k, xtype, att, H, D, 0.2f, out, lse, plan, stream);
    return gnn_gt_fused(csr, q, k, v, xtype, H, D, 0.0f, mode, out, lse, plan, stream);
  };
  auto time_it = [&](const gnn_plan_opts& o, gnn_gt_mode mode, float* ms) -> int {
    gnn_plan* plan = nullptr;
    GNN_TRY(gnn_plan_create(csr, &o, stream, &plan));
    int rc = run(plan, mode);  // untimed
    if (rc == GNN_OK && hipEventRecord(ev.a, s) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event record");
    for (int r = 0; rc == GNN_OK && r < reps; ++r) rc = run(plan, mode);
    if (rc == GNN_OK && hipEventRecord(ev.b, s) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event record");
    if (rc == GNN_OK && hipEventSynchronize(ev.b) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event sync");
    if (rc == GNN_OK && hipEventElapsedTime(ms, ev.a, ev.b) != hipSuccess) rc = fail(GNN_ERR_DEVICE, "event time");
    const int rd = gnn_plan_destroy(plan);
    if (rc != GNN_OK) return rc;
    if (rd != GNN_OK) return rd;
    *ms /= (float)reps;
    return GNN_OK;
  };

  float t_best = FLT_MAX;
  gnn_plan_opts o_best{};
  gnn_gt_mode m_best = GNN_GT_CSR;
  // CSR kernel: split threshold x chunk size x one-slot bound
  const float gammas[3] = {0.99f, 0.999f, -1.0f};
  const int32_t chunks[2] = {256, 1024};
  const int32_t slots[3] = {32, 128, 512};
  for (float gm : gammas)
    for (int32_t ch : chunks)
      for (int32_t sm : slots) {
        gnn_plan_opts o{};
        o.heavy_quantile = gm;
        o.chunk_edges = ch;
        o.att_slot_max = sm;
        float ms = 0.0f;
        GNN_TRY(time_it(o, GNN_GT_CSR, &ms));
        if (ms < t_best) {
          t_best = ms;
          o_best = o;
          m_best = GNN_GT_CSR;
        }
      }
  // block-sparse kernel (the choice AUTO makes from density), tile threshold tau
  const bool b16 = op == GNN_TUNE_GT && xtype == GNN_BF16 && csr->n_rows == csr->n_cols &&
                   (D == 32 || D == 64 || D == 128 || D == 256);
  if (b16) {
    const int32_t taus[3] = {1, 8, 32};
    for (int32_t tau : taus) {
      gnn_plan_opts o{};
      o.build_wsb = 1;
      o.wsb_min_nnz = tau;
      float ms = 0.0f;
      GNN_TRY(time_it(o, GNN_GT_BLOCK16, &ms));
      if (ms < t_best) {
        t_best = ms;
        o_best = o;
        m_best = GNN_GT_BLOCK16;
      }
    }
  }
  if (default_ms) {
    // the library's defaults: a default plan (with WSB tiles where BLOCK16 could run) and AUTO
    gnn_plan_opts o{};
    o.build_wsb = b16 ? 1 : 0;
    GNN_TRY(time_it(o, op == GNN_TUNE_GT ? GNN_GT_AUTO : GNN_GT_CSR, default_ms));
  }
  *best = o_best;
  *best_mode = m_best;
  *best_ms = t_best;
  GNN_HIP(hipStreamSynchronize(s));
  return GNN_OK;
}
