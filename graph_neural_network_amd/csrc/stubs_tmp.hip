#include "gnn_internal.h"
namespace gnn {
int launch_gt_block16(gnn_plan*, const void*, const void*, const void*, int32_t, int32_t, float, float*, float*, hipStream_t) { return fail(GNN_ERR_UNSUPPORTED, "not built yet"); }
int launch_reorder(const gnn_csr*, gnn_reorder_kind, int32_t*, int32_t*, int32_t*, hipStream_t) { return fail(GNN_ERR_UNSUPPORTED, "not built yet"); }
int plan_build_wsb(gnn_plan*, hipStream_t) { return fail(GNN_ERR_UNSUPPORTED, "not built yet"); }
}
