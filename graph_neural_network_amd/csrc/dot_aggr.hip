// dot-aggr: the reordering micro-benchmark of Fomina et al., "On efficient
// scaling of GNNs via IO-aware layer implementations" (Experiments, graph
// reordering, Figure 1; appendix E.1, Figure 2).  For every destination i,
//     y_i = sum over the sources j of row i of <x_i, x_j>   (D features),
// computed by one wave per node in either of two mappings that perform the
// same multiply-adds but touch memory differently:
//   FEATURE   lanes own features: the wave walks the row's sources one after
//             another and reads each source row with coalesced loads (one
//             row per load instruction);
//   NEIGHBOR  lanes own sources: each lane walks the features of its own
//             source row, so one load instruction gathers from up to 64
//             different rows (x_i is staged in LDS and read as a broadcast).
// Each lane loads 4 bytes (SCALAR) or 16 bytes (VEC16) per instruction.
//
// Rows longer than the plan's split threshold are cut into the plan's edge
// chunks (the degree-aware split of appendix D.1), one wave per chunk in the
// same launch; a second launch adds the chunk partials in chunk order.  Both mappings see the same
// split, so the comparison between them is unchanged, and no single
// hub row's chain of dependent loads sets the kernel time.
#include <algorithm>
#include <type_traits>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int kWaves = 4;  // nodes (or chunks) per workgroup

struct DotParams {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const float* X;
  int64_t ldx;
  float* y;
  const int4* items;   // (row, e_begin, e_end, multi index or -1)
  float* partial;      // [n_items] one per chunk of a split row
  int64_t n_items;     // chunk items (a bound when item_count is set)
  const int32_t* item_count;  // device: the plan's item count, or NULL
  int32_t n;
  int32_t D;
  int32_t split_thr;   // rows with more edges run as chunks
};

template <bool VEC>
using Elem = typename std::conditional<VEC, float4, float>::type;

__device__ __forceinline__ float fma_dot(float a, float b, float acc) { return fmaf(a, b, acc); }
__device__ __forceinline__ float fma_dot(const float4& a, const float4& b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

template <bool VEC>
__device__ __forceinline__ Elem<VEC> zero() {
  if constexpr (VEC) return make_float4(0.f, 0.f, 0.f, 0.f);
  else return 0.f;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// FEATURE mapping over edges [beg, end) of row i.  Lane l holds elements
// [W (l + 64 k), +W) of x_i for k < K; the sources are taken U at a time
// (column indices loaded 64 at once and read lane by lane), so U source rows
// are in flight per wave.
template <bool VEC, int K, int U>
__device__ __forceinline__ float feature_part(const DotParams& p, int64_t i, int32_t beg, int32_t end,
                                              int lane) {
  constexpr int W = VEC ? 4 : 1;
  const float* xi_row = p.X + i * p.ldx;
  Elem<VEC> xi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int f = W * (lane + 64 * k);
    xi[k] = f < p.D ? *reinterpret_cast<const Elem<VEC>*>(xi_row + f) : zero<VEC>();
  }
  float acc = 0.f;
  for (int32_t e0 = beg; e0 < end; e0 += 64) {
    const int cnt = min(64, end - e0);
    const int32_t c = lane < cnt ? p.col_idx[e0 + lane] : 0;
    for (int t = 0; t < cnt; t += U) {
      Elem<VEC> v[U][K];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = t + u < cnt;  // uniform
        const float* xr = p.X + (int64_t)__builtin_amdgcn_readlane(c, ok ? t + u : 0) * p.ldx;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int f = W * (lane + 64 * k);
          v[u][k] = ok && f < p.D ? *reinterpret_cast<const Elem<VEC>*>(xr + f) : zero<VEC>();
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < K; ++k) acc = fma_dot(xi[k], v[u][k], acc);
    }
  }
  return acc;
}

// NEIGHBOR mapping over edges [beg, end): lane l takes edges beg + l,
// beg + l + 64, ...; for each it walks all D features of its source row, U
// loads per step.  x_i comes from LDS (the same address in every lane).
// Scalar loads walk U interleaved segments of the row so that no two loads
// of a step are adjacent (the compiler would otherwise fuse them into wider
// loads); 16-byte loads walk the row front to back.
template <bool VEC, int U>
__device__ __forceinline__ float neighbor_part(const DotParams& p, const float* s_xi, int32_t beg,
                                               int32_t end, int lane) {
  constexpr int W = VEC ? 4 : 1;
  const int D = p.D;
  float acc = 0.f;
  for (int32_t e = beg + lane; e < end; e += 64) {
    const float* xr = p.X + (int64_t)p.col_idx[e] * p.ldx;
    if constexpr (VEC) {
      int d = 0;
      for (; d + U * W <= D; d += U * W) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float4*>(xr + d + u * W);
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fma_dot(*reinterpret_cast<const float4*>(s_xi + d + u * W), v[u], acc);
      }
      for (; d < D; d += W)
        acc = fma_dot(*reinterpret_cast<const float4*>(s_xi + d), *reinterpret_cast<const float4*>(xr + d), acc);
    } else {
      // U segments of seg >= 2 features (adjacent loads only within a
      // segment, one step apart), then the tail one load at a time
      const int seg = D >= 2 * U ? D / U : 0;
#pragma unroll 1
      for (int t = 0; t < seg; ++t) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = xr[u * seg + t];
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fmaf(s_xi[u * seg + t], v[u], acc);
      }
#pragma unroll 1
      for (int d = U * seg; d < D; ++d) acc = fmaf(s_xi[d], xr[d], acc);
    }
  }
  return acc;
}

// Copy x_i into this wave's LDS slice; only this wave reads it afterwards.
template <bool VEC>
__device__ __forceinline__ void stage_xi(const DotParams& p, int64_t i, float* s_xi, int lane) {
  constexpr int W = VEC ? 4 : 1;
  const float* src = p.X + i * p.ldx;
  for (int f = W * lane; f < p.D; f += 64 * W)
    *reinterpret_cast<Elem<VEC>*>(s_xi + f) = *reinterpret_cast<const Elem<VEC>*>(src + f);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

enum Map { FEATURE = 0, NEIGHBOR = 1 };

template <int MAP, bool VEC, int K, int U>
__device__ __forceinline__ float dot_range(const DotParams& p, float* s_xi, int64_t i, int32_t beg,
                                           int32_t end, int lane) {
  if constexpr (MAP == FEATURE) {
    return feature_part<VEC, K, U>(p, i, beg, end, lane);
  } else {
    stage_xi<VEC>(p, i, s_xi, lane);
    return neighbor_part<VEC, U>(p, s_xi, beg, end, lane);
  }
}

// One launch: first the chunk waves of split rows (hardware order spreads them
// over the XCDs; their workgroup count is padded to a multiple of 8), each
// writing its chunk's partial dot-sum; then one wave per node, workgroups
// remapped in per-XCD runs, skipping the split rows.
template <int MAP, bool VEC, int K, int U>
__global__ __launch_bounds__(64 * kWaves) void k_dot(DotParams p, int32_t n_item_blocks) {
  extern __shared__ __align__(16) float s_dyn[];  // NEIGHBOR: [kWaves][D]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float* s_xi = s_dyn + (size_t)w * p.D;
  const int32_t n_item_pad = (n_item_blocks + 7) & ~7;
  if ((int32_t)blockIdx.x < n_item_pad) {
    const int64_t it = (int64_t)blockIdx.x * kWaves + w;
    if (it >= p.n_items || (p.item_count && it >= *p.item_count)) return;
    const int4 item = p.items[it];
    if (item.w < 0) return;  // a whole-row item: that row runs as a node
    const float acc = wave_sum(dot_range<MAP, VEC, K, U>(p, s_xi, item.x, item.y, item.z, lane));
    if (lane == 0) p.partial[it] = acc;
    return;
  }
  const uint32_t nb = gridDim.x - (uint32_t)n_item_pad;
  const int64_t i = (int64_t)dev::xcd_remap(blockIdx.x - (uint32_t)n_item_pad, nb) * kWaves + w;
  if (i >= p.n) return;
  const int32_t beg = p.row_ptr[i], end = p.row_ptr[i + 1];
  if (end - beg > p.split_thr) return;
  const float acc = wave_sum(dot_range<MAP, VEC, K, U>(p, s_xi, i, beg, end, lane));
  if (lane == 0) p.y[i] = acc;
}

// y[row] = the row's chunk partials added in chunk order (deterministic).
__global__ __launch_bounds__(256) void k_dot_combine(DotParams p, const int4* multi, int64_t n_multi,
                                                     const int32_t* multi_count) {
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= n_multi || (multi_count && m >= *multi_count)) return;
  const int4 mr = multi[m];
  float s = 0.f;
  for (int k = 0; k < mr.z; ++k) s += p.partial[mr.y + k];
  p.y[mr.x] = s;
}

template <int MAP, bool VEC, int K, int U>
int launch_shape(gnn_plan* pl, const DotParams& p, hipStream_t s) {
  const size_t lds = MAP == NEIGHBOR ? (size_t)kWaves * p.D * sizeof(float) : 0;
  const int64_t nb = (p.n + kWaves - 1) / kWaves;
  const int64_t ib = (p.n_items + kWaves - 1) / kWaves;
  const int64_t grid = ((ib + 7) & ~(int64_t)7) + nb;
  if (grid > 0x7FFFFFFF) return fail(GNN_ERR_SIZE_OVERFLOW, "dot-aggr: grid too large");
  hipLaunchKernelGGL((k_dot<MAP, VEC, K, U>), dim3((unsigned)grid), dim3(64 * kWaves), lds, s, p, (int32_t)ib);
  GNN_LAUNCH_CHECK("k_dot");
  if (pl->n_multi > 0) {
    const unsigned cb = (unsigned)((pl->n_multi + 255) / 256);
    hipLaunchKernelGGL(k_dot_combine, dim3(cb), dim3(256), 0, s, p, (const int4*)pl->multi, pl->n_multi,
                       pl->multi_count);
    GNN_LAUNCH_CHECK("k_dot_combine");
  }
  return GNN_OK;
}

// Feature slots per lane K (smallest power of two covering D) and sources in
// flight U (about 16 loads per lane per step).
template <bool VEC>
int launch_feature(gnn_plan* pl, const DotParams& p, hipStream_t s) {
  const int per = 64 * (VEC ? 4 : 1);  // features covered per slot
  const int k = (p.D + per - 1) / per;
  if (k <= 1) return launch_shape<FEATURE, VEC, 1, 8>(pl, p, s);
  if (k <= 2) return launch_shape<FEATURE, VEC, 2, 8>(pl, p, s);
  if (k <= 4) return launch_shape<FEATURE, VEC, 4, 4>(pl, p, s);
  if constexpr (!VEC) {
    if (k <= 8) return launch_shape<FEATURE, VEC, 8, 2>(pl, p, s);
    if (k <= 16) return launch_shape<FEATURE, VEC, 16, 1>(pl, p, s);
  }
  return fail(GNN_ERR_UNSUPPORTED, "dot-aggr: D too large");
}

}  // namespace

int launch_dot_aggr(gnn_plan* pl, const float* X, int32_t D, int64_t ldx, int map, bool vec, float* y,
                    hipStream_t s) {
  DotParams p{};
  p.row_ptr = pl->row_ptr;
  p.col_idx = pl->col_idx;
  p.X = X;
  p.ldx = ldx;
  p.y = y;
  p.n = pl->n_rows;
  p.D = D;
  // the plan's split rule: a row runs as several chunks exactly when it is
  // longer than the light limit, the heavy threshold and one chunk
  p.split_thr = std::max(std::max(pl->light_max, pl->heavy_thr), pl->chunk_edges);
  if (pl->n_multi > 0) {
    // the chunks of split rows are the first n_slots items
    p.items = pl->items;
    p.n_items = pl->n_slots;
    p.item_count = pl->item_count;
    void* ws = nullptr;
    GNN_TRY(plan_workspace(pl, (size_t)pl->n_slots * sizeof(float), &ws));
    p.partial = static_cast<float*>(ws);
  }
  if (map == FEATURE) return vec ? launch_feature<true>(pl, p, s) : launch_feature<false>(pl, p, s);
  return vec ? launch_shape<NEIGHBOR, true, 1, 4>(pl, p, s) : launch_shape<NEIGHBOR, false, 1, 8>(pl, p, s);
}

}  // namespace gnn
