// Fused CSR attention: GATv2 and Graph Transformer forward in one pass over
// each destination's neighbours, with an online softmax, so that no per-edge
// logit, weight or message ever reaches memory.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations":
//   section 2.2 (iii): h_i' = sum_j alpha_ij v_j, alpha = softmax_j(e_ij);
//     GATv2 e_ij = a^T LeakyReLU(W_l h_i + W_r h_j), v_j = W_r h_j;
//     Graph Transformer e_ij = q_i . k_j / sqrt(D);
//   appendix D.2: fused CSR kernels, online softmax with the running
//     (max, sum) and the accumulator rescaled by exp(m_old - m_new), partial
//     states of parallel workers merged by rescaling each with
//     exp(m_w - m_global), logsumexp kept per (node, head).
//
// MI355X mapping.  An edge's feature row (all heads) is spread over a slot of
// LPE lanes, VB = 16 or 32 bytes per lane; the lanes of one head (LPH, a power
// of two: a head whose slices fill fewer lanes leaves the rest of its group
// idle) reduce the score with lane swaps.  Config examples: GATv2 H = 4,
// D = 32 bf16 is a 256-byte row = 16 lanes, four edges per wave instruction;
// GT H = 8, D = 64 bf16 is a 1-KB row = one full wave per edge for K and one
// for V.  Rows wider than a slot are cut into head groups of one slot each,
// one group per grid row (blockIdx.y); each group walks the same edges.
// Heads whose byte width is not a multiple of 16 take the generic mapping:
// 8-, 4- or 2-byte slices per lane, 64-lane slots, lanes per head known at
// run time (the pages' fallback beside the head-dimension specialisations,
// appendix D.2).  Each slot keeps its own (m, l, acc) state over U = 4 edges in
// flight; slots of a wave, waves of a workgroup and chunks of a split row
// are merged with the same rescaling rule.  Logits live in the log2 domain
// (log2 e folded into a or into q * scale) so every exponential is exp2.
//   light rows : one slot per row up to 128 edges, rows taken from the
//                plan's list in order of decreasing length, so that the four
//                slots of a wave run the same number of steps
//   items      : one workgroup per longer row or per chunk of a heavy row;
//                chunks of a heavy row leave partial (m, l, acc) states that a
//                combine kernel merges in chunk order.
#include <algorithm>

#include "att_common.h"

namespace gnn {
namespace {

using namespace att;

constexpr int WG = 256;
#ifndef GNN_ATT_U
#define GNN_ATT_U 4
#endif
#ifndef GNN_ATT_LIGHT_MAX
#define GNN_ATT_LIGHT_MAX 128
#endif
constexpr int32_t kAttLightMax = GNN_ATT_LIGHT_MAX;

enum { K_GATV2 = 0, K_GT = 1 };

struct AttParams {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* q;     // GATv2: x_l [n_rows, H, D]; GT: q
  const void* k;     // GATv2: x_r [n_cols, H, D]; GT: k
  const void* v;     // GT: v (GATv2: same as k)
  const float* att;  // GATv2: a [H, D]
  float* out;        // [n_rows, H, D]
  float* lse;        // [n_rows, H] or null
  const int4* items;
  float* pacc;       // [n_slots, H * D] partial accumulators of split rows
  float* pml;        // [n_slots, 2, H] partial (m, l) of split rows
  int32_t n_rows;
  int32_t H, D;
  int32_t row_elems;  // H * D
  int32_t lph;        // lanes per head (power of two)
  int32_t lph_data;   // of which hold data (D / VEL)
  int32_t hpg;        // heads per group (one group per grid row)
  int32_t dv;         // D / VEL: lane slices per head
  int32_t light_max;         // rows of at most this many edges take one slot
  const int32_t* att_rows;   // those rows, longest first
  const int32_t* att_count;  // device: how many
  int32_t n_item_blocks;
  const int32_t* item_count;  // device item count (NULL: n_item_blocks is exact)
  const int32_t* multi_count; // device split-row count (NULL: the launch's row count is exact)
  int32_t n_light_blocks;
  float slope;        // GATv2 LeakyReLU slope
  float qscale;       // GT: scale * log2(e)
  int32_t kv_bytes;   // bytes of K (and of V) when below 2^31, else 0
};

// Online-softmax state of one slot lane: running max m (log2 units), running
// sum l, accumulator acc over this lane's VEL output elements.
template <int VEL>
struct Soft {
  float m, l;
  float acc[VEL];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int k = 0; k < VEL; ++k) acc[k] = 0.0f;
  }
  // merge another state (m2, l2, acc2) into this one
  __device__ __forceinline__ void merge(float m2, float l2, const float (&a2)[VEL]) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;  // both empty
    const float c1 = ex2(m - mn), c2 = ex2(m2 - mn);
    l = l * c1 + l2 * c2;
#pragma unroll
    for (int k = 0; k < VEL; ++k) acc[k] = acc[k] * c1 + a2[k] * c2;
    m = mn;
  }
};

template <int VEL>
__device__ __forceinline__ void shfl_merge(Soft<VEL>& s, int lane_xor) {
  float m2 = __shfl_xor(s.m, lane_xor, 64);
  float l2 = __shfl_xor(s.l, lane_xor, 64);
  float a2[VEL];
#pragma unroll
  for (int k = 0; k < VEL; ++k) a2[k] = __shfl_xor(s.acc[k], lane_xor, 64);
  s.merge(m2, l2, a2);
}

// Process edges [eb, ee) of destination `row` for one slot, UU edges in
// flight.
//   qv / qraw : this lane's slice of the destination-side vector (GATv2: x_l
//               as float; GT: q, raw, its scale * log2 e applied after the
//               head reduction)
//   av, an    : GATv2 attention-vector slice times log2 e times (1 + slope) / 2
//               and (1 - slope) / 2 (unused for GT): a * LReLU(z) =
//               av * z + an * |z|, two multiply-adds (|z| is a free operand
//               modifier) instead of a multiply, a max and a multiply-add
template <typename T, int LPE, int VB, int KIND, int UU, int LPH>
__device__ __forceinline__ void scan_edges(const AttParams& p, int eb, int ee, int sl, int slot_base,
                                           uint32_t loff, const float (&qv)[VB / sizeof(T)],
                                           const RawB<VB>& qraw, const float (&av)[VB / sizeof(T)],
                                           const float (&an)[VB / sizeof(T)], Soft<VB / sizeof(T)>& st) {
  constexpr int VEL = VB / (int)sizeof(T);
  constexpr int NW = VB >= 4 ? VB / 4 : 1;
  const T* K = reinterpret_cast<const T*>(p.k);
  const T* V = reinterpret_cast<const T*>(p.v);
  // loff: this lane's slice of a row; lanes without data read their head
  // group's first slice (their query / attention-vector slices are zero, so
  // they add nothing)
  const int64_t ld = p.row_elems;
  const int row_bytes = p.row_elems * (int)sizeof(T);
  const uint32_t loff_b = loff * (uint32_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(K), (short)0, p.kv_bytes,
                                                                      kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(V), (short)0, p.kv_bytes,
                                                                      kBufferWord3);
  for (int e0 = eb; e0 < ee; e0 += LPE) {
    const int nb = min(LPE, ee - e0);
    const int my_c = (sl < nb) ? p.col_idx[e0 + sl] : 0;
    for (int u0 = 0; u0 < nb; u0 += UU) {
      int c[UU];
      RawB<VB> x[UU];
      RawB<VB> y[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u)
        c[u] = (LPE == 64) ? __builtin_amdgcn_readlane(my_c, u0 + u)  // one slot per wave: scalar
                           : __shfl(my_c, slot_base + u0 + u, 64);
      // every slot loads UU rows without branches: edges past the slot's end
      // re-read its first edge's row (finite values; their score is -inf, so
      // their weight is 0)
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int cu = (u0 + u < nb) ? c[u] : c[0];
        if constexpr (LPE == 64) {
          // the wave's row: its byte offset in a scalar register (one
          // descriptor over the array), or its base in one of its own
          if (p.kv_bytes > 0) {
            const uint32_t ro = (uint32_t)cu * (uint32_t)row_bytes;
            load_rawb_buf_so<VB>(rk, loff_b, ro, x[u]);
            if constexpr (KIND == K_GT) load_rawb_buf_so<VB>(rv, loff_b, ro, y[u]);
          } else {
            load_rawb_buf<VB>(row_rsrc(K + (int64_t)cu * ld, row_bytes), loff_b, x[u]);
            if constexpr (KIND == K_GT) load_rawb_buf<VB>(row_rsrc(V + (int64_t)cu * ld, row_bytes), loff_b, y[u]);
          }
        } else {
          load_rawb<T, VB>(row_at(K + loff, cu, (uint32_t)row_bytes), x[u]);
          if constexpr (KIND == K_GT) load_rawb<T, VB>(row_at(V + loff, cu, (uint32_t)row_bytes), y[u]);
        }
      }
      float s[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        float t = 0.0f;
        if constexpr (KIND == K_GATV2) {
#pragma unroll
          for (int k = 0; k < VEL; ++k) {
            const float z = qv[k] + elemb<T, VB>(x[u], k);
            t = fmaf(av[k], z, fmaf(an[k], fabsf(z), t));
          }
        } else if constexpr (sizeof(T) == 2) {
          // a 2-byte slice has a zero high half in both words
#pragma unroll
          for (int k = 0; k < NW; ++k)
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qraw.u[k]),
                                                __builtin_bit_cast(bf16x2_t, x[u].u[k]), t, false);
        } else {
#pragma unroll
          for (int k = 0; k < VEL; ++k) t = fmaf(qv[k], elemb<T, VB>(x[u], k), t);
        }
        if constexpr (LPH > 0) t = head_sum<LPH>(t);
        else t = head_sum_rt(t, p.lph);
        s[u] = (u0 + u < nb) ? t : -INFINITY;
      }
      // GT scores stay unscaled until the exponent: the batch maximum is
      // scaled once, each weight is exp2(fma(s, scale log2 e, -max))
      // (scale > 0; an edge past the slot's end gives exp2(-inf) = 0)
      float mx = s[0];
#pragma unroll
      for (int u = 1; u < UU; ++u) mx = fmaxf(mx, s[u]);
      const float qs = (KIND == K_GT) ? p.qscale : 1.0f;
      const float mn = fmaxf(st.m, (KIND == K_GT) ? mx * qs : mx);
      const float corr = ex2(st.m - mn);
      st.l *= corr;
#pragma unroll
      for (int k = 0; k < VEL; ++k) st.acc[k] *= corr;
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const float pu = ex2((KIND == K_GT) ? fmaf(s[u], qs, -mn) : s[u] - mn);
        st.l += pu;
#pragma unroll
        for (int k = 0; k < VEL; ++k)
          st.acc[k] = fmaf(pu, (KIND == K_GT) ? elemb<T, VB>(y[u], k) : elemb<T, VB>(x[u], k), st.acc[k]);
      }
      st.m = mn;
    }
  }
}

// Output slice of one slot: the head group's elements [goff, goff + gel) of
// the row; this lane's VEL elements sit at loff (valid when d_ok).  A lane
// with VEL > 4 holds more than 16 contiguous bytes, and stored directly each
// instruction would leave every 128-byte line half written (such rows reach
// HBM at a third of its write bandwidth), so the slice is staged in LDS
// (`stage`, LPE * VEL words of this slot) and stored as 16 contiguous bytes
// per lane.  Called by every lane of the slot.
template <int LPE, int VEL>
__device__ __forceinline__ void write_final(const AttParams& p, int64_t row, int head, bool d_ok, bool lead,
                                            uint32_t loff, uint32_t goff, int gel, int sl, const Soft<VEL>& st,
                                            float* stage) {
  float o[VEL];
  const float inv = st.l > 0.0f ? 1.0f / st.l : 0.0f;
#pragma unroll
  for (int k = 0; k < VEL; ++k) o[k] = st.acc[k] * inv;
  float* dst = p.out + row * p.row_elems;
  if constexpr (VEL <= 4) {
    if (d_ok) store_elems_nt<VEL>(dst + loff, o);
  } else {
    if (d_ok) store_row<VEL>(stage + (loff - goff), o);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < VEL / 4; ++j) {
      const int c = (j * LPE + sl) * 4;
      const float4 t = *reinterpret_cast<const float4*>(stage + c);
      if (c < gel)
        __builtin_nontemporal_store(nt_f32x4{t.x, t.y, t.z, t.w}, reinterpret_cast<nt_f32x4*>(dst + goff + c));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (p.lse && d_ok && lead)
    p.lse[row * p.H + head] = st.l > 0.0f ? st.m * kLn2 + logf(st.l) : -INFINITY;
}

// GATv2 asks for five waves per SIMD (90 VGPRs, no spills): left alone the
// compiler takes 103 and four, and the VALU-bound kernel runs 7% slower.
template <typename T, int LPE, int VB, int KIND, int UU, int LPH>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(KIND == K_GATV2 ? 5 : 1))) void k_attention(
    AttParams p) {
  constexpr int VEL = VB / (int)sizeof(T);  // elements per lane
  constexpr int SPW = 64 / LPE;
  constexpr int NWAVE = WG / 64;
  constexpr int NW = VB >= 4 ? VB / 4 : 1;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave; saying so keeps a 64-lane
  // slot's row, edge range and gathered row addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sw = lane / LPE, sl = lane % LPE;
  const int slot_base = sw * LPE;
  // head group of this grid row; this lane's head in it and slice of the head
  const int lph = LPH > 0 ? LPH : p.lph;
  const int hin = sl / lph, j = sl % lph;
  const int g0 = (int)blockIdx.y * p.hpg;
  const int hg = g0 + hin;
  const bool d_ok = hin < p.hpg && hg < p.H && j < p.lph_data;
  const int head = d_ok ? hg : 0;
  const uint32_t goff = (uint32_t)g0 * p.D;
  // a multiple of VEL by construction (D = dv * VEL), so slice loads and
  // stores stay vectorised
  const uint32_t loff = d_ok ? (uint32_t)((hg * p.dv + j) * VEL) : goff;
  const int gel = (min(p.H, g0 + p.hpg) - g0) * p.D;

  const int n_item_pad = (p.n_item_blocks + 7) & ~7;
  const bool is_item = (int)blockIdx.x < n_item_pad;
  int64_t row;
  int eb, ee, m_idx = -1, item = -1;
  if (is_item) {
    item = (int)dev::xcd_remap(blockIdx.x, n_item_pad);
    if (item >= p.n_item_blocks) return;
    if (p.item_count && item >= *p.item_count) return;
    const int4 it = p.items[item];
    // single-chunk rows short enough for the light path are processed there
    if (it.w < 0 && it.z - it.y <= p.light_max) return;
    row = it.x;
    m_idx = it.w;
    // split the item's edges over all slots of the workgroup
    const int nslots = SPW * NWAVE;
    const int slot = wave * SPW + sw;
    const int len = it.z - it.y;
    const int per = (len + nslots - 1) / nslots;
    eb = min(it.z, it.y + slot * per);
    ee = min(it.z, eb + per);
  } else {
    const uint32_t lb = dev::xcd_remap(blockIdx.x - n_item_pad, p.n_light_blocks);
    const int64_t idx = ((int64_t)lb * NWAVE + wave) * SPW + sw;
    if (idx >= *p.att_count) return;
    row = p.att_rows[idx];
    eb = p.row_ptr[row];
    ee = p.row_ptr[row + 1];
  }

  // destination-side slice (and the attention vector for GATv2)
  float qv[VEL], av[VEL], an[VEL];
  RawB<VB> qraw;
  if (d_ok) {
    load_rawb<T, VB>(reinterpret_cast<const T*>(p.q) + row * p.row_elems + loff, qraw);
#pragma unroll
    for (int k = 0; k < VEL; ++k) qv[k] = elemb<T, VB>(qraw, k);
    if constexpr (KIND == K_GATV2) {
#pragma unroll
      for (int k = 0; k < VEL; ++k) {
        const float a = p.att[loff + k] * kLog2e;
        av[k] = a * (0.5f + 0.5f * p.slope);
        an[k] = a * (0.5f - 0.5f * p.slope);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < NW; ++k) qraw.u[k] = 0u;
#pragma unroll
    for (int k = 0; k < VEL; ++k) qv[k] = av[k] = an[k] = 0.0f;
  }

  Soft<VEL> st;
  st.init();
  scan_edges<T, LPE, VB, KIND, UU, LPH>(p, eb, ee, sl, slot_base, loff, qv, qraw, av, an, st);

  // s_a merges the waves of an item; light rows stage their output in it
  // (one LPE x VEL region per slot)
  __shared__ __align__(16) float s_a[NWAVE][64][VEL];
  if (!is_item) {
    write_final<LPE, VEL>(p, row, head, d_ok, j == 0, loff, goff, gel, sl, st, &s_a[wave][slot_base][0]);
    return;
  }

  // merge the slots of each wave, then the waves through LDS
#pragma unroll
  for (int o = LPE; o < 64; o <<= 1) shfl_merge<VEL>(st, o);
  __shared__ float s_m[NWAVE][LPE], s_l[NWAVE][LPE];
  if (sw == 0) {
    s_m[wave][sl] = st.m;
    s_l[wave][sl] = st.l;
#pragma unroll
    for (int k = 0; k < VEL; ++k) s_a[wave][sl][k] = st.acc[k];
  }
  __syncthreads();
  if (wave != 0 || sw != 0) return;
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) {
    float a2[VEL];
#pragma unroll
    for (int k = 0; k < VEL; ++k) a2[k] = s_a[w][sl][k];
    st.merge(s_m[w][sl], s_l[w][sl], a2);
  }
  if (m_idx < 0) {
    write_final<LPE, VEL>(p, row, head, d_ok, j == 0, loff, goff, gel, sl, st, &s_a[0][0][0]);
  } else {
    if (!d_ok) return;
    store_elems<VEL>(p.pacc + (int64_t)item * p.row_elems + loff, st.acc);
    if (j == 0) {
      p.pml[((int64_t)item * 2 + 0) * p.H + head] = st.m;
      p.pml[((int64_t)item * 2 + 1) * p.H + head] = st.l;
    }
  }
}

// Merge the chunk states of each split row in chunk order (same rule).
__global__ __launch_bounds__(256) void k_att_combine(AttParams p, const int4* multi) {
  if (p.multi_count && (int)blockIdx.x >= *p.multi_count) return;
  const int4 mr = multi[blockIdx.x];
  const int row = mr.x, first = mr.y, cnt = mr.z;
  for (int t = threadIdx.x; t < p.row_elems; t += blockDim.x) {
    const int h = t / p.D;
    float m = -INFINITY, l = 0.0f, a = 0.0f;
    for (int c = 0; c < cnt; ++c) {
      const int64_t it = first + c;
      const float m2 = p.pml[(it * 2 + 0) * p.H + h];
      const float l2 = p.pml[(it * 2 + 1) * p.H + h];
      const float a2 = p.pacc[it * p.row_elems + t];
      const float mn = fmaxf(m, m2);
      if (mn == -INFINITY) continue;
      const float c1 = ex2(m - mn), c2 = ex2(m2 - mn);
      l = l * c1 + l2 * c2;
      a = a * c1 + a2 * c2;
      m = mn;
    }
    p.out[(int64_t)row * p.row_elems + t] = l > 0.0f ? a / l : 0.0f;
    if (p.lse && (t % p.D) == 0) p.lse[(int64_t)row * p.H + h] = l > 0.0f ? m * kLn2 + logf(l) : -INFINITY;
  }
}

template <typename T, int LPE, int VB, int KIND, int LPH>
int launch_att_h(gnn_plan* pl, AttParams& p, int groups, hipStream_t s) {
  constexpr int UU = GNN_ATT_U;
  constexpr int SPB = (64 / LPE) * (WG / 64);
  // the plan lists first the items this one-slot bound leaves to workgroups
  p.n_item_blocks = (int32_t)(p.light_max == pl->att_item_thr ? pl->n_att_items : pl->n_items);
  p.item_count = pl->item_count;
  p.multi_count = pl->multi_count;
  p.n_light_blocks = (int32_t)((p.n_rows + SPB - 1) / SPB);
  const int64_t gx = (((int64_t)p.n_item_blocks + 7) & ~7LL) + p.n_light_blocks;
  if (gx > 0x7FFFFFFF || groups > 65535) return fail(GNN_ERR_SIZE_OVERFLOW, "attention grid too large");
  hipLaunchKernelGGL((k_attention<T, LPE, VB, KIND, UU, LPH>), dim3((unsigned)gx, (unsigned)groups), dim3(WG), 0,
                     s, p);
  GNN_LAUNCH_CHECK("attention");
  if (pl->n_multi > 0) {
    hipLaunchKernelGGL(k_att_combine, dim3((unsigned)pl->n_multi), dim3(256), 0, s, p,
                       (const int4*)pl->multi);
    GNN_LAUNCH_CHECK("attention combine");
  }
  return GNN_OK;
}

// lanes per head is a power of two no larger than the slot
template <typename T, int LPE, int VB, int KIND>
int launch_att(gnn_plan* pl, AttParams& p, int groups, hipStream_t s) {
  switch (p.lph) {
    case 1: return launch_att_h<T, LPE, VB, KIND, 1>(pl, p, groups, s);
    case 2: return launch_att_h<T, LPE, VB, KIND, 2>(pl, p, groups, s);
    case 4: return launch_att_h<T, LPE, VB, KIND, 4>(pl, p, groups, s);
    case 8: return launch_att_h<T, LPE, VB, KIND, 8>(pl, p, groups, s);
    default: break;
  }
  if constexpr (LPE >= 16) if (p.lph == 16) return launch_att_h<T, LPE, VB, KIND, 16>(pl, p, groups, s);
  if constexpr (LPE >= 32) if (p.lph == 32) return launch_att_h<T, LPE, VB, KIND, 32>(pl, p, groups, s);
  if constexpr (LPE >= 64) if (p.lph == 64) return launch_att_h<T, LPE, VB, KIND, 64>(pl, p, groups, s);
  return fail(GNN_ERR_UNSUPPORTED, "lanes per head exceed the slot");
}

// Lane mapping of one call: bytes per lane, slot width, head groups.
struct Mapping {
  int vb = 16, lpe = 64, groups = 1;
};

template <typename T, int KIND>
int dispatch(gnn_plan* pl, AttParams& p, const Mapping& mp, hipStream_t s) {
  if (mp.vb < 16) {
    // generic mapping: one 64-lane slot per edge, lanes per head at run time
    if constexpr (sizeof(T) == 2) {
      if (mp.vb == 2) return launch_att_h<T, 64, 2, KIND, 0>(pl, p, mp.groups, s);
    }
    if (mp.vb == 4) return launch_att_h<T, 64, 4, KIND, 0>(pl, p, mp.groups, s);
    return launch_att_h<T, 64, 8, KIND, 0>(pl, p, mp.groups, s);
  }
  if (mp.vb == 32) {
    // GATv2 rows of more than 1 KB take head groups of 16-byte lanes, so only
    // GT instantiates the 32-bytes-per-lane kernels.
    if constexpr (KIND == K_GATV2) {
      return fail(GNN_ERR_UNSUPPORTED, "GATv2 has no 32-byte lane mapping");
    } else {
      switch (mp.lpe) {
        case 8: return launch_att<T, 8, 32, KIND>(pl, p, mp.groups, s);
        case 16: return launch_att<T, 16, 32, KIND>(pl, p, mp.groups, s);
        case 32: return launch_att<T, 32, 32, KIND>(pl, p, mp.groups, s);
        default: return launch_att<T, 64, 32, KIND>(pl, p, mp.groups, s);
      }
    }
  }
  switch (mp.lpe) {
    case 8: return launch_att<T, 8, 16, KIND>(pl, p, mp.groups, s);
    case 16: return launch_att<T, 16, 16, KIND>(pl, p, mp.groups, s);
    case 32: return launch_att<T, 32, 16, KIND>(pl, p, mp.groups, s);
    default: return launch_att<T, 64, 16, KIND>(pl, p, mp.groups, s);
  }
}

int pow2_at_least(int x) {
  int l = 1;
  while (l < x) l <<= 1;
  return l;
}

// The lane mapping for heads of D elements of esz bytes (the entry points
// checked H, D > 0 and 16-byte aligned bases).
//   - heads of a multiple of 16 bytes: 16-byte lane slices (32-byte ones for
//     GT rows of 1-2 KB whose heads fill a power of two of them); lanes per
//     head rounded up to a power of two; the row in one slot when it fits 64
//     lanes, else cut into groups of 64 / lph heads;
//   - other heads: the widest of 8-, 4- or 2-byte slices that divides the
//     head, at most 64 lanes per head, 64-lane slots, groups as above.
int choose_mapping(int kind, int esz, int H, int D, Mapping* mp, int* lph, int* lph_data, int* hpg) {
  const int64_t hb = (int64_t)D * esz, rowb = (int64_t)H * hb;
  const bool gt_wide = kind == K_GT && rowb > 1024 && rowb <= 2048 && hb % 32 == 0 &&
                       ((hb / 32) & (hb / 32 - 1)) == 0;
  if (gt_wide) {
    mp->vb = 32;
    *lph_data = *lph = (int)(hb / 32);
  } else if (hb % 16 == 0 && hb / 16 <= 64) {
    mp->vb = 16;
    *lph_data = (int)(hb / 16);
    *lph = pow2_at_least(*lph_data);
  } else {
    mp->vb = 0;
    for (int vb = 8; vb >= esz; vb >>= 1)
      if (hb % vb == 0 && hb / vb <= 64) {
        mp->vb = vb;
        break;
      }
    if (mp->vb == 0)
      return fail(GNN_ERR_UNSUPPORTED, "head too wide for the generic attention mapping: D * sizeof must be a "
                                       "multiple of 16 bytes up to 1 KB, or at most 64 slices of 8, 4 or 2 bytes");
    *lph_data = (int)(hb / mp->vb);
    *lph = pow2_at_least(*lph_data);
  }
  if (mp->vb >= 16 && (int64_t)H * *lph <= 64) {
    *hpg = H;
    mp->groups = 1;
    mp->lpe = std::max(8, pow2_at_least(H * *lph));
  } else {
    *hpg = 64 / *lph;
    mp->groups = (H + *hpg - 1) / *hpg;
    mp->lpe = 64;
  }
  return GNN_OK;
}

int setup(gnn_plan* pl, AttParams& p, int kind, gnn_dtype xt, int32_t H, int32_t D, Mapping* mp, hipStream_t s) {
  const int esz = xt == GNN_BF16 ? 2 : 4;
  GNN_TRY(choose_mapping(kind, esz, H, D, mp, &p.lph, &p.lph_data, &p.hpg));
  p.row_ptr = pl->row_ptr;
  p.col_idx = pl->col_idx;
  p.items = pl->items;
  p.n_rows = pl->n_rows;
  p.H = H;
  p.D = D;
  p.row_elems = H * D;
  const int64_t kvb = (int64_t)pl->n_cols * H * D * esz;
  p.kv_bytes = kvb < ((int64_t)1 << 31) ? (int32_t)kvb : 0;
  p.dv = (int32_t)((int64_t)D * esz / mp->vb);
  // One slot per row up to kAttLightMax edges, never below the plan's own
  // light threshold (its longer rows are the plan's items) and never above
  // its heavy threshold (split rows go through the items alone).  The rows
  // are listed longest first, so that the slots of a wave see rows of one
  // length and finish together.
  const int32_t slot_max = pl->opts.att_slot_max > 0 ? pl->opts.att_slot_max : kAttLightMax;
  p.light_max = std::max(pl->light_max, std::min(slot_max, pl->heavy_thr));
  GNN_TRY(plan_att_rows(pl, p.light_max, s));
  p.att_rows = pl->att_rows;
  p.att_count = pl->att_count;
  if (pl->n_multi > 0) {
    void* ws = nullptr;
    size_t need = (size_t)pl->n_slots * (H * D + 2 * H) * 4;
    GNN_TRY(plan_workspace(pl, need, &ws));
    p.pacc = (float*)ws;
    p.pml = p.pacc + (size_t)pl->n_slots * H * D;
  }
  return GNN_OK;
}

}  // namespace

int launch_gatv2(gnn_plan* pl, const void* xl, const void* xr, gnn_dtype xt, const float* att,
                 int32_t H, int32_t D, float slope, float* out, float* lse, hipStream_t s) {
  AttParams p{};
  Mapping mp;
  GNN_TRY(setup(pl, p, K_GATV2, xt, H, D, &mp, s));
  p.q = xl;
  p.k = xr;
  p.v = xr;
  p.att = att;
  p.out = out;
  p.lse = lse;
  p.slope = slope;
  if (xt == GNN_BF16) return dispatch<uint16_t, K_GATV2>(pl, p, mp, s);
  return dispatch<float, K_GATV2>(pl, p, mp, s);
}

int launch_gt_csr(gnn_plan* pl, const void* q, const void* k, const void* v, gnn_dtype xt, int32_t H,
                  int32_t D, float scale, float* out, float* lse, hipStream_t s) {
  AttParams p{};
  Mapping mp;
  GNN_TRY(setup(pl, p, K_GT, xt, H, D, &mp, s));
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.qscale = scale * kLog2e;
  if (xt == GNN_BF16) return dispatch<uint16_t, K_GT>(pl, p, mp, s);
  return dispatch<float, K_GT>(pl, p, mp, s);
}

int attention_mapping_supported(int gt, gnn_dtype xt, int32_t H, int32_t D) {
  Mapping mp;
  int a, b, c;
  return choose_mapping(gt ? K_GT : K_GATV2, xt == GNN_BF16 ? 2 : 4, H, D, &mp, &a, &b, &c);
}

}  // namespace gnn
