// Backward of the fused CSR attention layers (Graph Transformer, GATv2).
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", attention appendix, backward passes: only the per-(node,
// head) logsumexp L of the forward is kept, the weights are recomputed on the
// fly as alpha_ij = exp(e_ij - L_i), Delta[i, h] = <O[i, h, :], dO[i, h, :]>
// (for GATv2 the same statistic is G_{i,h} = sum_j alpha_ij <dO_i, r_j>), a
// walk over the transposed CSR gathers the gradients of the source-side
// tensors, and the attention-vector gradient of GATv2 is reduced over nodes.
// With de_ij = alpha_ij (<dO_i, v_j> - Delta_i):
//   Graph Transformer (e = s <q_i, k_j>): dq_i = s sum_j de_ij k_j,
//     dk_j = s sum_i de_ij q_i, dv_j = sum_i alpha_ij dO_i;
//   GATv2 (e = a . LReLU(l_i + r_j), v_j = r_j): dl_i = sum_j de_ij a (.) LReLU'(z_ij),
//     dr_j = sum_i (alpha_ij dO_i + de_ij a (.) LReLU'(z_ij)),
//     da = sum_ij de_ij LReLU(z_ij).
//
// MI355X mapping: two walks and no atomics.  The destination walk (rows of
// the CSR) forms Delta_i from O_i and dO_i, then per entry alpha and de, and
// accumulates the destination gradient (dq_i, or dl_i and the workgroup's
// share of da).  The source walk (rows of the plan's transpose) recomputes
// the same alpha and de per entry from the stored L_i and Delta_i and
// accumulates the source gradients.  Short rows take one slot each, in the
// plan's length-sorted row list (as the forward kernels).  Every output row is
// summed by one slot,
// one workgroup, or ordered chunk partials (hub rows), so results are
// deterministic; the pages' own backward instead updates one gradient with
// atomic adds along the transposed walk, which at H * D = 512 would be 512
// fp32 atomics per entry.  Lanes hold 16-byte slices of a node row and
// per-head dot products use the DPP lane sums, as in the forward kernels.
#include <algorithm>

#include "att_common.h"

namespace gnn {
namespace {

using namespace att;

constexpr int WG = 256;
constexpr int UB = 4;                 // entries in flight per slot
constexpr int32_t kBwdLightMax = 128;  // one slot per row up to this many entries

enum { B_GT_DST = 0, B_GT_SRC = 1, B_GAT_DST = 2, B_GAT_SRC = 3 };

struct BwdParams {
  // the walked graph (the CSR, or the plan's transpose) and its work split
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int4* items;
  int32_t n_rows;
  int32_t light_max;
  const int32_t* light_rows;   // rows of at most light_max entries, by length within windows
  const int32_t* light_count;  // device: how many
  int32_t n_item_blocks;
  const int32_t* item_count;  // device item count (NULL: n_item_blocks is exact)
  int32_t n_light_blocks;
  // tensors: "dst" are indexed by destinations (rows of the CSR), "src" by sources
  const void* q;     // dst: GT q; GATv2 x_l
  const void* k;     // src: GT k; GATv2 x_r
  const void* v;     // src: GT v; GATv2 x_r
  const float* att;  // GATv2 a [H, D]
  const float* out;  // dst: forward output
  const float* lse;  // dst: forward logsumexp (natural log)
  const float* dout; // dst: gradient of the output
  float* delta;      // dst [.., H]: written by the destination walk, read by the source walk
  float* g0;         // GT dst: dq; GT src: dk; GATv2 dst: dl; GATv2 src: dr
  float* g1;         // GT src: dv
  float* dapart;     // GATv2 dst: [gridDim.x, H * D] per-workgroup shares of da
  float* part;       // split rows: [n_slots, 2, H * D] chunk partials
  int32_t H, D, row_elems;
  // lane mapping (as in the forward): a slot covers the heads of one group
  // (blockIdx.y), LPH lanes per head of which lph_data hold data
  int32_t hpg, lph_data;
  float scale;       // GT score scale
  float slope;       // GATv2 LeakyReLU slope
  // bytes of the gathered arrays when each is below 2^31 (else 0): k / v
  // (rows = sources), q (rows = destinations), dO (fp32, destinations)
  int32_t kv_bytes, q_bytes, do_bytes, lse_bytes;
};

template <int VEL>
__device__ __forceinline__ void load_f32(const float* p, float (&o)[VEL]) {
#pragma unroll
  for (int k = 0; k < VEL; k += 4) {
    const float4 t = *reinterpret_cast<const float4*>(p + k);
    o[k] = t.x; o[k + 1] = t.y; o[k + 2] = t.z; o[k + 3] = t.w;
  }
}

template <typename T, int NV>
__device__ __forceinline__ void decode(const Raw<NV>& r, float (&o)[(16 / sizeof(T)) * NV]) {
#pragma unroll
  for (int k = 0; k < (16 / (int)sizeof(T)) * NV; ++k) o[k] = elem<T, NV>(r, k);
}

// Per-row state: the row's own data and the accumulators.
template <typename T, int NV, int KIND>
struct Row {
  static constexpr int VEL = (16 / (int)sizeof(T)) * NV;
  Raw<NV> own;        // GT dst: q_i; GT src: k_j
  float f0[VEL];      // dst: dO_i; GT src: v_j; GATv2 src: r_j
  float f1[VEL];      // GATv2 dst: l_i
  // GATv2: a (1 + slope) / 2 and a (1 - slope) / 2: a LeakyReLU(z) = av z +
  // an |z|, and a LeakyReLU'(z) = av + an for z > 0, av - an otherwise
  float av[VEL], an[VEL];
  float sde = 0.0f;   // GATv2: sum of de over the slot's entries (the av part of acc0)
  float L2 = 0.0f;    // dst: L_i * log2 e
  float delta = 0.0f; // dst: Delta_i
  float acc0[VEL], acc1[VEL];
  // GT destination walk with bf16 rows: dO_i split into bf16 pairs hi + lo
  // (dO - hi - lo is below 2^-16 |dO|), so that dO_i . v_j takes dot2 steps
  uint32_t dhi[VEL / 2], dlo[VEL / 2];
};

__device__ __forceinline__ uint32_t pack_bf16x2(__bf16 a, __bf16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Work on entries [eb, ee) of walk row `row` for one slot (LPE lanes).
template <typename T, int LPE, int NV, int KIND, int LPH>
__device__ __forceinline__ void scan(const BwdParams& p, int eb, int ee, int sl, int slot_base, bool d_ok,
                                     int head, int loff, Row<T, NV, KIND>& R) {
  constexpr int VEL = (16 / (int)sizeof(T)) * NV;
  const int64_t ld = p.row_elems;
  const uint32_t rb = (uint32_t)(p.row_elems * (int)sizeof(T)), rb4 = (uint32_t)(p.row_elems * 4);
  const float sc2 = p.scale * kLog2e;
  const __amdgpu_buffer_rsrc_t rk = row_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = row_rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rq = row_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rd = row_rsrc(p.dout, p.do_bytes);
  const __amdgpu_buffer_rsrc_t rl = row_rsrc(p.lse, p.lse_bytes);
  const __amdgpu_buffer_rsrc_t rdl = row_rsrc(p.delta, p.lse_bytes);
  for (int e0 = eb; e0 < ee; e0 += LPE) {
    const int nb = min(LPE, ee - e0);
    const int my_c = (sl < nb) ? p.col_idx[e0 + sl] : 0;
    for (int u0 = 0; u0 < nb; u0 += UB) {
      int c[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u)
        c[u] = (LPE == 64) ? __builtin_amdgcn_readlane(my_c, u0 + u) : __shfl(my_c, slot_base + u0 + u, 64);
      // gathers of the other end of each entry
      Raw<NV> x[UB], y[UB];
      float g[UB][VEL];
      float Lc[UB], Dc[UB];
      if constexpr (LPE == 64) {
        if (p.kv_bytes > 0 && p.q_bytes > 0 && p.do_bytes > 0) {
          // one slot per wave: the entry's row offset is a scalar operand of
          // buffer loads over the whole array, and an entry past the slot's
          // end or a lane without data reads at an offset beyond the array,
          // which returns zeros: no per-lane addresses, no branches
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const bool ok = u0 + u < nb && d_ok;
            const uint32_t so = (uint32_t)c[u] * (uint32_t)(ld * (int64_t)sizeof(T));
            const uint32_t vo = ok ? (uint32_t)(loff * (int)sizeof(T)) : 0x80000000u;
            if constexpr (KIND == B_GT_DST) {
              load_rawb_buf_so<16 * NV>(rk, vo, so, x[u]);
              load_rawb_buf_so<16 * NV>(rv, vo, so, y[u]);
            } else if constexpr (KIND == B_GAT_DST) {
              load_rawb_buf_so<16 * NV>(rk, vo, so, x[u]);
            } else {
              load_rawb_buf_so<16 * NV>(rq, vo, so, x[u]);
              RawB<4 * VEL> gr;
              load_rawb_buf_so<4 * VEL>(rd, ok ? (uint32_t)(loff * 4) : 0x80000000u,
                                        (uint32_t)c[u] * (uint32_t)(ld * 4), gr);
#pragma unroll
              for (int k = 0; k < VEL; ++k) g[u][k] = __uint_as_float(gr.u[k]);
              // the destination's (L, Delta) of this lane's head, zero past the end
              const uint32_t ho = ok ? (uint32_t)(head * 4) : 0x80000000u, hs = (uint32_t)c[u] * (uint32_t)(p.H * 4);
              Lc[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, ho, hs, 0));
              Dc[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdl, ho, hs, 0));
            }
          }
          goto gathered;
        }
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const bool ok = u0 + u < nb && d_ok;
        const int o = loff;  // the lane's slice; rows by row_at
        if constexpr (KIND == B_GT_DST) {
          if (ok) {
            load_raw<T, NV>(row_at(reinterpret_cast<const T*>(p.k) + o, c[u], rb), x[u]);
            load_raw<T, NV>(row_at(reinterpret_cast<const T*>(p.v) + o, c[u], rb), y[u]);
          } else {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t) x[u].u[t] = y[u].u[t] = 0u;
          }
        } else if constexpr (KIND == B_GAT_DST) {
          if (ok) load_raw<T, NV>(row_at(reinterpret_cast<const T*>(p.k) + o, c[u], rb), x[u]);
          else {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t) x[u].u[t] = 0u;
          }
        } else {  // source walks: the destination's q / l, dO, L and Delta
          if (ok) {
            load_raw<T, NV>(row_at(reinterpret_cast<const T*>(p.q) + o, c[u], rb), x[u]);
            load_f32<VEL>(row_at(p.dout + o, c[u], rb4), g[u]);
            Lc[u] = p.lse[(int64_t)c[u] * p.H + head];
            Dc[u] = p.delta[(int64_t)c[u] * p.H + head];
          } else {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t) x[u].u[t] = 0u;
#pragma unroll
            for (int k = 0; k < VEL; ++k) g[u][k] = 0.0f;
            Lc[u] = 0.0f;
            Dc[u] = 0.0f;
          }
        }
      }
    gathered:
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const bool valid = u0 + u < nb;
        if constexpr (KIND == B_GT_DST) {
          float dot = 0.0f, gv = 0.0f;
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t)
              dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, R.own.u[t]),
                                                    __builtin_bit_cast(bf16x2_t, x[u].u[t]), dot, false);
          } else {
#pragma unroll
            for (int k = 0; k < VEL; ++k) dot = fmaf(elem<T, NV>(R.own, k), elem<T, NV>(x[u], k), dot);
          }
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t) {
              gv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, R.dhi[t]),
                                                   __builtin_bit_cast(bf16x2_t, y[u].u[t]), gv, false);
              gv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, R.dlo[t]),
                                                   __builtin_bit_cast(bf16x2_t, y[u].u[t]), gv, false);
            }
          } else {
#pragma unroll
            for (int k = 0; k < VEL; ++k) gv = fmaf(R.f0[k], elem<T, NV>(y[u], k), gv);
          }
          dot = head_sum<LPH>(dot);
          gv = head_sum<LPH>(gv);
          const float al = valid ? ex2(dot * sc2 - R.L2) : 0.0f;
          const float w = p.scale * al * (gv - R.delta);
#pragma unroll
          for (int k = 0; k < VEL; ++k) R.acc0[k] = fmaf(w, elem<T, NV>(x[u], k), R.acc0[k]);
        } else if constexpr (KIND == B_GT_SRC) {
          float dot = 0.0f, gv = 0.0f;
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int t = 0; t < 4 * NV; ++t)
              dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x[u].u[t]),
                                                    __builtin_bit_cast(bf16x2_t, R.own.u[t]), dot, false);
          } else {
#pragma unroll
            for (int k = 0; k < VEL; ++k) dot = fmaf(elem<T, NV>(x[u], k), elem<T, NV>(R.own, k), dot);
          }
#pragma unroll
          for (int k = 0; k < VEL; ++k) gv = fmaf(g[u][k], R.f0[k], gv);
          dot = head_sum<LPH>(dot);
          gv = head_sum<LPH>(gv);
          // L in natural-log units, scaled where it is used (its load need not
          // have arrived before the batch's first products).  An entry past the
          // slot's end has zero q, dO, L and Delta, so it adds nothing.
          const float al = ex2(fmaf(dot, p.scale, -Lc[u]) * kLog2e);
          const float w = p.scale * al * (gv - Dc[u]);
#pragma unroll
          for (int k = 0; k < VEL; ++k) {
            R.acc0[k] = fmaf(w, elem<T, NV>(x[u], k), R.acc0[k]);
            R.acc1[k] = fmaf(al, g[u][k], R.acc1[k]);
          }
        } else if constexpr (KIND == B_GAT_DST) {
          float e = 0.0f, gv = 0.0f, z[VEL];
#pragma unroll
          for (int k = 0; k < VEL; ++k) {
            const float r = elem<T, NV>(x[u], k);
            z[k] = R.f1[k] + r;
            e = fmaf(R.av[k], z[k], fmaf(R.an[k], fabsf(z[k]), e));
            gv = fmaf(R.f0[k], r, gv);
          }
          e = head_sum<LPH>(e);
          gv = head_sum<LPH>(gv);
          const float al = valid ? ex2(e * kLog2e - R.L2) : 0.0f;
          const float de = al * (gv - R.delta);
          R.sde += de;
#pragma unroll
          for (int k = 0; k < VEL; ++k) {
            R.acc0[k] = fmaf(de, z[k] > 0.0f ? R.an[k] : -R.an[k], R.acc0[k]);
            R.acc1[k] = fmaf(de, fmaxf(z[k], p.slope * z[k]), R.acc1[k]);
          }
        } else {  // B_GAT_SRC
          float e = 0.0f, gv = 0.0f, z[VEL];
#pragma unroll
          for (int k = 0; k < VEL; ++k) {
            z[k] = elem<T, NV>(x[u], k) + R.f0[k];
            e = fmaf(R.av[k], z[k], fmaf(R.an[k], fabsf(z[k]), e));
            gv = fmaf(g[u][k], R.f0[k], gv);
          }
          e = head_sum<LPH>(e);
          gv = head_sum<LPH>(gv);
          // as in the GT source walk: past the slot's end every term is zero
          const float al = ex2((e - Lc[u]) * kLog2e);
          const float de = al * (gv - Dc[u]);
          R.sde += de;
#pragma unroll
          for (int k = 0; k < VEL; ++k)
            R.acc0[k] = fmaf(al, g[u][k], fmaf(de, z[k] > 0.0f ? R.an[k] : -R.an[k], R.acc0[k]));
        }
      }
    }
  }
}

template <typename T, int LPE, int NV, int KIND, int LPH>
__global__ __launch_bounds__(WG) void k_att_bwd(BwdParams p) {
  constexpr int VEL = (16 / (int)sizeof(T)) * NV;
  constexpr int SPW = 64 / LPE;
  constexpr int NWAVE = WG / 64;
  constexpr bool DST = KIND == B_GT_DST || KIND == B_GAT_DST;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sw = lane / LPE, sl = lane % LPE;
  const int slot_base = sw * LPE;
  const int hin = sl / LPH, hj = sl % LPH;
  const int head_g = (int)blockIdx.y * p.hpg + hin;
  const bool d_ok = hin < p.hpg && head_g < p.H && hj < p.lph_data;
  const int head = d_ok ? head_g : 0;
  const int loff = d_ok ? head * p.D + hj * VEL : 0;  // the lane's slice of a row

  const int n_item_pad = (p.n_item_blocks + 7) & ~7;
  const bool is_item = (int)blockIdx.x < n_item_pad;
  int64_t row = -1;
  int eb = 0, ee = 0, m_idx = -1, item = -1;
  bool active = true;  // GATv2 dst workgroups reach the block reduction even when idle
  if (is_item) {
    item = (int)dev::xcd_remap(blockIdx.x, n_item_pad);
    active = item < p.n_item_blocks && (!p.item_count || item < *p.item_count);
    if (active) {
      const int4 it = p.items[item];
      active = !(it.w < 0 && it.z - it.y <= p.light_max);  // short rows: light path
      row = it.x;
      m_idx = it.w;
      const int nslots = SPW * NWAVE, slot = wave * SPW + sw;
      const int len = it.z - it.y, per = (len + nslots - 1) / nslots;
      eb = min(it.z, it.y + slot * per);
      ee = min(it.z, eb + per);
    }
  } else {
    const uint32_t lb = dev::xcd_remap(blockIdx.x - n_item_pad, p.n_light_blocks);
    const int64_t idx = ((int64_t)lb * NWAVE + wave) * SPW + sw;
    active = idx < *p.light_count;
    if (active) {
      row = p.light_rows[idx];
      eb = p.row_ptr[row];
      ee = p.row_ptr[row + 1];
    }
  }
  if (KIND != B_GAT_DST && !active) return;  // uniform over the workgroup for items, over the slot otherwise

  Row<T, NV, KIND> R;
#pragma unroll
  for (int k = 0; k < VEL; ++k) R.acc0[k] = R.acc1[k] = R.av[k] = R.an[k] = R.f0[k] = R.f1[k] = 0.0f;
#pragma unroll
  for (int k = 0; k < VEL / 2; ++k) R.dhi[k] = R.dlo[k] = 0u;  // lanes without data join the head sums
#pragma unroll
  for (int t = 0; t < 4 * NV; ++t) R.own.u[t] = 0u;
  const int64_t ro = row * (int64_t)p.row_elems + loff;
  if (active && d_ok) {
    if constexpr (DST) {
      float o[VEL];
      load_f32<VEL>(p.dout + ro, R.f0);
      load_f32<VEL>(p.out + ro, o);
      float t = 0.0f;
#pragma unroll
      for (int k = 0; k < VEL; ++k) t = fmaf(R.f0[k], o[k], t);
      R.delta = t;
      if constexpr (KIND == B_GT_DST && sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < VEL / 2; ++q) {
          const float a = R.f0[2 * q], b = R.f0[2 * q + 1];
          const __bf16 ha = (__bf16)a, hb = (__bf16)b;
          R.dhi[q] = pack_bf16x2(ha, hb);
          R.dlo[q] = pack_bf16x2((__bf16)(a - (float)ha), (__bf16)(b - (float)hb));
        }
      }
      R.L2 = p.lse[row * p.H + head] * kLog2e;
      if constexpr (KIND == B_GT_DST) load_raw<T, NV>(reinterpret_cast<const T*>(p.q) + ro, R.own);
      else {
        Raw<NV> l;
        load_raw<T, NV>(reinterpret_cast<const T*>(p.q) + ro, l);
        decode<T, NV>(l, R.f1);
      }
    } else {
      Raw<NV> f;
      if constexpr (KIND == B_GT_SRC) {
        load_raw<T, NV>(reinterpret_cast<const T*>(p.k) + ro, R.own);
        load_raw<T, NV>(reinterpret_cast<const T*>(p.v) + ro, f);
      } else {
        load_raw<T, NV>(reinterpret_cast<const T*>(p.k) + ro, f);
      }
      decode<T, NV>(f, R.f0);
    }
    if constexpr (KIND == B_GAT_DST || KIND == B_GAT_SRC) {
#pragma unroll
      for (int k = 0; k < VEL; ++k) {
        const float a = p.att[loff + k];
        R.av[k] = a * (0.5f + 0.5f * p.slope);
        R.an[k] = a * (0.5f - 0.5f * p.slope);
      }
    }
  }
  if constexpr (DST) R.delta = head_sum<LPH>(R.delta);
  if (DST && active && d_ok && hj == 0 && (!is_item || m_idx < 0 || p.items[item].y == p.row_ptr[row]))
    p.delta[row * p.H + head] = R.delta;  // once per row: the light slot, the single item, or chunk 0

  if (active) scan<T, LPE, NV, KIND, LPH>(p, eb, ee, sl, slot_base, d_ok, head, loff, R);
  if constexpr (KIND == B_GAT_DST || KIND == B_GAT_SRC) {
#pragma unroll
    for (int k = 0; k < VEL; ++k) R.acc0[k] = fmaf(R.av[k], R.sde, R.acc0[k]);
  }


  __shared__ __align__(16) float s_acc[NWAVE][2][64 * VEL];

  if constexpr (KIND == B_GAT_DST) {
    // the workgroup's share of da: the sum of acc1 over every slot, in slot order
#pragma unroll
    for (int o = LPE; o < 64; o <<= 1)
#pragma unroll
      for (int k = 0; k < VEL; ++k) R.acc1[k] += __shfl_xor(R.acc1[k], o, 64);
    if (sw == 0) {
#pragma unroll
      for (int k = 0; k < VEL; ++k) s_acc[wave][1][sl * VEL + k] = R.acc1[k];
    }
    __syncthreads();
    if (wave == 0 && sw == 0 && d_ok) {
#pragma unroll
      for (int k = 0; k < VEL; ++k) {
        float t = s_acc[0][1][sl * VEL + k];
        for (int w = 1; w < NWAVE; ++w) t += s_acc[w][1][sl * VEL + k];
        p.dapart[(int64_t)blockIdx.x * p.row_elems + loff + k] = t;
      }
    }
  }

  if (!is_item) {
    if (active && d_ok) {
      store_row_nt<VEL>(p.g0 + ro, R.acc0);
      if constexpr (KIND == B_GT_SRC) store_row_nt<VEL>(p.g1 + ro, R.acc1);
    }
    return;
  }
  if (!active) return;  // uniform over an item workgroup

  // an item: sum the slots of each wave, then the waves in order
#pragma unroll
  for (int o = LPE; o < 64; o <<= 1)
#pragma unroll
    for (int k = 0; k < VEL; ++k) {
      R.acc0[k] += __shfl_xor(R.acc0[k], o, 64);
      if constexpr (KIND == B_GT_SRC) R.acc1[k] += __shfl_xor(R.acc1[k], o, 64);
    }
  if (KIND == B_GAT_DST) __syncthreads();  // s_acc[.][1] was read above
  if (sw == 0) {
#pragma unroll
    for (int k = 0; k < VEL; ++k) {
      s_acc[wave][0][sl * VEL + k] = R.acc0[k];
      if constexpr (KIND == B_GT_SRC) s_acc[wave][1][sl * VEL + k] = R.acc1[k];
    }
  }
  __syncthreads();
  if (wave != 0 || sw != 0 || !d_ok) return;
#pragma unroll
  for (int k = 0; k < VEL; ++k) {
    float t0 = s_acc[0][0][sl * VEL + k], t1 = s_acc[0][1][sl * VEL + k];
    for (int w = 1; w < NWAVE; ++w) {
      t0 += s_acc[w][0][sl * VEL + k];
      if constexpr (KIND == B_GT_SRC) t1 += s_acc[w][1][sl * VEL + k];
    }
    R.acc0[k] = t0;
    R.acc1[k] = t1;
  }
  if (m_idx < 0) {
    store_row_nt<VEL>(p.g0 + ro, R.acc0);
    if constexpr (KIND == B_GT_SRC) store_row_nt<VEL>(p.g1 + ro, R.acc1);
  } else {
    const int64_t po = (int64_t)item * 2 * p.row_elems + loff;
    store_row<VEL>(p.part + po, R.acc0);
    if constexpr (KIND == B_GT_SRC) store_row<VEL>(p.part + po + p.row_elems, R.acc1);
  }
}

// Rows split into chunks: sum the chunk partials in chunk order.
__global__ __launch_bounds__(256) void k_bwd_combine(const float* part, const int4* multi,
                                                     const int32_t* multi_count, int32_t row_elems, int two,
                                                     float* g0, float* g1) {
  if (multi_count && (int)blockIdx.x >= *multi_count) return;
  const int4 mr = multi[blockIdx.x];
  const int row = mr.x, first = mr.y, cnt = mr.z;
  for (int t = threadIdx.x; t < row_elems; t += blockDim.x) {
    float a = 0.0f, b = 0.0f;
    for (int c = 0; c < cnt; ++c) {
      a += part[(int64_t)(first + c) * 2 * row_elems + t];
      if (two) b += part[(int64_t)(first + c) * 2 * row_elems + row_elems + t];
    }
    g0[(int64_t)row * row_elems + t] = a;
    if (two) g1[(int64_t)row * row_elems + t] = b;
  }
}

// da = sum over workgroups of their shares, as a tree of ordered levels:
// block b of a level sums rows [b * per, (b + 1) * per) of its input.
__global__ __launch_bounds__(256) void k_da_level(const float* in, int64_t rows, int64_t per, int32_t cols,
                                                  float* out) {
  const int64_t r0 = (int64_t)blockIdx.x * per, r1 = min(rows, r0 + per);
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    float t = 0.0f;
    for (int64_t r = r0; r < r1; ++r) t += in[r * cols + c];
    out[(int64_t)blockIdx.x * cols + c] = t;
  }
}

template <typename T, int LPE, int NV, int KIND, int LPH>
int launch_walk(gnn_plan* pl, BwdParams p, int groups, hipStream_t s) {
  constexpr int SPB = (64 / LPE) * (WG / 64);
  p.row_ptr = pl->row_ptr;
  p.col_idx = pl->col_idx;
  p.items = pl->items;
  p.n_rows = pl->n_rows;
  const int32_t slot_max = pl->opts.att_slot_max > 0 ? pl->opts.att_slot_max : kBwdLightMax;
  p.light_max = std::max(pl->light_max, std::min(slot_max, pl->heavy_thr));
  GNN_TRY(plan_att_rows(pl, p.light_max, s));
  p.light_rows = pl->att_rows;
  p.light_count = pl->att_count;
  // the plan lists first the items this one-slot bound leaves to workgroups
  p.n_item_blocks = (int32_t)(p.light_max == pl->att_item_thr ? pl->n_att_items : pl->n_items);
  p.item_count = pl->item_count;
  p.n_light_blocks = (int32_t)((p.n_rows + SPB - 1) / SPB);
  const int64_t gx = (((int64_t)p.n_item_blocks + 7) & ~7LL) + p.n_light_blocks;
  if (gx > 0x7FFFFFFF || groups > 65535) return fail(GNN_ERR_SIZE_OVERFLOW, "attention backward grid too large");
  const size_t part_b = ((size_t)std::max<int64_t>(pl->n_slots, 1) * 2 * p.row_elems * 4 + 255) & ~(size_t)255;
  const size_t da_b = KIND == B_GAT_DST ? (size_t)gx * p.row_elems * 4 : 0;
  void* ws = nullptr;
  const size_t mid_b = 2 * (size_t)((gx + 15) / 16 + 1) * p.row_elems * 4;
  GNN_TRY(plan_workspace(pl, part_b + da_b + (KIND == B_GAT_DST ? mid_b : 0) + 256, &ws));
  p.part = (float*)ws;
  p.dapart = KIND == B_GAT_DST ? (float*)((char*)ws + part_b) : nullptr;
  if (gx > 0) {
    hipLaunchKernelGGL((k_att_bwd<T, LPE, NV, KIND, LPH>), dim3((unsigned)gx, (unsigned)groups), dim3(WG), 0, s, p);
    GNN_LAUNCH_CHECK("attention backward");
  }
  if (pl->n_multi > 0) {
    hipLaunchKernelGGL(k_bwd_combine, dim3((unsigned)pl->n_multi), dim3(256), 0, s, p.part,
                       (const int4*)pl->multi, pl->multi_count, p.row_elems, KIND == B_GT_SRC ? 1 : 0, p.g0, p.g1);
    GNN_LAUNCH_CHECK("attention backward combine");
  }
  if constexpr (KIND == B_GAT_DST) {
    // da: the workgroup shares summed by an ordered tree, 16 rows per block
    // and level (two scratch areas of ceil(gx / 16) rows alternate)
    constexpr int64_t PER = 16;
    float* mid[2] = {(float*)((char*)ws + part_b + da_b), nullptr};
    mid[1] = mid[0] + ((gx + PER - 1) / PER + 1) * p.row_elems;
    const float* in = p.dapart;
    int64_t rows = gx;
    int lvl = 0;
    while (rows > PER) {
      const int64_t nb = (rows + PER - 1) / PER;
      hipLaunchKernelGGL(k_da_level, dim3((unsigned)nb), dim3(256), 0, s, in, rows, PER, p.row_elems, mid[lvl]);
      in = mid[lvl];
      rows = nb;
      lvl ^= 1;
    }
    hipLaunchKernelGGL(k_da_level, dim3(1), dim3(256), 0, s, in, rows, PER, p.row_elems, p.g1);
    GNN_LAUNCH_CHECK("attention backward da");
  }
  return GNN_OK;
}

template <typename T, int LPE, int NV, int KIND>
int by_lph(gnn_plan* pl, const BwdParams& p, int lph, int groups, hipStream_t s) {
  switch (lph) {
    case 1: return launch_walk<T, LPE, NV, KIND, 1>(pl, p, groups, s);
    case 2: return launch_walk<T, LPE, NV, KIND, 2>(pl, p, groups, s);
    case 4: return launch_walk<T, LPE, NV, KIND, 4>(pl, p, groups, s);
    case 8: return launch_walk<T, LPE, NV, KIND, 8>(pl, p, groups, s);
    default: break;
  }
  if constexpr (LPE >= 16) if (lph == 16) return launch_walk<T, LPE, NV, KIND, 16>(pl, p, groups, s);
  if constexpr (LPE >= 32) if (lph == 32) return launch_walk<T, LPE, NV, KIND, 32>(pl, p, groups, s);
  if constexpr (LPE >= 64) if (lph == 64) return launch_walk<T, LPE, NV, KIND, 64>(pl, p, groups, s);
  return fail(GNN_ERR_UNSUPPORTED, "lanes per head exceed the slot");
}

template <typename T, int KIND>
int by_shape(gnn_plan* pl, const BwdParams& p, int lpe, int nv, int lph, int groups, hipStream_t s) {
  if (nv == 2) {
    switch (lpe) {
      case 8: return by_lph<T, 8, 2, KIND>(pl, p, lph, groups, s);
      case 16: return by_lph<T, 16, 2, KIND>(pl, p, lph, groups, s);
      case 32: return by_lph<T, 32, 2, KIND>(pl, p, lph, groups, s);
      default: return by_lph<T, 64, 2, KIND>(pl, p, lph, groups, s);
    }
  }
  switch (lpe) {
    case 8: return by_lph<T, 8, 1, KIND>(pl, p, lph, groups, s);
    case 16: return by_lph<T, 16, 1, KIND>(pl, p, lph, groups, s);
    case 32: return by_lph<T, 32, 1, KIND>(pl, p, lph, groups, s);
    default: return by_lph<T, 64, 1, KIND>(pl, p, lph, groups, s);
  }
}

// Lane layout of a row of H * D elements, as in the forward kernels: 16-byte
// lane slices (32-byte ones for rows of 1-2 KB whose heads fill a power of
// two of them), lanes per head rounded up to a power of two (the extra lanes
// hold no data), the row in one slot when it fits 64 lanes, else cut into
// groups of 64 / lph heads, one grid row per group.  Heads whose byte width
// is not a multiple of 16 are not served.
struct BwdShape {
  int lpe, nv, lph, lph_data, hpg, groups;
};

int pow2_at_least(int x) {
  int l = 1;
  while (l < x) l <<= 1;
  return l;
}

int shape(gnn_dtype xt, int32_t H, int32_t D, BwdShape* sh) {
  const int64_t esz = xt == GNN_BF16 ? 2 : 4, hb = (int64_t)D * esz, rowb = (int64_t)H * hb;
  if (hb % 16 != 0)
    return fail(GNN_ERR_UNSUPPORTED, "attention backward: D * element size must be a multiple of 16 bytes");
  sh->nv = (rowb > 1024 && rowb <= 2048 && hb % 32 == 0 && (((hb / 32) & (hb / 32 - 1)) == 0)) ? 2 : 1;
  sh->lph_data = (int)(hb / (16 * sh->nv));
  sh->lph = pow2_at_least(sh->lph_data);
  if (sh->lph > 64) return fail(GNN_ERR_UNSUPPORTED, "attention backward: head wider than 64 lane slices");
  if ((int64_t)H * sh->lph <= 64) {
    sh->hpg = H;
    sh->groups = 1;
    sh->lpe = std::max(8, pow2_at_least(H * sh->lph));
  } else {
    sh->hpg = 64 / sh->lph;
    sh->groups = (H + sh->hpg - 1) / sh->hpg;
    sh->lpe = 64;
  }
  return GNN_OK;
}

template <int KIND>
int run(gnn_plan* pl, const BwdParams& p, gnn_dtype xt, const BwdShape& sh, hipStream_t s) {
  return xt == GNN_BF16 ? by_shape<uint16_t, KIND>(pl, p, sh.lpe, sh.nv, sh.lph, sh.groups, s)
                        : by_shape<float, KIND>(pl, p, sh.lpe, sh.nv, sh.lph, sh.groups, s);
}

// Sizes of the gathered arrays for the buffer loads of one-slot walks (0:
// 2 GB or more, where those walks use per-lane addresses).
void set_gather_bytes(const gnn_plan* pl, gnn_dtype xt, BwdParams& p) {
  const int64_t esz = xt == GNN_BF16 ? 2 : 4, lim = (int64_t)1 << 31;
  const int64_t kv = (int64_t)pl->n_cols * p.row_elems * esz, q = (int64_t)pl->n_rows * p.row_elems * esz;
  const int64_t d = (int64_t)pl->n_rows * p.row_elems * 4;
  p.kv_bytes = kv < lim ? (int32_t)kv : 0;
  p.q_bytes = q < lim ? (int32_t)q : 0;
  p.do_bytes = d < lim ? (int32_t)d : 0;
  // (L, Delta) [n_rows, H] are smaller than dO: valid whenever dO's size is
  p.lse_bytes = p.do_bytes > 0 ? (int32_t)((int64_t)pl->n_rows * p.H * 4) : 0;
}

}  // namespace

int launch_gt_backward(gnn_plan* pl, const void* q, const void* k, const void* v, gnn_dtype xt, int32_t H,
                       int32_t D, float scale, const float* out, const float* lse, const float* dout,
                       float* dq, float* dk, float* dv, hipStream_t s) {
  BwdShape sh;
  GNN_TRY(shape(xt, H, D, &sh));
  GNN_TRY(plan_transpose(pl, s));
  BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.dout = dout;
  p.H = H;
  p.D = D;
  p.row_elems = H * D;
  p.hpg = sh.hpg;
  p.lph_data = sh.lph_data;
  set_gather_bytes(pl, xt, p);
  p.scale = scale > 0.0f ? scale : 1.0f / sqrtf((float)D);
  // Delta lives in the plan of the destinations, sized [n_rows, H]
  GNN_TRY(plan_grow(pl, (void**)&pl->delta, &pl->delta_cap, (size_t)std::max(pl->n_rows, 1) * H * 4));
  p.delta = pl->delta;
  p.g0 = dq;
  GNN_TRY(run<B_GT_DST>(pl, p, xt, sh, s));
  p.g0 = dk;
  p.g1 = dv;
  return run<B_GT_SRC>(pl->tplan, p, xt, sh, s);
}

int launch_gatv2_backward(gnn_plan* pl, const void* xl, const void* xr, gnn_dtype xt, const float* att,
                          int32_t H, int32_t D, float slope, const float* out, const float* lse,
                          const float* dout, float* dxl, float* dxr, float* datt, hipStream_t s) {
  BwdShape sh;
  GNN_TRY(shape(xt, H, D, &sh));
  GNN_TRY(plan_transpose(pl, s));
  BwdParams p{};
  p.q = xl;
  p.k = xr;
  p.v = xr;
  p.att = att;
  p.out = out;
  p.lse = lse;
  p.dout = dout;
  p.H = H;
  p.D = D;
  p.row_elems = H * D;
  p.hpg = sh.hpg;
  p.lph_data = sh.lph_data;
  set_gather_bytes(pl, xt, p);
  p.slope = slope;
  GNN_TRY(plan_grow(pl, (void**)&pl->delta, &pl->delta_cap, (size_t)std::max(pl->n_rows, 1) * H * 4));
  p.delta = pl->delta;
  p.g0 = dxl;
  p.g1 = datt;
  GNN_TRY(run<B_GAT_DST>(pl, p, xt, sh, s));
  p.g0 = dxr;
  p.g1 = nullptr;
  return run<B_GAT_SRC>(pl->tplan, p, xt, sh, s);
}

}  // namespace gnn
