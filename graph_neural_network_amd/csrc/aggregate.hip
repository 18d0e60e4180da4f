// Neighbourhood aggregation kernels: SpMM (Y = A_norm X) and the segmented
// reductions sum / mean / max / min.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations": section 2.2 (i) and (ii) define the operators; appendix
// D.1 gives the degree-aware design (light rows feature-parallel, heavy rows
// split into edge chunks, partial max / min merged by one 64-bit atomic on a
// packed (order-preserving key, source index) word, then an unpack kernel);
// appendix D.4 the normalisation modes.  The forward pass reads about
// M * F * sizeof(dtype) bytes of neighbour features whatever the mapping.
//
// MI355X mapping.  A wave64 gathers neighbour rows with one 16-byte load per
// lane: a row of F elements spans LPR = F * sizeof(T) / 16 lanes (a "slot"),
// and a wave holds 64 / LPR slots.  F = 128 float32 or F = 256 bf16 is a
// 512-byte row: two slots per wave, each slot one dwordx4 wave-half load per
// edge, 8 edges kept in flight per slot.
//   light rows  (deg <= light_max): LPR consecutive rows per slot, their
//               edges walked as one flat sequence so that short rows still
//               keep U gathers in flight; the slot loads up to LPR column
//               indices with one coalesced access and broadcasts them lane to
//               lane (ds_bpermute).
//   items       (medium rows, and chunks of heavy rows): one workgroup of
//               four waves per item; each slot takes a contiguous part of the
//               item's edges, the slots are merged in LDS in slot order.
//               Single-item rows write Y directly; multi-item rows write
//               float partials (sum, combined later in item order, so the
//               sum is deterministic) or packed 64-bit words merged with
//               atomicMax / atomicMin (max, min) and unpacked afterwards.
// Both kinds of work run in one launch (items first, then light rows).
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int WG = 256;  // 4 waves
constexpr int U = 8;     // edges in flight per slot
// At most this many item workgroups, each taking items blockIdx.x + k x
// kItemBlocks: a workgroup per item spends launch slots on short items and,
// for plans that hold only a bound of their item count, on empty ones
// (measured on the 1M-node R-MAT reduction: 1.45 ms with one workgroup per
// item, 1.37 ms at 4096, 1.40 ms at 1024 and 16384).
constexpr int32_t kItemBlocks = 4096;

// K_ALL: sum, mean, max and min (with source indices) of one pass.
enum Kind { K_SUM = 0, K_MAX = 1, K_MIN = 2, K_ALL = 3 };

struct AggParams {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const float* edge_val;   // nullable
  const int32_t* deg_out;  // for RIGHT / BOTH
  const void* X;
  int64_t ldx;
  uint32_t ldx_b;          // ldx in bytes (below 2^32): a gathered row's offset is one 32 x 32 -> 64 multiply-add
  float* Y;
  int64_t ldy;
  int32_t* arg;            // nullable, ld = F
  const int4* items;
  float* partial;          // [n_slots, F] chunk partials of split rows
  unsigned long long* packed;  // [n_multi, F]
  int32_t n_rows;
  int32_t F;
  int32_t light_max;
  int32_t n_item_blocks;   // item workgroups in grid.x (each takes items blockIdx.x + k n_item_blocks)
  int32_t n_items;         // items (an upper bound when item_count is set)
  const int32_t* item_count;  // device item count (NULL: n_items is exact)
  const int32_t* multi_count; // device split-row count (NULL: the launch's row count is exact)
  int32_t n_light_blocks;
  int32_t rps;             // light rows per slot (LPR on large graphs)
  int32_t norm;            // gnn_norm (SpMM); MEAN is expressed as LEFT
  int32_t weighted;        // edge_val present or RIGHT / BOTH
  // K_ALL outputs (each nullable; Y above is the sum), and the min words
  float* Ymean;
  float* Ymax;
  float* Ymin;
  int32_t* argmax;
  int32_t* argmin;
  unsigned long long* packed2;
};

// ---------------------------------------------------------------------------
// vector loads / stores of VE elements per lane
// ---------------------------------------------------------------------------

// Gathered rows are kept as raw words until use (a bf16 row slice is 4
// registers raw, 8 decoded), which keeps U rows in flight within the
// register budget of four waves per SIMD.
template <typename T, int VE> struct RawOf;
template <> struct RawOf<float, 4> { using type = float4; };
template <> struct RawOf<uint16_t, 8> { using type = uint4; };
template <> struct RawOf<float, 1> { using type = float; };
template <> struct RawOf<uint16_t, 1> { using type = uint16_t; };

// Row c of X at this lane's slice: c (a column index, >= 0) times the row
// stride in bytes, as one unsigned 32 x 32 -> 64 multiply-add
// (v_mad_u64_u32) instead of a signed 64-bit product.
template <typename T>
__device__ __forceinline__ const T* row_at(const T* base, int c, uint32_t ld_bytes) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + (uint64_t)(uint32_t)c * ld_bytes);
}

template <typename T, int VE>
__device__ __forceinline__ typename RawOf<T, VE>::type load_raw(const T* p) {
  return *reinterpret_cast<const typename RawOf<T, VE>::type*>(p);
}
__device__ __forceinline__ void decode(const float4& v, float (&o)[4]) {
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void decode(const uint4& v, float (&o)[8]) {
  o[0] = dev::bf16_lo(v.x); o[1] = dev::bf16_hi(v.x);
  o[2] = dev::bf16_lo(v.y); o[3] = dev::bf16_hi(v.y);
  o[4] = dev::bf16_lo(v.z); o[5] = dev::bf16_hi(v.z);
  o[6] = dev::bf16_lo(v.w); o[7] = dev::bf16_hi(v.w);
}
__device__ __forceinline__ void decode(const float& v, float (&o)[1]) { o[0] = v; }
__device__ __forceinline__ void decode(const uint16_t& v, float (&o)[1]) {
  o[0] = __uint_as_float((uint32_t)v << 16);
}

// Outputs and column indices are touched once: non-temporal accesses keep
// them from displacing the gathered feature rows in L2 / the MALL.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int VE>
__device__ __forceinline__ void storev(float* p, const float (&v)[VE]) {
  if constexpr (VE == 1) {
    __builtin_nontemporal_store(v[0], p);
  } else {
#pragma unroll
    for (int k = 0; k < VE; k += 4) {
      f32x4_t t = {v[k], v[k + 1], v[k + 2], v[k + 3]};
      __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p + k));
    }
  }
}
template <int VE>
__device__ __forceinline__ void storei(int32_t* p, const int (&v)[VE]) {
  if constexpr (VE == 1) {
    __builtin_nontemporal_store(v[0], p);
  } else {
#pragma unroll
    for (int k = 0; k < VE; k += 4) {
      i32x4_t t = {v[k], v[k + 1], v[k + 2], v[k + 3]};
      __builtin_nontemporal_store(t, reinterpret_cast<i32x4_t*>(p + k));
    }
  }
}

// ---------------------------------------------------------------------------
// per-lane reduction state
// ---------------------------------------------------------------------------

// SUM keeps float accumulators.  MAX / MIN keep, per element, one 64-bit
// word (order_key << 32) | t with t = 0xFFFFFFFF - source (MAX) or source
// (MIN): one unsigned 64-bit compare then picks the larger (smaller) value
// and, on equal values, the smaller source index; without an index output
// the 32-bit key alone is kept.
template <int KIND, int VE, bool ARG>
struct State {
  float acc[VE];
  uint32_t key[VE];
  unsigned long long pk[VE];   // MAX / MIN word (K_ALL: the max word)
  unsigned long long pk2[VE];  // K_ALL: the min word

  static constexpr unsigned long long kInit = (KIND == K_MIN) ? ~0ull : 0ull;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int v = 0; v < VE; ++v) {
      acc[v] = 0.0f;
      key[v] = (KIND == K_MIN) ? 0xFFFFFFFFu : 0u;
      pk[v] = kInit;
      pk2[v] = ~0ull;
    }
  }
  __device__ __forceinline__ static uint32_t tie(int j) {
    return (KIND == K_MAX) ? ~(uint32_t)j : (uint32_t)j;
  }
  __device__ __forceinline__ void add(const float (&x)[VE], float w, int j) {
    const uint32_t t = tie(j);
#pragma unroll
    for (int v = 0; v < VE; ++v) {
      if constexpr (KIND == K_SUM) {
        acc[v] = fmaf(w, x[v], acc[v]);
      } else if constexpr (KIND == K_ALL) {
        acc[v] += x[v];
        const unsigned long long kk = (unsigned long long)dev::order_key(x[v]) << 32;
        const unsigned long long cmax = kk | ~(uint32_t)j, cmin = kk | (uint32_t)j;
        pk[v] = cmax > pk[v] ? cmax : pk[v];
        pk2[v] = cmin < pk2[v] ? cmin : pk2[v];
      } else if constexpr (ARG) {
        const unsigned long long c = ((unsigned long long)dev::order_key(x[v]) << 32) | t;
        pk[v] = (KIND == K_MAX) ? (c > pk[v] ? c : pk[v]) : (c < pk[v] ? c : pk[v]);
      } else {
        const uint32_t k = dev::order_key(x[v]);
        key[v] = (KIND == K_MAX) ? max(key[v], k) : min(key[v], k);
      }
    }
  }
  // value and source index of a packed word / key
  __device__ __forceinline__ float value(int v) const {
    return dev::key_to_float(ARG ? (uint32_t)(pk[v] >> 32) : key[v]);
  }
  __device__ __forceinline__ int index(int v) const {
    const uint32_t lo = (uint32_t)pk[v];
    return (int)((KIND == K_MAX) ? ~lo : lo);
  }
};

// Edge weight of SpMM entry e (source j): edge value, times 1/deg_out(j)
// (RIGHT) or deg_out(j)^-1/2 (BOTH).  The destination's factor is applied
// once per row at the end.
__device__ __forceinline__ float edge_weight(const AggParams& p, int e, int j) {
  float w = p.edge_val ? p.edge_val[e] : 1.0f;
  if (p.norm == GNN_NORM_RIGHT) w = w / (float)p.deg_out[j];
  else if (p.norm == GNN_NORM_BOTH) w = w * rsqrtf((float)p.deg_out[j]);
  return w;
}

__device__ __forceinline__ float row_factor(const AggParams& p, float acc, int deg) {
  // the mean as a product with the rounded reciprocal of the degree (one
  // division per row, within an ulp of the quotient), the same in every path
  if (p.norm == GNN_NORM_LEFT) return deg > 0 ? acc * (1.0f / (float)deg) : 0.0f;
  if (p.norm == GNN_NORM_BOTH) return deg > 0 ? acc * rsqrtf((float)deg) : 0.0f;
  return acc;
}

// Scan edges [eb, ee) for one slot (LPR lanes, lane sl), accumulating into st.
// `f_ok` says whether this lane's feature group exists (lanes past F still
// load column indices for the slot).  slot_base = first lane of the slot.
template <typename T, int LPR, int VE, int KIND, bool ARG>
__device__ __forceinline__ void scan_edges(const AggParams& p, int eb, int ee, int sl, int slot_base,
                                           const T* Xf, bool f_ok, State<KIND, VE, ARG>& st) {
  for (int e0 = eb; e0 < ee; e0 += LPR) {
    const int nb = min(LPR, ee - e0);
    const int my_e = e0 + sl;
    int my_c = 0;
    float my_w = 1.0f;
    if (sl < nb) {
      my_c = __builtin_nontemporal_load(p.col_idx + my_e);
      if (KIND == K_SUM && p.weighted) my_w = edge_weight(p, my_e, my_c);
    }
    for (int u0 = 0; u0 < nb; u0 += U) {
      int c[U];
      float w[U];
      typename RawOf<T, VE>::type x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        c[u] = __shfl(my_c, slot_base + u0 + u, 64);
        if (KIND == K_SUM) w[u] = p.weighted ? __shfl(my_w, slot_base + u0 + u, 64) : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u0 + u < nb && f_ok) x[u] = load_raw<T, VE>(row_at(Xf, c[u], p.ldx_b));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u0 + u < nb && f_ok) {
          float xv[VE];
          decode(x[u], xv);
          st.add(xv, KIND == K_SUM ? w[u] : 1.0f, c[u]);
        }
    }
  }
}

// Store one lane group's part of an output row tile (`tile` = the row's first
// element of this feature tile, `nvalid` = elements of the tile inside F).
// With VE <= 4 a lane stores its own 16 bytes and one wave store covers whole
// 128-byte lines.  With VE == 8 a lane owns 32 contiguous bytes: stored
// directly, each store instruction leaves every line half written, and such
// rows reach HBM at a third of its write bandwidth.  There the slot's tile is
// staged in LDS (`stage`, LPR * 8 words of this slot) and stored as 16
// contiguous bytes per lane.  Called by every lane of the slot.
template <int LPR, int VE>
__device__ __forceinline__ void put_tile(float* tile, const float (&v)[VE], int sl, int nvalid,
                                         float* stage) {
  if constexpr (VE == 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) stage[sl * 8 + i] = v[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = stage[sl * 4 + i];
      hi[i] = stage[LPR * 4 + sl * 4 + i];
    }
    // the stage is rewritten by the next tile only after every lane read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (sl * 4 < nvalid) storev<4>(tile + sl * 4, lo);
    if (LPR * 4 + sl * 4 < nvalid) storev<4>(tile + LPR * 4 + sl * 4, hi);
  } else {
    if (sl * VE < nvalid) storev<VE>(tile + sl * VE, v);
  }
}
template <int LPR, int VE>
__device__ __forceinline__ void put_tile_i(int32_t* tile, const int (&v)[VE], int sl, int nvalid,
                                           float* stage) {
  if constexpr (VE == 8) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __int_as_float(v[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) stage[sl * 8 + i] = f[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = __float_as_int(stage[sl * 4 + i]);
      hi[i] = __float_as_int(stage[LPR * 4 + sl * 4 + i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (sl * 4 < nvalid) storei<4>(tile + sl * 4, lo);
    if (LPR * 4 + sl * 4 < nvalid) storei<4>(tile + LPR * 4 + sl * 4, hi);
  } else {
    if (sl * VE < nvalid) storei<VE>(tile + sl * VE, v);
  }
}

// Write row `row` of the light path from the slot's state.  `ft0` = first
// feature of this tile; every lane of the slot takes part.
template <typename T, int LPR, int VE, int KIND, bool ARG>
__device__ __forceinline__ void finish_row(const AggParams& p, int row, int deg, int ft0, int sl,
                                           float* stage, State<KIND, VE, ARG>& st) {
  const int nvalid = min(LPR * VE, p.F - ft0);
  const int64_t oy = (int64_t)row * p.ldy + ft0, oa = (int64_t)row * p.F + ft0;
  if constexpr (KIND == K_ALL) {
    float o[VE];
    int ai[VE];
    if (p.Y) {
#pragma unroll
      for (int v = 0; v < VE; ++v) o[v] = st.acc[v];
      put_tile<LPR, VE>(p.Y + oy, o, sl, nvalid, stage);
    }
    if (p.Ymean) {
#pragma unroll
      for (int v = 0; v < VE; ++v) o[v] = deg > 0 ? st.acc[v] * (1.0f / (float)deg) : 0.0f;
      put_tile<LPR, VE>(p.Ymean + oy, o, sl, nvalid, stage);
    }
    if (p.Ymax) {
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        o[v] = deg > 0 ? dev::key_to_float((uint32_t)(st.pk[v] >> 32)) : 0.0f;
        ai[v] = deg > 0 ? (int)~(uint32_t)st.pk[v] : -1;
      }
      put_tile<LPR, VE>(p.Ymax + oy, o, sl, nvalid, stage);
      if (p.argmax) put_tile_i<LPR, VE>(p.argmax + oa, ai, sl, nvalid, stage);
    }
    if (p.Ymin) {
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        o[v] = deg > 0 ? dev::key_to_float((uint32_t)(st.pk2[v] >> 32)) : 0.0f;
        ai[v] = deg > 0 ? (int)(uint32_t)st.pk2[v] : -1;
      }
      put_tile<LPR, VE>(p.Ymin + oy, o, sl, nvalid, stage);
      if (p.argmin) put_tile_i<LPR, VE>(p.argmin + oa, ai, sl, nvalid, stage);
    }
    return;
  }
  float out[VE];
  int ai[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) {
    if constexpr (KIND == K_SUM) {
      out[v] = row_factor(p, st.acc[v], deg);
    } else {
      out[v] = deg > 0 ? st.value(v) : 0.0f;
      if constexpr (ARG) ai[v] = deg > 0 ? st.index(v) : -1;
    }
  }
  put_tile<LPR, VE>(p.Y + oy, out, sl, nvalid, stage);
  if constexpr (ARG) put_tile_i<LPR, VE>(p.arg + oa, ai, sl, nvalid, stage);
}

// The bf16 sum (SpMM) asks for six waves per SIMD: 80 VGPRs with 10-12
// spilled instead of 94 and five waves, and runs 2-6% faster
// on a 16M-node graph.  The fused four-way reduction keeps four waves (116
// VGPRs): at five it spills 19 and runs 5% slower.
template <typename T, int LPR, int VE, int KIND, bool ARG>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && KIND == K_SUM ? 6 : 1))) void k_aggregate(AggParams p) {
  constexpr int SPW = 64 / LPR;          // slots per wave
  constexpr int SPB = SPW * (WG / 64);   // slots per workgroup
  constexpr int FT = LPR * VE;           // features per tile
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sw = lane / LPR, sl = lane % LPR;
  const int slot = wave * SPW + sw;
  const int slot_base = sw * LPR;
  const int f0 = blockIdx.y * FT + sl * VE;
  const bool f_ok = f0 < p.F;
  const T* Xf = reinterpret_cast<const T*>(p.X) + f0;
  // item workgroups merge their slots here; light workgroups stage output
  // tiles in the same memory (each array holds at least SPB * FT words)
  __shared__ __align__(16) float s_acc[(KIND == K_SUM || KIND == K_ALL) ? SPB * FT : 1];
  __shared__ __align__(16) uint32_t s_key[(KIND == K_MAX || KIND == K_MIN) && !ARG ? SPB * FT : 1];
  __shared__ __align__(16) unsigned long long s_pk[(KIND == K_ALL || (KIND != K_SUM && ARG)) ? SPB * FT : 1];
  __shared__ unsigned long long s_pk2[(KIND == K_ALL) ? SPB * FT : 1];

  // Item workgroups come first (hardware order spreads them over the XCDs);
  // their count is padded to a multiple of 8 so that the light part starts on
  // XCD 0 and can be remapped to per-XCD runs of consecutive row ranges.
  const int n_item_pad = (p.n_item_blocks + 7) & ~7;
  if ((int)blockIdx.x < n_item_pad) {
    // ---------------- work items, strided over the item workgroups ----------------
    if ((int)blockIdx.x >= p.n_item_blocks) return;
    const int n_items = p.item_count ? min(p.n_items, *p.item_count) : p.n_items;
    for (int lid = blockIdx.x; lid < n_items; lid += p.n_item_blocks) {
      if (lid != (int)blockIdx.x) __syncthreads();  // the previous item's merge has read the LDS slots
      const int4 it = p.items[lid];
      const int row = it.x, eb = it.y, ee = it.z, m = it.w;
      const int len = ee - eb;
      const int per = (len + SPB - 1) / SPB;
      const int sb = min(ee, eb + slot * per);
      const int se = min(ee, sb + per);
      State<KIND, VE, ARG> st;
      st.init();
      scan_edges<T, LPR, VE, KIND, ARG>(p, sb, se, sl, slot_base, Xf, f_ok, st);

      // merge the slots in LDS, in slot order
  #pragma unroll
      for (int v = 0; v < VE; ++v) {
        const int t = sl * VE + v;
        if constexpr (KIND == K_ALL) {
          s_acc[slot * FT + t] = st.acc[v];
          s_pk[slot * FT + t] = st.pk[v];
          s_pk2[slot * FT + t] = st.pk2[v];
        } else if constexpr (KIND == K_SUM) {
          s_acc[slot * FT + t] = st.acc[v];
        } else if constexpr (ARG) {
          s_pk[slot * FT + t] = st.pk[v];
        } else {
          s_key[slot * FT + t] = st.key[v];
        }
      }
      __syncthreads();
      for (int t = threadIdx.x; t < FT; t += WG) {
        const int f = blockIdx.y * FT + t;
        if (f >= p.F) continue;
        float a = 0.0f;
        uint32_t k = (KIND == K_MIN) ? 0xFFFFFFFFu : 0u;
        unsigned long long w = State<KIND, VE, ARG>::kInit, w2 = ~0ull;
        for (int s2 = 0; s2 < SPB; ++s2) {
          if constexpr (KIND == K_ALL) {
            a += s_acc[s2 * FT + t];
            const unsigned long long c = s_pk[s2 * FT + t], c2 = s_pk2[s2 * FT + t];
            w = c > w ? c : w;
            w2 = c2 < w2 ? c2 : w2;
          } else if constexpr (KIND == K_SUM) {
            a += s_acc[s2 * FT + t];
          } else if constexpr (ARG) {
            const unsigned long long c = s_pk[s2 * FT + t];
            w = (KIND == K_MAX) ? (c > w ? c : w) : (c < w ? c : w);
          } else {
            const uint32_t c = s_key[s2 * FT + t];
            k = (KIND == K_MAX) ? max(k, c) : min(k, c);
          }
        }
        if constexpr (KIND != K_SUM && !ARG) w = ((unsigned long long)k << 32) | State<KIND, VE, ARG>::tie(0);
        if constexpr (KIND == K_ALL) {
          const int64_t oy = (int64_t)row * p.ldy + f, oa = (int64_t)row * p.F + f;
          if (m < 0) {
            if (p.Y) __builtin_nontemporal_store(a, p.Y + oy);
            if (p.Ymean) __builtin_nontemporal_store(a * (1.0f / (float)len), p.Ymean + oy);
            if (p.Ymax) __builtin_nontemporal_store(dev::key_to_float((uint32_t)(w >> 32)), p.Ymax + oy);
            if (p.argmax) __builtin_nontemporal_store((int)~(uint32_t)w, p.argmax + oa);
            if (p.Ymin) __builtin_nontemporal_store(dev::key_to_float((uint32_t)(w2 >> 32)), p.Ymin + oy);
            if (p.argmin) __builtin_nontemporal_store((int)(uint32_t)w2, p.argmin + oa);
          } else {
            p.partial[(int64_t)lid * p.F + f] = a;
            atomicMax(p.packed + (int64_t)m * p.F + f, w);
            atomicMin(p.packed2 + (int64_t)m * p.F + f, w2);
          }
          continue;
        }
        if (m < 0) {
          const int deg = len;  // single item covers the whole row
          if constexpr (KIND == K_SUM) {
            __builtin_nontemporal_store(row_factor(p, a, deg), p.Y + (int64_t)row * p.ldy + f);
          } else {
            const uint32_t lo = (uint32_t)w;
            __builtin_nontemporal_store(dev::key_to_float((uint32_t)(w >> 32)), p.Y + (int64_t)row * p.ldy + f);
            if constexpr (ARG)
              __builtin_nontemporal_store((int)((KIND == K_MAX) ? ~lo : lo), p.arg + (int64_t)row * p.F + f);
          }
        } else {
          if constexpr (KIND == K_SUM) {
            p.partial[(int64_t)lid * p.F + f] = a;
          } else {
            unsigned long long* dst = p.packed + (int64_t)m * p.F + f;
            if constexpr (KIND == K_MAX) atomicMax(dst, w);
            else atomicMin(dst, w);
          }
        }
      }
    }
    return;
  }

  // ---------------- light rows: rps <= LPR consecutive rows per slot ----------------
  // The slot's first rps lanes hold one row each: a prefix sum of the light degrees
  // lays the rows' edges out as one flat sequence, which the slot walks with
  // U gathers in flight across row boundaries; a row is written when the
  // walk leaves it.  Rows of the other classes inside the range count as
  // empty here (their items write them); empty light rows get the identity.
  const uint32_t lb = dev::xcd_remap(blockIdx.x - n_item_pad, p.n_light_blocks);
  const int64_t r0 = ((int64_t)lb * (WG / LPR) + slot) * p.rps;
  if (r0 >= p.n_rows) return;
  const int ft0 = blockIdx.y * FT;
  float* stage = ((KIND == K_SUM || KIND == K_ALL) ? s_acc
                  : (KIND != K_SUM && ARG) ? reinterpret_cast<float*>(s_pk)
                                           : reinterpret_cast<float*>(s_key)) + slot * FT;
  const int64_t myr = r0 + sl;
  int rs = 0, dr = -1;
  if (sl < p.rps && myr < p.n_rows) {
    rs = p.row_ptr[myr];
    dr = p.row_ptr[myr + 1] - rs;
  }
  const bool lt = dr >= 0 && dr <= p.light_max;
  const int d = lt ? dr : 0;
  int incl = d;
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) {
    const int t = __shfl_up(incl, o, LPR);
    if (sl >= o) incl += t;
  }
  const int off = rs - (incl - d);  // edge position of flat index k in this row: off + k
  const int total = __shfl(incl, slot_base + LPR - 1, 64);
  {
    const unsigned long long b = __ballot(lt && dr == 0);
    unsigned long long em = (LPR == 64) ? b : (b >> slot_base) & ((1ull << (LPR & 63)) - 1);
    State<KIND, VE, ARG> z;
    z.init();
    while (em) {
      const int t = __builtin_ctzll(em);
      em &= em - 1;
      finish_row<T, LPR, VE, KIND, ARG>(p, (int)(r0 + t), 0, ft0, sl, stage, z);
    }
  }
  State<KIND, VE, ARG> st;
  st.init();
  int cur = -1;
  for (int kb = 0; kb < total; kb += LPR) {
    const int nb = min(LPR, total - kb);
    const int k = kb + sl;
    // local row of flat edge k: the number of rows whose inclusive end is <= k
    int lo = 0;
#pragma unroll
    for (int step = LPR / 2; step >= 1; step >>= 1)
      if (__shfl(incl, slot_base + lo + step - 1, 64) <= k) lo += step;
    const int my_off = __shfl(off, slot_base + lo, 64);
    int my_c = 0;
    float my_w = 1.0f;
    if (sl < nb) {
      const int e = my_off + k;
      my_c = __builtin_nontemporal_load(p.col_idx + e);
      if (KIND == K_SUM && p.weighted) my_w = edge_weight(p, e, my_c);
    }
    for (int u0 = 0; u0 < nb; u0 += U) {
      int c[U], tr[U];
      float w[U];
      typename RawOf<T, VE>::type x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        c[u] = __shfl(my_c, slot_base + u0 + u, 64);
        tr[u] = __shfl(lo, slot_base + u0 + u, 64);
        if (KIND == K_SUM) w[u] = p.weighted ? __shfl(my_w, slot_base + u0 + u, 64) : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u0 + u < nb && f_ok) x[u] = load_raw<T, VE>(row_at(Xf, c[u], p.ldx_b));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u0 + u < nb) {
          if (tr[u] != cur) {  // uniform over the slot
            if (cur >= 0) {
              const int dd = __shfl(d, slot_base + cur, 64);
              finish_row<T, LPR, VE, KIND, ARG>(p, (int)(r0 + cur), dd, ft0, sl, stage, st);
            }
            cur = tr[u];
            st.init();
          }
          if (f_ok) {
            float xv[VE];
            decode(x[u], xv);
            st.add(xv, KIND == K_SUM ? w[u] : 1.0f, c[u]);
          }
        }
      }
    }
  }
  if (cur >= 0) {
    const int dd = __shfl(d, slot_base + cur, 64);
    finish_row<T, LPR, VE, KIND, ARG>(p, (int)(r0 + cur), dd, ft0, sl, stage, st);
  }
}

// Sum of a heavy row's item partials, in item order (deterministic).
__global__ __launch_bounds__(256) void k_combine_sum(AggParams p, const int4* multi) {
  if (p.multi_count && (int)blockIdx.x >= *p.multi_count) return;
  const int4 mr = multi[blockIdx.x];
  const int row = mr.x, first = mr.y, cnt = mr.z;
  const int deg = p.row_ptr[row + 1] - p.row_ptr[row];
  for (int f = threadIdx.x; f < p.F; f += blockDim.x) {
    float a = 0.0f;
    for (int c = 0; c < cnt; ++c) a += p.partial[(int64_t)(first + c) * p.F + f];
    p.Y[(int64_t)row * p.ldy + f] = row_factor(p, a, deg);
  }
}

// K_ALL: sum / mean from the item partials (item order), max / min unpacked.
__global__ __launch_bounds__(256) void k_combine_all(AggParams p, const int4* multi) {
  if (p.multi_count && (int)blockIdx.x >= *p.multi_count) return;
  const int4 mr = multi[blockIdx.x];
  const int row = mr.x, first = mr.y, cnt = mr.z;
  const int deg = p.row_ptr[row + 1] - p.row_ptr[row];
  for (int f = threadIdx.x; f < p.F; f += blockDim.x) {
    float a = 0.0f;
    for (int c = 0; c < cnt; ++c) a += p.partial[(int64_t)(first + c) * p.F + f];
    const int64_t oy = (int64_t)row * p.ldy + f, oa = (int64_t)row * p.F + f;
    if (p.Y) p.Y[oy] = a;
    if (p.Ymean) p.Ymean[oy] = a * (1.0f / (float)deg);
    const unsigned long long w = p.packed[(int64_t)blockIdx.x * p.F + f];
    const unsigned long long w2 = p.packed2[(int64_t)blockIdx.x * p.F + f];
    if (p.Ymax) p.Ymax[oy] = dev::key_to_float((uint32_t)(w >> 32));
    if (p.argmax) p.argmax[oa] = (int)~(uint32_t)w;
    if (p.Ymin) p.Ymin[oy] = dev::key_to_float((uint32_t)(w2 >> 32));
    if (p.argmin) p.argmin[oa] = (int)(uint32_t)w2;
  }
}

// Packed (key, index) words of heavy rows back to value and source index.
template <int KIND, bool ARG>
__global__ __launch_bounds__(256) void k_unpack(AggParams p, const int4* multi) {
  if (p.multi_count && (int)blockIdx.x >= *p.multi_count) return;
  const int row = multi[blockIdx.x].x;
  for (int f = threadIdx.x; f < p.F; f += blockDim.x) {
    unsigned long long w = p.packed[(int64_t)blockIdx.x * p.F + f];
    uint32_t k = (uint32_t)(w >> 32), lo = (uint32_t)w;
    p.Y[(int64_t)row * p.ldy + f] = dev::key_to_float(k);
    if constexpr (ARG) p.arg[(int64_t)row * p.F + f] = (int)(KIND == K_MAX ? 0xFFFFFFFFu - lo : lo);
  }
}

// p[0, n) = v; with rows set, only the first *rows * per words of them.
__global__ void k_fill_u64(unsigned long long* p, int64_t n, unsigned long long v, const int32_t* rows,
                           int32_t per) {
  if (rows) n = min(n, (int64_t)*rows * per);
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <typename T, int LPR, int VE, int KIND, bool ARG>
int launch_one(gnn_plan* pl, AggParams& p, hipStream_t s) {
  constexpr int FT = LPR * VE;
  const int ftiles = (p.F + FT - 1) / FT;
  p.n_items = (int32_t)pl->n_items;
  p.n_item_blocks = std::min<int32_t>(p.n_items, kItemBlocks);
  p.item_count = pl->item_count;
  p.multi_count = pl->multi_count;
  // a light workgroup covers (WG / LPR) * rps rows: 64 / LPR slots per wave,
  // rps rows per slot.  rps = LPR unless that leaves fewer than 1024
  // workgroups (four per CU): a slot walks its rows' edges as one dependent
  // sequence, so on small graphs fewer rows per slot cut the latency chain.
  const int64_t spw = WG / LPR;
  int rps = LPR;
  while (rps > 1 && (p.n_rows + spw * rps - 1) / (spw * rps) * ftiles < 1024) rps >>= 1;
  p.rps = rps;
  p.n_light_blocks = (int32_t)((p.n_rows + spw * rps - 1) / (spw * rps));
  const int64_t gx = (((int64_t)p.n_item_blocks + 7) & ~7LL) + p.n_light_blocks;
  if (gx > 0x7FFFFFFF) return fail(GNN_ERR_SIZE_OVERFLOW, "aggregate grid too large");
  if (KIND != K_SUM && pl->n_multi > 0) {
    int64_t nw = pl->n_multi * p.F;
    const unsigned nb = (unsigned)std::min<int64_t>((nw + 255) / 256, 16384);
    hipLaunchKernelGGL(k_fill_u64, dim3(nb), dim3(256), 0, s, p.packed, nw, KIND == K_MIN ? ~0ull : 0ull,
                       pl->multi_count, p.F);
    GNN_LAUNCH_CHECK("fill packed");
    if (KIND == K_ALL) {
      hipLaunchKernelGGL(k_fill_u64, dim3(nb), dim3(256), 0, s, p.packed2, nw, ~0ull, pl->multi_count, p.F);
      GNN_LAUNCH_CHECK("fill packed");
    }
  }
  if (gx > 0) {
    hipLaunchKernelGGL((k_aggregate<T, LPR, VE, KIND, ARG>), dim3((unsigned)gx, (unsigned)ftiles),
                       dim3(WG), 0, s, p);
    GNN_LAUNCH_CHECK("aggregate");
  }
  if (pl->n_multi > 0) {
    if constexpr (KIND == K_ALL) {
      hipLaunchKernelGGL(k_combine_all, dim3((unsigned)pl->n_multi), dim3(256), 0, s, p,
                         (const int4*)pl->multi);
    } else if constexpr (KIND == K_SUM) {
      hipLaunchKernelGGL(k_combine_sum, dim3((unsigned)pl->n_multi), dim3(256), 0, s, p,
                         (const int4*)pl->multi);
    } else {
      hipLaunchKernelGGL((k_unpack<KIND, ARG>), dim3((unsigned)pl->n_multi), dim3(256), 0, s, p,
                         (const int4*)pl->multi);
    }
    GNN_LAUNCH_CHECK("merge heavy rows");
  }
  return GNN_OK;
}

template <typename T, int VE, int KIND, bool ARG>
int pick_lpr(gnn_plan* pl, AggParams& p, int lpr, hipStream_t s) {
  if constexpr (VE == 1) {
    return launch_one<T, 64, 1, KIND, ARG>(pl, p, s);
  } else {
    switch (lpr) {
      case 8: return launch_one<T, 8, VE, KIND, ARG>(pl, p, s);
      case 16: return launch_one<T, 16, VE, KIND, ARG>(pl, p, s);
      case 32: return launch_one<T, 32, VE, KIND, ARG>(pl, p, s);
      default: return launch_one<T, 64, VE, KIND, ARG>(pl, p, s);
    }
  }
}

template <typename T, int VE>
int pick_kind(gnn_plan* pl, AggParams& p, int kind, bool arg, int lpr, hipStream_t s) {
  if (kind == K_ALL) return pick_lpr<T, VE, K_ALL, true>(pl, p, lpr, s);
  if (kind == K_SUM) return pick_lpr<T, VE, K_SUM, false>(pl, p, lpr, s);
  if (kind == K_MAX)
    return arg ? pick_lpr<T, VE, K_MAX, true>(pl, p, lpr, s) : pick_lpr<T, VE, K_MAX, false>(pl, p, lpr, s);
  return arg ? pick_lpr<T, VE, K_MIN, true>(pl, p, lpr, s) : pick_lpr<T, VE, K_MIN, false>(pl, p, lpr, s);
}

}  // namespace

int launch_aggregate(gnn_plan* pl, const void* X, gnn_dtype xt, int32_t F, int64_t ldx, float* Y,
                     int64_t ldy, int mode, gnn_norm norm, const float* edge_val, int32_t* arg,
                     hipStream_t s) {
  if (mode == AGG_SPMM && (norm == GNN_NORM_RIGHT || norm == GNN_NORM_BOTH)) GNN_TRY(plan_deg_out(pl, s));
  AggParams p{};
  p.row_ptr = pl->row_ptr;
  p.col_idx = pl->col_idx;
  p.edge_val = (mode == AGG_SPMM) ? edge_val : nullptr;
  p.deg_out = pl->deg_out;
  p.X = X;
  p.ldx = ldx;
  p.Y = Y;
  p.ldy = ldy;
  p.arg = arg;
  p.items = pl->items;
  p.n_rows = pl->n_rows;
  p.F = F;
  p.light_max = pl->light_max;
  p.norm = (mode == AGG_SPMM) ? (int)norm : (mode == AGG_MEAN ? (int)GNN_NORM_LEFT : 0);
  p.weighted = (p.edge_val != nullptr) || p.norm == GNN_NORM_RIGHT || p.norm == GNN_NORM_BOTH;
  const int kind = (mode == AGG_MAX) ? K_MAX : (mode == AGG_MIN ? K_MIN : K_SUM);

  // workspace: partials for sums of heavy rows, packed words for max / min
  if (pl->n_multi > 0) {
    void* ws = nullptr;
    size_t need = (kind == K_SUM) ? (size_t)pl->n_slots * F * 4 : (size_t)pl->n_multi * F * 8;
    GNN_TRY(plan_workspace(pl, need, &ws));
    p.partial = (float*)ws;
    p.packed = (unsigned long long*)ws;
  }

  const int esz = (xt == GNN_BF16) ? 2 : 4;
  const int64_t rowb = (int64_t)F * esz;
  if (ldx * esz > (int64_t)UINT32_MAX) return fail(GNN_ERR_SIZE_OVERFLOW, "X row stride of 4 GB or more");
  p.ldx_b = (uint32_t)(ldx * esz);
  const bool vec_ok = (rowb % 16 == 0) && ((ldx * esz) % 16 == 0) && ((uintptr_t)X % 16 == 0) &&
                      ((uintptr_t)Y % 16 == 0) && (ldy % 4 == 0) &&
                      (arg == nullptr || ((uintptr_t)arg % 16 == 0 && F % 4 == 0));
  int lpr = 64;
  if (vec_ok) {
    int lanes = (int)std::min<int64_t>(rowb / 16, 64);
    lpr = 8;
    while (lpr < lanes) lpr <<= 1;
  }
  if (xt == GNN_BF16) {
    return vec_ok ? pick_kind<uint16_t, 8>(pl, p, kind, arg != nullptr, lpr, s)
                  : pick_kind<uint16_t, 1>(pl, p, kind, arg != nullptr, lpr, s);
  }
  return vec_ok ? pick_kind<float, 4>(pl, p, kind, arg != nullptr, lpr, s)
                : pick_kind<float, 1>(pl, p, kind, arg != nullptr, lpr, s);
}

size_t reduce_multi_ws_bytes(const gnn_plan* pl, int32_t F) {
  if (pl->n_multi <= 0) return 0;
  const size_t part = ((size_t)pl->n_slots * F * 4 + 255) & ~(size_t)255;
  const size_t words = (size_t)pl->n_multi * F * 8;
  return part + 2 * words;
}

int launch_reduce_multi(gnn_plan* pl, const void* X, gnn_dtype xt, int32_t F, int64_t ldx,
                        float* Ysum, float* Ymean, float* Ymax, int32_t* argmax, float* Ymin,
                        int32_t* argmin, int64_t ldy, hipStream_t s, void* ws_given) {
  AggParams p{};
  p.row_ptr = pl->row_ptr;
  p.col_idx = pl->col_idx;
  p.deg_out = pl->deg_out;
  p.X = X;
  p.ldx = ldx;
  p.Y = Ysum;
  p.Ymean = Ymean;
  p.Ymax = Ymax;
  p.Ymin = Ymin;
  p.argmax = argmax;
  p.argmin = argmin;
  p.ldy = ldy;
  p.items = pl->items;
  p.n_rows = pl->n_rows;
  p.F = F;
  p.light_max = pl->light_max;
  if (pl->n_multi > 0) {
    // split rows: item partial sums, then the packed max and min words
    void* ws = ws_given;
    const size_t part = ((size_t)pl->n_slots * F * 4 + 255) & ~(size_t)255;
    const size_t words = (size_t)pl->n_multi * F * 8;
    if (!ws) GNN_TRY(plan_workspace(pl, part + 2 * words, &ws));
    p.partial = (float*)ws;
    p.packed = (unsigned long long*)((char*)ws + part);
    p.packed2 = (unsigned long long*)((char*)ws + part + words);
  }
  const int esz = (xt == GNN_BF16) ? 2 : 4;
  const int64_t rowb = (int64_t)F * esz;
  if (ldx * esz > (int64_t)UINT32_MAX) return fail(GNN_ERR_SIZE_OVERFLOW, "X row stride of 4 GB or more");
  p.ldx_b = (uint32_t)(ldx * esz);
  const uintptr_t outs = (uintptr_t)Ysum | (uintptr_t)Ymean | (uintptr_t)Ymax | (uintptr_t)Ymin |
                         (uintptr_t)argmax | (uintptr_t)argmin;
  const bool vec_ok = (rowb % 16 == 0) && ((ldx * esz) % 16 == 0) && ((uintptr_t)X % 16 == 0) &&
                      (outs % 16 == 0) && (ldy % 4 == 0) && (F % 4 == 0);
  int lpr = 64;
  if (vec_ok) {
    int lanes = (int)std::min<int64_t>(rowb / 16, 64);
    lpr = 8;
    while (lpr < lanes) lpr <<= 1;
  }
  if (xt == GNN_BF16)
    return vec_ok ? pick_kind<uint16_t, 8>(pl, p, K_ALL, true, lpr, s)
                  : pick_kind<uint16_t, 1>(pl, p, K_ALL, true, lpr, s);
  return vec_ok ? pick_kind<float, 4>(pl, p, K_ALL, true, lpr, s)
                : pick_kind<float, 1>(pl, p, K_ALL, true, lpr, s);
}

}  // namespace gnn
