// SpMM on 16 x 16 block-sparse tiles with fp32 matrix cores (WSB-SpMM).
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.3: the windowed segmented bitmap format
// (16-row windows, blocks of 8 distinct source columns with a 128-bit mask)
// serves the SpMM convolution as well as attention: per window, each dense
// 16 x 16 tile of A multiplies the 16 gathered feature rows of its columns,
// so a gathered row serves every entry of its column in the window instead of
// one.  The plan's residual CSR (entries of tiles below the density
// threshold) is added by a plain loop into the same accumulators.
//
// MI355X mapping.  One workgroup per (window, 256-feature slice); wave w owns
// features 64 w .. 64 w + 63 of the slice as four 16-wide chunks.  For each
// dense tile the workgroup stages the 16 X rows (the slice of each) in LDS,
// double-buffered (the next tile's rows are loaded into registers while the
// current one computes).  A is built in registers from the tile bitmap and the
// column weights; every product is exact in fp32 and accumulates in fp32, as
// in the CSR kernel:
//   bf16 X: per chunk one v_mfma_f32_16x16x16_bf16 over the tile's 16
//     columns, B read from LDS with the transpose read.  A column weight that
//     is not 1 (RIGHT, BOTH) is split exactly into three bf16 parts, w = hi +
//     mid + lo (8 significant bits each, 24 in all), one MFMA each: a
//     bf16 x bf16 product is exact in fp32, so the sum of the three products
//     is w x up to the fp32 accumulation.
//   fp32 X: 4 k-steps x 4 chunks of v_mfma_f32_16x16x4_f32.
// Lane layouts (checked on the device): 16x16x4 f32: A: lane l holds
// A[l % 16][l / 16]; B: B[l / 16][l % 16].  16x16x16 bf16: A: lane l holds
// A[l % 16][4 (l / 16) .. +3]; B: B[4 (l / 16) .. +3][l % 16].  Both: D: lane
// l holds D[4 (l / 16) + r][l % 16], r = 0..3.  The window's tile
// metadata (columns, weights, bitmap words) is staged in LDS up front, so a
// tile's row gathers wait on one memory latency instead of three dependent
// ones.  Output rows are staged through LDS so that each store writes whole
// lines.
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int FW = 256;   // features per workgroup
constexpr int LDX = FW + 8;  // staged row stride: 16 rows of one transpose read land on distinct LDS banks
constexpr int MAXT = 16;  // tiles whose metadata is staged at once
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The B operand of a 16x16x16 bf16 MFMA (lane 16g + r: rows 4g .. 4g + 3 of
// column r) from a 16 x 16 block stored row-major in LDS (row stride ld), by
// the gfx950 LDS transpose read: within each 16 lanes, lane 16g + 4i + a
// names row 4g + i, columns 4a .. 4a + 3, and lane 16g + 4a + j receives
// element j of the rows named by lanes 16g + a, 16g + 4 + a, ...  Needs every
// lane active.
__device__ __forceinline__ s16x4 lds_tr_operand(const uint16_t* blk, int ld, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* a = blk + (4 * g + (r >> 2)) * ld + 4 * (r & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
}

struct B16SpmmParams {
  const int32_t* row_ptr;
  const int32_t* deg_out;
  const int32_t* win_ptr;
  const int32_t* blk_col;
  const unsigned long long* blk_bits;
  const int32_t* tile_ptr;
  const int32_t* tile_blk;
  const int32_t* res_ptr;
  const int32_t* res_col;
  const void* X;
  int64_t ldx;
  float* Y;
  int64_t ldy;
  int32_t F;
  int32_t n_rows;
  int32_t norm;
};

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// weight of a column j (the destination's factor is applied per row at the end)
__device__ __forceinline__ float col_weight(const B16SpmmParams& p, int j) {
  if (p.norm == GNN_NORM_RIGHT) return 1.0f / (float)p.deg_out[j];
  if (p.norm == GNN_NORM_BOTH) return rsqrtf((float)p.deg_out[j]);
  return 1.0f;
}

// bf16: seven waves per SIMD (72 VGPRs, no spills; 19.4 KB of LDS per
// workgroup). Eight waves cap the kernel at 64 VGPRs and spill three, which
// measured 7% slower.
// WIDE: 64-bit block-column offsets, for layouts of 2^28 blocks or more (the
// 32-bit form costs two fewer registers and runs about 5% faster).
template <typename T, bool WIDE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 7 : 4))) void k_spmm_b16(B16SpmmParams p) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = FW / EPC;              // chunks per staged row slice
  constexpr int CPT = 16 * CPR / 256;        // chunks per thread per tile
  __shared__ __align__(16) T s_x[2][16][LDX];
  // the window's tile metadata, MAXT tiles at a time: the 16 columns of each
  // tile, their weights (0 for padding) and the two blocks' bitmap words
  __shared__ int32_t s_tcol[MAXT][16];
  __shared__ float s_tw[MAXT][16];
  __shared__ unsigned long long s_tbits[MAXT][4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int w = (int)dev::xcd_remap(blockIdx.x, gridDim.x);
  const int f0 = blockIdx.y * FW;                 // first feature of the slice
  const int fw = f0 + wave * 64;                  // first feature of this wave
  const int t_beg = p.tile_ptr[w], t_end = p.tile_ptr[w + 1];
  const int b_end = p.win_ptr[w + 1];
  const T* X = reinterpret_cast<const T*>(p.X);

  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // this thread's share of the 16 staged rows of local tile k
  uint4 pre[CPT];
  auto load_tile = [&](int k) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int chunk = threadIdx.x + q * 256;   // 0 .. 16 * CPR - 1
      const int r = chunk / CPR, cc = chunk % CPR;
      const int col = s_tcol[k][r];
      const int f = f0 + cc * EPC;
      // row col at a byte stride below 4 GB: one unsigned 32 x 32 -> 64 multiply-add
      const T* xr = reinterpret_cast<const T*>(reinterpret_cast<const char*>(X) +
                                               (uint64_t)(uint32_t)col * (uint32_t)(p.ldx * (int64_t)sizeof(T)));
      pre[q] = (f < p.F) ? *reinterpret_cast<const uint4*>(xr + f) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int chunk = threadIdx.x + q * 256;
      const int r = chunk / CPR, cc = chunk % CPR;
      *reinterpret_cast<uint4*>(&s_x[buf][r][cc * EPC]) = pre[q];
    }
  };

  for (int tb = t_beg; tb < t_end; tb += MAXT) {
    const int nt = min(MAXT, t_end - tb);
    __syncthreads();  // the previous batch is done with the metadata and the buffers
    for (int q = threadIdx.x; q < nt * 16; q += 256) {
      const int k = q >> 4, c = q & 15;
      const int blk = p.tile_blk[tb + k] + (c >> 3);
      const bool have = !((c >> 3) == 1 && blk >= b_end);   // second block past the window: padding
      int col = 0;
      if (have) {
        if constexpr (WIDE) col = p.blk_col[(int64_t)blk * 8 + (c & 7)];
        else col = p.blk_col[blk * 8 + (c & 7)];
      }
      s_tcol[k][c] = col;
      s_tw[k][c] = have ? col_weight(p, col) : 0.0f;
      if (c < 4) {
        const int bb = p.tile_blk[tb + k] + (c >> 1);
        const bool hb = !((c >> 1) == 1 && bb >= b_end);
        s_tbits[k][c] = hb ? p.blk_bits[(int64_t)bb * 2 + (c & 1)] : 0ull;
      }
    }
    __syncthreads();
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int k = 0; k < nt; ++k) {
      const int buf = k & 1;
      if (k + 1 < nt) load_tile(k + 1);
      if constexpr (sizeof(T) == 2) {
        // A values of this lane: row li, tile columns 4 lg .. 4 lg + 3; the
        // four B operands of its chunks
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * lg + i;
          const unsigned long long word = s_tbits[k][(c >> 3) * 2 + (li >> 3)];
          const bool bit = (word >> ((li & 7) * 8 + (c & 7))) & 1ull;
          a[i] = bit ? s_tw[k][c] : 0.0f;
        }
        s16x4 b[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch)
          b[ch] = lds_tr_operand(reinterpret_cast<const uint16_t*>(&s_x[buf][0][wave * 64 + ch * 16]), LDX, lane);
        // the weights in exact bf16 parts, high to low: a part is a rounded
        // to bf16, and a keeps the (exact) remainder; one part when every
        // weight is 1
        const int parts = (p.norm == GNN_NORM_RIGHT || p.norm == GNN_NORM_BOTH) ? 3 : 1;
        for (int q = 0; q < parts; ++q) {
          s16x4 ap;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint16_t h = f2bf(a[i]);
            ap[i] = (short)h;
            a[i] -= bf2f(h);
          }
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ap, b[ch], acc[ch], 0, 0, 0);
        }
      } else {
        // A values of this lane: row li, tile columns 4 s + lg
        float a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = 4 * s + lg;
          const unsigned long long word = s_tbits[k][(c >> 3) * 2 + (li >> 3)];
          const bool bit = (word >> ((li & 7) * 8 + (c & 7))) & 1ull;
          a[s] = bit ? s_tw[k][c] : 0.0f;
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const int fl = wave * 64 + ch * 16 + li;   // feature within the slice
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float b = to_f32<T>(s_x[buf][4 * s + lg][fl]);
            acc[ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b, acc[ch], 0, 0, 0);
          }
        }
      }
      __syncthreads();  // every wave is done with the other buffer before it is refilled
      if (k + 1 < nt) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // residual entries of the window's rows: lane (li, lg) owns rows 4 lg .. 4 lg + 3 of
  // feature fw + 16 ch + li
  const int row0 = w * 16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * lg + r;
    if (row >= p.n_rows) continue;
    const int e1 = p.res_ptr[row + 1];
    for (int e = p.res_ptr[row]; e < e1; ++e) {
      const int j = p.res_col[e];
      const float wj = col_weight(p, j);
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int f = fw + ch * 16 + li;
        if (f < p.F) acc[ch][r] = fmaf(wj, to_f32<T>(X[(int64_t)j * p.ldx + f]), acc[ch][r]);
      }
    }
  }

  // destination factor, then stage the 16 x FW slice in LDS and store whole rows
  float* s_y = reinterpret_cast<float*>(&s_x[0][0][0]);   // 16 x FW floats fit the two buffers
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * lg + r;
    float rf = 1.0f;
    if (row < p.n_rows && (p.norm == GNN_NORM_LEFT || p.norm == GNN_NORM_BOTH)) {
      const int d = p.row_ptr[row + 1] - p.row_ptr[row];
      rf = d > 0 ? (p.norm == GNN_NORM_LEFT ? 1.0f / (float)d : rsqrtf((float)d)) : 0.0f;
    }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) s_y[(4 * lg + r) * FW + wave * 64 + ch * 16 + li] = acc[ch][r] * rf;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 16 * FW / 4; q += 256) {
    const int r = q / (FW / 4), f = f0 + (q % (FW / 4)) * 4;
    const int row = row0 + r;
    if (row < p.n_rows && f < p.F)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(s_y + r * FW + (f - f0)),
                                  reinterpret_cast<f32x4_t*>(p.Y + (int64_t)row * p.ldy + f));
  }
}

}  // namespace

int launch_spmm_block16(gnn_plan* pl, const void* X, gnn_dtype xt, int32_t F, int64_t ldx, float* Y, int64_t ldy,
                        gnn_norm norm, hipStream_t s) {
  if (norm == GNN_NORM_RIGHT || norm == GNN_NORM_BOTH) GNN_TRY(plan_deg_out(pl, s));
  B16SpmmParams p{};
  p.row_ptr = pl->row_ptr;
  p.deg_out = pl->deg_out;
  p.win_ptr = pl->wsb.win_ptr;
  p.blk_col = pl->wsb.blk_col;
  p.blk_bits = (const unsigned long long*)pl->wsb.blk_bits;
  p.tile_ptr = pl->wsb.tile_ptr;
  p.tile_blk = pl->wsb.tile_blk;
  p.res_ptr = pl->wsb.res_ptr;
  p.res_col = pl->wsb.res_col;
  p.X = X;
  p.ldx = ldx;
  if (ldx * (xt == GNN_BF16 ? 2 : 4) > (int64_t)UINT32_MAX) return fail(GNN_ERR_SIZE_OVERFLOW, "X row stride of 4 GB or more");
  p.Y = Y;
  p.ldy = ldy;
  p.F = F;
  p.n_rows = pl->n_rows;
  p.norm = (int)norm;
  if (pl->wsb.n_windows == 0) return GNN_OK;
  const dim3 grid((unsigned)pl->wsb.n_windows, (unsigned)((F + FW - 1) / FW));
  const bool wide = pl->wsb.n_blocks * 8 >= (int64_t)1 << 31;
  if (xt == GNN_BF16) {
    if (wide) hipLaunchKernelGGL((k_spmm_b16<uint16_t, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_spmm_b16<uint16_t, false>), grid, dim3(256), 0, s, p);
  } else {
    if (wide) hipLaunchKernelGGL((k_spmm_b16<float, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_spmm_b16<float, false>), grid, dim3(256), 0, s, p);
  }
  GNN_LAUNCH_CHECK("spmm block16");
  return GNN_OK;
}

}  // namespace gnn
