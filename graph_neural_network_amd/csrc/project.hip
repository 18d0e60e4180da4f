// Per-vertex linear projections of the attention layers on bf16 matrix cores.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", section 2.2 (iii): GATv2 scores a^T LeakyReLU(W_l h_i +
// W_r h_j) with values v_j = W_r h_j; the Graph Transformer's q_i = W_Q h_i,
// k_j = W_K h_j, v_j = W_V h_j.  Appendix D.2 runs the fused kernels on these
// vectors precomputed once per vertex; this file computes them:
//   Y_m[i, o] = sum_k X[i, k] W_m[o, k]   for m < n_mat (up to three weights),
// X [n, f_in] bf16, W_m [f_out, f_in] bf16 (one row per output feature),
// products exact in fp32, fp32 accumulation, output rounded to bf16 (nearest
// even).  A dense contraction: it belongs on the matrix cores.
//
// MI355X mapping.  A wave owns 16 * MR rows of X and keeps their K = f_in
// columns in registers as B operands of v_mfma_f32_16x16x32_bf16, loaded
// straight from memory in operand layout (lane l: row l % 16, k 8 (l / 16)
// .. +7, 16 contiguous bytes).  For every 16-feature output tile it streams
// the weight rows in as A operands (W is tiny and stays in L1 / L2) and
// forms Y^T = W X^T, so lane l ends with Y[row l % 16][o 4 (l / 16) .. +3]:
// four consecutive outputs of one row, converted to bf16 in one instruction
// and written as 8 bytes to the wave's LDS staging tile.  The staged
// 16 * MR x 64 block is then stored as 16 contiguous bytes per lane, whole
// lines per instruction.  Each weight fragment serves MR row tiles.
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int WG = 256;
constexpr int OCH = 64;            // output features staged per pass
constexpr int SROW = OCH + 8;      // staging row stride (bf16), padded against bank conflicts
constexpr size_t kProjLdsMax = 160 * 1024;  // LDS of one CU

struct ProjParams {
  const uint16_t* X;
  const uint16_t* W[3];
  uint16_t* Y[3];
  int64_t ldx;
  int32_t n;
  int32_t f_out;
  int32_t n_mat;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int KS, int MR>
__global__ __launch_bounds__(WG) void k_project(ProjParams p) {
  constexpr int K = 32 * KS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t r_base = ((int64_t)blockIdx.x * (WG / 64) + wave) * 16 * MR;
  if (r_base >= p.n) return;  // the whole wave leaves; staging is wave-private
  const int lr = lane & 15, lk = lane >> 4;

  // B operands: this wave's rows of X (rows past n re-read the last row)
  bf16x8 xf[MR][KS];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const int64_t row = min<int64_t>(r_base + 16 * r + lr, (int64_t)p.n - 1);
    const uint16_t* src = p.X + row * p.ldx + 8 * lk;
#pragma unroll
    for (int k = 0; k < KS; ++k) xf[r][k] = *reinterpret_cast<const bf16x8*>(src + 32 * k);
  }

  __shared__ __align__(16) uint16_t stage[WG / 64][16 * MR][SROW];
  uint16_t(*st)[SROW] = stage[wave];
  const int n_here = (int)min<int64_t>(16 * MR, (int64_t)p.n - r_base);

  // output chunks of OCH features of each of the n_mat weights in turn
  const int cpm = (p.f_out + OCH - 1) / OCH;  // chunks per weight
  for (int cidx = 0; cidx < p.n_mat * cpm; ++cidx) {
    const int m = cidx / cpm, o0 = (cidx % cpm) * OCH;
    const uint16_t* W = p.W[m];
    uint16_t* Y = p.Y[m];
    const int ow = min(OCH, p.f_out - o0);  // a multiple of 16
    // weight fragments of the next 16-feature tile are loaded while the
    // current tile's products run
    bf16x8 wcur[KS], wnxt[KS];
    const uint16_t* w0 = W + (int64_t)(o0 + lr) * K + 8 * lk;
#pragma unroll
    for (int k = 0; k < KS; ++k) wcur[k] = *reinterpret_cast<const bf16x8*>(w0 + 32 * k);
    for (int t = 0; t < ow; t += 16) {
      const int tn = t + 16 < ow ? t + 16 : t;  // the last tile re-reads itself
      const uint16_t* wn = W + (int64_t)(o0 + tn + lr) * K + 8 * lk;
#pragma unroll
      for (int k = 0; k < KS; ++k) wnxt[k] = *reinterpret_cast<const bf16x8*>(wn + 32 * k);
      f32x4 acc[MR];
#pragma unroll
      for (int r = 0; r < MR; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[k], xf[r][k], acc[r], 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < KS; ++k) wcur[k] = wnxt[k];
      // lane: row 16 r + lr, outputs t + 4 lk .. +3
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const uint2 w2 = make_uint2(pack_bf16(acc[r][0], acc[r][1]), pack_bf16(acc[r][2], acc[r][3]));
        *reinterpret_cast<uint2*>(&st[16 * r + lr][t + 4 * lk]) = w2;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // store the staged rows: ow / 8 lanes of 16 bytes per row
    const int lpr = ow / 8;
    for (int q = lane; q < n_here * lpr; q += 64) {
      const int row = q / lpr, c = (q % lpr) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(&st[row][c]);
      *reinterpret_cast<uint4*>(Y + (r_base + row) * p.f_out + o0 + c) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// The same products with the weights in LDS, for weights that fit there:
// one resident workgroup per CU of NWV waves loads every weight once
// (cooperatively, rows padded by 8 bf16 so that the 16 rows an A-operand read
// touches fall in distinct banks) and its waves then take 16 * MR-row tiles
// of X in turn.  Reading the weights from L2 for every wave (k_project)
// moves 64 KB per 64 rows of X at f_in = 128 with two 128-wide weights: the
// GATv2 layer's projection (200k rows) took 0.058 ms that way, 0.037 ms here.
// Loading the next tile's rows during the current one's products measured
// no faster.
template <int KS, int MR, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_project_lds(ProjParams p) {
  constexpr int K = 32 * KS;
  constexpr int WROW = K + 8;  // padded weight row (bf16)
  extern __shared__ __align__(16) uint16_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  uint16_t* wl = lds;  // [n_mat * f_out][WROW]
  uint16_t(*st)[SROW] = reinterpret_cast<uint16_t(*)[SROW]>(lds + (size_t)p.n_mat * p.f_out * WROW +
                                                              (size_t)wave * 16 * MR * SROW);
  {
    const int per_row = K / 8, rows = p.n_mat * p.f_out;
    for (int q = threadIdx.x; q < rows * per_row; q += 64 * NWV) {
      const int r = q / per_row, c = (q % per_row) * 8;
      const int m = r / p.f_out, o = r % p.f_out;
      *reinterpret_cast<uint4*>(wl + (size_t)r * WROW + c) =
          *reinterpret_cast<const uint4*>(p.W[m] + (int64_t)o * K + c);
    }
  }
  __syncthreads();
  const int64_t n_tiles = ((int64_t)p.n + 16 * MR - 1) / (16 * MR);
  const int cpm = (p.f_out + OCH - 1) / OCH;  // chunks per weight
  for (int64_t tile = (int64_t)blockIdx.x * NWV + wave; tile < n_tiles; tile += (int64_t)gridDim.x * NWV) {
    const int64_t r_base = tile * 16 * MR;
    bf16x8 xf[MR][KS];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int64_t row = min<int64_t>(r_base + 16 * r + lr, (int64_t)p.n - 1);
      const uint16_t* src = p.X + row * p.ldx + 8 * lk;
#pragma unroll
      for (int k = 0; k < KS; ++k) xf[r][k] = *reinterpret_cast<const bf16x8*>(src + 32 * k);
    }
    const int n_here = (int)min<int64_t>(16 * MR, (int64_t)p.n - r_base);
    for (int cidx = 0; cidx < p.n_mat * cpm; ++cidx) {
      const int m = cidx / cpm, o0 = (cidx % cpm) * OCH;
      uint16_t* Y = p.Y[m];
      const int ow = min(OCH, p.f_out - o0);  // a multiple of 16
      for (int t = 0; t < ow; t += 16) {
        const uint16_t* w0 = wl + (size_t)(m * p.f_out + o0 + t + lr) * WROW + 8 * lk;
        bf16x8 wf[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) wf[k] = *reinterpret_cast<const bf16x8*>(w0 + 32 * k);
        f32x4 acc[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
#pragma unroll
          for (int r = 0; r < MR; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[k], xf[r][k], acc[r], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          const uint2 w2 = make_uint2(pack_bf16(acc[r][0], acc[r][1]), pack_bf16(acc[r][2], acc[r][3]));
          *reinterpret_cast<uint2*>(&st[16 * r + lr][t + 4 * lk]) = w2;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int lpr = ow / 8;
      for (int q = lane; q < n_here * lpr; q += 64) {
        const int row = q / lpr, c = (q % lpr) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(&st[row][c]);
        *reinterpret_cast<uint4*>(Y + (r_base + row) * p.f_out + o0 + c) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <int KS>
int launch_ks(ProjParams& p, hipStream_t s) {
  // MR * KS * 4 VGPRs hold the rows of X: at most 64
  constexpr int MR = KS <= 4 ? 4 : (KS <= 8 ? 2 : 1);
  constexpr int NWV = 16, MRL = MR > 2 ? 2 : MR;  // 16 waves of 32-row tiles: 0.037 ms on config 3 (8 waves of 64 rows: 0.041)
  const size_t lds = ((size_t)p.n_mat * p.f_out * (32 * KS + 8) + (size_t)NWV * 16 * MRL * SROW) * 2;
  if (lds <= kProjLdsMax &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_project_lds<KS, MRL, NWV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess) {
    int dev = 0, cus = 0;
    GNN_HIP(hipGetDevice(&dev));
    GNN_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const int64_t tiles = ((int64_t)p.n + 16 * MRL - 1) / (16 * MRL);
    const int64_t blocks = std::min<int64_t>(cus, (tiles + NWV - 1) / NWV);
    hipLaunchKernelGGL((k_project_lds<KS, MRL, NWV>), dim3((unsigned)std::max<int64_t>(blocks, 1)),
                       dim3(64 * NWV), lds, s, p);
    GNN_LAUNCH_CHECK("projection");
    return GNN_OK;
  }
  const int64_t rows_per_block = (int64_t)(WG / 64) * 16 * MR;
  const int64_t blocks = (p.n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return fail(GNN_ERR_SIZE_OVERFLOW, "projection grid too large");
  hipLaunchKernelGGL((k_project<KS, MR>), dim3((unsigned)blocks), dim3(WG), 0, s, p);
  GNN_LAUNCH_CHECK("projection");
  return GNN_OK;
}

}  // namespace

int launch_project(const void* X, int32_t n, int32_t f_in, int64_t ldx, int32_t n_mat, const void* const* W,
                   int32_t f_out, void* const* Y, hipStream_t s) {
  ProjParams p{};
  p.X = (const uint16_t*)X;
  p.ldx = ldx;
  p.n = n;
  p.f_out = f_out;
  p.n_mat = n_mat;
  for (int m = 0; m < n_mat; ++m) {
    p.W[m] = (const uint16_t*)W[m];
    p.Y[m] = (uint16_t*)Y[m];
  }
  switch (f_in / 32) {
    case 1: return launch_ks<1>(p, s);
    case 2: return launch_ks<2>(p, s);
    case 3: return launch_ks<3>(p, s);
    case 4: return launch_ks<4>(p, s);
    case 5: return launch_ks<5>(p, s);
    case 6: return launch_ks<6>(p, s);
    case 7: return launch_ks<7>(p, s);
    case 8: return launch_ks<8>(p, s);
    case 9: return launch_ks<9>(p, s);
    case 10: return launch_ks<10>(p, s);
    case 11: return launch_ks<11>(p, s);
    case 12: return launch_ks<12>(p, s);
    case 13: return launch_ks<13>(p, s);
    case 14: return launch_ks<14>(p, s);
    case 15: return launch_ks<15>(p, s);
    case 16: return launch_ks<16>(p, s);
    default: return fail(GNN_ERR_UNSUPPORTED, "projection needs f_in a multiple of 32, at most 512");
  }
}

}  // namespace gnn
