// Graph Transformer forward on 16 x 16 block-sparse tiles with bf16 MFMA.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.3 "Tensor Core attention (Graph Transformer) on
// WSB": per row window and head, the 16-row query block meets one 16-column
// key/value block per tile: S = Q_win K_blk^T, entries without an edge set to
// -inf by the tile bitmap, a per-row online softmax (m, l), and
// acc <- acc * exp(m_old - m_new) + exp(S - m_new) V_blk; finally acc / l and
// the logsumexp per row.  Every loaded key then serves 16 queries and every
// query 16 keys.
//
// MI355X mapping.  One workgroup of two waves per window; wave w handles
// heads w, w + 2, ... (D in {32, 64, 128, 256}, any number of heads).  The window's tile metadata (columns, bitmaps) is staged
// in LDS once, and each wave keeps the next tile's K / V loads in flight
// while it computes the current one.  For a tile the wave computes the transposed scores
// S^T = K_blk Q_win^T with v_mfma_f32_16x16x32_bf16 (A = 16 key rows, B = the
// window's queries, both loaded straight from memory in operand layout), so
// that lane l holds S[row l % 16][cols 4 (l / 16) .. +3]: exactly the B-operand
// layout of v_mfma_f32_16x16x16_bf16 for O^T += V_blk^T P^T.  The value block
// is transposed through LDS (V rows are dimension-contiguous, the MFMA needs
// column-contiguous k), read back with the LDS transpose read.  P is rounded to bf16 for that product; l sums the
// rounded weights.  Edges of tiles too sparse for the matrix cores (the
// residual CSR of the plan) are then streamed per row into the same (m, l,
// acc) state, the four lanes of a row splitting the head dimension.
// Windows are mapped to XCDs in runs of consecutive windows, so the windows of
// one locally dense cluster share an L2.
#include <type_traits>

#include "gnn_internal.h"

namespace gnn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short s16x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLn2 = 0.6931471805599453f;
// 2^x on v_exp_f32 alone: every argument is a difference from the running
// maximum (<= 0), and results below 2^-126 of it, which the hardware may
// flush to zero, do not change any sum at fp32 precision.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

struct B16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* out;
  float* lse;
  const int32_t* win_ptr;
  const int32_t* blk_col;
  const unsigned long long* blk_bits;
  const int32_t* tile_ptr;
  const int32_t* tile_blk;
  const int32_t* res_ptr;
  const int32_t* res_col;
  int32_t n_rows;
  int32_t n_windows;
  int32_t H;
  float scale_log2;  // scale * log2(e)
};

// Max / sum over the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48) with
// the gfx950 lane-swap instructions, on the VALU (a shuffle would go through
// the LDS crossbar).  v_permlane32_swap(x, x) leaves x[l] and x[l ^ 32] in
// the pair at every lane, v_permlane16_swap x[l] and x[l ^ 16]; every lane
// of the row ends with the same value.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// A 16x16x16 bf16 MFMA operand holding, in lane 16g + r, rows 4g .. 4g + 3 of
// column r of a 16 x 16 block stored row-major in LDS (row stride ld), read
// with the gfx950 LDS transpose read: within each 16 lanes, lane 16g + 4i + a
// names row 4g + i, columns 4a .. 4a + 3, and lane 16g + 4a + j receives
// element j of the rows named by lanes 16g + a, 16g + 4 + a, ...  Needs every
// lane active.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_tr_operand(const uint16_t* blk, int ld, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* a = blk + (4 * g + (r >> 2)) * ld + 4 * (r & 3);
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)a);
  return __builtin_bit_cast(s16x4, v);
}

// dot of 8 bf16 pairs on v_dot2_f32_bf16
__device__ __forceinline__ float dot8(const s16x8& a, const s16x8& b, float acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const s16x2 x = {a[2 * t], a[2 * t + 1]}, y = {b[2 * t], b[2 * t + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y),
                                          acc, false);
  }
  return acc;
}

constexpr int MAXT = 32;  // tiles of a window staged in LDS (larger windows read metadata directly)

// Latency decides this kernel's speed (each wave keeps one tile of K / V in
// flight while it computes another), so D <= 64 asks for four waves per SIMD
// (at most 128 VGPRs) rather than the three its natural allocation allows.
// At D = 256 a tile's K and V slices alone take 64 registers per lane and the
// output block 64 more: one tile at a time, two waves per SIMD.
template <int D, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 4 : 2)))
void k_gt_block16(B16Params p) {
  constexpr int KC = D / 32;   // k-chunks of the score product
  constexpr int MB = D / 16;   // 16-dim blocks of the output
  constexpr int LDV = D + 8;   // padded LDS row (bf16 elements)
  constexpr int LDO = D + 4;   // padded LDS row of the output stage (floats)
  // per wave: the value block of the current tile during the tile loop, the
  // output block of the head after it (never both at once)
  constexpr int STAGE_BYTES = 16 * LDO * 4 > 16 * LDV * 2 ? 16 * LDO * 4 : 16 * LDV * 2;
  __shared__ __align__(16) unsigned char s_stage[NWAVE][STAGE_BYTES];
  __shared__ int32_t s_col[MAXT][16];                // the 16 columns of each tile
  __shared__ unsigned long long s_bits[MAXT][4];     // block 0 words 0-1, block 1 words 0-1

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int w = (int)dev::xcd_remap(blockIdx.x, gridDim.x);
  const int row = w * 16 + r;
  const bool row_ok = row < p.n_rows;
  const int t_beg = p.tile_ptr[w], t_end = p.tile_ptr[w + 1];
  const int b_end = p.win_ptr[w + 1];
  const int nt = t_end - t_beg;
  const bool staged = nt <= MAXT;
  const int res_b = row_ok ? p.res_ptr[row] : 0, res_e = row_ok ? p.res_ptr[row + 1] : 0;
  const int64_t ldr = (int64_t)p.H * D;  // elements per node row
  uint16_t* lv = reinterpret_cast<uint16_t*>(s_stage[wave]);
  float* lo = reinterpret_cast<float*>(s_stage[wave]);

  // tile metadata of the window, one cooperative pass
  if (staged) {
    for (int i = threadIdx.x; i < nt * 16; i += NWAVE * 64) {
      const int t = i >> 4, c = i & 15;
      const int blk = p.tile_blk[t_beg + t] + (c >> 3);
      s_col[t][c] = ((c >> 3) == 1 && blk >= b_end) ? 0 : p.blk_col[(int64_t)blk * 8 + (c & 7)];
    }
    for (int i = threadIdx.x; i < nt * 4; i += NWAVE * 64) {
      const int t = i >> 2, q = i & 3;
      const int blk = p.tile_blk[t_beg + t] + (q >> 1);
      s_bits[t][q] = ((q >> 1) == 1 && blk >= b_end) ? 0ull : p.blk_bits[(int64_t)blk * 2 + (q & 1)];
    }
  }
  __syncthreads();

  // Tile metadata from LDS (ST) or from memory.  The two are separate
  // instantiations of the tile loop: a metadata load from memory inside the
  // loop would make the compiler wait for every outstanding load (the next
  // tile's K / V included) before using it.
  auto tile_col = [&](auto st, int t) -> int {
    if constexpr (decltype(st)::value) {
      return s_col[t - t_beg][r];
    } else {
      const int blk = p.tile_blk[t] + (r >> 3);
      return ((r >> 3) == 1 && blk >= b_end) ? 0 : p.blk_col[(int64_t)blk * 8 + (r & 7)];
    }
  };
  auto tile_word = [&](auto st, int t) -> unsigned long long {
    const int ub = g >> 1;  // which 16x8 block holds this lane's four columns
    if constexpr (decltype(st)::value) {
      return s_bits[t - t_beg][ub * 2 + (r >> 3)];
    } else {
      const int blk = p.tile_blk[t] + ub;
      return (ub == 1 && blk >= b_end) ? 0ull : p.blk_bits[(int64_t)blk * 2 + (r >> 3)];
    }
  };

  for (int h = wave; h < p.H; h += NWAVE) {
    // queries of the window in B-operand layout: lane l holds Q[row][kc*32 + 8g .. +7]
    s16x8 qb[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (row_ok)
        qb[kc] = *reinterpret_cast<const s16x8*>(p.q + (int64_t)row * ldr + h * D + kc * 32 + 8 * g);
      else
        qb[kc] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    float m = -INFINITY, lsum = 0.0f;
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_kv = [&](auto st, int t, s16x8 (&ka)[KC], s16x8 (&va)[KC]) {
      const int col = tile_col(st, t);
      // row col at a byte stride below 4 GB: one unsigned 32 x 32 -> 64 multiply-add
      const uint64_t ro = (uint64_t)(uint32_t)col * (uint32_t)(ldr * 2);
      const uint16_t* krow = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(p.k) + ro) + h * D;
      const uint16_t* vrow = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(p.v) + ro) + h * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        ka[kc] = *reinterpret_cast<const s16x8*>(krow + kc * 32 + 8 * g);
        va[kc] = *reinterpret_cast<const s16x8*>(vrow + kc * 32 + 8 * g);
      }
    };

    auto process = [&](auto stg, int t, const s16x8 (&ka)[KC], const s16x8 (&va)[KC]) {
      const unsigned long long word = tile_word(stg, t);
      const int base = (r & 7) * 8 + 4 * (g & 1);
      f32x4 st = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kc]),
                                                     __builtin_bit_cast(bf16x8, qb[kc]), st, 0, 0, 0);
      float s[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = ((word >> (base + i)) & 1ull) ? st[i] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[i]);
      }
      mx = row4_max(mx);
      const float mn = fmaxf(m, mx);
      float corr = 1.0f;
      uint16_t pb[4];
      float rs = 0.0f;
      if (mn != -INFINITY) {
        corr = ex2(m - mn);
        // weights rounded to bf16 (nearest even) two at a time by v_cvt_pk_bf16_f32
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          bf16x2 w2;
          w2[0] = (__bf16)ex2(s[i] - mn);
          w2[1] = (__bf16)ex2(s[i + 1] - mn);
          const uint32_t u = __builtin_bit_cast(uint32_t, w2);
          pb[i] = (uint16_t)(u & 0xffffu);
          pb[i + 1] = (uint16_t)(u >> 16);
          rs += __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = 0;
      }
      rs = row4_sum(rs);
      lsum = lsum * corr + rs;
      m = mn;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] *= corr;

      // value block -> LDS as [col][dim], then read transposed
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        *reinterpret_cast<s16x8*>(lv + r * LDV + kc * 32 + 8 * g) = va[kc];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const s16x4 pt = s16x4{(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const s16x4 vt = lds_tr_operand(lv + mb * 16, LDV, lane);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pt, acc[mb], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    auto tiles = [&](auto st) {
      if constexpr (D <= 128) {
        // two-deep pipeline: the next tile's K / V are in flight while one
        // computes.  The loop runs while both prefetches exist, and the last
        // one or two tiles follow it: a prefetch under a branch inside the
        // loop leaves the compiler two load counts to reconcile at the join,
        // and it then waits for the prefetched tile with the current one.
        if (t_beg < t_end) {
          s16x8 kA[KC], vA[KC], kB[KC], vB[KC];
          load_kv(st, t_beg, kA, vA);
          int t = t_beg;
          for (; t + 2 < t_end; t += 2) {
            load_kv(st, t + 1, kB, vB);
            process(st, t, kA, vA);
            load_kv(st, t + 2, kA, vA);
            process(st, t + 1, kB, vB);
          }
          if (t + 1 < t_end) {
            load_kv(st, t + 1, kB, vB);
            process(st, t, kA, vA);
            process(st, t + 1, kB, vB);
          } else {
            process(st, t, kA, vA);
          }
        }
      } else {
        s16x8 kA[KC], vA[KC];
        for (int t = t_beg; t < t_end; ++t) {
          load_kv(st, t, kA, vA);
          process(st, t, kA, vA);
        }
      }
    };
    if (staged) tiles(std::true_type{});
    else tiles(std::false_type{});

    // residual edges of this row: the row's four lanes split the head dims
    int j_next = (res_b < res_e) ? p.res_col[res_b] : 0;
    for (int e = res_b; e < res_e; ++e) {
      const int j = j_next;
      if (e + 1 < res_e) j_next = p.res_col[e + 1];
      const uint16_t* kr = p.k + (int64_t)j * ldr + h * D;
      const uint16_t* vr = p.v + (int64_t)j * ldr + h * D;
      s16x8 kv[KC];
      s16x4 vv[MB];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kv[kc] = *reinterpret_cast<const s16x8*>(kr + kc * 32 + 8 * g);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) vv[mb] = *reinterpret_cast<const s16x4*>(vr + mb * 16 + 4 * g);
      float dot = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) dot = dot8(qb[kc], kv[kc], dot);
      dot = row4_sum(dot);
      const float sc = dot * p.scale_log2;
      const float mn = fmaxf(m, sc);
      const float corr = ex2(m - mn);
      const float pe = ex2(sc - mn);
      lsum = lsum * corr + pe;
      m = mn;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] = fmaf(pe, bf((uint16_t)vv[mb][i]), acc[mb][i] * corr);
    }

    // Lane (r, g) holds dims mb * 16 + 4g .. +3 of its row: stored directly,
    // each instruction would write half of every 128-byte line.  Stage the
    // window's 16 x D head slice in LDS and store whole row slices instead
    // (256 / D rows per instruction, 16 contiguous bytes per lane).
    {
      const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        *reinterpret_cast<f32x4*>(lo + r * LDO + mb * 16 + 4 * g) =
            f32x4{acc[mb][0] * inv, acc[mb][1] * inv, acc[mb][2] * inv, acc[mb][3] * inv};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int LPRW = D / 4;        // lanes per row slice
      constexpr int RPI = 64 / LPRW;     // rows per store instruction
      const int r0 = lane / LPRW, dd = (lane % LPRW) * 4;
      const float* lsrc = lo + r0 * LDO + dd;
      float* odst = p.out + (int64_t)(w * 16 + r0) * ldr + h * D + dd;
      const int rows_left = p.n_rows - (w * 16 + r0);
#pragma unroll
      for (int q = 0; q < 16 / RPI; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(lsrc + q * RPI * LDO);
        if (q * RPI < rows_left) __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(odst + (int64_t)q * RPI * ldr));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (row_ok && p.lse && g == 0)
        p.lse[(int64_t)row * p.H + h] = lsum > 0.0f ? m * kLn2 + logf(lsum) : -INFINITY;
    }
  }
}

}  // namespace

int launch_gt_block16(gnn_plan* pl, const void* q, const void* k, const void* v, int32_t H,
                      int32_t D, float scale, float* out, float* lse, hipStream_t s) {
  B16Params p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = out;
  p.lse = lse;
  p.win_ptr = pl->wsb.win_ptr;
  p.blk_col = pl->wsb.blk_col;
  p.blk_bits = (const unsigned long long*)pl->wsb.blk_bits;
  p.tile_ptr = pl->wsb.tile_ptr;
  p.tile_blk = pl->wsb.tile_blk;
  p.res_ptr = pl->wsb.res_ptr;
  p.res_col = pl->wsb.res_col;
  p.n_rows = pl->n_rows;
  p.n_windows = pl->wsb.n_windows;
  p.H = H;
  p.scale_log2 = scale * 1.4426950408889634f;
  // two waves per window, each looping over half of the heads: the window's
  // tile metadata is staged once per workgroup and amortised over the heads
  const dim3 grid((unsigned)p.n_windows);
#define GNN_B16(DD) hipLaunchKernelGGL((k_gt_block16<DD, 2>), grid, dim3(2 * 64), 0, s, p)
  if (D == 32) GNN_B16(32);
  else if (D == 64) GNN_B16(64);
  else if (D == 128) GNN_B16(128);
  else if (D == 256) GNN_B16(256);
  else return fail(GNN_ERR_UNSUPPORTED, "BLOCK16 head dim must be 32, 64, 128 or 256");
#undef GNN_B16
  GNN_LAUNCH_CHECK("gt block16");
  return GNN_OK;
}

}  // namespace gnn
