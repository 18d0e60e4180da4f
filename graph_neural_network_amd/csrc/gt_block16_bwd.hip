// Graph Transformer backward on 16 x 16 block-sparse tiles with bf16 MFMA.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations": appendix D.2 (backward with cached statistics: only the
// per-(row, head) logsumexp L_i of the forward is kept; alpha_ij =
// exp(e_ij - L_i), Delta_i = <dO_i, O_i>, dS_ij = alpha_ij (<dO_i, v_j> -
// Delta_i)) and appendix D.3 (the windowed block-sparse layout, here used for
// training as well as inference).  With e_ij = scale <q_i, k_j>:
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i alpha_ij dO_i.
//
// Two walks, no atomics, as in the CSR backward:
//   destination walk (WSB tiles of A, 16 destination rows per window): per
//     dense tile S^T = K_blk Q_win^T and dP^T = V_blk dO_win^T (16x16x32 bf16
//     MFMA, both operands straight from memory), alpha and dS per entry, then
//     dQ_win += dS K_blk (16x16x16 bf16 MFMA; dS is already in A-operand
//     layout, K_blk is read transposed from LDS).  Writes Delta and dO in
//     bf16 for the other walk, which gathers them per tile.
//   source walk (WSB tiles of A^T, 16 source columns per window): per dense
//     tile S'^T = Q_blk K_win^T and dP'^T = dO_blk V_win^T, alpha and dS, then
//     dK_win += dS^T Q_blk and dV_win += alpha^T dO_blk.
// The transposed B operands come from LDS through the gfx950 transpose read
// (ds_read_b64_tr_b16), one instruction per 16 x 16 block.
// Entries of tiles below the density threshold (the residual CSR of each
// layout) are added per row by the row's four lanes, each holding a quarter of
// the head dimension, into row-layout partial sums placed in LDS before the
// tile loop and merged with the tile results at the end.
// The matrix cores take dO, alpha and dS rounded to bf16 (q, k, v are bf16
// already): the results carry bf16 rounding of those three, as the
// block-sparse forward carries it for alpha.
#include "gnn_internal.h"

namespace gnn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short s16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int MAXT = 32;  // tiles of a window whose metadata is staged in LDS
template <int D>
constexpr int ldk() { return D + 8; }  // padded LDS row (bf16)
template <int D>
constexpr int ldo() { return D + 4; }  // padded LDS row (floats)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 rounding to nearest even on v_cvt_pk_bf16_f32
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Sum over the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48) on the VALU
// lane-swap instructions: v_permlane32_swap(x, x) leaves x[l] and x[l ^ 32]
// in the pair at every lane, v_permlane16_swap x[l] and x[l ^ 16].
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// dot of 8 bf16 pairs on v_dot2_f32_bf16
__device__ __forceinline__ float dot8(const s16x8& a, const s16x8& b, float acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const s16x2 x = {a[2 * t], a[2 * t + 1]}, y = {b[2 * t], b[2 * t + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc,
                                          false);
  }
  return acc;
}

// The B operand of a 16x16x16 bf16 MFMA (lane 16g + r: rows 4g .. 4g + 3 of
// column r) from a 16 x 16 block stored row-major in LDS (row stride ld), by
// the LDS transpose read: within each 16 lanes, lane 16g + 4i + a names row
// 4g + i, columns 4a .. 4a + 3, and lane 16g + 4a + j receives element j of
// the four rows named by lanes 16g + a, 16g + 4 + a, ...  Needs every lane
// active.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_b_operand(const uint16_t* blk, int ld, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* a = blk + (4 * g + (r >> 2)) * ld + 4 * (r & 3);
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)a);
  return __builtin_bit_cast(s16x4, v);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct B16BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* out;
  const float* lse;
  const float* dout;
  float* delta;   // [destinations, H]: written by the destination walk, read by the source walk
  uint16_t* dob;  // [destinations, H, D] dO in bf16: the same hand-over
  float* g0;     // destination walk: dq; source walk: dk
  float* g1;     // source walk: dv
  // block-sparse layout of the walked matrix (A, or A^T for the source walk)
  const int32_t* win_ptr;
  const int32_t* blk_col;
  const unsigned long long* blk_bits;
  const int32_t* tile_ptr;
  const int32_t* tile_blk;
  const int32_t* res_ptr;
  const int32_t* res_col;
  int32_t n_rows;  // rows of the walked matrix
  int32_t H;
  float scale;
};

// A row slice of 8 * KC elements of this lane (dims kc * 32 + 8g .. +7).
template <int KC>
__device__ __forceinline__ void load_bf(const uint16_t* row, int g, s16x8 (&x)[KC]) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) x[kc] = *reinterpret_cast<const s16x8*>(row + kc * 32 + 8 * g);
}
template <int KC>
__device__ __forceinline__ void load_f32(const float* row, int g, float (&x)[KC][8]) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + kc * 32 + 8 * g);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + kc * 32 + 8 * g + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[kc][t] = a[t];
      x[kc][4 + t] = b[t];
    }
  }
}
template <int KC>
__device__ __forceinline__ void to_bf(const float (&x)[KC][8], s16x8 (&y)[KC]) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int t = 0; t < 8; ++t) y[kc][t] = (short)f2bf(x[kc][t]);
}

// Window tile metadata (columns and bitmap words), staged in LDS when the
// window has at most MAXT tiles.
struct Tiles {
  int t_beg, t_end, b_end;
  bool staged;
};

template <int NWAVE>
__device__ __forceinline__ Tiles stage_tiles(const B16BwdParams& p, int w, int32_t (*s_col)[16],
                                             unsigned long long (*s_bits)[4]) {
  Tiles T;
  T.t_beg = p.tile_ptr[w];
  T.t_end = p.tile_ptr[w + 1];
  T.b_end = p.win_ptr[w + 1];
  const int nt = T.t_end - T.t_beg;
  T.staged = nt <= MAXT;
  if (T.staged) {
    for (int i = threadIdx.x; i < nt * 16; i += NWAVE * 64) {
      const int t = i >> 4, c = i & 15;
      const int blk = p.tile_blk[T.t_beg + t] + (c >> 3);
      s_col[t][c] = ((c >> 3) == 1 && blk >= T.b_end) ? 0 : p.blk_col[(int64_t)blk * 8 + (c & 7)];
    }
    for (int i = threadIdx.x; i < nt * 4; i += NWAVE * 64) {
      const int t = i >> 2, q = i & 3;
      const int blk = p.tile_blk[T.t_beg + t] + (q >> 1);
      s_bits[t][q] = ((q >> 1) == 1 && blk >= T.b_end) ? 0ull : p.blk_bits[(int64_t)blk * 2 + (q & 1)];
    }
  }
  __syncthreads();
  return T;
}

// Column c (0..15) of tile t.  ST (staged) is a template parameter: with a
// run-time choice the compiler merges the LDS and global reads into one flat
// load, whose wait then also waits for every prefetch in flight.
template <bool ST>
__device__ __forceinline__ int tile_col(const B16BwdParams& p, const Tiles& T, const int32_t (*s_col)[16], int t,
                                        int c) {
  if constexpr (ST) {
    return s_col[t - T.t_beg][c];
  } else {
    const int blk = p.tile_blk[t] + (c >> 3);
    return ((c >> 3) == 1 && blk >= T.b_end) ? 0 : p.blk_col[(int64_t)blk * 8 + (c & 7)];
  }
}
// bitmap word holding window row r, tile columns 4g .. 4g + 3
template <bool ST>
__device__ __forceinline__ unsigned long long tile_word(const B16BwdParams& p, const Tiles& T,
                                                        const unsigned long long (*s_bits)[4], int t, int r,
                                                        int g) {
  const int ub = g >> 1;
  if constexpr (ST) {
    return s_bits[t - T.t_beg][ub * 2 + (r >> 3)];
  } else {
    const int blk = p.tile_blk[t] + ub;
    return (ub == 1 && blk >= T.b_end) ? 0ull : p.blk_bits[(int64_t)blk * 2 + (r >> 3)];
  }
}

// Row-layout partial results (lane l: row r, dims kc*32 + 8g + t) placed in
// a 16 x D LDS tile.
template <int D>
__device__ __forceinline__ void put_rows(float* lo, const float (&res)[D / 32][8], int lane) {
  constexpr int KC = D / 32, LDO = ldo<D>();
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int t = 0; t < 8; ++t) lo[r * LDO + kc * 32 + 8 * g + t] = res[kc][t];
}

// A D-layout accumulator set (lane l: rows 4g + i, dims mb*16 + r) into the
// LDS tile: stored, or added to what is there.
template <int D, bool ADD>
__device__ __forceinline__ void put_acc(float* lo, const f32x4 (&acc)[D / 16], int lane) {
  constexpr int MB = D / 16, LDO = ldo<D>();
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float& x = lo[(4 * g + i) * LDO + mb * 16 + r];
      x = ADD ? x + acc[mb][i] : acc[mb][i];
    }
}

// Add row-layout partial results (lane l: row r, dims kc*32 + 8g + t).
template <int D>
__device__ __forceinline__ void add_rows(float* lo, const float (&res)[D / 32][8], int lane) {
  constexpr int KC = D / 32, LDO = ldo<D>();
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int t = 0; t < 8; ++t) lo[r * LDO + kc * 32 + 8 * g + t] += res[kc][t];
}

// Store the LDS tile as the window's rows of head h, 16 contiguous bytes per
// lane (rows past the end skipped).
template <int D>
__device__ __forceinline__ void write_rows(const float* lo, float* dst, int64_t ldr, int h, int w, int n_rows,
                                           int lane) {
  constexpr int LDO = ldo<D>();
  constexpr int LPRW = D / 4;     // lanes per row slice
  constexpr int RPI = 64 / LPRW;  // rows per store instruction
  wave_sync();
  const int r0 = lane / LPRW, dd = (lane % LPRW) * 4;
  const float* lsrc = lo + r0 * LDO + dd;
  float* odst = dst + (int64_t)(w * 16 + r0) * ldr + h * D + dd;
  const int rows_left = n_rows - (w * 16 + r0);
#pragma unroll
  for (int q = 0; q < 16 / RPI; ++q) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(lsrc + q * RPI * LDO);
    if (q * RPI < rows_left) __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(odst + (int64_t)q * RPI * ldr));
  }
  wave_sync();
}

// Add a D-layout accumulator set to the LDS tile and store it.
template <int D>
__device__ __forceinline__ void store_rows(float* lo, const f32x4 (&acc)[D / 16], float* dst, int64_t ldr, int h,
                                           int w, int n_rows, int lane) {
  wave_sync();
  put_acc<D, true>(lo, acc, lane);
  write_rows<D>(lo, dst, ldr, h, w, n_rows, lane);
}

// ---------------------------------------------------------------------------
// destination walk: dq (and Delta)
// ---------------------------------------------------------------------------
template <int D, int NWAVE, bool ST>
__device__ __forceinline__ void dst_walk(const B16BwdParams& p, const Tiles& T, int w, const int32_t (*s_col)[16],
                                         const unsigned long long (*s_bits)[4], uint16_t* lk, float* lo) {
  constexpr int KC = D / 32, MB = D / 16;
  constexpr int LDK = ldk<D>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int row = w * 16 + r;
  const bool row_ok = row < p.n_rows;
  const int res_b = row_ok ? p.res_ptr[row] : 0, res_e = row_ok ? p.res_ptr[row + 1] : 0;
  const int64_t ldr = (int64_t)p.H * D;
  const float sc2 = p.scale * kLog2e;

  for (int h = wave; h < p.H; h += NWAVE) {
    // this lane's slices of the row: q, dO (rounded to bf16 for the matrix
    // cores, and stored so for the source walk) in B-operand layout; Delta =
    // <dO, O> over the head, lse
    s16x8 qb[KC], gb[KC];
    float L2 = 0.0f, dl = 0.0f;
    if (row_ok) {
      const int64_t ro = (int64_t)row * ldr + h * D;
      load_bf<KC>(p.q + ro, g, qb);
      float go[KC][8], o[KC][8];
      load_f32<KC>(p.dout + ro, g, go);
      load_f32<KC>(p.out + ro, g, o);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int t = 0; t < 8; ++t) dl = fmaf(go[kc][t], o[kc][t], dl);
      to_bf<KC>(go, gb);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) *reinterpret_cast<s16x8*>(p.dob + ro + kc * 32 + 8 * g) = gb[kc];
      L2 = p.lse[(int64_t)row * p.H + h] * kLog2e;
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qb[kc] = gb[kc] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    dl = row4_sum(dl);
    if (row_ok && g == 0) p.delta[(int64_t)row * p.H + h] = dl;
    {
      float res[KC][8];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int t = 0; t < 8; ++t) res[kc][t] = 0.0f;
      // residual entries of this row: the row's four lanes each hold a
      // quarter of the head dimension
      for (int e = res_b; e < res_e; ++e) {
        const int64_t co = (int64_t)p.res_col[e] * ldr + h * D;
        s16x8 kv[KC], vv[KC];
        load_bf<KC>(p.k + co, g, kv);
        load_bf<KC>(p.v + co, g, vv);
        float s = 0.0f, dpv = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          s = dot8(qb[kc], kv[kc], s);
          dpv = dot8(gb[kc], vv[kc], dpv);
        }
        s = row4_sum(s);
        dpv = row4_sum(dpv);
        const float ds = ex2(s * sc2 - L2) * (dpv - dl) * p.scale;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int t = 0; t < 8; ++t) res[kc][t] = fmaf(ds, bf((uint16_t)kv[kc][t]), res[kc][t]);
      }
      put_rows<D>(lo, res, lane);
    }
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto load_kv = [&](int t, s16x8 (&ka)[KC], s16x8 (&va)[KC]) {
      const int64_t co = (int64_t)tile_col<ST>(p, T, s_col, t, r) * ldr + h * D;
      load_bf<KC>(p.k + co, g, ka);
      load_bf<KC>(p.v + co, g, va);
    };
    auto process = [&](int t, const s16x8 (&ka)[KC], const s16x8 (&va)[KC]) {
      // lane holds S and dP of row r, tile columns 4g .. 4g + 3
      f32x4 st = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, dp = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kc]),
                                                     __builtin_bit_cast(bf16x8, qb[kc]), st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[kc]),
                                                     __builtin_bit_cast(bf16x8, gb[kc]), dp, 0, 0, 0);
      }
      const unsigned long long word = tile_word<ST>(p, T, s_bits, t, r, g);
      const int base = (r & 7) * 8 + 4 * (g & 1);
      s16x4 dsb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = ((word >> (base + i)) & 1ull) ? ex2(st[i] * sc2 - L2) : 0.0f;
        dsb[i] = (short)f2bf(a * (dp[i] - dl) * p.scale);
      }
      // K block to LDS as [column][dim], read transposed as the B operand
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) *reinterpret_cast<s16x8*>(lk + r * LDK + kc * 32 + 8 * g) = ka[kc];
      wave_sync();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const s16x4 kt = lds_b_operand(lk + mb * 16, LDK, lane);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dsb, kt, acc[mb], 0, 0, 0);
      }
      wave_sync();
    };

    // two-deep pipeline over the window's dense tiles
    s16x8 kA[KC], vA[KC], kB[KC], vB[KC];
    if (T.t_beg < T.t_end) load_kv(T.t_beg, kA, vA);
    for (int t = T.t_beg; t < T.t_end; t += 2) {
      if (t + 1 < T.t_end) load_kv(t + 1, kB, vB);
      process(t, kA, vA);
      if (t + 1 < T.t_end) {
        if (t + 2 < T.t_end) load_kv(t + 2, kA, vA);
        process(t + 1, kB, vB);
      }
    }

    store_rows<D>(lo, acc, p.g0, ldr, h, w, p.n_rows, lane);
  }
}

// (waves_per_eu: without it the compiler splits the registers into VGPRs
// and AGPRs and loses a wave of occupancy)
template <int D, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2))) void k_gt_b16_bwd_dst(
    B16BwdParams p) {
  __shared__ uint16_t s_k[NWAVE][16 * ldk<D>()];
  __shared__ __align__(16) float s_o[NWAVE][16 * ldo<D>()];
  __shared__ int32_t s_col[MAXT][16];
  __shared__ unsigned long long s_bits[MAXT][4];
  const int wave = threadIdx.x >> 6;
  const int w = (int)dev::xcd_remap(blockIdx.x, gridDim.x);
  const Tiles T = stage_tiles<NWAVE>(p, w, s_col, s_bits);
  if (T.staged) dst_walk<D, NWAVE, true>(p, T, w, s_col, s_bits, s_k[wave], s_o[wave]);
  else dst_walk<D, NWAVE, false>(p, T, w, s_col, s_bits, s_k[wave], s_o[wave]);
}

// ---------------------------------------------------------------------------
// source walk over A^T: dk, dv
// ---------------------------------------------------------------------------
// buf: the wave's LDS: during the tile loop the tile's q and dO rows
// ([destination][dim], bf16), after it the window's dk rows (fp32); lo2: the
// window's dv rows
template <int D, int NWAVE, bool ST>
__device__ __forceinline__ void src_walk(const B16BwdParams& p, const Tiles& T, int w, const int32_t (*s_col)[16],
                                         const unsigned long long (*s_bits)[4], char* buf, float* lo2) {
  constexpr int KC = D / 32, MB = D / 16;
  constexpr int LDK = ldk<D>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int row = w * 16 + r;  // a source node (row of A^T)
  const bool row_ok = row < p.n_rows;
  const int res_b = row_ok ? p.res_ptr[row] : 0, res_e = row_ok ? p.res_ptr[row + 1] : 0;
  const int64_t ldr = (int64_t)p.H * D;
  const float sc2 = p.scale * kLog2e;
  uint16_t* lq = reinterpret_cast<uint16_t*>(buf);
  uint16_t* lg = lq + 16 * LDK;
  float* lo = reinterpret_cast<float*>(buf);

  // one destination row's slices for this lane: q, dO (bf16), lse, Delta
  // (lse raw: arithmetic on it at load time would wait for the loads)
  struct Dst {
    s16x8 q[KC], g[KC];
    float lse, dl;
  };
  for (int h = wave; h < p.H; h += NWAVE) {
    // this lane's slices of its source row: k and v in B-operand layout
    s16x8 kb[KC], vb[KC];
    if (row_ok) {
      const int64_t ro = (int64_t)row * ldr + h * D;
      load_bf<KC>(p.k + ro, g, kb);
      load_bf<KC>(p.v + ro, g, vb);
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kb[kc] = vb[kc] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    f32x4 acck[MB], accv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acck[mb] = accv[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto load_dst = [&](int t, Dst& d) {
      const int i = tile_col<ST>(p, T, s_col, t, r);
      const int64_t io = (int64_t)i * ldr + h * D;
      load_bf<KC>(p.q + io, g, d.q);
      load_bf<KC>(p.dob + io, g, d.g);
      d.lse = p.lse[(int64_t)i * p.H + h];
      d.dl = p.delta[(int64_t)i * p.H + h];
    };
    auto process = [&](int t, const Dst& d) {
      // lane holds S and dP of source r with destinations 4g .. 4g + 3 of the tile
      f32x4 st = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, dp = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d.q[kc]),
                                                     __builtin_bit_cast(bf16x8, kb[kc]), st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d.g[kc]),
                                                     __builtin_bit_cast(bf16x8, vb[kc]), dp, 0, 0, 0);
      }
      const unsigned long long word = tile_word<ST>(p, T, s_bits, t, r, g);
      const int base = (r & 7) * 8 + 4 * (g & 1);
      s16x4 dsb, ab;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float Lc = __shfl(d.lse, 4 * g + i, 64) * kLog2e;  // lane c (0..15) holds destination c
        const float Dc = __shfl(d.dl, 4 * g + i, 64);
        const float a = ((word >> (base + i)) & 1ull) ? ex2(st[i] * sc2 - Lc) : 0.0f;
        ab[i] = (short)f2bf(a);
        dsb[i] = (short)f2bf(a * (dp[i] - Dc) * p.scale);
      }
      // the tile's q and dO rows to LDS as [destination][dim], read transposed
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        *reinterpret_cast<s16x8*>(lq + r * LDK + kc * 32 + 8 * g) = d.q[kc];
        *reinterpret_cast<s16x8*>(lg + r * LDK + kc * 32 + 8 * g) = d.g[kc];
      }
      wave_sync();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const s16x4 qt = lds_b_operand(lq + mb * 16, LDK, lane);
        const s16x4 gt = lds_b_operand(lg + mb * 16, LDK, lane);
        acck[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dsb, qt, acck[mb], 0, 0, 0);
        accv[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, gt, accv[mb], 0, 0, 0);
      }
      wave_sync();
    };

    // two-deep pipeline over the window's dense tiles
    Dst dA, dB;
    if (T.t_beg < T.t_end) load_dst(T.t_beg, dA);
    for (int t = T.t_beg; t < T.t_end; t += 2) {
      if (t + 1 < T.t_end) load_dst(t + 1, dB);
      process(t, dA);
      if (t + 1 < T.t_end) {
        if (t + 2 < T.t_end) load_dst(t + 2, dA);
        process(t + 1, dB);
      }
    }

    // tile results to LDS: dk over the q / dO staging, which the tiles no
    // longer need, dv beside it
    wave_sync();
    put_acc<D, false>(lo, acck, lane);
    put_acc<D, false>(lo2, accv, lane);

    float resk[KC][8], resv[KC][8];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int t = 0; t < 8; ++t) resk[kc][t] = resv[kc][t] = 0.0f;
    // residual entries of this source row (destinations i)
    for (int e = res_b; e < res_e; ++e) {
      const int i = p.res_col[e];
      const int64_t io = (int64_t)i * ldr + h * D;
      s16x8 qv[KC], gv[KC];
      load_bf<KC>(p.q + io, g, qv);
      load_bf<KC>(p.dob + io, g, gv);
      const float L2 = p.lse[(int64_t)i * p.H + h] * kLog2e;
      const float dl = p.delta[(int64_t)i * p.H + h];
      float s = 0.0f, dpv = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        s = dot8(qv[kc], kb[kc], s);
        dpv = dot8(gv[kc], vb[kc], dpv);
      }
      s = row4_sum(s);
      dpv = row4_sum(dpv);
      const float a = ex2(s * sc2 - L2);
      const float ds = a * (dpv - dl) * p.scale;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          resk[kc][t] = fmaf(ds, bf((uint16_t)qv[kc][t]), resk[kc][t]);
          resv[kc][t] = fmaf(a, bf((uint16_t)gv[kc][t]), resv[kc][t]);
        }
    }

    wave_sync();
    add_rows<D>(lo, resk, lane);
    add_rows<D>(lo2, resv, lane);
    write_rows<D>(lo, p.g0, ldr, h, w, p.n_rows, lane);
    write_rows<D>(lo2, p.g1, ldr, h, w, p.n_rows, lane);
  }
}

// (D <= 64: three waves per SIMD, a few registers spilled and reloaded once
// per head, faster than two; D = 128: two waves with some spills, faster than
// one without)
template <int D, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2))) void k_gt_b16_bwd_src(
    B16BwdParams p) {
  constexpr int BUF = 2 * 16 * ldk<D>() * 2 > 16 * ldo<D>() * 4 ? 2 * 16 * ldk<D>() * 2 : 16 * ldo<D>() * 4;
  __shared__ __align__(16) char s_buf[NWAVE][BUF];
  __shared__ __align__(16) float s_o2[NWAVE][16 * ldo<D>()];
  __shared__ int32_t s_col[MAXT][16];
  __shared__ unsigned long long s_bits[MAXT][4];
  const int wave = threadIdx.x >> 6;
  const int w = (int)dev::xcd_remap(blockIdx.x, gridDim.x);
  const Tiles T = stage_tiles<NWAVE>(p, w, s_col, s_bits);
  if (T.staged) src_walk<D, NWAVE, true>(p, T, w, s_col, s_bits, s_buf[wave], s_o2[wave]);
  else src_walk<D, NWAVE, false>(p, T, w, s_col, s_bits, s_buf[wave], s_o2[wave]);
}

void fill_layout(B16BwdParams& p, const gnn_plan* pl) {
  p.win_ptr = pl->wsb.win_ptr;
  p.blk_col = pl->wsb.blk_col;
  p.blk_bits = (const unsigned long long*)pl->wsb.blk_bits;
  p.tile_ptr = pl->wsb.tile_ptr;
  p.tile_blk = pl->wsb.tile_blk;
  p.res_ptr = pl->wsb.res_ptr;
  p.res_col = pl->wsb.res_col;
  p.n_rows = pl->n_rows;
}

}  // namespace

int launch_gt_backward_block16(gnn_plan* pl, const void* q, const void* k, const void* v, int32_t H, int32_t D,
                               float scale, const float* out, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, hipStream_t s) {
  if (D != 32 && D != 64 && D != 128)
    return fail(GNN_ERR_UNSUPPORTED, "block-sparse GT backward needs D in {32, 64, 128}");
  GNN_TRY(plan_transpose(pl, s));
  GNN_TRY(plan_transpose_wsb(pl, s));
  GNN_TRY(plan_grow(pl, (void**)&pl->delta, &pl->delta_cap, (size_t)std::max(pl->n_rows, 1) * H * 4));
  GNN_TRY(plan_grow(pl, (void**)&pl->dob, &pl->dob_cap, (size_t)std::max(pl->n_rows, 1) * H * D * 2));
  B16BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = out;
  p.lse = lse;
  p.dout = dout;
  p.delta = pl->delta;
  p.dob = pl->dob;
  p.H = H;
  p.scale = scale;
  constexpr int NW = 2;  // waves per window, each looping over half of the heads
  fill_layout(p, pl);
  p.g0 = dq;
  if (pl->wsb.n_windows > 0) {
    const dim3 grid((unsigned)pl->wsb.n_windows);
    if (D == 32) hipLaunchKernelGGL((k_gt_b16_bwd_dst<32, NW>), grid, dim3(NW * 64), 0, s, p);
    else if (D == 64) hipLaunchKernelGGL((k_gt_b16_bwd_dst<64, NW>), grid, dim3(NW * 64), 0, s, p);
    else hipLaunchKernelGGL((k_gt_b16_bwd_dst<128, NW>), grid, dim3(NW * 64), 0, s, p);
    GNN_LAUNCH_CHECK("block-sparse GT backward (destinations)");
  }
  const gnn_plan* tp = pl->tplan;
  fill_layout(p, tp);
  p.g0 = dk;
  p.g1 = dv;
  if (tp->wsb.n_windows > 0) {
    const dim3 grid((unsigned)tp->wsb.n_windows);
    if (D == 32) hipLaunchKernelGGL((k_gt_b16_bwd_src<32, NW>), grid, dim3(NW * 64), 0, s, p);
    else if (D == 64) hipLaunchKernelGGL((k_gt_b16_bwd_src<64, NW>), grid, dim3(NW * 64), 0, s, p);
    else hipLaunchKernelGGL((k_gt_b16_bwd_src<128, NW>), grid, dim3(NW * 64), 0, s, p);
    GNN_LAUNCH_CHECK("block-sparse GT backward (sources)");
  }
  return GNN_OK;
}

}  // namespace gnn
