// Weighted block-sparse (WSB) layout built on the GPU.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.3 "WSB format and TCB construction":
// destination rows are cut into windows of R = 16; each window's distinct
// source columns are sorted and cut into blocks of W = 8 columns (zero-padded
// column list), each block carrying a 16 x 8 occupancy bitmap in two 64-bit
// words; two consecutive blocks form one 16 x 16 tile for the matrix cores.
// "Storage costs" in the same appendix: 32 bytes of columns plus 16 bytes of
// bitmap per block.
//
// Tile routing (the pages' "WSB pays off only where windows are locally
// dense"): a tile whose two blocks hold fewer than tau edges is not sent to
// the matrix cores; its edges form a residual CSR that the block-sparse
// kernel streams with the CSR loop into the same softmax state.
//
// Steps (all on the GPU):
//   1. key(e) = (window(row(e)) << colbits) | col(e); stable radix sort.
//   2. distinct keys -> per-window distinct column count -> blocks per window
//      (ceil(count / 8)) -> win_ptr by a scan; block column lists filled.
//   3. every CSR edge finds its column among its window's sorted distinct
//      columns (binary search, one workgroup per window, the columns in LDS)
//      and sets its bit in the window's LDS bitmaps, stored once.
//   4. tiles: block pairs (0,1), (2,3), ... of each window; dense when their
//      bit count >= tau -> tile list per window (scan).
//   5. residual CSR: edges of non-dense tiles, in CSR order per row (scan).
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

// One workgroup per window of 16 rows: the window's entries are contiguous
// in the CSR, so no entry has to search for its row or window.
constexpr int kWinThreads = 256;
constexpr int kWinLdsBlocks = 512;  // windows with at most this many blocks keep columns and bits in LDS

__global__ __launch_bounds__(kWinThreads) void k_wsb_keys(const int32_t* row_ptr, const int32_t* col_idx,
                                                          int32_t n, int colbits, uint64_t* keys) {
  const int w = blockIdx.x;
  const int64_t e0 = row_ptr[w * 16], e1 = row_ptr[min(w * 16 + 16, n)];
  const uint64_t hi = (uint64_t)w << colbits;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += kWinThreads) keys[e] = hi | (uint32_t)col_idx[e];
}

__global__ void k_wsb_flags(const uint64_t* keys, int64_t nnz, int32_t* flag) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= nnz) return;
  flag[e] = (e == 0 || keys[e] != keys[e - 1]) ? 1 : 0;
}

// distinct columns and blocks per window
__global__ void k_wsb_wcount(const int32_t* row_ptr, int32_t n, int32_t nw, const int32_t* uidx,
                             int32_t* ucnt, int32_t* nblk) {
  int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= nw) return;
  const int b = row_ptr[w * 16], e = row_ptr[min(w * 16 + 16, n)];
  const int u = uidx[e] - uidx[b];
  ucnt[w] = u;
  nblk[w] = (u + 7) / 8;
}

__global__ void k_wsb_fill_cols(const uint64_t* keys, const int32_t* flag, const int32_t* uidx,
                                int64_t nnz, const int32_t* row_ptr, int32_t n, int colbits,
                                const int32_t* win_ptr, int32_t* blk_col) {
  int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nnz || !flag[s]) return;
  const uint64_t k = keys[s];
  const int w = (int)(k >> colbits);
  const int col = (int)(k & ((1ull << colbits) - 1));
  const int p = uidx[s] - uidx[row_ptr[w * 16]];
  blk_col[(int64_t)(win_ptr[w] + p / 8) * 8 + (p % 8)] = col;
}

// position of `col` among the window's sorted distinct columns
__device__ __forceinline__ int col_pos(const int32_t* wcols, int u, int col) {
  int lo = 0, hi = u - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (wcols[mid] < col) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// The window's row starts, its sorted distinct columns (in LDS when the
// window has at most kWinLdsBlocks blocks) and, for entry e of the window,
// its row within the window and its column's position among the distinct
// columns.
struct WinStage {
  int32_t rp[17];
  int32_t cols[kWinLdsBlocks * 8];
};

__device__ __forceinline__ void stage_window(WinStage& ws, const int32_t* row_ptr, int32_t n, int w,
                                             const int32_t* wcols, int u, bool inl, int& nr) {
  nr = min(16, n - w * 16);
  if ((int)threadIdx.x <= nr) ws.rp[threadIdx.x] = row_ptr[w * 16 + threadIdx.x];
  if (inl)
    for (int i = threadIdx.x; i < u; i += kWinThreads) ws.cols[i] = wcols[i];
}

__device__ __forceinline__ int row_in_window(const WinStage& ws, int nr, int e) {
  int lo = 0, hi = nr - 1;  // largest i with rp[i] <= e
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ws.rp[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Each entry sets its bit of the window's 16 x 8 block bitmaps: LDS atomics
// on the window's words, stored once (device-scope atomics, about 27 G/s on
// this part, were the cost of the per-entry version).  Windows with more
// than kWinLdsBlocks blocks set their bits in memory directly.
__global__ __launch_bounds__(kWinThreads) void k_wsb_bits(const int32_t* row_ptr, const int32_t* col_idx, int32_t n,
                                                          const int32_t* win_ptr, const int32_t* ucnt,
                                                          const int32_t* blk_col, unsigned long long* bits) {
  __shared__ WinStage ws;
  __shared__ unsigned long long lb[kWinLdsBlocks * 2];
  const int w = blockIdx.x;
  const int b0 = win_ptr[w], nb = win_ptr[w + 1] - b0, u = ucnt[w];
  const int32_t* wcols = blk_col + (int64_t)b0 * 8;
  const bool inl = nb <= kWinLdsBlocks;
  int nr;
  stage_window(ws, row_ptr, n, w, wcols, u, inl, nr);
  if (inl)
    for (int i = threadIdx.x; i < 2 * nb; i += kWinThreads) lb[i] = 0ull;
  __syncthreads();
  const int e0 = ws.rp[0], e1 = ws.rp[nr];
  for (int e = e0 + threadIdx.x; e < e1; e += kWinThreads) {
    const int i = row_in_window(ws, nr, e);
    const int c = col_idx[e];
    const int pos = inl ? col_pos(ws.cols, u, c) : col_pos(wcols, u, c);
    const int bit = i * 8 + (pos & 7);
    const int word = (pos >> 3) * 2 + (bit >> 6);
    if (inl) atomicOr(&lb[word], 1ull << (bit & 63));
    else atomicOr(&bits[(int64_t)b0 * 2 + word], 1ull << (bit & 63));
  }
  if (inl) {
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * nb; i += kWinThreads) bits[(int64_t)b0 * 2 + i] = lb[i];
  }
}

__device__ __forceinline__ int window_of_block(const int32_t* win_ptr, int32_t nw, int blk) {
  int lo = 0, hi = nw - 1;  // largest w with win_ptr[w] <= blk
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (win_ptr[mid] <= blk) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// dense[blk] = 1 for the first block of a dense tile
__global__ void k_wsb_dense(const int32_t* win_ptr, int32_t nw, int64_t nblocks,
                            const unsigned long long* bits, int tau, int32_t* dense) {
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const int w = window_of_block(win_ptr, nw, (int)blk);
  int d = 0;
  if (((blk - win_ptr[w]) & 1) == 0) {
    int cnt = __popcll(bits[blk * 2]) + __popcll(bits[blk * 2 + 1]);
    if (blk + 1 < win_ptr[w + 1]) cnt += __popcll(bits[blk * 2 + 2]) + __popcll(bits[blk * 2 + 3]);
    d = cnt >= tau ? 1 : 0;
  }
  dense[blk] = d;
}

__global__ void k_wsb_tiles(const int32_t* dense, const int32_t* tscan, int64_t nblocks,
                            int32_t* tile_blk) {
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks || !dense[blk]) return;
  tile_blk[tscan[blk]] = (int)blk;
}

__global__ void k_wsb_tile_ptr(const int32_t* win_ptr, const int32_t* tscan, int32_t nw,
                               int32_t* tile_ptr) {
  int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w > nw) return;
  tile_ptr[w] = tscan[win_ptr[w]];
}

// rflag[e] = 1 for an entry outside the dense tiles (the residual CSR).
__global__ __launch_bounds__(kWinThreads) void k_wsb_resid_flags(const int32_t* row_ptr, const int32_t* col_idx,
                                                                 int32_t n, const int32_t* win_ptr,
                                                                 const int32_t* ucnt, const int32_t* blk_col,
                                                                 const int32_t* dense, int32_t* rflag) {
  __shared__ WinStage ws;
  const int w = blockIdx.x;
  const int b0 = win_ptr[w], nb = win_ptr[w + 1] - b0, u = ucnt[w];
  const int32_t* wcols = blk_col + (int64_t)b0 * 8;
  const bool inl = nb <= kWinLdsBlocks;
  int nr;
  stage_window(ws, row_ptr, n, w, wcols, u, inl, nr);
  __syncthreads();
  const int e0 = ws.rp[0], e1 = ws.rp[nr];
  for (int e = e0 + threadIdx.x; e < e1; e += kWinThreads) {
    const int c = col_idx[e];
    const int pos = inl ? col_pos(ws.cols, u, c) : col_pos(wcols, u, c);
    const int first = b0 + ((pos >> 3) & ~1);  // first block of the entry's tile
    rflag[e] = dense[first] ? 0 : 1;
  }
}

__global__ void k_wsb_resid_fill(const int32_t* col_idx, int64_t nnz, const int32_t* rflag,
                                 const int32_t* rscan, int32_t* res_col) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= nnz || !rflag[e]) return;
  res_col[rscan[e]] = col_idx[e];
}

__global__ void k_wsb_res_ptr(const int32_t* row_ptr, const int32_t* rscan, int32_t n,
                              int32_t* res_ptr) {
  int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r > n) return;
  res_ptr[r] = rscan[row_ptr[r]];
}

unsigned nblk(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

int plan_build_wsb(gnn_plan* p, hipStream_t s) {
  const int32_t n = p->n_rows;
  const int64_t nnz = p->nnz;
  const int32_t nw = (n + 15) / 16;
  WsbLayout& L = p->wsb;
  L.n_windows = nw;
  int colbits = 1;
  while ((1ll << colbits) < std::max(p->n_cols, 2)) ++colbits;
  int winbits = 1;
  while ((1ll << winbits) < std::max(nw, 2)) ++winbits;
  if (colbits + winbits > 64) return fail(GNN_ERR_SIZE_OVERFLOW, "WSB keys exceed 64 bits");

  GNN_TRY(plan_alloc(p, (void**)&L.win_ptr, ((size_t)nw + 1) * 4));
  GNN_TRY(plan_alloc(p, (void**)&L.tile_ptr, ((size_t)nw + 1) * 4));
  GNN_TRY(plan_alloc(p, (void**)&L.res_ptr, ((size_t)n + 1) * 4));
  if (nnz == 0) {
    GNN_HIP(hipMemsetAsync(L.win_ptr, 0, ((size_t)nw + 1) * 4, s));
    GNN_HIP(hipMemsetAsync(L.tile_ptr, 0, ((size_t)nw + 1) * 4, s));
    GNN_HIP(hipMemsetAsync(L.res_ptr, 0, ((size_t)n + 1) * 4, s));
    GNN_TRY(plan_alloc(p, (void**)&L.blk_col, 32));
    GNN_TRY(plan_alloc(p, (void**)&L.blk_bits, 16));
    GNN_TRY(plan_alloc(p, (void**)&L.tile_blk, 4));
    GNN_TRY(plan_alloc(p, (void**)&L.res_col, 4));
    p->has_wsb = true;
    return GNN_OK;
  }

  uint64_t *keys = nullptr, *tmp = nullptr;
  int32_t *flag = nullptr, *uidx = nullptr, *ucnt = nullptr, *nbk = nullptr;
  StreamTemps tt(s);
  GNN_TRY(tt.get(&keys, nnz * 8));
  GNN_TRY(tt.get(&tmp, nnz * 8));
  GNN_TRY(tt.get(&flag, (nnz + 1) * 4));
  GNN_TRY(tt.get(&uidx, (nnz + 1) * 4));
  GNN_TRY(tt.get(&ucnt, (size_t)nw * 4));
  GNN_TRY(tt.get(&nbk, (size_t)nw * 4));

  hipLaunchKernelGGL(k_wsb_keys, dim3((unsigned)nw), dim3(kWinThreads), 0, s, p->row_ptr, p->col_idx, n, colbits,
                     keys);
  GNN_LAUNCH_CHECK("wsb keys");
  GNN_TRY(radix_sort_u64(keys, tmp, nnz, 0, colbits + winbits, s));
  hipLaunchKernelGGL(k_wsb_flags, dim3(nblk(nnz)), dim3(256), 0, s, keys, nnz, flag);
  GNN_LAUNCH_CHECK("wsb flags");
  GNN_TRY(exclusive_scan_i32(flag, uidx, nnz, s));
  hipLaunchKernelGGL(k_wsb_wcount, dim3(nblk(nw)), dim3(256), 0, s, p->row_ptr, n, nw, uidx, ucnt, nbk);
  GNN_LAUNCH_CHECK("wsb counts");
  GNN_TRY(exclusive_scan_i32(nbk, L.win_ptr, nw, s));
  int32_t nb32 = 0;
  GNN_HIP(hipMemcpyAsync(&nb32, L.win_ptr + nw, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  L.n_blocks = nb32;

  GNN_TRY(plan_alloc(p, (void**)&L.blk_col, (size_t)std::max<int64_t>(L.n_blocks, 1) * 32));
  GNN_TRY(plan_alloc(p, (void**)&L.blk_bits, (size_t)std::max<int64_t>(L.n_blocks, 1) * 16));
  GNN_HIP(hipMemsetAsync(L.blk_col, 0, (size_t)std::max<int64_t>(L.n_blocks, 1) * 32, s));
  GNN_HIP(hipMemsetAsync(L.blk_bits, 0, (size_t)std::max<int64_t>(L.n_blocks, 1) * 16, s));
  hipLaunchKernelGGL(k_wsb_fill_cols, dim3(nblk(nnz)), dim3(256), 0, s, keys, flag, uidx, nnz,
                     p->row_ptr, n, colbits, L.win_ptr, L.blk_col);
  GNN_LAUNCH_CHECK("wsb cols");
  hipLaunchKernelGGL(k_wsb_bits, dim3((unsigned)nw), dim3(kWinThreads), 0, s, p->row_ptr, p->col_idx, n,
                     L.win_ptr, ucnt, L.blk_col, (unsigned long long*)L.blk_bits);
  GNN_LAUNCH_CHECK("wsb bits");

  // dense tiles
  int32_t *dense = nullptr, *tscan = nullptr;
  GNN_TRY(tt.get(&dense, (size_t)(L.n_blocks + 1) * 4));
  GNN_TRY(tt.get(&tscan, (size_t)(L.n_blocks + 1) * 4));
  hipLaunchKernelGGL(k_wsb_dense, dim3(nblk(L.n_blocks)), dim3(256), 0, s, L.win_ptr, nw, L.n_blocks,
                     (const unsigned long long*)L.blk_bits, p->opts.wsb_min_nnz, dense);
  GNN_LAUNCH_CHECK("wsb dense");
  GNN_TRY(exclusive_scan_i32(dense, tscan, L.n_blocks, s));
  int32_t nt32 = 0;
  GNN_HIP(hipMemcpyAsync(&nt32, tscan + L.n_blocks, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  L.n_tiles = nt32;
  GNN_TRY(plan_alloc(p, (void**)&L.tile_blk, (size_t)std::max<int64_t>(L.n_tiles, 1) * 4));
  hipLaunchKernelGGL(k_wsb_tiles, dim3(nblk(L.n_blocks)), dim3(256), 0, s, dense, tscan, L.n_blocks,
                     L.tile_blk);
  GNN_LAUNCH_CHECK("wsb tiles");
  hipLaunchKernelGGL(k_wsb_tile_ptr, dim3(nblk(nw + 1)), dim3(256), 0, s, L.win_ptr, tscan, nw,
                     L.tile_ptr);
  GNN_LAUNCH_CHECK("wsb tile ptr");

  // residual CSR
  hipLaunchKernelGGL(k_wsb_resid_flags, dim3((unsigned)nw), dim3(kWinThreads), 0, s, p->row_ptr, p->col_idx, n,
                     L.win_ptr, ucnt, L.blk_col, dense, flag);
  GNN_LAUNCH_CHECK("wsb residual flags");
  GNN_TRY(exclusive_scan_i32(flag, uidx, nnz, s));
  int32_t nr32 = 0;
  GNN_HIP(hipMemcpyAsync(&nr32, uidx + nnz, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  L.n_resid = nr32;
  GNN_TRY(plan_alloc(p, (void**)&L.res_col, (size_t)std::max<int64_t>(L.n_resid, 1) * 4));
  hipLaunchKernelGGL(k_wsb_resid_fill, dim3(nblk(nnz)), dim3(256), 0, s, p->col_idx, nnz, flag, uidx,
                     L.res_col);
  GNN_LAUNCH_CHECK("wsb residual fill");
  hipLaunchKernelGGL(k_wsb_res_ptr, dim3(nblk(n + 1)), dim3(256), 0, s, p->row_ptr, uidx, n,
                     L.res_ptr);
  GNN_LAUNCH_CHECK("wsb residual ptr");

  GNN_TRY(tt.release());
  p->has_wsb = true;
  return GNN_OK;
}

}  // namespace gnn
