// Plan construction: degrees, the degree-quantile threshold, degree bins and
// edge-chunk work items.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.1: destinations are split into light and heavy
// sets by a graph-specific degree threshold, the gamma-quantile of the degree
// distribution (gamma in [0.99, 0.999]); heavy rows are cut into chunks of
// EDGES_PER_BLOCK edges processed by separate blocks.  Appendix D.4: degrees
// are precomputed once per graph and cached.
//
// Bins used here (the MI355X mapping):
//   light  : deg <= light_max           one 32-lane slot per row
//   medium : light_max < deg <= thr     one workgroup per row
//   heavy  : deg > thr                  ceil(deg / chunk) workgroups, merged
#include <algorithm>

#include <string.h>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;                       // per thread
constexpr int kScanTile = kScanThreads * kScanItems;  // 4096 elements per block
constexpr int kHistBins = 65536;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Block-wide exclusive scan of one value per thread; returns the block total.
__device__ int block_excl_scan(int v, int* lds_waves, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = kScanThreads / 64;
  int inc = wave_incl_scan(v);
  if (lane == 63) lds_waves[wave] = inc;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int s = lds_waves[w];
    if (w < wave) off += s;
    total += s;
  }
  __syncthreads();
  return off + inc - v;
}

// A thread's kScanItems consecutive inputs; a tile inside the array with
// 16-byte aligned arrays (VEC) is read with four 16-byte loads per thread.
template <bool VEC>
__device__ __forceinline__ void scan_load(const int32_t* in, int64_t n, int64_t base, int (&v)[kScanItems]) {
  if (VEC && (int64_t)(blockIdx.x + 1) * kScanTile <= n) {
    const int4* p = reinterpret_cast<const int4*>(in + base);
#pragma unroll
    for (int q = 0; q < kScanItems / 4; ++q) {
      const int4 t = p[q];
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) v[k] = (base + k < n) ? in[base + k] : 0;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void k_scan_block_sums(const int32_t* in, int64_t n,
                                                                  int32_t* sums) {
  __shared__ int lw[kScanThreads / 64];
  int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
  int v[kScanItems];
  scan_load<VEC>(in, n, base, v);
  int s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) s += v[k];
  int total;
  block_excl_scan(s, lw, total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void k_scan_tiles(const int32_t* in, int64_t n,
                                                             const int32_t* block_off,
                                                             int32_t* out) {
  __shared__ int lw[kScanThreads / 64];
  int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
  int v[kScanItems];
  scan_load<VEC>(in, n, base, v);
  int s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) s += v[k];
  int total;
  int run = block_excl_scan(s, lw, total) + (block_off ? block_off[blockIdx.x] : 0);
  if (VEC && (int64_t)(blockIdx.x + 1) * kScanTile <= n) {
    int4* p = reinterpret_cast<int4*>(out + base);
#pragma unroll
    for (int q = 0; q < kScanItems / 4; ++q) {
      int4 t;
      t.x = run;
      run += v[4 * q];
      t.y = run;
      run += v[4 * q + 1];
      t.z = run;
      run += v[4 * q + 2];
      t.w = run;
      run += v[4 * q + 3];
      p[q] = t;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      if (base + k < n) out[base + k] = run;
      run += v[k];
    }
  }
  // the last element's successor: out[n] = grand total
  if (base + kScanItems >= n && base < n) out[n] = run;
  if (n == 0 && blockIdx.x == 0 && threadIdx.x == 0) out[0] = 0;
}

// ---------------------------------------------------------------------------

// Degree histogram.  Low degrees are very common on power-law graphs (most
// rows have degree 0 or 1), so each workgroup counts bins below kLdsBins in
// LDS and flushes its non-zero bins once; larger degrees go straight to the
// global histogram.
constexpr int kLdsBins = 4096;

__global__ __launch_bounds__(256) void k_deg_hist(const int32_t* row_ptr, int32_t n, int32_t* hist) {
  __shared__ int32_t lh[kLdsBins];
  for (int b = threadIdx.x; b < kLdsBins; b += blockDim.x) lh[b] = 0;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n; base += stride) {
    const int64_t i = base + threadIdx.x;
    const bool ok = i < n;
    const int d = ok ? row_ptr[i + 1] - row_ptr[i] : -1;
    // degrees 0 and 1 are counted per wave by ballot, the rest by atomics
    const unsigned long long b0 = __ballot(d == 0), b1 = __ballot(d == 1);
    if ((threadIdx.x & 63) == 0) {
      if (b0) atomicAdd(&lh[0], (int)__popcll(b0));
      if (b1) atomicAdd(&lh[1], (int)__popcll(b1));
    }
    if (d >= 2) {
      if (d < kLdsBins) atomicAdd(&lh[d], 1);
      else atomicAdd(&hist[d < kHistBins - 1 ? d : kHistBins - 1], 1);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kLdsBins; b += blockDim.x)
    if (lh[b]) atomicAdd(&hist[b], lh[b]);
}

// Smallest degree d with #{rows with deg <= d} >= ceil(gamma * n): the
// gamma-quantile.  One block; the histogram is scanned serially in chunks.
__global__ __launch_bounds__(256) void k_quantile(const int32_t* hist, int32_t n, float gamma,
                                                  int32_t* out) {
  __shared__ int lw[4];
  __shared__ int carry;
  __shared__ int found;
  if (threadIdx.x == 0) {
    carry = 0;
    found = kHistBins - 1;
  }
  __syncthreads();
  int64_t target = (int64_t)ceil((double)gamma * (double)n);
  if (target < 1) target = 1;
  for (int base = 0; base < kHistBins; base += 256) {
    int v = hist[base + threadIdx.x];
    int total;
    // reuse the generic block scan (256 threads)
    int ex = block_excl_scan(v, lw, total);
    int incl = carry + ex + v;
    if (incl >= target && (carry + ex) < target) found = base + threadIdx.x;
    __syncthreads();
    if (threadIdx.x == 0) carry += total;
    __syncthreads();
    if (carry >= target) break;
  }
  if (threadIdx.x == 0) *out = found;
}

// Row classes.  Each workgroup writes its (light, medium, heavy, max chunks)
// totals to part[blockIdx.x]; k_stats_total folds them.  (One atomic per wave
// on four shared counters serialises at the L2 on large graphs.)
// Work items of a row of d entries: none up to light_max, one up to thr,
// else one per chunk.
__device__ __forceinline__ int row_items(int d, int32_t light_max, int32_t thr, int32_t chunk) {
  return d <= light_max ? 0 : (d <= thr ? 1 : (d + chunk - 1) / chunk);
}

// Per-block counts of light, medium and heavy rows and the largest item
// count of a row (for the plan's statistics).
__global__ __launch_bounds__(256) void k_classify(const int32_t* row_ptr, int32_t n, int32_t light_max,
                                                  int32_t thr, int32_t chunk, unsigned long long* part) {
  __shared__ unsigned long long ws[4][4];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int c = 0;
  if (i < n) {
    c = row_items(row_ptr[i + 1] - row_ptr[i], light_max, thr, chunk);
  }
  const unsigned long long l = __popcll(__ballot(i < n && c == 0));
  const unsigned long long m = __popcll(__ballot(i < n && c == 1));
  const unsigned long long h = __popcll(__ballot(i < n && c > 1));
  int cm = c;
  for (int d = 32; d >= 1; d >>= 1) cm = max(cm, __shfl_xor(cm, d));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ws[wave][0] = l;
    ws[wave][1] = m;
    ws[wave][2] = h;
    ws[wave][3] = (unsigned long long)cm;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    unsigned long long v = 0;
    for (int w = 0; w < 4; ++w)
      v = threadIdx.x == 3 ? (ws[w][3] > v ? ws[w][3] : v) : v + ws[w][threadIdx.x];
    part[(int64_t)blockIdx.x * 4 + threadIdx.x] = v;
  }
}

// Sum (the first three words) and maximum (the fourth) of nb partials.
__global__ __launch_bounds__(256) void k_stats_total(const unsigned long long* part, int64_t nb,
                                                     unsigned long long* stats) {
  __shared__ unsigned long long red[4][256];
  unsigned long long a[4] = {0, 0, 0, 0};
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
    for (int k = 0; k < 3; ++k) a[k] += part[b * 4 + k];
    a[3] = part[b * 4 + 3] > a[3] ? part[b * 4 + 3] : a[3];
  }
  for (int k = 0; k < 4; ++k) red[k][threadIdx.x] = a[k];
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      for (int k = 0; k < 3; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + o];
      red[3][threadIdx.x] = red[3][threadIdx.x + o] > red[3][threadIdx.x] ? red[3][threadIdx.x + o]
                                                                          : red[3][threadIdx.x];
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) stats[threadIdx.x] = red[threadIdx.x][0];
}

// Fingerprint samples: out[k] = row_ptr[k n / (K - 1)], out[K + k] =
// col_idx[k (nnz - 1) / (K - 1)] (0 for an empty graph), k < K.
__global__ void k_fingerprint(const int32_t* row_ptr, int32_t n, const int32_t* col_idx, int64_t nnz, int32_t K,
                              int32_t* out) {
  const int k = threadIdx.x;
  if (k >= K) return;
  out[k] = row_ptr[(int64_t)k * n / (K - 1)];
  out[K + k] = nnz > 0 ? col_idx[(int64_t)k * (nnz - 1) / (K - 1)] : 0;
}

// The item list, built in two passes over the rows.  Layout: the chunks of
// split rows (chunk q of a row at its split offset + q, so that an item index
// below the chunk total is also the row's partial slot), then the medium rows
// longer than att_thr, then the other medium rows, each group in row order.
// multi[m] = (row, first chunk item, chunk count, 0).  The attention kernels
// run rows of up to att_thr entries one per slot, so they launch only the
// items before the short medium rows.
// Pass one: per tile of kScanTile rows, the sums of items, split chunks,
// split rows and long medium rows, stored as four runs of nb entries
// (sums[k nb + b]); one exclusive scan over all 4 nb entries turns them into
// per-tile offsets (minus each run's first entry).  Pass two: the same
// per-row counts, scanned inside the tile, give every row its positions.
struct RowCounts {
  int c, sc, m, g;  // items, split chunks, split rows, long medium rows
};

__device__ __forceinline__ RowCounts row_counts(const int32_t* row_ptr, int64_t i, int32_t light_max, int32_t thr,
                                                int32_t chunk, int32_t att_thr) {
  const int d = row_ptr[i + 1] - row_ptr[i];
  const int r = row_items(d, light_max, thr, chunk);
  return RowCounts{r, r > 1 ? r : 0, r > 1 ? 1 : 0, (r == 1 && d > att_thr) ? 1 : 0};
}

__global__ __launch_bounds__(kScanThreads) void k_items_sums(const int32_t* row_ptr, int64_t n, int32_t light_max,
                                                             int32_t thr, int32_t chunk, int32_t att_thr,
                                                             int32_t* sums) {
  __shared__ int lw[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
  RowCounts t{0, 0, 0, 0};
  for (int k = 0; k < kScanItems; ++k) {
    if (base + k >= n) break;
    const RowCounts r = row_counts(row_ptr, base + k, light_max, thr, chunk, att_thr);
    t.c += r.c;
    t.sc += r.sc;
    t.m += r.m;
    t.g += r.g;
  }
  int t0, t1, t2, t3;
  (void)block_excl_scan(t.c, lw, t0);
  (void)block_excl_scan(t.sc, lw, t1);
  (void)block_excl_scan(t.m, lw, t2);
  (void)block_excl_scan(t.g, lw, t3);
  if (threadIdx.x == 0) {
    sums[blockIdx.x] = t0;
    sums[gridDim.x + blockIdx.x] = t1;
    sums[2 * gridDim.x + blockIdx.x] = t2;
    sums[3 * gridDim.x + blockIdx.x] = t3;
  }
}

// cs: the exclusive scan of the 4 nb sums (4 nb + 1 entries).  counts
// (optional): [0] = items, [1] = split rows.
__global__ __launch_bounds__(kScanThreads) void k_items_fill(const int32_t* row_ptr, int64_t n, int32_t light_max,
                                                             int32_t thr, int32_t chunk, int32_t att_thr,
                                                             const int32_t* cs, int4* items, int4* multi,
                                                             int32_t* counts) {
  __shared__ int lw[kScanThreads / 64];
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const int64_t base = (int64_t)b * kScanTile + (int64_t)threadIdx.x * kScanItems;
  RowCounts r[kScanItems];
  RowCounts t{0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    r[k] = base + k < n ? row_counts(row_ptr, base + k, light_max, thr, chunk, att_thr) : RowCounts{0, 0, 0, 0};
    t.c += r[k].c;
    t.sc += r[k].sc;
    t.m += r[k].m;
    t.g += r[k].g;
  }
  int tot;
  int io = block_excl_scan(t.c, lw, tot) + cs[b];
  int so = block_excl_scan(t.sc, lw, tot) + cs[nb + b] - cs[nb];
  int mo = block_excl_scan(t.m, lw, tot) + cs[2 * nb + b] - cs[2 * nb];
  int go = block_excl_scan(t.g, lw, tot) + cs[3 * nb + b] - cs[3 * nb];
  const int n_chunks = cs[2 * nb] - cs[nb], n_long = cs[4 * nb] - cs[3 * nb];
  if (counts && b == 0 && threadIdx.x == 0) {
    counts[0] = cs[nb];
    counts[1] = cs[3 * nb] - cs[2 * nb];
  }
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    if (r[k].c == 0) continue;
    const int64_t i = base + k;
    const int e0 = row_ptr[i], e1 = row_ptr[i + 1];
    if (r[k].c == 1) {
      // medium rows before this one: io - so; long ones among them: go
      const int pos = r[k].g ? n_chunks + go : n_chunks + n_long + (io - so - go);
      items[pos] = make_int4((int)i, e0, e1, -1);
    } else {
      for (int q = 0; q < r[k].c; ++q) {
        const int eb = e0 + q * chunk;
        items[so + q] = make_int4((int)i, eb, min(e1, eb + chunk), mo);
      }
      multi[mo] = make_int4((int)i, so, r[k].c, 0);
    }
    io += r[k].c;
    so += r[k].sc;
    mo += r[k].m;
    go += r[k].g;
  }
}

// The attention row list.  Rows of at most lmax edges are ordered by window
// of 2^kAttWindowBits consecutive rows, then by decreasing length, then by
// row: waves get rows of one length while the rows a window's workgroups
// touch stay close (neighbourhoods of nearby rows overlap on clustered
// graphs).  Longer rows are not listed.  One workgroup per window counts its
// listed rows; after an exclusive scan of the counts, one workgroup per
// window sorts its rows in LDS and writes them at the window's offset.
#ifndef GNN_ATT_WINDOW_BITS
#define GNN_ATT_WINDOW_BITS 10
#endif
constexpr int kAttWindowBits = GNN_ATT_WINDOW_BITS;
constexpr int kAttWindow = 1 << kAttWindowBits;
static_assert(kAttWindowBits >= 8 && kAttWindowBits <= 12, "window of 256 to 4096 rows");

__global__ __launch_bounds__(256) void k_att_win_count(const int32_t* row_ptr, int32_t n, int32_t lmax,
                                                       int32_t* cnt) {
  __shared__ int32_t red[4];
  const int64_t base = (int64_t)blockIdx.x * kAttWindow;
  int c = 0;
  for (int k = threadIdx.x; k < kAttWindow; k += 256) {
    const int64_t i = base + k;
    if (i < n && row_ptr[i + 1] - row_ptr[i] <= lmax) ++c;
  }
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cnt[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// Sort key of a row inside its window: (lmax - length) above the row's
// position (longer first, then by row), all ones for a row that is not
// listed.  The length field saturates at 2^(32 - kAttWindowBits) - 1: rows
// that much shorter than lmax keep row order among themselves.
__global__ __launch_bounds__(256) void k_att_win_sort(const int32_t* row_ptr, int32_t n, int32_t lmax,
                                                      const int32_t* woff, int32_t* rows) {
  __shared__ uint32_t key[kAttWindow];
  const int64_t base = (int64_t)blockIdx.x * kAttWindow;
  constexpr uint32_t kLenMax = (1u << (32 - kAttWindowBits)) - 2;
  for (int k = threadIdx.x; k < kAttWindow; k += 256) {
    const int64_t i = base + k;
    uint32_t v = 0xFFFFFFFFu;
    if (i < n) {
      const int d = row_ptr[i + 1] - row_ptr[i];
      if (d <= lmax) v = (min((uint32_t)(lmax - d), kLenMax) << kAttWindowBits) | (uint32_t)k;
    }
    key[k] = v;
  }
  __syncthreads();
  // bitonic sorting network, ascending
  for (int size = 2; size <= kAttWindow; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < kAttWindow / 2; t += 256) {
        const int a = 2 * t - (t & (j - 1)), b = a + j;
        const uint32_t x = key[a], y = key[b];
        if ((x > y) == ((a & size) == 0)) {
          key[a] = y;
          key[b] = x;
        }
      }
      __syncthreads();
    }
  }
  const int32_t off = woff[blockIdx.x], cnt = woff[blockIdx.x + 1] - off;
  for (int k = threadIdx.x; k < cnt; k += 256) rows[off + k] = (int32_t)(base + (key[k] & (kAttWindow - 1)));
}

}  // namespace

int plan_att_rows(gnn_plan* p, int32_t lmax, hipStream_t s) {
  if (p->att_lmax == lmax) return GNN_OK;
  const int32_t n = p->n_rows;
  const int64_t nw = ((int64_t)n + kAttWindow - 1) / kAttWindow;
  if (!p->att_rows) GNN_TRY(plan_alloc(p, (void**)&p->att_rows, (size_t)std::max(n, 1) * 4));
  if (!p->att_count) {
    // listed rows before each window; the last entry is the count
    int32_t* woff = nullptr;
    GNN_TRY(plan_alloc(p, (void**)&woff, (size_t)(nw + 1) * 4));
    p->att_woff = woff;
    p->att_count = woff + nw;
  }
  if (n == 0) {
    GNN_HIP(hipMemsetAsync(p->att_count, 0, 4, s));
  } else {
    StreamTemps tt(s);
    int32_t* cnt = nullptr;
    GNN_TRY(tt.get(&cnt, (size_t)nw * 4));
    hipLaunchKernelGGL(k_att_win_count, dim3((unsigned)nw), dim3(256), 0, s, p->row_ptr, n, lmax, cnt);
    GNN_LAUNCH_CHECK("attention row counts");
    GNN_TRY(exclusive_scan_i32(cnt, p->att_woff, nw, s));
    hipLaunchKernelGGL(k_att_win_sort, dim3((unsigned)nw), dim3(256), 0, s, p->row_ptr, n, lmax, p->att_woff,
                       p->att_rows);
    GNN_LAUNCH_CHECK("attention row list");
    GNN_TRY(tt.release());
  }
  p->att_lmax = lmax;
  return GNN_OK;
}

size_t scan_scratch_bytes(int64_t n) {
  const int64_t nb = (n + kScanTile - 1) / kScanTile;
  if (nb <= 1) return 0;
  return Arena::round((size_t)nb * 4) + Arena::round((size_t)(nb + 1) * 4) + scan_scratch_bytes(nb);
}

int exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, hipStream_t s, void* scratch) {
  int64_t nb = (n + kScanTile - 1) / kScanTile;
  const bool in16 = (uintptr_t)in % 16 == 0, vec = in16 && (uintptr_t)out % 16 == 0;
  if (nb <= 1) {
    if (vec) hipLaunchKernelGGL(k_scan_tiles<true>, dim3(1), dim3(kScanThreads), 0, s, in, n, nullptr, out);
    else hipLaunchKernelGGL(k_scan_tiles<false>, dim3(1), dim3(kScanThreads), 0, s, in, n, nullptr, out);
    GNN_LAUNCH_CHECK("scan");
    return GNN_OK;
  }
  StreamTemps tmp(s);
  if (!scratch) GNN_TRY(tmp.get(&scratch, scan_scratch_bytes(n)));
  Arena a{static_cast<char*>(scratch), scan_scratch_bytes(n), 0};
  int32_t* sums = a.take<int32_t>(nb);
  int32_t* offs = a.take<int32_t>(nb + 1);
  if (in16) hipLaunchKernelGGL(k_scan_block_sums<true>, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, sums);
  else hipLaunchKernelGGL(k_scan_block_sums<false>, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, sums);
  GNN_LAUNCH_CHECK("scan sums");
  int rc = exclusive_scan_i32(sums, offs, nb, s, a.base + a.off);
  if (rc == GNN_OK) {
    if (vec)
      hipLaunchKernelGGL(k_scan_tiles<true>, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, offs, out);
    else
      hipLaunchKernelGGL(k_scan_tiles<false>, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, offs, out);
    GNN_LAUNCH_CHECK("scan tiles");
  }
  if (rc != GNN_OK) return rc;
  return tmp.release();
}

int plan_alloc(gnn_plan* p, void** ptr, size_t bytes) {
  if (p->n_allocs >= (int)(sizeof(p->allocs) / sizeof(p->allocs[0])))
    return fail(GNN_ERR_DEVICE, "plan: too many allocations");
  void* q = nullptr;
  if (p->async_mem) GNN_TRY(dev_malloc_async(&q, bytes ? bytes : 16, p->stream));
  else GNN_TRY(dev_malloc(&q, bytes ? bytes : 16));
  p->allocs[p->n_allocs++] = q;
  *ptr = q;
  return GNN_OK;
}

int plan_workspace(gnn_plan* p, size_t bytes, void** out) {
  if (bytes <= p->ws_bytes && p->ws) {
    *out = p->ws;
    return GNN_OK;
  }
  if (p->ws) {
    if (p->async_mem) {
      GNN_TRY(dev_free_async(p->ws, p->stream));
    } else {
      GNN_HIP(hipStreamSynchronize(p->stream));
      GNN_HIP(hipFree(p->ws));
    }
    p->ws = nullptr;
    p->ws_bytes = 0;
  }
  void* q = nullptr;
  if (p->async_mem) GNN_TRY(dev_malloc_async(&q, bytes, p->stream));
  else GNN_TRY(dev_malloc(&q, bytes));
  p->ws = q;
  p->ws_bytes = bytes;
  *out = q;
  return GNN_OK;
}

int plan_grow(gnn_plan* p, void** buf, size_t* cap, size_t bytes) {
  if (*buf && *cap >= bytes) return GNN_OK;
  if (*buf) {
    if (p->async_mem) {
      GNN_TRY(dev_free_async(*buf, p->stream));
    } else {
      GNN_HIP(hipStreamSynchronize(p->stream));
      GNN_HIP(hipFree(*buf));
    }
    *buf = nullptr;
    *cap = 0;
  }
  if (p->async_mem) GNN_TRY(dev_malloc_async(buf, bytes, p->stream));
  else GNN_TRY(dev_malloc(buf, bytes));
  *cap = bytes;
  return GNN_OK;
}

int plan_sample_fingerprint(gnn_plan* p, hipStream_t s) {
  hipLaunchKernelGGL(k_fingerprint, dim3(1), dim3(gnn_plan::kFingerprint), 0, s, p->row_ptr, p->n_rows, p->col_idx,
                     p->nnz, (int32_t)gnn_plan::kFingerprint, p->fp_dev);
  GNN_LAUNCH_CHECK("fingerprint");
  return GNN_OK;
}

int plan_verify(gnn_plan* p, hipStream_t s) {
  int32_t now[2 * gnn_plan::kFingerprint];
  GNN_TRY(plan_sample_fingerprint(p, s));
  GNN_HIP(hipMemcpyAsync(now, p->fp_dev, sizeof(now), hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  if (memcmp(now, p->fp_host, sizeof(now)) != 0)
    return fail(GNN_ERR_PLAN_MISMATCH, "the CSR arrays changed since the plan was built (sampled entries differ)");
  return GNN_OK;
}

int plan_deg_out(gnn_plan* p, hipStream_t s) {
  if (p->deg_out) return GNN_OK;
  int32_t* d = nullptr;
  GNN_TRY(plan_alloc(p, (void**)&d, (size_t)std::max(p->n_cols, 1) * 4));
  GNN_TRY(count_out_degrees(p->col_idx, p->nnz, p->n_cols, d, s));
  p->deg_out = d;
  return GNN_OK;
}

int plan_build_async(const gnn_csr* csr, hipStream_t s, gnn_plan* p, int32_t light_max) {
  p->n_rows = csr->n_rows;
  p->n_cols = csr->n_cols;
  p->nnz = csr->nnz;
  p->row_ptr = csr->row_ptr;
  p->col_idx = csr->col_idx;
  p->stream = s;
  p->async_mem = true;
  p->opts.wsb_min_nnz = 8;
  p->light_max = light_max;
  p->chunk_edges = std::max(1024, 2 * (light_max + 1));  // keeps the item bound below valid
  // no degree quantile (it needs a read-back): every row longer than one
  // chunk is split
  p->heavy_thr = p->chunk_edges;
  const int32_t n = p->n_rows;
  const int64_t nnz = p->nnz, lm = p->light_max, ch = p->chunk_edges;
  // out-degrees on first use (plan_deg_out)
  // Host bounds of the device counts.  A row of d > light_max entries gives
  // one item, or ceil(d / chunk) <= d / (light_max + 1) chunks when split,
  // so items <= nnz / (light_max + 1), and <= rows + nnz / chunk; split rows
  // have more than one chunk of entries, so there are at most nnz / (chunk + 1)
  // of them and at most nnz / chunk + nnz / (chunk + 1) chunks.
  p->n_items = std::min<int64_t>(nnz / (lm + 1), (int64_t)n + nnz / ch);
  p->n_multi = std::min<int64_t>(n, nnz / (ch + 1));
  p->n_slots = std::min<int64_t>(p->n_items, nnz / ch + p->n_multi);
  p->att_item_thr = light_max;
  p->n_att_items = p->n_items;
  GNN_TRY(plan_alloc(p, (void**)&p->item_count, 16));
  p->multi_count = p->item_count + 1;
  GNN_TRY(plan_alloc(p, (void**)&p->items, (size_t)std::max<int64_t>(p->n_items, 1) * sizeof(int4)));
  GNN_TRY(plan_alloc(p, (void**)&p->multi, (size_t)std::max<int64_t>(p->n_multi, 1) * sizeof(int4)));
  if (n == 0 || p->n_items == 0) {
    GNN_HIP(hipMemsetAsync(p->item_count, 0, 8, s));
    return GNN_OK;
  }
  StreamTemps tt(s);
  const int64_t nb = ((int64_t)n + kScanTile - 1) / kScanTile;
  int32_t *sums = nullptr, *cs = nullptr;
  GNN_TRY(tt.get(&sums, (size_t)nb * 4 * 4));
  GNN_TRY(tt.get(&cs, ((size_t)nb * 4 + 1) * 4));
  // every medium row counts as long (att_thr = light_max): row order
  hipLaunchKernelGGL(k_items_sums, dim3((unsigned)nb), dim3(kScanThreads), 0, s, p->row_ptr, (int64_t)n,
                     p->light_max, p->heavy_thr, p->chunk_edges, p->light_max, sums);
  GNN_LAUNCH_CHECK("item sums");
  GNN_TRY(exclusive_scan_i32(sums, cs, nb * 4, s));
  hipLaunchKernelGGL(k_items_fill, dim3((unsigned)nb), dim3(kScanThreads), 0, s, p->row_ptr, (int64_t)n,
                     p->light_max, p->heavy_thr, p->chunk_edges, p->light_max, cs, p->items, p->multi,
                     p->item_count);
  GNN_LAUNCH_CHECK("fill items");
  return tt.release();
}

int plan_build(const gnn_csr* csr, const gnn_plan_opts* opts, hipStream_t s, gnn_plan* p) {
  p->n_rows = csr->n_rows;
  p->n_cols = csr->n_cols;
  p->nnz = csr->nnz;
  p->row_ptr = csr->row_ptr;
  p->col_idx = csr->col_idx;
  p->stream = s;
  if (opts) p->opts = *opts;
  float gamma = p->opts.heavy_quantile == 0.0f ? 0.99f : p->opts.heavy_quantile;
  p->light_max = p->opts.light_max_deg > 0 ? p->opts.light_max_deg : 32;
  p->chunk_edges = p->opts.chunk_edges > 0 ? p->opts.chunk_edges : 1024;
  if (p->opts.wsb_min_nnz <= 0) p->opts.wsb_min_nnz = 8;

  const int32_t n = p->n_rows;
  GNN_TRY(plan_alloc(p, (void**)&p->deg_out, (size_t)std::max(p->n_cols, 1) * 4));
  GNN_TRY(plan_alloc(p, (void**)&p->fp_dev, sizeof(p->fp_host)));
  GNN_TRY(plan_sample_fingerprint(p, s));
  GNN_HIP(hipMemcpyAsync(p->fp_host, p->fp_dev, sizeof(p->fp_host), hipMemcpyDeviceToHost, s));
  GNN_TRY(count_out_degrees(p->col_idx, p->nnz, p->n_cols, p->deg_out, s));

  // gamma-quantile degree threshold
  StreamTemps tt(s);
  int32_t* hist = nullptr;
  int32_t* tmp = nullptr;  // [threshold]
  GNN_TRY(tt.get(&hist, kHistBins * 4 + 16));
  tmp = hist + kHistBins;
  int32_t thr_host = INT32_MAX;
  if (gamma > 0.0f && n > 0) {
    GNN_HIP(hipMemsetAsync(hist, 0, kHistBins * 4, s));
    int64_t blocks = std::min<int64_t>((n + 255) / 256, 512);
    hipLaunchKernelGGL(k_deg_hist, dim3((unsigned)blocks), dim3(256), 0, s, p->row_ptr, n, hist);
    GNN_LAUNCH_CHECK("deg_hist");
    hipLaunchKernelGGL(k_quantile, dim3(1), dim3(256), 0, s, hist, n, std::min(gamma, 1.0f), tmp);
    GNN_LAUNCH_CHECK("quantile");
    GNN_HIP(hipMemcpyAsync(&thr_host, tmp, 4, hipMemcpyDeviceToHost, s));
    GNN_HIP(hipStreamSynchronize(s));
    // a row is heavy only if it also exceeds one chunk
    thr_host = std::max(thr_host, p->chunk_edges);
  }
  p->heavy_thr = thr_host;

  // statistics, then the item list (totals read back to size it)
  unsigned long long* stats = nullptr;
  const int64_t ncb = std::max<int64_t>((n + 255) / 256, 1);
  GNN_TRY(tt.get(&stats, (4 + ncb * 4) * 8));
  GNN_HIP(hipMemsetAsync(stats, 0, (4 + ncb * 4) * 8, s));
  // the attention kernels' one-slot bound for this plan
  p->att_item_thr = std::max(p->light_max, std::min(p->opts.att_slot_max > 0 ? p->opts.att_slot_max : kAttSlotRows,
                                                    p->heavy_thr));
  const int64_t nb = std::max<int64_t>(((int64_t)n + kScanTile - 1) / kScanTile, 1);
  int32_t *sums = nullptr, *cs = nullptr;
  GNN_TRY(tt.get(&sums, (size_t)nb * 4 * 4));
  GNN_TRY(tt.get(&cs, ((size_t)nb * 4 + 1) * 4));
  int32_t tot[5] = {0, 0, 0, 0, 0};
  if (n > 0) {
    hipLaunchKernelGGL(k_classify, dim3((unsigned)ncb), dim3(256), 0, s, p->row_ptr, n, p->light_max,
                       p->heavy_thr, p->chunk_edges, stats + 4);
    GNN_LAUNCH_CHECK("classify");
    hipLaunchKernelGGL(k_stats_total, dim3(1), dim3(256), 0, s, stats + 4, ncb, stats);
    GNN_LAUNCH_CHECK("classify totals");
    hipLaunchKernelGGL(k_items_sums, dim3((unsigned)nb), dim3(kScanThreads), 0, s, p->row_ptr, (int64_t)n,
                       p->light_max, p->heavy_thr, p->chunk_edges, p->att_item_thr, sums);
    GNN_LAUNCH_CHECK("item sums");
    GNN_TRY(exclusive_scan_i32(sums, cs, nb * 4, s));
    for (int k = 0; k < 5; ++k) GNN_HIP(hipMemcpyAsync(&tot[k], cs + k * nb, 4, hipMemcpyDeviceToHost, s));
  }
  unsigned long long st[4] = {0, 0, 0, 0};
  GNN_HIP(hipMemcpyAsync(st, stats, 32, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  p->n_items = tot[1] - tot[0];
  p->n_slots = tot[2] - tot[1];
  p->n_multi = tot[3] - tot[2];
  p->n_att_items = p->n_slots + (tot[4] - tot[3]);
  p->n_light = (int64_t)st[0];
  p->n_medium = (int64_t)st[1];
  p->n_heavy = (int64_t)st[2];
  p->max_items_per_row = (int32_t)st[3];
  GNN_TRY(plan_alloc(p, (void**)&p->items, (size_t)std::max<int64_t>(p->n_items, 1) * sizeof(int4)));
  GNN_TRY(plan_alloc(p, (void**)&p->multi, (size_t)std::max<int64_t>(p->n_multi, 1) * sizeof(int4)));
  if (n > 0) {
    hipLaunchKernelGGL(k_items_fill, dim3((unsigned)nb), dim3(kScanThreads), 0, s, p->row_ptr, (int64_t)n,
                       p->light_max, p->heavy_thr, p->chunk_edges, p->att_item_thr, cs, p->items, p->multi,
                       (int32_t*)nullptr);
    GNN_LAUNCH_CHECK("fill items");
  }
  GNN_TRY(tt.release());
  if (p->opts.build_wsb) GNN_TRY(plan_build_wsb(p, s));
  GNN_HIP(hipStreamSynchronize(s));
  return GNN_OK;
}

}  // namespace gnn
