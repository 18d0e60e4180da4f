// Out-degrees of a CSR's columns: deg_out[j] = #{e : col_idx[e] = j}.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", appendix D.4: degrees are computed once per graph and
// cached with it; the out-degree serves the right and symmetric
// normalisations and the transposed CSR of the backward passes.
//
// The plain way, one device-scope atomic add per entry, runs at about 27 G
// atomics/s on MI355X whatever the degree distribution (agent-scope atomics
// are carried out past the XCD's L2), i.e. ~0.6 ms for 16 M entries.  Here
// the counting happens in LDS instead, after a partition by column range:
//   1. per segment of entries, an LDS histogram of the column buckets
//      (bucket = column >> shift, at most 4096 buckets);
//   2. an exclusive scan of those counts, bucket-major, gives every
//      (bucket, segment) pair its output range;
//   3. each segment writes the low `shift` bits of its columns into its
//      ranges (16 bits per entry; the order inside a bucket is irrelevant);
//   4. one workgroup per bucket (several for a bucket much longer than the
//      average) counts the bucket's columns in an LDS histogram and stores
//      the bucket's degrees; only the parts of a split bucket add theirs
//      atomically, one atomic per non-zero column per part.
// About 7 bytes of HBM traffic per entry and no contended atomics.  Small
// graphs (launch latency dominates) and graphs with more than 2^26 columns
// (the buckets no longer fit the LDS histogram) take the atomic kernel.
// Entries whose column lies outside [0, n_cols) are not counted.
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int kMaxBuckets = 4096;
constexpr int kMinShift = 4;
constexpr int kMaxShift = 14;           // 16384 columns per bucket: 64 KB of LDS counters
constexpr int kSegThreads = 512;        // partition kernels
constexpr int kHistThreads = 512;       // per-bucket histogram kernel
constexpr int64_t kAtomicBelow = 1 << 18;  // entries: below this, the atomic kernel

__global__ void k_deg_out_atomic(const int32_t* col_idx, int64_t nnz, int32_t n_cols, int32_t* deg_out) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; e < nnz; e += stride) {
    const int32_t c = col_idx[e];
    if ((uint32_t)c < (uint32_t)n_cols) atomicAdd(&deg_out[c], 1);
  }
}

// h[v] += 1 for every lane's v.  A column with a large in-degree fills many
// lanes of a wave with the same value, and same-address LDS atomics are
// serialised: lanes sharing the first pending lane's value add once, by
// their count, for as long as such a value is shared by two lanes or more
// (at most three rounds); the rest add one each.
__device__ __forceinline__ void wave_hist_add(int32_t* h, uint32_t v, bool valid) {
  bool pending = valid;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const unsigned long long act = __ballot(pending);
    if (!act) return;
    const int src = __ffsll((long long)act) - 1;
    const uint32_t u = (uint32_t)__builtin_amdgcn_readlane((int)v, src);
    const unsigned long long same = __ballot(pending && v == u);
    const int k = __popcll(same);
    if (k < 2) break;
    if ((int)(threadIdx.x & 63) == src) atomicAdd(&h[u], k);
    pending = pending && v != u;
  }
  if (pending) atomicAdd(&h[v], 1);
}

// Visit the columns of entries [e0, e1): f4(c) with four consecutive columns
// (an int4) over the 16-byte aligned middle when col_idx is 16-byte aligned
// (e0 is a multiple of 4 in every caller), four loads in flight per thread;
// f(c) with single columns otherwise.
template <typename Fn, typename Fn4>
__device__ __forceinline__ void for_each_col(const int32_t* col, int64_t e0, int64_t e1, bool vec, Fn&& f,
                                             Fn4&& f4) {
  int64_t e = e0;
  if (vec) {
    const int64_t step = 16 * (int64_t)blockDim.x;
    for (; e + step <= e1; e += step) {
      int4 c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        c[k] = *reinterpret_cast<const int4*>(col + e + 4 * ((int64_t)threadIdx.x + (int64_t)k * blockDim.x));
#pragma unroll
      for (int k = 0; k < 4; ++k) f4(c[k]);
    }
  }
  for (e += threadIdx.x; e < e1; e += blockDim.x) f(col[e]);
}

// cnt[b * G + g] = entries of segment g whose column falls in bucket b.
__global__ __launch_bounds__(kSegThreads) void k_dego_count(const int32_t* col, int64_t nnz, int32_t n_cols,
                                                            int shift, int nb, int64_t seg, bool vec,
                                                            int32_t* cnt) {
  __shared__ int32_t h[kMaxBuckets];
  for (int b = threadIdx.x; b < nb; b += blockDim.x) h[b] = 0;
  __syncthreads();
  const int64_t g = blockIdx.x, G = gridDim.x;
  const int64_t e0 = g * seg, e1 = std::min(nnz, e0 + seg);
  // consecutive entries often share a bucket (a row's sources in one
  // cluster, sorted columns): four equal buckets add once
  auto one = [&](int32_t c) {
    if ((uint32_t)c < (uint32_t)n_cols) atomicAdd(&h[(uint32_t)c >> shift], 1);
  };
  for_each_col(col, e0, e1, vec, one, [&](int4 c) {
    const uint32_t b = (uint32_t)c.x >> shift;
    const uint32_t nc = (uint32_t)n_cols;
    if ((uint32_t)c.x < nc && (uint32_t)c.y < nc && (uint32_t)c.z < nc && (uint32_t)c.w < nc &&
        ((uint32_t)c.y >> shift) == b && ((uint32_t)c.z >> shift) == b && ((uint32_t)c.w >> shift) == b) {
      atomicAdd(&h[b], 4);
    } else {
      one(c.x);
      one(c.y);
      one(c.z);
      one(c.w);
    }
  });
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x) cnt[(int64_t)b * G + g] = h[b];
}

// Segment g writes the low bits of its columns into bucket b's range from
// off[b * G + g] on.  The segment is taken kSub entries at a time: the
// entries are ranked within their bucket in LDS, staged in bucket order, and
// written out in that order, so that a wave's stores fall into one or two
// runs of consecutive positions instead of 64 scattered ones.
constexpr int kSub = 8192;                 // entries per staging round
constexpr int kPer = kSub / kSegThreads;   // 16 per thread

// Block exclusive scan in place over v[0..nb) (nb <= 4096), v[nb] = total.
__device__ void block_scan_buckets(int32_t* v, int nb, int32_t* wsum) {
  constexpr int PER = kMaxBuckets / kSegThreads;  // 8
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int x[PER];
  int s = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = t * PER + k;
    x[k] = b < nb ? v[b] : 0;
    s += x[k];
  }
  int inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int run = inc - s, total = 0;
#pragma unroll
  for (int w = 0; w < kSegThreads / 64; ++w) {
    run += (w < wave) ? wsum[w] : 0;
    total += wsum[w];
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = t * PER + k;
    if (b < nb) v[b] = run;
    run += x[k];
  }
  if (t == 0) v[nb] = total;
}

__global__ __launch_bounds__(kSegThreads, 4) void k_dego_scatter(const int32_t* col, int64_t nnz, int32_t n_cols,
                                                              int shift, int nb, int64_t seg, bool vec,
                                                              const int32_t* off, uint16_t* low) {
  __shared__ int32_t cur[kMaxBuckets];       // next global position per bucket
  __shared__ int32_t lst[kMaxBuckets + 1];   // round: counts, then exclusive starts
  __shared__ uint32_t stage[kSub];           // (bucket << 16) | low bits, in bucket order
  __shared__ int32_t wsum[kSegThreads / 64];
  const int t = threadIdx.x;
  const int64_t g = blockIdx.x, G = gridDim.x;
  for (int b = t; b < nb; b += kSegThreads) cur[b] = off[(int64_t)b * G + g];
  const int64_t e0 = g * seg, e1 = std::min(nnz, e0 + seg);
  const uint32_t mask = (1u << shift) - 1;
  for (int64_t r0 = e0; r0 < e1; r0 += kSub) {
    const int64_t n_r = std::min<int64_t>(kSub, e1 - r0);
    for (int b = t; b < nb; b += kSegThreads) lst[b] = 0;
    __syncthreads();
    int c[kPer], rank[kPer];
    if (vec && n_r == kSub) {
#pragma unroll
      for (int k = 0; k < kPer / 4; ++k) {
        const int4 q = *reinterpret_cast<const int4*>(col + r0 + 4 * (t + k * kSegThreads));
        c[4 * k] = q.x;
        c[4 * k + 1] = q.y;
        c[4 * k + 2] = q.z;
        c[4 * k + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int64_t i = t + (int64_t)k * kSegThreads;
        c[k] = i < n_r ? col[r0 + i] : -1;
      }
    }
    // ranks within the bucket; four consecutive entries of one bucket (the
    // groups of a 16-byte load) take four ranks from one atomic
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const uint32_t b = (uint32_t)c[4 * q] >> shift;
      bool four = vec && n_r == kSub;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        four = four && (uint32_t)c[4 * q + j] < (uint32_t)n_cols && ((uint32_t)c[4 * q + j] >> shift) == b;
      if (four) {
        const int base = atomicAdd(&lst[b], 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) rank[4 * q + j] = base + j;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t cj = (uint32_t)c[4 * q + j];
          rank[4 * q + j] = cj < (uint32_t)n_cols ? atomicAdd(&lst[cj >> shift], 1) : -1;
        }
      }
    }
    __syncthreads();
    block_scan_buckets(lst, nb, wsum);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (rank[k] >= 0) {
        const uint32_t b = (uint32_t)c[k] >> shift;
        stage[lst[b] + rank[k]] = (b << 16) | ((uint32_t)c[k] & mask);
      }
    __syncthreads();
    const int total = lst[nb];
    for (int i = t; i < total; i += kSegThreads) {
      const uint32_t v = stage[i];
      const int b = (int)(v >> 16);
      low[cur[b] + (i - lst[b])] = (uint16_t)(v & 0xffffu);
    }
    __syncthreads();
    for (int b = t; b < nb; b += kSegThreads) cur[b] += lst[b + 1] - lst[b];
    __syncthreads();
  }
}

// Parts per bucket: one, or one per seg3 entries of a longer bucket;
// part_off = their exclusive scan (part_off[nb] = the number of parts), and
// part_bucket[q] = the bucket of part q.  One workgroup of 1024 threads,
// nb <= 4096.
__global__ __launch_bounds__(1024) void k_dego_parts(const int32_t* off, int64_t G, int nb, int64_t seg3,
                                                     int32_t* part_off, int32_t* part_bucket) {
  __shared__ int32_t ws[16];
  constexpr int PER = kMaxBuckets / 1024;
  int v[PER];
  int s = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = threadIdx.x * PER + k;
    int parts = 0;
    if (b < nb) {
      const int64_t len = (int64_t)off[(int64_t)(b + 1) * G] - off[(int64_t)b * G];
      parts = (int)std::max<int64_t>(1, (len + seg3 - 1) / seg3);
    }
    v[k] = parts;
    s += parts;
  }
  // block exclusive scan of s
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    before += (w < wave) ? ws[w] : 0;
    total += ws[w];
  }
  int run = before + inc - s;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = threadIdx.x * PER + k;
    if (b < nb) {
      part_off[b] = run;
      for (int j = 0; j < v[k]; ++j) part_bucket[run + j] = b;
    }
    run += v[k];
  }
  if (threadIdx.x == 0) part_off[nb] = total;
}

// Workgroup g takes part p of bucket b (part_off[b] <= g < part_off[b + 1]):
// entries [start + p * seg3, ...) of the bucket's range, counted in LDS.
// Dynamic LDS: 4 << shift bytes.
__global__ __launch_bounds__(kHistThreads) void k_dego_hist(const uint16_t* low, const int32_t* off, int64_t G,
                                                            const int32_t* part_off, const int32_t* part_bucket,
                                                            int nb, int shift, int64_t seg3, int32_t n_cols,
                                                            int32_t* deg_out) {
  extern __shared__ int32_t h[];
  const int g = blockIdx.x;
  if (g >= part_off[nb]) return;
  const int b = part_bucket[g], p = g - part_off[b], np = part_off[b + 1] - part_off[b];
  const int W = 1 << shift;
  for (int t = threadIdx.x; t < W; t += blockDim.x) h[t] = 0;
  __syncthreads();
  const int64_t s0 = off[(int64_t)b * G], s1 = off[(int64_t)(b + 1) * G];
  const int64_t a = s0 + (int64_t)p * seg3, z = std::min(s1, a + seg3);
  // 16-byte loads of 8 entries over the aligned middle, two in flight; the
  // unaligned head and tail (fewer than 8 entries each) one per lane
  const int64_t a8 = std::min(z, (a + 7) & ~(int64_t)7), z8 = std::max(a8, z & ~(int64_t)7);
  for (int64_t e = a; e < a8; e += blockDim.x) {
    const int64_t i = e + threadIdx.x;
    wave_hist_add(h, i < a8 ? low[i] : 0u, i < a8);
  }
  for (int64_t e = z8; e < z; e += blockDim.x) {
    const int64_t i = e + threadIdx.x;
    wave_hist_add(h, i < z ? low[i] : 0u, i < z);
  }
  constexpr int64_t kStep = 8 * kHistThreads;
  for (int64_t base = a8; base < z8; base += 2 * kStep) {
    const int64_t e = base + 8 * (int64_t)threadIdx.x;
    uint4 q[2] = {};
    const bool ok0 = e < z8, ok1 = e + kStep < z8;
    if (ok0) q[0] = *reinterpret_cast<const uint4*>(low + e);
    if (ok1) q[1] = *reinterpret_cast<const uint4*>(low + e + kStep);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool ok = k ? ok1 : ok0;
      const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wave_hist_add(h, w[j] & 0xffffu, ok);
        wave_hist_add(h, w[j] >> 16, ok);
      }
    }
  }
  __syncthreads();
  const int64_t c0 = (int64_t)b << shift;
  const int cw = (int)std::min<int64_t>(W, n_cols - c0);
  if (np == 1) {
    for (int t = threadIdx.x; t < cw; t += blockDim.x) deg_out[c0 + t] = h[t];
  } else {
    for (int t = threadIdx.x; t < cw; t += blockDim.x)
      if (h[t]) atomicAdd(&deg_out[c0 + t], h[t]);
  }
}

int ceil_log2(int64_t v) {
  int k = 0;
  while (((int64_t)1 << k) < v) ++k;
  return k;
}

}  // namespace

int count_out_degrees(const int32_t* col_idx, int64_t nnz, int32_t n_cols, int32_t* deg_out, hipStream_t s) {
  if (n_cols <= 0) return GNN_OK;
  GNN_HIP(hipMemsetAsync(deg_out, 0, (size_t)n_cols * 4, s));
  if (nnz <= 0) return GNN_OK;
  // about 1024 buckets; wider ones (at most 2^14 columns) past 2^24 columns
  const int shift = std::min(kMaxShift, std::max(kMinShift, ceil_log2(n_cols) - 10));
  const int64_t nb64 = ((int64_t)n_cols + (1 << shift) - 1) >> shift;
  if (nnz < kAtomicBelow || nb64 > kMaxBuckets) {
    const int64_t blocks = std::min<int64_t>((nnz + 255) / 256, 65536);
    hipLaunchKernelGGL(k_deg_out_atomic, dim3((unsigned)blocks), dim3(256), 0, s, col_idx, nnz, n_cols, deg_out);
    GNN_LAUNCH_CHECK("deg_out");
    return GNN_OK;
  }
  const int nb = (int)nb64;
  // segments of at least 32 entries per bucket, so the count table stays
  // below nnz / 32 entries
  const int64_t seg = std::max<int64_t>(32768, ((int64_t)nb * 32 + kSub - 1) / kSub * kSub);
  const int64_t G = (nnz + seg - 1) / seg;
  const int64_t ncnt = (int64_t)nb * G;
  // a bucket is split only when it is more than 4x the average length
  const int64_t seg3 = std::max<int64_t>(16384, 4 * ((nnz + nb - 1) / nb));
  const int64_t max_parts = nb + (nnz + seg3 - 1) / seg3;
  const bool vec = (reinterpret_cast<uintptr_t>(col_idx) & 15) == 0;

  StreamTemps tt(s);
  int32_t *cnt = nullptr, *off = nullptr, *part_off = nullptr, *part_bucket = nullptr;
  uint16_t* low = nullptr;
  GNN_TRY(tt.get(&cnt, (size_t)ncnt * 4));
  GNN_TRY(tt.get(&off, (size_t)(ncnt + 1) * 4));
  GNN_TRY(tt.get(&part_off, (size_t)(nb + 1) * 4));
  GNN_TRY(tt.get(&part_bucket, (size_t)max_parts * 4));
  GNN_TRY(tt.get(&low, (size_t)nnz * 2));
  hipLaunchKernelGGL(k_dego_count, dim3((unsigned)G), dim3(kSegThreads), 0, s, col_idx, nnz, n_cols, shift, nb, seg,
                     vec, cnt);
  GNN_LAUNCH_CHECK("deg_out: bucket counts");
  GNN_TRY(exclusive_scan_i32(cnt, off, ncnt, s));
  hipLaunchKernelGGL(k_dego_scatter, dim3((unsigned)G), dim3(kSegThreads), 0, s, col_idx, nnz, n_cols, shift, nb,
                     seg, vec, off, low);
  GNN_LAUNCH_CHECK("deg_out: partition");
  hipLaunchKernelGGL(k_dego_parts, dim3(1), dim3(1024), 0, s, off, G, nb, seg3, part_off, part_bucket);
  GNN_LAUNCH_CHECK("deg_out: parts");
  hipLaunchKernelGGL(k_dego_hist, dim3((unsigned)max_parts), dim3(kHistThreads), (size_t)4 << shift, s, low, off, G,
                     part_off, part_bucket, nb, shift, seg3, n_cols, deg_out);
  GNN_LAUNCH_CHECK("deg_out: bucket histograms");
  return tt.release();
}

}  // namespace gnn
