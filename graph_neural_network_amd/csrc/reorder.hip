// Vertex reordering on the GPU: degree sort and reverse Cuthill-McKee, and the
// relabelled CSR P A P^T.
//
// Fomina et al., "On efficient scaling of GNNs via IO-aware layer
// implementations", section 2.4 and the reordering discussion of section 4:
// a permutation that places co-accessed vertices close together helps
// gather-dominated (neighbour-parallel) kernels.  RCM is named in Tang et
// al., "A High-Throughput Solver for Marginalized Graph Kernels on GPU",
// section on graph reordering, as the bandwidth-reduction heuristic; its
// steps are the textbook Cuthill-McKee ones.
//
// Degree sort: perm sorts vertices by descending row length, ties by
// ascending id; one stable radix sort of ((maxdeg - deg) << idbits | id) on
// the degree bits only.
//
// RCM (readings fixed where the pages are silent): symmetrised pattern
// A u A^T without self loops; delta(v) its degree; every connected component
// is started at its vertex of smallest (delta, id), components taken in that
// order; a FIFO breadth-first search appends each popped vertex's unvisited
// neighbours in increasing (delta, id); the visit order is reversed.
// Level-synchronous form computed here, which yields exactly that order:
//   - rank(v) = position of v in the global (delta, id) order; adjacency lists
//     sorted by rank;
//   - component label = smallest rank in the component (union-find over
//     ranks, each root hooked under the smaller one);
//   - all components advance together, one BFS level per step: every
//     unvisited neighbour of level L is claimed by its earliest parent
//     (atomicMin of the parent's position in level L) and emitted in the
//     parent's rank-sorted adjacency order, so level L+1 is grouped by parent
//     in parent order, as the queue would produce it;
//   - a stable sort of the concatenated levels by component label gives
//     (component, level, position) order = the queue order; then reverse.
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

unsigned nb(int64_t n) { return (unsigned)((n + 255) / 256); }

int bits_for(int64_t v) {
  int b = 1;
  while ((1ll << b) <= v) ++b;
  return b;
}

// ---- segment of an entry ----
// Kernels over the entries of a segmented array (CSR rows, a frontier's
// flattened adjacency) need each entry's segment: the largest k with
// ptr[k] <= e.  A workgroup takes kSegSpan consecutive entries, finds the
// segments of its first and last entry in global memory once, stages the
// offsets between them in LDS and searches there (entries are not looked up
// one by one across the whole offset array: that is ~24 dependent loads on a
// 16M-row graph).  A span over more than kSegCap segments (many empty ones)
// searches global memory, bounded by the same two segments.
constexpr int kSegEPT = 8;              // entries per thread
constexpr int kSegSpan = 256 * kSegEPT; // entries per workgroup of 256
constexpr int kSegCap = 4096;           // staged offsets

unsigned nb_seg(int64_t n) { return (unsigned)((n + kSegSpan - 1) / kSegSpan); }

// largest k in [lo, hi] with ptr[k] <= e, given ptr[lo] <= e
__device__ __forceinline__ int seg_search(const int32_t* ptr, int lo, int hi, int64_t e) {
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ptr[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// This workgroup's entries [e0, e1] (of n) and their segments [r0, r1] (of
// nseg); the offsets ptr[r0 .. r1 + 1] are staged in s_ptr (kSegCap + 1
// words) when r1 - r0 < kSegCap.
struct SegSpan {
  int64_t e0, e1;
  int r0, r1;
};

// Called by every thread of the workgroup (s_r: two words of LDS).
__device__ __forceinline__ SegSpan seg_stage(const int32_t* ptr, int32_t nseg, int64_t n, int32_t* s_ptr,
                                             int32_t* s_r) {
  SegSpan sp;
  sp.e0 = (int64_t)blockIdx.x * kSegSpan;
  sp.e1 = min(n, sp.e0 + kSegSpan) - 1;
  if (threadIdx.x < 2) s_r[threadIdx.x] = seg_search(ptr, 0, nseg - 1, threadIdx.x == 0 ? sp.e0 : sp.e1);
  __syncthreads();
  sp.r0 = s_r[0];
  sp.r1 = s_r[1];
  const int cnt = sp.r1 - sp.r0 + 1;
  if (cnt <= kSegCap)
    for (int i = threadIdx.x; i <= cnt; i += blockDim.x) s_ptr[i] = ptr[sp.r0 + i];
  __syncthreads();
  return sp;
}

// j-th entry of this thread in the span (-1 past its end)
__device__ __forceinline__ int64_t seg_entry(const SegSpan& sp, int j) {
  const int64_t e = sp.e0 + (int64_t)j * blockDim.x + threadIdx.x;
  return e <= sp.e1 ? e : -1;
}

__device__ __forceinline__ int seg_find(const int32_t* ptr, const int32_t* s_ptr, const SegSpan& sp, int64_t e) {
  if (sp.r1 - sp.r0 + 1 > kSegCap) return seg_search(ptr, sp.r0, sp.r1, e);
  return sp.r0 + seg_search(s_ptr, 0, sp.r1 - sp.r0, e);
}

// ptr[k] for k in [r0, r1 + 1]
__device__ __forceinline__ int seg_at(const int32_t* ptr, const int32_t* s_ptr, const SegSpan& sp, int k) {
  return sp.r1 - sp.r0 + 1 > kSegCap ? ptr[k] : s_ptr[k - sp.r0];
}

// ---- compaction of a span's kept entries ----
// A counting pass stores, per wave and round of its span, the ballot of kept
// entries (words in entry order) and the span's count; after a scan of the
// counts, a writing pass places each kept entry at its span's offset plus
// the kept entries before it.  No flag or position per entry goes through
// memory.
constexpr int kSpanWords = kSegEPT * 4;  // ballot words per span (4 waves)

// this wave's ballot of round j into the span's words kw; c counts them
__device__ __forceinline__ void span_keep(bool kept, unsigned long long* kw, int j, int& c) {
  const unsigned long long b = __ballot(kept);
  if ((threadIdx.x & 63) == 0) kw[j * 4 + (threadIdx.x >> 6)] = b;
  c += __popcll(b);
}

// the span's count; every thread calls (s_c: four words of LDS)
__device__ __forceinline__ void span_count(int c, int32_t* s_c, int32_t* cnt) {
  if ((threadIdx.x & 63) == 0) s_c[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cnt[blockIdx.x] = s_c[0] + s_c[1] + s_c[2] + s_c[3];
}

// s_pre[w] = kept entries before ballot word w of the span; every thread calls
__device__ __forceinline__ void span_prefix(const unsigned long long* kw, int32_t* s_pre) {
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const int c = t < kSpanWords ? __popcll(kw[t]) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (t >= o) incl += v;
    }
    if (t < kSpanWords) s_pre[t] = incl - c;
  }
  __syncthreads();
}

// whether this lane's entry of round j is kept, and if so its output position
__device__ __forceinline__ bool span_pos(const unsigned long long* kw, const int32_t* s_pre, int j, int base,
                                         int& pos) {
  const int lane = threadIdx.x & 63, w = j * 4 + (threadIdx.x >> 6);
  const unsigned long long b = kw[w];
  if (!((b >> lane) & 1ull)) return false;
  pos = base + s_pre[w] + __popcll(b & (lane ? (~0ull >> (64 - lane)) : 0ull));
  return true;
}

// Largest row length: a grid-stride walk, one atomic per workgroup (one per
// wave serialises 250k atomics on one word for a 16M-row graph).
__global__ __launch_bounds__(256) void k_max_deg(const int32_t* row_ptr, int32_t n, int32_t* out) {
  __shared__ int32_t s_m[4];
  int d = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    d = max(d, row_ptr[i + 1] - row_ptr[i]);
  for (int o = 32; o >= 1; o >>= 1) d = max(d, __shfl_xor(d, o));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = d;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, max(max(s_m[0], s_m[1]), max(s_m[2], s_m[3])));
}

// ---- segmented sort of 32-bit values ----
// Sorts every segment [ptr[k], ptr[k+1]) of `in` ascending into the same
// positions of `out` (equal values are interchangeable: their order is not
// kept).  Four tiers by segment length L:
//   L <= kSortSmall: each value counts the smaller values of its segment and
//     the equal ones before it, which is its place;
//   L <= kSortWave: one wave per segment, bitonic sort in registers (the
//     four waves of a workgroup sort four segments, without LDS or barriers);
//   L <= kSortBlock: one workgroup per segment, bitonic sort in LDS;
//   longer: (long-segment index, value) keys through the global radix sort,
//     written back segment by segment.
// The rows of a CSR or an adjacency are already grouped, so this replaces a
// radix sort of (row, value) keys over all entries.
constexpr int kSortSmall = 16;
constexpr int kSortWave = 1024;
constexpr int kSortBlock = 4096;
constexpr int kSortBlocks = 4096;  // workgroups striding over the medium segments
constexpr int kClassPer = 8;       // segments per thread when classifying

__global__ __launch_bounds__(256) void k_sseg_small(const uint32_t* in, uint32_t* out, const int32_t* ptr,
                                                    int32_t nseg, int64_t n) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  const SegSpan sp = seg_stage(ptr, nseg, n, s_ptr, s_r);
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t e = seg_entry(sp, j);
    if (e < 0) break;
    const int k = seg_find(ptr, s_ptr, sp, e);
    const int b = seg_at(ptr, s_ptr, sp, k);
    const int len = seg_at(ptr, s_ptr, sp, k + 1) - b;
    if (len > kSortSmall) continue;
    const uint32_t x = in[e];
    const int me = (int)(e - b);
    int rank = 0;
    for (int t = 0; t < len; ++t) {
      const uint32_t y = in[b + t];
      rank += (y < x || (y == x && t < me)) ? 1 : 0;
    }
    out[b + rank] = x;
  }
}

// Lists the wave-sorted segments (wmid), the workgroup-sorted ones (mid) and
// the long ones (big, with lengths); cnt = {mid count, long count, entries of
// long segments, wmid count}.  Positions in the lists are reserved with one
// global atomic per list and workgroup.
__global__ __launch_bounds__(256) void k_sseg_classify(const int32_t* ptr, int32_t nseg, int32_t* mid,
                                                       int32_t* big, int32_t* big_len, int32_t* wmid,
                                                       int32_t* cnt) {
  __shared__ int32_t s_n[3], s_base[3], s_tot;
  if (threadIdx.x < 3) s_n[threadIdx.x] = 0;
  if (threadIdx.x == 0) s_tot = 0;
  __syncthreads();
  int cls[kClassPer], pos[kClassPer], len[kClassPer];
  const int64_t k0 = (int64_t)blockIdx.x * 256 * kClassPer + threadIdx.x;
#pragma unroll
  for (int j = 0; j < kClassPer; ++j) {
    const int64_t k = k0 + (int64_t)j * 256;
    len[j] = k < nseg ? ptr[k + 1] - ptr[k] : 0;
    cls[j] = len[j] > kSortBlock ? 2 : (len[j] > kSortWave ? 1 : (len[j] > kSortSmall ? 3 : 0));
    pos[j] = cls[j] ? atomicAdd(&s_n[cls[j] - 1], 1) : 0;
    if (cls[j] == 2) atomicAdd(&s_tot, len[j]);
  }
  __syncthreads();
  if (threadIdx.x < 3 && s_n[threadIdx.x] > 0)
    s_base[threadIdx.x] = atomicAdd(&cnt[threadIdx.x == 2 ? 3 : threadIdx.x], s_n[threadIdx.x]);
  if (threadIdx.x == 0 && s_tot > 0) atomicAdd(&cnt[2], s_tot);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kClassPer; ++j) {
    const int k = (int)(k0 + (int64_t)j * 256);
    if (cls[j] == 1) mid[s_base[0] + pos[j]] = k;
    if (cls[j] == 2) {
      big[s_base[1] + pos[j]] = k;
      big_len[s_base[1] + pos[j]] = len[j];
    }
    if (cls[j] == 3) wmid[s_base[2] + pos[j]] = k;
  }
}

// Bitonic sorting network over values held in registers by one wave: the
// wave holds positions t0 .. t0 + 64 R - 1, position t0 + t in slot t / 64
// of lane t % 64.  A compare-exchange of positions t and t ^ j (j < 64 R)
// pairs two slots of one lane when j >= 64 and two lanes' equal slots
// otherwise (one lane swap), so no stage touches LDS.  Each stage sorts
// ascending where position & k is 0.  Fully unrolled: slots are registers.
template <int R, int J>
__device__ __forceinline__ void regs_stage(uint32_t (&v)[R], int lane, int t0, int k) {
  if constexpr (J >= 64) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      constexpr int dr = J >> 6;
      if ((r ^ dr) > r) {
        const bool up = ((t0 + r * 64) & k) == 0;  // k > J >= 64: the same for every lane
        const uint32_t x = v[r], y = v[r ^ dr];
        v[r] = up ? min(x, y) : max(x, y);
        v[r ^ dr] = up ? max(x, y) : min(x, y);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t y = __shfl_xor(v[r], J, 64);
      const bool up = ((t0 + r * 64 + lane) & k) == 0;
      const bool lower = (lane & J) == 0;
      v[r] = (lower == up) ? min(v[r], y) : max(v[r], y);
    }
  }
}

// stages J, J / 2, ..., 1 of merge step k
template <int R, int J>
__device__ __forceinline__ void regs_merge(uint32_t (&v)[R], int lane, int t0, int k) {
  regs_stage<R, J>(v, lane, t0, k);
  if constexpr (J > 1) regs_merge<R, J / 2>(v, lane, t0, k);
}

// merge steps K, 2 K, ..., 64 R: the wave's positions end sorted (ascending
// or descending by bit 64 R of t0, as the network needs)
template <int R, int K>
__device__ __forceinline__ void regs_sort_from(uint32_t (&v)[R], int lane, int t0) {
  regs_merge<R, K / 2>(v, lane, t0, K);
  if constexpr (K < 64 * R) regs_sort_from<R, 2 * K>(v, lane, t0);
}

template <int R>
__device__ __forceinline__ void wave_sort_regs(uint32_t (&v)[R], int lane, int t0 = 0) {
  regs_sort_from<R, 2>(v, lane, t0);
}

template <int R>
__device__ __forceinline__ void wave_sort_segment(const uint32_t* in, uint32_t* out, int b, int len, int lane) {
  uint32_t v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = r * 64 + lane;
    v[r] = t < len ? in[b + t] : 0xFFFFFFFFu;
  }
  wave_sort_regs<R>(v, lane, 0);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = r * 64 + lane;
    if (t < len) out[b + t] = v[r];
  }
}

// One segment per wave, waves striding over the list.
__global__ __launch_bounds__(256) void k_sseg_wave(const uint32_t* in, uint32_t* out, const int32_t* ptr,
                                                   const int32_t* wmid, const int32_t* cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = cnt[3];
  for (int i = blockIdx.x * 4 + wave; i < nw; i += gridDim.x * 4) {
    const int k = wmid[i];
    const int b = ptr[k], len = ptr[k + 1] - b;
    if (len <= 64) wave_sort_segment<1>(in, out, b, len, lane);
    else if (len <= 128) wave_sort_segment<2>(in, out, b, len, lane);
    else if (len <= 256) wave_sort_segment<4>(in, out, b, len, lane);
    else if (len <= 512) wave_sort_segment<8>(in, out, b, len, lane);
    else wave_sort_segment<16>(in, out, b, len, lane);
  }
}

// One segment of up to 4 x 64 R values per workgroup: each wave sorts its
// quarter in registers (directions from the positions in the whole segment),
// then every merge step of the whole runs its stages across quarters through
// LDS and the rest in registers.
template <int R>
__device__ __forceinline__ void block_sort_segment(const uint32_t* in, uint32_t* out, int b, int len,
                                                   uint32_t* sv) {
  constexpr int Q = 64 * R, P = 4 * Q;
  const int lane = threadIdx.x & 63, t0 = (threadIdx.x >> 6) * Q;
  uint32_t v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r * 64 + lane;
    v[r] = t < len ? in[b + t] : 0xFFFFFFFFu;
  }
  wave_sort_regs<R>(v, lane, t0);
  for (int k = 2 * Q; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= Q; j >>= 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) sv[t0 + r * 64 + lane] = v[r];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int t = t0 + r * 64 + lane;
        const uint32_t y = sv[t ^ j];
        v[r] = (((t & j) == 0) == ((t & k) == 0)) ? min(v[r], y) : max(v[r], y);
      }
      __syncthreads();
    }
    regs_merge<R, Q / 2>(v, lane, t0, k);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r * 64 + lane;
    if (t < len) out[b + t] = v[r];
  }
}

__global__ __launch_bounds__(256) void k_sseg_mid(const uint32_t* in, uint32_t* out, const int32_t* ptr,
                                                  const int32_t* mid, const int32_t* cnt) {
  __shared__ uint32_t sv[kSortBlock];
  const int nmid = cnt[0];
  for (int i = blockIdx.x; i < nmid; i += gridDim.x) {
    const int k = mid[i];
    const int b = ptr[k], len = ptr[k + 1] - b;
    if (len <= 2048) block_sort_segment<8>(in, out, b, len, sv);
    else block_sort_segment<16>(in, out, b, len, sv);
  }
}

// keys of long segment i (one workgroup per segment): (i << vbits) | value
__global__ __launch_bounds__(256) void k_sseg_big_keys(const uint32_t* in, const int32_t* ptr, const int32_t* big,
                                                       const int32_t* big_off, int vbits, uint64_t* keys) {
  const int i = blockIdx.x;
  const int b = ptr[big[i]], o = big_off[i], len = big_off[i + 1] - o;
  for (int t = threadIdx.x; t < len; t += blockDim.x)
    keys[(int64_t)o + t] = ((uint64_t)i << vbits) | in[b + t];
}

__global__ void k_sseg_big_out(const uint64_t* keys, int64_t nk, const int32_t* ptr, const int32_t* big,
                               const int32_t* big_off, int vbits, uint32_t* out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= nk) return;
  const uint64_t key = keys[q];
  const int i = (int)(key >> vbits);
  out[ptr[big[i]] + (q - big_off[i])] = (uint32_t)(key & ((1ull << vbits) - 1));
}

// Values are below vmax.  One host synchronisation (the long segments' entry
// count); temporaries are stream-ordered.
int segmented_sort_u32(const uint32_t* in, uint32_t* out, const int32_t* ptr, int32_t nseg, int64_t n,
                       uint32_t vmax, hipStream_t s) {
  if (n <= 0 || nseg <= 0) return GNN_OK;
  const int64_t big_max = std::min<int64_t>(nseg, n / (kSortBlock + 1) + 1);
  StreamTemps own(s);
  int32_t *cnt = nullptr, *mid = nullptr, *wmid = nullptr, *big = nullptr, *big_len = nullptr, *big_off = nullptr;
  GNN_TRY(own.get(&cnt, 16));
  GNN_TRY(own.get(&mid, (size_t)std::min<int64_t>(nseg, n / (kSortWave + 1) + 1) * 4));
  GNN_TRY(own.get(&wmid, (size_t)std::min<int64_t>(nseg, n / (kSortSmall + 1) + 1) * 4));
  GNN_TRY(own.get(&big, (size_t)big_max * 4));
  GNN_TRY(own.get(&big_len, (size_t)big_max * 4));
  GNN_TRY(own.get(&big_off, (size_t)(big_max + 1) * 4));
  GNN_HIP(hipMemsetAsync(cnt, 0, 16, s));
  const unsigned ncls = (unsigned)((nseg + 256 * kClassPer - 1) / (256 * kClassPer));
  hipLaunchKernelGGL(k_sseg_classify, dim3(ncls), dim3(256), 0, s, ptr, nseg, mid, big, big_len, wmid, cnt);
  GNN_LAUNCH_CHECK("segment classes");
  hipLaunchKernelGGL(k_sseg_small, dim3(nb_seg(n)), dim3(256), 0, s, in, out, ptr, nseg, n);
  GNN_LAUNCH_CHECK("short segments");
  hipLaunchKernelGGL(k_sseg_mid, dim3((unsigned)std::min<int64_t>(nseg, kSortBlocks)), dim3(256), 0, s, in, out,
                     ptr, mid, cnt);
  GNN_LAUNCH_CHECK("medium segments");
  hipLaunchKernelGGL(k_sseg_wave, dim3((unsigned)std::min<int64_t>((nseg + 3) / 4, 4 * kSortBlocks)), dim3(256), 0, s,
                     in, out, ptr, wmid, cnt);
  GNN_LAUNCH_CHECK("wave segments");
  int32_t hc[3] = {0, 0, 0};
  GNN_HIP(hipMemcpyAsync(hc, cnt, 12, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  const int32_t nbig = hc[1];
  const int64_t nk = hc[2];
  if (nbig < 0 || nbig > big_max || nk < 0 || nk > n) return fail(GNN_ERR_DEVICE, "segmented sort: bad counts");
  if (nbig > 0) {
    GNN_TRY(exclusive_scan_i32(big_len, big_off, nbig, s));
    const int vbits = bits_for((int64_t)std::max<uint32_t>(vmax, 1) - 1);
    const int ibits = bits_for(nbig - 1);
    if (vbits + ibits > 64) return fail(GNN_ERR_SIZE_OVERFLOW, "segmented sort keys exceed 64 bits");
    uint64_t *keys = nullptr, *tmp = nullptr;
    GNN_TRY(own.get(&keys, (size_t)nk * 8));
    GNN_TRY(own.get(&tmp, (size_t)nk * 8));
    hipLaunchKernelGGL(k_sseg_big_keys, dim3((unsigned)nbig), dim3(256), 0, s, in, ptr, big, big_off, vbits, keys);
    GNN_LAUNCH_CHECK("long segment keys");
    GNN_TRY(radix_sort_u64(keys, tmp, nk, 0, vbits + ibits, s));
    hipLaunchKernelGGL(k_sseg_big_out, dim3(nb(nk)), dim3(256), 0, s, keys, nk, ptr, big, big_off, vbits, out);
    GNN_LAUNCH_CHECK("long segments");
  }
  return own.release();
}

__global__ void k_deg_keys(const int32_t* row_ptr, int32_t n, int32_t maxdeg, int idbits,
                           uint64_t* keys) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int d = row_ptr[i + 1] - row_ptr[i];
  keys[i] = ((uint64_t)(maxdeg - d) << idbits) | (uint64_t)i;
}

__global__ void k_low_bits(const uint64_t* keys, int64_t n, int idbits, int32_t* out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (int32_t)(keys[i] & ((1ull << idbits) - 1));
}

// ---- relabelled CSR ----

__global__ void k_inverse(const int32_t* perm, int32_t n, int32_t* inv) {
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p < n) inv[perm[p]] = (int32_t)p;
}

__global__ void k_new_deg(const int32_t* row_ptr, const int32_t* perm, int32_t n, int32_t* deg) {
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p < n) deg[p] = row_ptr[perm[p] + 1] - row_ptr[perm[p]];
}

// new column of every entry of P A P^T, rows in their new places (the
// entries of new row p are those of old row perm[p], in their old order)
__global__ __launch_bounds__(256) void k_perm_cols(const int32_t* row_ptr, const int32_t* col_idx,
                                                   const int32_t* perm, const int32_t* inv,
                                                   const int32_t* new_ptr, int32_t n, int64_t nnz,
                                                   uint32_t* cols) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  const SegSpan sp = seg_stage(new_ptr, n, nnz, s_ptr, s_r);
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t q = seg_entry(sp, j);
    if (q < 0) break;
    const int p = seg_find(new_ptr, s_ptr, sp, q);
    const int64_t old_e = row_ptr[perm[p]] + (q - new_ptr[p]);
    cols[q] = (uint32_t)inv[col_idx[old_e]];
  }
}

// ---- RCM ----

// both directions of every non-loop edge, compacted: the counting pass keeps
// entries whose column is not their row, the writing pass emits the keys
__global__ __launch_bounds__(256) void k_loop_count(const int32_t* row_ptr, const int32_t* col_idx, int32_t n,
                                                    int64_t nnz, unsigned long long* keep, int32_t* cnt) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  __shared__ int32_t s_c[4];
  const SegSpan sp = seg_stage(row_ptr, n, nnz, s_ptr, s_r);
  int c = 0;
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t e = seg_entry(sp, j);
    const bool kept = e >= 0 && col_idx[e] != seg_find(row_ptr, s_ptr, sp, e);
    span_keep(kept, keep + (int64_t)blockIdx.x * kSpanWords, j, c);
  }
  span_count(c, s_c, cnt);
}

__global__ __launch_bounds__(256) void k_sym_keys(const int32_t* row_ptr, const int32_t* col_idx, int32_t n,
                                                  int64_t nnz, const unsigned long long* keep, const int32_t* off,
                                                  int idbits, uint64_t* keys) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  __shared__ int32_t s_pre[kSpanWords];
  const SegSpan sp = seg_stage(row_ptr, n, nnz, s_ptr, s_r);
  const unsigned long long* kw = keep + (int64_t)blockIdx.x * kSpanWords;
  span_prefix(kw, s_pre);
  const int base = off[blockIdx.x];
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t e = seg_entry(sp, j);
    int p;
    if (e < 0) break;
    if (!span_pos(kw, s_pre, j, base, p)) continue;
    const uint64_t i = (uint64_t)seg_find(row_ptr, s_ptr, sp, e), c = (uint64_t)col_idx[e];
    keys[2 * (int64_t)p] = (i << idbits) | c;
    keys[2 * (int64_t)p + 1] = (c << idbits) | i;
  }
}

// sorted keys: keep the first of each run of equal keys
__global__ __launch_bounds__(256) void k_uniq_count(const uint64_t* keys, int64_t m2, unsigned long long* keep,
                                                    int32_t* cnt) {
  __shared__ int32_t s_c[4];
  const int64_t e0 = (int64_t)blockIdx.x * kSegSpan;
  int c = 0;
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t e = e0 + (int64_t)j * blockDim.x + threadIdx.x;
    const bool kept = e < m2 && (e == 0 || keys[e] != keys[e - 1]);
    span_keep(kept, keep + (int64_t)blockIdx.x * kSpanWords, j, c);
  }
  span_count(c, s_c, cnt);
}

__global__ __launch_bounds__(256) void k_sym_fill(const uint64_t* keys, int64_t m2, const unsigned long long* keep,
                                                  const int32_t* off, int idbits, int32_t* adj, int32_t* adj_row) {
  __shared__ int32_t s_pre[kSpanWords];
  const unsigned long long* kw = keep + (int64_t)blockIdx.x * kSpanWords;
  span_prefix(kw, s_pre);
  const int64_t e0 = (int64_t)blockIdx.x * kSegSpan;
  const int base = off[blockIdx.x];
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t e = e0 + (int64_t)j * blockDim.x + threadIdx.x;
    int p;
    if (e >= m2) break;
    if (!span_pos(kw, s_pre, j, base, p)) continue;
    adj[p] = (int32_t)(keys[e] & ((1ull << idbits) - 1));
    adj_row[p] = (int32_t)(keys[e] >> idbits);
  }
}

// Row pointers of the symmetrised pattern: adj_row is sorted, so row r starts
// at the first entry not below r (a binary search per row; r = n gives m).
// Counting entries per row with atomics instead serialises on hub rows.
__global__ void k_row_bounds(const int32_t* adj_row, int64_t m, int32_t n, int32_t* sym_ptr) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r > n) return;
  int64_t lo = 0, hi = m;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (adj_row[mid] < r) lo = mid + 1;
    else hi = mid;
  }
  sym_ptr[r] = (int32_t)lo;
}

__global__ void k_rank_keys(const int32_t* sym_ptr, int32_t n, int idbits, uint64_t* keys) {
  int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n) return;
  keys[v] = ((uint64_t)(sym_ptr[v + 1] - sym_ptr[v]) << idbits) | (uint64_t)v;
}

__global__ void k_rank(const uint64_t* keys, int32_t n, int idbits, int32_t* order, int32_t* rank) {
  int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  const int v = (int)(keys[r] & ((1ull << idbits) - 1));
  order[r] = v;
  rank[v] = (int32_t)r;
}

__global__ void k_adj_ranks(const int32_t* adj, const int32_t* rank, int64_t m, uint32_t* rk) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m) return;
  rk[e] = (uint32_t)rank[adj[e]];
}

__global__ void k_adj_from_ranks(const uint32_t* rk, const int32_t* order, int64_t m, int32_t* adj) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m) return;
  adj[e] = order[rk[e]];
}

// ---- component labels: union-find over ranks ----
// P[r] is the parent of rank r, a root its own parent.  A hook only attaches
// a root under a smaller root, so every parent is smaller than its child, a
// tree's root is its smallest rank (the component's label) and every walk up
// a tree ends.  Parents are read with agent-scope atomic loads (past the
// per-CU cache); a stale read costs only a failed compare-and-swap, which
// returns the current parent to retry from.
__device__ __forceinline__ int uf_parent(const int32_t* P, int x) {
  return __hip_atomic_load(P + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Root of x, re-pointing each visited node to its grandparent (path halving):
// the grandparent is an ancestor in the same tree and smaller than the
// parent, so concurrent walks and hooks keep every tree valid.
__device__ int uf_root(int32_t* P, int x) {
  for (;;) {
    const int p = uf_parent(P, x);
    if (p == x) return x;
    const int g = uf_parent(P, p);
    if (g == p) return p;
    __hip_atomic_store(P + x, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    x = g;
  }
}

__global__ void k_iota(int32_t* p, int32_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = (int32_t)i;
}

// Joins the trees of ranks a and b: attaches the larger root under the
// smaller one.  A failed swap means that root was attached elsewhere
// meanwhile: the larger of the two roots strictly decreases with every retry.
__device__ void uf_hook(int32_t* P, int a, int b) {
  a = uf_root(P, a);
  b = uf_root(P, b);
  while (a != b) {
    if (a < b) {
      const int t = a;
      a = b;
      b = t;
    }
    const int old = atomicCAS(P + a, a, b);
    if (old == a) return;
    a = uf_root(P, old);
    b = uf_root(P, b);
  }
}

// Neighbour sampling (the components of most graphs are found from a few
// edges per vertex): every vertex with more than j neighbours is joined to
// its j-th one.
__global__ void k_cc_link_nth(const int32_t* sym_ptr, const int32_t* adj, const int32_t* rank, int32_t n, int j,
                              int32_t* P) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n) return;
  const int b = sym_ptr[v];
  if (sym_ptr[v + 1] - b > j) uf_hook(P, rank[v], rank[adj[b + j]]);
}

// Every rank points at its root (no hooks run meanwhile; concurrent walks
// may leave a few entries one step short, which only costs later walks).
__global__ void k_cc_compress(int32_t n, int32_t* P) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n) __hip_atomic_store(P + r, uf_root(P, (int)r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The most frequent root among 1024 spread sample ranks (one workgroup of
// 256): the component whose vertices skip the full pass.
__global__ __launch_bounds__(256) void k_cc_giant(int32_t n, int32_t* P, int32_t* giant) {
  __shared__ int32_t s_root[1024];
  __shared__ unsigned long long s_best;
  if (threadIdx.x == 0) s_best = 0;
  for (int i = threadIdx.x; i < 1024; i += 256)
    s_root[i] = uf_root(P, (int)(((uint64_t)i * 2654435761u) % (uint64_t)n));
  __syncthreads();
  for (int i = threadIdx.x; i < 1024; i += 256) {
    int c = 0;
    for (int t = 0; t < 1024; ++t) c += s_root[t] == s_root[i];
    atomicMax(&s_best, ((unsigned long long)c << 32) | (uint32_t)s_root[i]);
  }
  __syncthreads();
  if (threadIdx.x == 0) *giant = (int32_t)(uint32_t)s_best;
}

// skip[v] = v's tree is the sampled giant one
__global__ void k_cc_skip(const int32_t* rank, int32_t n, int32_t* P, const int32_t* giant, int32_t* skip) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v < n) skip[v] = uf_root(P, rank[v]) == *giant ? 1 : 0;
}

// Every entry (u, v) of a vertex outside the giant tree is hooked.  An edge
// between two giant-tree vertices joins vertices already in one tree; an
// edge with one end outside is hooked from that end (the pattern holds both
// directions).
__global__ void k_cc_hook(const int32_t* adj, const int32_t* adj_row, const int32_t* rank, const int32_t* skip,
                          int64_t m, int32_t* P) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m) return;
  const int u = adj_row[e];
  if (skip[u]) return;
  uf_hook(P, rank[u], rank[adj[e]]);
}

__global__ void k_cc_label(const int32_t* rank, int32_t n, int32_t* P, int32_t* label) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v < n) label[v] = uf_root(P, rank[v]);
}

__global__ void k_start_flags(const int32_t* order, const int32_t* label, int32_t n, int32_t* flag) {
  int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  flag[r] = (label[order[r]] == (int32_t)r) ? 1 : 0;
}

__global__ void k_start_fill(const int32_t* order, const int32_t* flag, const int32_t* pos, int32_t n,
                             int32_t* level, int32_t* claim) {
  int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n || !flag[r]) return;
  const int v = order[r];
  level[pos[r]] = v;
  claim[v] = -1;
}

// ---- one BFS level over the frontier's flattened adjacency ----
// Frontier edge q (0 <= q < E_f) belongs to frontier position k with
// eoff[k] <= q < eoff[k+1]; its target is adj[sym_ptr[front[k]] + q - eoff[k]].
// Edges are numbered in (frontier position, adjacency order), so emitting
// them in q order keeps the queue order.  claim[w] is -1 once w is visited,
// else the smallest frontier position claiming it (INT_MAX: none), so one
// word per vertex serves both tests.

__global__ void k_front_deg(const int32_t* front, int32_t f, const int32_t* sym_ptr, int32_t* deg) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < f) deg[k] = sym_ptr[front[k] + 1] - sym_ptr[front[k]];
}

__global__ __launch_bounds__(256) void k_claim(const int32_t* front, int32_t f, const int32_t* eoff,
                                               int64_t ef, const int32_t* sym_ptr, const int32_t* adj,
                                               int32_t* claim) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  const SegSpan sp = seg_stage(eoff, f, ef, s_ptr, s_r);
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t q = seg_entry(sp, j);
    if (q < 0) break;
    const int k = seg_find(eoff, s_ptr, sp, q);
    const int w = adj[sym_ptr[front[k]] + (q - eoff[k])];
    if (claim[w] > k) atomicMin(&claim[w], k);
  }
}

// Children of the level: frontier edge q keeps its target w when its
// frontier position k won w's claim; kept targets are compacted in q order.
__global__ __launch_bounds__(256) void k_child_count(const int32_t* front, int32_t f, const int32_t* eoff,
                                                     int64_t ef, const int32_t* sym_ptr, const int32_t* adj,
                                                     const int32_t* claim, unsigned long long* keep,
                                                     int32_t* cnt) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  __shared__ int32_t s_c[4];
  const SegSpan sp = seg_stage(eoff, f, ef, s_ptr, s_r);
  int c = 0;
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t q = seg_entry(sp, j);
    bool kept = false;
    if (q >= 0) {
      const int k = seg_find(eoff, s_ptr, sp, q);
      kept = claim[adj[sym_ptr[front[k]] + (q - eoff[k])]] == k;
    }
    span_keep(kept, keep + (int64_t)blockIdx.x * kSpanWords, j, c);
  }
  span_count(c, s_c, cnt);
}

__global__ __launch_bounds__(256) void k_child_emit(const int32_t* front, int32_t f, const int32_t* eoff,
                                                    int64_t ef, const int32_t* sym_ptr, const int32_t* adj,
                                                    const unsigned long long* keep, const int32_t* off,
                                                    int32_t* next) {
  __shared__ int32_t s_ptr[kSegCap + 1];
  __shared__ int32_t s_r[2];
  __shared__ int32_t s_pre[kSpanWords];
  const SegSpan sp = seg_stage(eoff, f, ef, s_ptr, s_r);
  const unsigned long long* kw = keep + (int64_t)blockIdx.x * kSpanWords;
  span_prefix(kw, s_pre);
  const int base = off[blockIdx.x];
  for (int j = 0; j < kSegEPT; ++j) {
    const int64_t q = seg_entry(sp, j);
    int p;
    if (q < 0) break;
    if (!span_pos(kw, s_pre, j, base, p)) continue;
    const int k = seg_find(eoff, s_ptr, sp, q);
    next[p] = adj[sym_ptr[front[k]] + (q - eoff[k])];
  }
}

__global__ void k_mark(const int32_t* next, int32_t f, int32_t* claim) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < f) claim[next[k]] = -1;
}

__global__ void k_final_keys(const int32_t* concat, const int32_t* label, int32_t n, int idbits,
                             uint64_t* keys) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  keys[i] = ((uint64_t)label[concat[i]] << idbits) | (uint64_t)i;
}

__global__ void k_final_perm(const uint64_t* keys, const int32_t* concat, int32_t n, int idbits,
                             int32_t* perm) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  perm[n - 1 - i] = concat[keys[i] & ((1ull << idbits) - 1)];
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------

size_t degree_bytes(int32_t n) {
  return Arena::round(4) + 2 * Arena::round((size_t)n * 8) + radix_scratch_bytes(n);
}

int degree_perm(const gnn_csr* c, int32_t* perm, Arena& ar, hipStream_t s) {
  const int32_t n = c->n_rows;
  int32_t* mx = ar.take<int32_t>(1);
  uint64_t* keys = ar.take<uint64_t>(n);
  uint64_t* tmp = ar.take<uint64_t>(n);
  void* ws = ar.base + ar.off;
  GNN_HIP(hipMemsetAsync(mx, 0, 4, s));
  hipLaunchKernelGGL(k_max_deg, dim3(std::min<unsigned>(nb(n), 2048)), dim3(256), 0, s, c->row_ptr, n, mx);
  GNN_LAUNCH_CHECK("max degree");
  int32_t maxdeg = 0;
  GNN_HIP(hipMemcpyAsync(&maxdeg, mx, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  const int idbits = bits_for(n);
  const int dbits = bits_for(maxdeg);
  if (idbits + dbits > 64) return fail(GNN_ERR_SIZE_OVERFLOW, "degree keys exceed 64 bits");
  hipLaunchKernelGGL(k_deg_keys, dim3(nb(n)), dim3(256), 0, s, c->row_ptr, n, maxdeg, idbits, keys);
  GNN_LAUNCH_CHECK("degree keys");
  GNN_TRY(radix_sort_u64(keys, tmp, n, idbits, idbits + dbits, s, ws));
  hipLaunchKernelGGL(k_low_bits, dim3(nb(n)), dim3(256), 0, s, keys, (int64_t)n, idbits, perm);
  GNN_LAUNCH_CHECK("degree perm");
  return GNN_OK;
}

// Temporaries of rcm_perm: two small slabs (per-span counts of kept entries
// and their offsets, one word per span of the 2 nnz symmetric entries), two
// key arrays, the symmetrised adjacency with its row ids, nine
// per-vertex arrays, and scan / sort scratch.
size_t rcm_bytes(int32_t n, int64_t nnz) {
  // key arrays: 2 nnz symmetric keys, n rank keys, the BFS's ballot words
  // (kSpanWords per span of frontier edges: at most 1/64 of them plus one span's)
  const int64_t M2 = std::max<int64_t>(2 * nnz, 1), NN = std::max<int64_t>({M2, (int64_t)n, 2 * kSpanWords});
  size_t b = 2 * Arena::round((size_t)(M2 / kSegSpan + 2) * 4) + 2 * Arena::round((size_t)NN * 8) +
             2 * Arena::round((size_t)M2 * 4) + 3 * Arena::round((size_t)(n + 1) * 4) +
             6 * Arena::round((size_t)n * 4);
  return b + std::max(scan_scratch_bytes(NN + 1), radix_scratch_bytes(NN));
}

int rcm_perm(const gnn_csr* c, int32_t* perm, Arena& ar, hipStream_t s) {
  const int32_t n = c->n_rows;
  const int64_t nnz = c->nnz;
  const int idbits = bits_for(n);
  if (2 * idbits > 64) return fail(GNN_ERR_SIZE_OVERFLOW, "RCM keys exceed 64 bits");
  // key arrays: 2 nnz symmetric keys, n rank keys, the BFS's ballot words
  // (kSpanWords per span of frontier edges: at most 1/64 of them plus one span's)
  const int64_t M2 = std::max<int64_t>(2 * nnz, 1), NN = std::max<int64_t>({M2, (int64_t)n, 2 * kSpanWords});
  int32_t* slab0 = ar.take<int32_t>(M2 / kSegSpan + 2);
  int32_t* slab1 = ar.take<int32_t>(M2 / kSegSpan + 2);
  uint64_t* keys = ar.take<uint64_t>(NN);
  uint64_t* tmp = ar.take<uint64_t>(NN);
  int32_t* adj = ar.take<int32_t>(M2);
  int32_t* adj_row = ar.take<int32_t>(M2);
  int32_t* sym_ptr = ar.take<int32_t>(n + 1);
  int32_t* ccnt = ar.take<int32_t>(n + 1);
  int32_t* coff = ar.take<int32_t>(n + 1);
  int32_t* order = ar.take<int32_t>(n);
  int32_t* rank = ar.take<int32_t>(n);
  int32_t* label = ar.take<int32_t>(n);
  int32_t* concat = ar.take<int32_t>(n);
  int32_t* skip = ar.take<int32_t>(n);
  int32_t* claim = ar.take<int32_t>(n);
  void* ws = ar.base + ar.off;  // scan and sort scratch

  // 1. symmetrised pattern without loops, as sorted unique (row, col) keys;
  // span counts and their offsets in the slabs, the spans' ballot words in
  // the second key array (free outside the sort)
  int32_t *cnt = slab0, *off = slab1;
  unsigned long long* keep = reinterpret_cast<unsigned long long*>(tmp);
  const unsigned nsp1 = nb_seg(nnz);
  if (nnz > 0) {
    hipLaunchKernelGGL(k_loop_count, dim3(nsp1), dim3(256), 0, s, c->row_ptr, c->col_idx, n, nnz, keep, cnt);
    GNN_LAUNCH_CHECK("rcm loop counts");
  }
  GNN_TRY(exclusive_scan_i32(cnt, off, nsp1, s, ws));
  int32_t nl = 0;
  GNN_HIP(hipMemcpyAsync(&nl, off + nsp1, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  const int64_t m2 = 2 * (int64_t)nl;
  if (m2 >= 0x7FFFFFFF) return fail(GNN_ERR_SIZE_OVERFLOW, "RCM: symmetrised pattern too large");
  if (nnz > 0) {
    hipLaunchKernelGGL(k_sym_keys, dim3(nsp1), dim3(256), 0, s, c->row_ptr, c->col_idx, n, nnz, keep, off,
                       idbits, keys);
    GNN_LAUNCH_CHECK("rcm sym keys");
  }
  GNN_TRY(radix_sort_u64(keys, tmp, m2, 0, 2 * idbits, s, ws));
  const unsigned nsp2 = nb_seg(m2);
  if (m2 > 0) {
    hipLaunchKernelGGL(k_uniq_count, dim3(nsp2), dim3(256), 0, s, keys, m2, keep, cnt);
    GNN_LAUNCH_CHECK("rcm unique");
  }
  GNN_TRY(exclusive_scan_i32(cnt, off, nsp2, s, ws));
  int32_t m32 = 0;
  GNN_HIP(hipMemcpyAsync(&m32, off + nsp2, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  const int64_t m = m32;  // entries of the symmetrised pattern
  if (m2 > 0) {
    hipLaunchKernelGGL(k_sym_fill, dim3(nsp2), dim3(256), 0, s, keys, m2, keep, off, idbits, adj, adj_row);
    GNN_LAUNCH_CHECK("rcm sym fill");
  }
  hipLaunchKernelGGL(k_row_bounds, dim3(nb((int64_t)n + 1)), dim3(256), 0, s, adj_row, m, n, sym_ptr);
  GNN_LAUNCH_CHECK("rcm row bounds");

  // 2. global (delta, id) order and ranks
  hipLaunchKernelGGL(k_rank_keys, dim3(nb(n)), dim3(256), 0, s, sym_ptr, n, idbits, keys);
  GNN_LAUNCH_CHECK("rcm rank keys");
  GNN_TRY(radix_sort_u64(keys, tmp, n, idbits, idbits + bits_for(m + 1), s, ws));
  hipLaunchKernelGGL(k_rank, dim3(nb(n)), dim3(256), 0, s, keys, n, idbits, order, rank);
  GNN_LAUNCH_CHECK("rcm rank");

  // 3. adjacency lists in rank order: each row's neighbour ranks sorted
  if (m > 0) {
    uint32_t* rk = reinterpret_cast<uint32_t*>(keys);
    uint32_t* rk_sorted = reinterpret_cast<uint32_t*>(tmp);
    hipLaunchKernelGGL(k_adj_ranks, dim3(nb(m)), dim3(256), 0, s, adj, rank, m, rk);
    GNN_LAUNCH_CHECK("rcm adj ranks");
    GNN_TRY(segmented_sort_u32(rk, rk_sorted, sym_ptr, n, m, (uint32_t)n, s));
    hipLaunchKernelGGL(k_adj_from_ranks, dim3(nb(m)), dim3(256), 0, s, rk_sorted, order, m, adj);
    GNN_LAUNCH_CHECK("rcm adj sort");
  }

  // 4. component labels: smallest rank in the component, by union-find over
  // ranks: two rounds of neighbour sampling, then every entry of the
  // vertices outside the sampled giant tree (the claim array holds the
  // parents)
  {
    int32_t* P = claim;
    hipLaunchKernelGGL(k_iota, dim3(nb(n)), dim3(256), 0, s, P, n);
    GNN_LAUNCH_CHECK("rcm parents");
    if (m > 0) {
      for (int j = 0; j < 2; ++j) {
        hipLaunchKernelGGL(k_cc_link_nth, dim3(nb(n)), dim3(256), 0, s, sym_ptr, adj, rank, n, j, P);
        hipLaunchKernelGGL(k_cc_compress, dim3(nb(n)), dim3(256), 0, s, n, P);
        GNN_LAUNCH_CHECK("rcm sampled links");
      }
      int32_t* giant = ccnt;  // one word, free until the BFS
      hipLaunchKernelGGL(k_cc_giant, dim3(1), dim3(256), 0, s, n, P, giant);
      hipLaunchKernelGGL(k_cc_skip, dim3(nb(n)), dim3(256), 0, s, rank, n, P, giant, skip);
      hipLaunchKernelGGL(k_cc_hook, dim3(nb(m)), dim3(256), 0, s, adj, adj_row, rank, skip, m, P);
      GNN_LAUNCH_CHECK("rcm hooks");
    }
    hipLaunchKernelGGL(k_cc_label, dim3(nb(n)), dim3(256), 0, s, rank, n, P, label);
    GNN_LAUNCH_CHECK("rcm labels");
  }

  // 5. level-synchronous BFS of all components at once (kept frontier edges
  // compacted through cnt, off and keep as in step 1)
  hipLaunchKernelGGL(k_fill_i32, dim3(nb(n)), dim3(256), 0, s, claim, (int64_t)n, 0x7FFFFFFF);
  GNN_LAUNCH_CHECK("rcm claim init");
  hipLaunchKernelGGL(k_start_flags, dim3(nb(n)), dim3(256), 0, s, order, label, n, ccnt);
  GNN_LAUNCH_CHECK("rcm starts");
  GNN_TRY(exclusive_scan_i32(ccnt, coff, n, s, ws));
  hipLaunchKernelGGL(k_start_fill, dim3(nb(n)), dim3(256), 0, s, order, ccnt, coff, n, concat, claim);
  GNN_LAUNCH_CHECK("rcm level 0");
  int32_t f = 0;
  GNN_HIP(hipMemcpyAsync(&f, coff + n, 4, hipMemcpyDeviceToHost, s));
  GNN_HIP(hipStreamSynchronize(s));
  int64_t base = 0;
  while (f > 0 && base + f < n) {
    const int32_t* front = concat + base;
    int32_t* next = concat + base + f;
    // frontier degrees -> offsets of the flattened frontier adjacency
    hipLaunchKernelGGL(k_front_deg, dim3(nb(f)), dim3(256), 0, s, front, f, sym_ptr, ccnt);
    GNN_LAUNCH_CHECK("rcm frontier degrees");
    GNN_TRY(exclusive_scan_i32(ccnt, coff, f, s, ws));
    int32_t ef = 0;
    GNN_HIP(hipMemcpyAsync(&ef, coff + f, 4, hipMemcpyDeviceToHost, s));
    GNN_HIP(hipStreamSynchronize(s));
    if (ef < 0 || ef > m) return fail(GNN_ERR_DEVICE, "RCM: frontier adjacency larger than the graph");
    int32_t nf = 0;
    if (ef > 0) {
      hipLaunchKernelGGL(k_claim, dim3(nb_seg(ef)), dim3(256), 0, s, front, f, coff, (int64_t)ef, sym_ptr,
                         adj, claim);
      hipLaunchKernelGGL(k_child_count, dim3(nb_seg(ef)), dim3(256), 0, s, front, f, coff, (int64_t)ef,
                         sym_ptr, adj, claim, keep, cnt);
      GNN_LAUNCH_CHECK("rcm level counts");
      GNN_TRY(exclusive_scan_i32(cnt, off, nb_seg(ef), s, ws));
      GNN_HIP(hipMemcpyAsync(&nf, off + nb_seg(ef), 4, hipMemcpyDeviceToHost, s));
      GNN_HIP(hipStreamSynchronize(s));
    }
    if (nf < 0 || base + f + nf > n) return fail(GNN_ERR_DEVICE, "RCM: level larger than the graph");
    if (nf > 0) {
      hipLaunchKernelGGL(k_child_emit, dim3(nb_seg(ef)), dim3(256), 0, s, front, f, coff, (int64_t)ef,
                         sym_ptr, adj, keep, off, next);
      GNN_LAUNCH_CHECK("rcm level emit");
      hipLaunchKernelGGL(k_mark, dim3(nb(nf)), dim3(256), 0, s, next, nf, claim);
      GNN_LAUNCH_CHECK("rcm mark");
    }
    base += f;
    f = nf;
  }
  if (base + f != n) return fail(GNN_ERR_DEVICE, "RCM: levels do not cover every vertex");

  // 6. (component, level, position) order by a stable sort on the label; reverse
  hipLaunchKernelGGL(k_final_keys, dim3(nb(n)), dim3(256), 0, s, concat, label, n, idbits, keys);
  GNN_LAUNCH_CHECK("rcm final keys");
  GNN_TRY(radix_sort_u64(keys, tmp, n, idbits, 2 * idbits, s, ws));
  hipLaunchKernelGGL(k_final_perm, dim3(nb(n)), dim3(256), 0, s, keys, concat, n, idbits, perm);
  GNN_LAUNCH_CHECK("rcm perm");
  return GNN_OK;
}

size_t permute_bytes(int32_t n, int64_t nnz) {
  const int64_t m = std::max<int64_t>(nnz, 1);
  return 2 * Arena::round((size_t)n * 4) + Arena::round((size_t)m * 4) + scan_scratch_bytes(n);
}

int permute_csr(const gnn_csr* c, const int32_t* perm, int32_t* rp_out, int32_t* ci_out, Arena& ar,
                hipStream_t s) {
  const int32_t n = c->n_rows;
  const int64_t nnz = c->nnz;
  int32_t* inv = ar.take<int32_t>(n);
  int32_t* deg = ar.take<int32_t>(n);
  uint32_t* cols = ar.take<uint32_t>(std::max<int64_t>(nnz, 1));
  void* ws = ar.base + ar.off;
  hipLaunchKernelGGL(k_inverse, dim3(nb(n)), dim3(256), 0, s, perm, n, inv);
  hipLaunchKernelGGL(k_new_deg, dim3(nb(n)), dim3(256), 0, s, c->row_ptr, perm, n, deg);
  GNN_LAUNCH_CHECK("permute degrees");
  GNN_TRY(exclusive_scan_i32(deg, rp_out, n, s, ws));
  if (nnz > 0) {
    hipLaunchKernelGGL(k_perm_cols, dim3(nb_seg(nnz)), dim3(256), 0, s, c->row_ptr, c->col_idx, perm, inv,
                       rp_out, n, nnz, cols);
    GNN_LAUNCH_CHECK("permute cols");
    GNN_TRY(segmented_sort_u32(cols, reinterpret_cast<uint32_t*>(ci_out), rp_out, n, nnz, (uint32_t)n, s));
  }
  return GNN_OK;
}

}  // namespace

// One device block per call holds every temporary (the permutation step, then
// the relabelling, which reuses it in stream order).
int launch_reorder(const gnn_csr* csr, gnn_reorder_kind kind, int32_t* perm, int32_t* rp_out,
                   int32_t* ci_out, hipStream_t s) {
  const int32_t n = csr->n_rows;
  size_t need = kind == GNN_REORDER_DEGREE ? degree_bytes(n) : rcm_bytes(n, csr->nnz);
  if (rp_out) need = std::max(need, permute_bytes(n, csr->nnz));
  void* blk = nullptr;
  GNN_TRY(dev_malloc_async(&blk, need, s));
  Arena ar{static_cast<char*>(blk), need, 0};
  int rc = kind == GNN_REORDER_DEGREE ? degree_perm(csr, perm, ar, s) : rcm_perm(csr, perm, ar, s);
  if (rc == GNN_OK && rp_out) {
    ar.off = 0;
    rc = permute_csr(csr, perm, rp_out, ci_out, ar, s);
  }
  const int r1 = dev_free_async(blk, s);
  const hipError_t e2 = hipStreamSynchronize(s);
  if (rc != GNN_OK) return rc;
  if (r1 != GNN_OK) return r1;
  if (e2 != hipSuccess) return fail(GNN_ERR_DEVICE, std::string("reorder: ") + hipGetErrorString(e2));
  return GNN_OK;
}

}  // namespace gnn
