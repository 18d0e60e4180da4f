// Stable LSD radix sort of 64-bit keys on the GPU (8-bit digits), used by
// the preprocessing steps (WSB column lists, degree order, RCM levels).
//
// One pass per digit: (1) each workgroup counts the digits of its tile of
// 4096 keys; (2) an exclusive scan over the digit-major count table gives
// every (digit, tile) its output offset; (3) each workgroup re-reads its tile
// in rounds of 256 keys and writes every key at offset + its rank among equal
// digits in the tile, ranks taken in input order (wave ballots give the rank
// inside a wave, LDS counters across waves and rounds), which keeps the pass
// stable.
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int RT = 256;          // threads
constexpr int RI = 16;           // rounds per tile
constexpr int RTILE = RT * RI;   // keys per tile
constexpr int NW = RT / 64;

__global__ __launch_bounds__(RT) void k_rs_hist(const uint64_t* keys, int64_t n, int shift,
                                                int32_t* hist, int32_t ntiles) {
  __shared__ int32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RTILE;
  for (int r = 0; r < RI; ++r) {
    const int64_t i = base + (int64_t)r * RT + threadIdx.x;
    if (i < n) atomicAdd(&h[(keys[i] >> shift) & 0xFF], 1);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(RT) void k_rs_scatter(const uint64_t* keys, uint64_t* out, int64_t n,
                                                   int shift, const int32_t* offs, int32_t ntiles) {
  __shared__ int32_t run[256];      // keys of each digit already placed by earlier rounds
  __shared__ int32_t wcnt[NW][256]; // per-wave digit counts of the current round
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  run[threadIdx.x] = offs[(int64_t)threadIdx.x * ntiles + blockIdx.x];
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * RTILE;
  for (int r = 0; r < RI; ++r) {
#pragma unroll
    for (int w = 0; w < NW; ++w) wcnt[w][threadIdx.x] = 0;
    __syncthreads();
    const int64_t i = base + (int64_t)r * RT + threadIdx.x;
    const bool ok = i < n;
    const uint64_t key = ok ? keys[i] : 0;
    const int d = ok ? (int)((key >> shift) & 0xFF) : 256;  // 256: no key
    // lanes of this wave holding the same digit
    unsigned long long peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const unsigned long long m = __ballot(ok && ((d >> b) & 1));
      peers &= ((d >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    if (ok && rank == 0) wcnt[wave][d] = __popcll(peers);
    __syncthreads();
    if (ok) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w][d];
      out[run[d] + before + rank] = key;
    }
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += wcnt[w][threadIdx.x];
    run[threadIdx.x] += tot;
    __syncthreads();
  }
}

}  // namespace

size_t radix_scratch_bytes(int64_t n) {
  const int64_t ntiles = (n + RTILE - 1) / RTILE;
  return Arena::round((size_t)ntiles * 256 * 4) + Arena::round((size_t)(ntiles * 256 + 1) * 4) +
         scan_scratch_bytes(ntiles * 256);
}

// Sorts keys[0..n) by bits [begin_bit, end_bit) ascending, stably; the result
// ends up in `keys` (tmp is scratch of the same size).  n < 2^31.
int radix_sort_u64(uint64_t* keys, uint64_t* tmp, int64_t n, int begin_bit, int end_bit,
                   hipStream_t s, void* scratch) {
  if (n <= 1 || end_bit <= begin_bit) return GNN_OK;
  const int64_t ntiles = (n + RTILE - 1) / RTILE;
  if (ntiles * 256 >= 0x7FFFFFFF) return fail(GNN_ERR_SIZE_OVERFLOW, "radix sort too large");
  StreamTemps own(s);
  if (!scratch) GNN_TRY(own.get(&scratch, radix_scratch_bytes(n)));
  Arena a{static_cast<char*>(scratch), radix_scratch_bytes(n), 0};
  int32_t* hist = a.take<int32_t>(ntiles * 256);
  int32_t* offs = a.take<int32_t>(ntiles * 256 + 1);
  void* scan_ws = a.base + a.off;
  uint64_t* src = keys;
  uint64_t* dst = tmp;
  int rc = GNN_OK;
  for (int shift = begin_bit; shift < end_bit && rc == GNN_OK; shift += 8) {
    hipLaunchKernelGGL(k_rs_hist, dim3((unsigned)ntiles), dim3(RT), 0, s, src, n, shift, hist,
                       (int32_t)ntiles);
    GNN_LAUNCH_CHECK("radix hist");
    rc = exclusive_scan_i32(hist, offs, ntiles * 256, s, scan_ws);
    if (rc != GNN_OK) break;
    hipLaunchKernelGGL(k_rs_scatter, dim3((unsigned)ntiles), dim3(RT), 0, s, src, dst, n, shift, offs,
                       (int32_t)ntiles);
    GNN_LAUNCH_CHECK("radix scatter");
    std::swap(src, dst);
  }
  if (rc == GNN_OK && src != keys)
    GNN_HIP(hipMemcpyAsync(keys, src, n * 8, hipMemcpyDeviceToDevice, s));
  if (rc != GNN_OK) return rc;
  return own.release();
}

}  // namespace gnn
