// Stable LSD radix sort of 64-bit keys on the GPU (8-bit digits), used by
// the preprocessing steps (WSB column lists, degree order, RCM levels).
//
// One pass per digit: (1) each workgroup counts the digits of its tile of
// 4096 keys (one LDS histogram per wave: plain LDS atomics measured faster
// than matching equal digits with ballots first); (2) an exclusive scan over the digit-major count table gives
// every (digit, tile) its output offset; (3) each workgroup sorts its tile by
// the digit in LDS and writes every digit's keys as one contiguous run.
// In (3) each wave ranks a contiguous quarter of the tile in rounds of 64
// keys: lanes holding the same digit find each other with eight ballots,
// take their rank among them in lane order, and add to the wave's running
// count of that digit, so a key's place in the tile is (digit start, keys of
// that digit in earlier waves, then earlier in its own wave): input order
// among equal digits, which keeps the pass stable.  Writing runs instead of
// single keys keeps the stores coalesced (on average 16 keys, 128 bytes, per
// digit and tile).
#include <algorithm>

#include "gnn_internal.h"

namespace gnn {
namespace {

constexpr int RT = 256;          // threads
constexpr int RI = 16;           // rounds per wave
constexpr int NW = RT / 64;      // waves
constexpr int RTILE = RT * RI;   // keys per tile
constexpr int KPW = RTILE / NW;  // keys per wave

// Lanes of this wave whose digit equals this lane's (d in [0, 256), or 256
// for a lane without a key; `ok` = the lane holds a key).
__device__ __forceinline__ unsigned long long digit_peers(bool ok, int d) {
  unsigned long long peers = __ballot(ok);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const unsigned long long m = __ballot(ok && ((d >> b) & 1));
    peers &= ((d >> b) & 1) ? m : ~m;
  }
  return peers;
}

// Orders this wave's LDS accesses around the call (different lanes touch
// the same words: one lane writes what others read in the next round).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(RT) void k_rs_hist(const uint64_t* keys, int64_t n, int shift,
                                                int32_t* hist, int32_t ntiles) {
  __shared__ int32_t h[NW][256];
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int w = 0; w < NW; ++w) h[w][threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RTILE;
  uint64_t kv[RI];
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int64_t i = base + (int64_t)r * RT + threadIdx.x;
    kv[r] = i < n ? keys[i] : 0;
  }
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int64_t i = base + (int64_t)r * RT + threadIdx.x;
    if (i < n) atomicAdd(&h[wave][(kv[r] >> shift) & 0xFF], 1);
  }
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += h[w][threadIdx.x];
  hist[(int64_t)threadIdx.x * ntiles + blockIdx.x] = t;
}

__global__ __launch_bounds__(RT) void k_rs_scatter(const uint64_t* keys, uint64_t* out, int64_t n,
                                                   int shift, const int32_t* offs, int32_t ntiles) {
  __shared__ uint64_t s_keys[RTILE];  // the tile in digit order
  __shared__ int32_t wcnt[NW][256];   // per-wave digit counts, then each wave's start per digit
  __shared__ int32_t s_loc[256];      // tile position of each digit's first key
  __shared__ int32_t s_cnt[256];      // keys of each digit in the tile
  __shared__ int32_t s_out[256];      // output position of each digit's first key
  __shared__ int32_t s_wsum[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * RTILE;
  const int64_t wbase = base + (int64_t)wave * KPW;
  for (int t = lane; t < 256; t += 64) wcnt[wave][t] = 0;
  wave_sync_lds();

  // the wave's keys, all loads issued before the ranking
  uint64_t kv[RI];
  int rk[RI];
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int64_t i = wbase + (int64_t)r * 64 + lane;
    kv[r] = i < n ? keys[i] : 0;
  }
  // rank them: rk = earlier keys of the same digit in this wave
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const bool ok = wbase + (int64_t)r * 64 + lane < n;
    const uint64_t key = kv[r];
    const int d = ok ? (int)((key >> shift) & 0xFF) : 256;
    const unsigned long long peers = digit_peers(ok, d);
    const int before = ok ? wcnt[wave][d] : 0;
    wave_sync_lds();
    if (ok && (peers & lt) == 0) wcnt[wave][d] = before + __popcll(peers);
    wave_sync_lds();
    rk[r] = before + __popcll(peers & lt);
  }
  __syncthreads();

  // digit starts in the tile (exclusive scan of the counts over the digits)
  // and each wave's start within its digit
  {
    const int t = threadIdx.x;
    int c[NW], tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      c[w] = wcnt[w][t];
      tot += c[w];
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int loc = incl - tot;
    for (int w = 0; w < wave; ++w) loc += s_wsum[w];
    s_loc[t] = loc;
    s_cnt[t] = tot;
    s_out[t] = offs[(int64_t)t * ntiles + blockIdx.x];
    int run = loc;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wcnt[w][t] = run;
      run += c[w];
    }
  }
  __syncthreads();

  // the tile in digit order (a key's slot is below the tile's key count)
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int64_t i = wbase + (int64_t)r * 64 + lane;
    if (i < n) {
      const int d = (int)((kv[r] >> shift) & 0xFF);
      const int slot = wcnt[wave][d] + rk[r];
      if (slot < RTILE) s_keys[slot] = kv[r];
    }
  }
  __syncthreads();

  // each digit's keys as one contiguous run of the output
  const int tile_n = (int)min((int64_t)RTILE, n - base);
  for (int i = threadIdx.x; i < tile_n; i += RT) {
    const uint64_t key = s_keys[i];
    const int d = (int)((key >> shift) & 0xFF);
    const int j = i - s_loc[d];
    if (j >= 0 && j < s_cnt[d]) out[(int64_t)s_out[d] + j] = key;
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
