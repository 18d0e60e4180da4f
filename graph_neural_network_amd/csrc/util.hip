// Small data-movement kernels: row gather for reordered features and a plain
// streaming copy used to calibrate bandwidth figures and hardware counters.
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "gnn_internal.h"

namespace gnn {

// The allocation-failure hook: with GNN_FAIL_ALLOC=k or k:tag, the k-th
// allocation counted from when the variable last took its value fails.
static std::mutex g_fault_mu;
static std::string g_fault_value;
static long g_fault_count = 0;

static bool alloc_fault() {
  const char* e = getenv("GNN_FAIL_ALLOC");
  std::lock_guard<std::mutex> lock(g_fault_mu);
  if (!e || !*e) {
    g_fault_value.clear();
    return false;
  }
  if (g_fault_value != e) {
    g_fault_value = e;
    g_fault_count = 0;
  }
  return ++g_fault_count == atol(e);
}

int dev_malloc(void** p, size_t bytes) {
  *p = nullptr;
  if (alloc_fault()) return fail(GNN_ERR_OUT_OF_MEMORY, "device allocation failed (GNN_FAIL_ALLOC)");
  const hipError_t e = hipMalloc(p, bytes ? bytes : 16);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(e == hipErrorOutOfMemory ? GNN_ERR_OUT_OF_MEMORY : GNN_ERR_DEVICE,
                std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  return GNN_OK;
}

// Block cache of the stream-ordered allocations.  A block that
// dev_free_async releases stays with the library, with an event recorded on
// the releasing stream, and serves a later dev_malloc_async request on the
// same device: the requesting stream first waits for that event, so the new
// work starts after the last use of the block, with no host wait.  (The
// runtime's own stream-ordered free can block the host until the device
// catches up, which leaves the device idle between the steps of a call
// without a plan.)  A request takes the smallest cached block of at least its
// rounded size and at most twice that.  Above kCacheCap cached bytes on a
// device the oldest blocks go back to the runtime; so do all of the device's
// blocks when an allocation fails for lack of memory (then the allocation is
// tried once more) and on release_cached_memory.  Giving a block back waits
// for its event.
namespace {
struct CachedBlock {
  void* p;
  size_t bytes;
  int dev;
  hipEvent_t ev;  // recorded when the block was released
};
struct LiveBlock {
  size_t bytes;
  int dev;
  hipEvent_t ev;  // the block's event from an earlier release, or NULL
};
constexpr size_t kCacheCap = (size_t)8 << 30;
std::mutex g_cache_mu;
std::vector<CachedBlock> g_cached;            // released, oldest first
std::unordered_map<void*, LiveBlock> g_live;  // handed out by dev_malloc_async

// 4 KiB minimum; above that, multiples of an eighth of the power of two below
size_t round_block(size_t b) {
  if (b <= 4096) return 4096;
  const int lg = 63 - __builtin_clzll((unsigned long long)b);
  const size_t g = std::max<size_t>(4096, (size_t)1 << (lg - 3));
  return (b + g - 1) / g * g;
}

size_t cached_bytes(int dev) {
  size_t t = 0;
  for (const CachedBlock& c : g_cached)
    if (c.dev == dev) t += c.bytes;
  return t;
}

// Gives the current device's cached blocks back to the runtime, oldest
// first, until at most `keep` bytes remain (caller holds the lock).
hipError_t trim_cache(int dev, size_t keep) {
  hipError_t first = hipSuccess;
  auto note = [&first](hipError_t e) {
    if (e != hipSuccess && first == hipSuccess) first = e;
  };
  size_t have = cached_bytes(dev);
  for (size_t i = 0; i < g_cached.size() && have > keep;) {
    const CachedBlock c = g_cached[i];
    if (c.dev != dev) {
      ++i;
      continue;
    }
    note(hipEventSynchronize(c.ev));
    note(hipFreeAsync(c.p, nullptr));
    note(hipEventDestroy(c.ev));
    have -= c.bytes;
    g_cached.erase(g_cached.begin() + (std::ptrdiff_t)i);
  }
  return first;
}
}  // namespace

int dev_malloc_async(void** p, size_t bytes, hipStream_t s) {
  *p = nullptr;
  if (alloc_fault()) return fail(GNN_ERR_OUT_OF_MEMORY, "device allocation failed (GNN_FAIL_ALLOC)");
  int dev = 0;
  GNN_HIP(hipGetDevice(&dev));
  const size_t want = round_block(bytes);
  std::lock_guard<std::mutex> lock(g_cache_mu);
  int best = -1;
  for (int i = 0; i < (int)g_cached.size(); ++i) {
    const CachedBlock& c = g_cached[i];
    if (c.dev == dev && c.bytes >= want && c.bytes <= 2 * want && (best < 0 || c.bytes < g_cached[best].bytes))
      best = i;
  }
  if (best >= 0) {
    const CachedBlock c = g_cached[best];
    GNN_HIP(hipStreamWaitEvent(s, c.ev, 0));
    g_cached.erase(g_cached.begin() + best);
    g_live[c.p] = LiveBlock{c.bytes, dev, c.ev};
    *p = c.p;
    return GNN_OK;
  }
  hipError_t e = hipMallocAsync(p, want, s);
  if (e == hipErrorOutOfMemory && cached_bytes(dev) > 0) {
    (void)hipGetLastError();
    (void)trim_cache(dev, 0);
    e = hipMallocAsync(p, want, s);
  }
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(e == hipErrorOutOfMemory ? GNN_ERR_OUT_OF_MEMORY : GNN_ERR_DEVICE,
                std::string("hipMallocAsync: ") + hipGetErrorString(e));
  }
  g_live[*p] = LiveBlock{want, dev, nullptr};
  return GNN_OK;
}

int dev_free_async(void* p, hipStream_t s) {
  if (!p) return GNN_OK;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto it = g_live.find(p);
  if (it == g_live.end()) {
    GNN_HIP(hipFreeAsync(p, s));
    return GNN_OK;
  }
  LiveBlock b = it->second;
  hipError_t e = hipSuccess;
  if (!b.ev) e = hipEventCreateWithFlags(&b.ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(b.ev, s);
  if (e != hipSuccess) {
    // no event: give the block back in stream order instead
    g_live.erase(it);
    if (b.ev) (void)hipEventDestroy(b.ev);
    (void)hipFreeAsync(p, s);
    return fail(GNN_ERR_DEVICE, std::string("releasing a device block: ") + hipGetErrorString(e));
  }
  g_live.erase(it);
  g_cached.push_back(CachedBlock{p, b.bytes, b.dev, b.ev});
  if (cached_bytes(b.dev) > kCacheCap) {
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && cur == b.dev) {
      const hipError_t t = trim_cache(cur, kCacheCap);
      if (t != hipSuccess) return fail(GNN_ERR_DEVICE, std::string("trimming the block cache: ") + hipGetErrorString(t));
    }
  }
  return GNN_OK;
}

int release_cached_memory() {
  int dev = 0;
  GNN_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  const hipError_t e = trim_cache(dev, 0);
  if (e != hipSuccess) return fail(GNN_ERR_DEVICE, std::string("releasing cached blocks: ") + hipGetErrorString(e));
  return GNN_OK;
}

namespace {

// One wave per destination row; 16-byte accesses when the row allows it.
__global__ __launch_bounds__(256) void k_permute_rows16(const int32_t* perm, int32_t n,
                                                        const uint4* X, int64_t ldx16, uint4* Y,
                                                        int64_t ldy16, int32_t row16) {
  int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const uint4* src = X + (int64_t)perm[r] * ldx16;
  uint4* dst = Y + r * ldy16;
  for (int c = threadIdx.x & 63; c < row16; c += 64) dst[c] = src[c];
}

__global__ __launch_bounds__(256) void k_permute_rows_b(const int32_t* perm, int32_t n,
                                                        const uint8_t* X, int64_t ldxb, uint8_t* Y,
                                                        int64_t ldyb, int32_t rowb, int esz) {
  int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const uint8_t* src = X + (int64_t)perm[r] * ldxb;
  uint8_t* dst = Y + r * ldyb;
  if (esz == 2) {
    for (int c = threadIdx.x & 63; c < rowb / 2; c += 64)
      reinterpret_cast<uint16_t*>(dst)[c] = reinterpret_cast<const uint16_t*>(src)[c];
  } else {
    for (int c = threadIdx.x & 63; c < rowb / 4; c += 64)
      reinterpret_cast<uint32_t*>(dst)[c] = reinterpret_cast<const uint32_t*>(src)[c];
  }
}

__global__ __launch_bounds__(256) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ void k_copy_tail(const uint8_t* src, uint8_t* dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

int launch_permute_rows(const int32_t* perm, int32_t n, const void* X, int esz, int32_t F,
                        int64_t ldx, void* Xout, int64_t ldo, hipStream_t s) {
  const int64_t rowb = (int64_t)F * esz;
  const unsigned blocks = (unsigned)((n + 3) / 4);
  if (rowb % 16 == 0 && (ldx * esz) % 16 == 0 && (ldo * esz) % 16 == 0 &&
      ((uintptr_t)X | (uintptr_t)Xout) % 16 == 0) {
    hipLaunchKernelGGL(k_permute_rows16, dim3(blocks), dim3(256), 0, s, perm, n, (const uint4*)X,
                       ldx * esz / 16, (uint4*)Xout, ldo * esz / 16, (int32_t)(rowb / 16));
  } else {
    hipLaunchKernelGGL(k_permute_rows_b, dim3(blocks), dim3(256), 0, s, perm, n, (const uint8_t*)X,
                       ldx * esz, (uint8_t*)Xout, ldo * esz, (int32_t)rowb, esz);
  }
  GNN_LAUNCH_CHECK("permute_rows");
  return GNN_OK;
}

int launch_copy(const void* src, void* dst, int64_t n, hipStream_t s) {
  int64_t head = 0;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 == 0) {
    int64_t n16 = n / 16;
    if (n16 > 0) {
      int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 256 * 64);
      hipLaunchKernelGGL(k_copy16, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4*)src,
                         (uint4*)dst, n16);
      GNN_LAUNCH_CHECK("copy");
    }
    head = n16 * 16;
  }
  int64_t rest = n - head;
  if (rest > 0) {
    hipLaunchKernelGGL(k_copy_tail, dim3((unsigned)((rest + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)src + head, (uint8_t*)dst + head, rest);
    GNN_LAUNCH_CHECK("copy tail");
  }
  return GNN_OK;
}

}  // namespace gnn
