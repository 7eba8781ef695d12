// validate.hip -- the graph check behind GATTN_FLAG_VALIDATE, on the device.
//
// One grid-stride pass reads row_ptr, col_idx and (when given) the edge-id
// map once and raises a flag word if row_ptr[0] != 0, row_ptr[N] != nnz, a
// row pointer decreases, a column index lies outside [0, N) or an edge id
// outside [0, nnz).  The flag words are a small file-scope array (one copy
// per GPU, its address taken once per device with hipGetSymbolAddress), so
// the check allocates nothing; each call takes the next of kSlots words, so
// that checks issued concurrently from different host threads use different
// words (more than kSlots at once on one GPU would share them).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "internal.hpp"

namespace gattn {

namespace {

constexpr int kSlots = 64;
__device__ __align__(256) uint32_t validate_flags[kSlots];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
uint32_t* g_flags[kMaxDevices] = {};
std::atomic<uint32_t> g_next{0};

__global__ __launch_bounds__(64) void clear_flag(uint32_t* flag) {
  if (threadIdx.x == 0) *flag = 0u;
}

__global__ __launch_bounds__(256) void validate_kernel(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       const int32_t* __restrict__ ids, uint32_t* flag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t last = nnz > (int64_t)n ? nnz : (int64_t)n;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= last; i += stride) {
    if (i <= n) {
      const int32_t v = row_ptr[i];
      if ((i == 0 && v != 0) || (i == n && (int64_t)v != nnz)) bad = true;
      if (i < n && row_ptr[i + 1] < v) bad = true;
    }
    if (i < nnz) {
      const int32_t c = col_idx[i];
      if (c < 0 || c >= n) bad = true;
      if (ids) {
        const int32_t r = ids[i];
        if (r < 0 || (int64_t)r >= nnz) bad = true;
      }
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
}

hipError_t flag_word(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_flags[dev]) {
      void* p = nullptr;
      if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(validate_flags))) != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_flags[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_flags[dev] + (g_next.fetch_add(1, std::memory_order_relaxed) % kSlots);
  }
  return hipSuccess;
}

}  // namespace

hipError_t validate_on_device(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                              const int32_t* ids, hipStream_t s, bool* ok) {
  uint32_t* flag = nullptr;
  hipError_t e = flag_word(&flag);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_flag, dim3(1), dim3(64), 0, s, flag);
  const int64_t items = std::max<int64_t>((int64_t)n + 1, nnz);
  const unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>(ceil_div(items, 256), 1), 4096);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(256), 0, s, n, nnz, row_ptr, col_idx, ids, flag);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint32_t h = 1u;
  if ((e = hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  *ok = h == 0u;
  return hipSuccess;
}

}  // namespace gattn
