// scan.hip -- exclusive prefix sum of int32 counts (reduce, scan the block
// sums in one workgroup, scan again with offsets) and a fill kernel.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;

// inclusive scan across a 256-thread block; returns the block total in *total
__device__ __forceinline__ int32_t block_incl_scan(int32_t x, int32_t* s_wave, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const int32_t v = s_wave[w];
    if (w < wave) off += v;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return x + off;
}

__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const int32_t* __restrict__ in, int64_t n,
                                                                   int32_t* __restrict__ blocksums) {
  __shared__ int32_t s_wave[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i)
    if (base + i < n) s += in[base + i];
  int32_t total;
  block_incl_scan(s, s_wave, &total);
  if (threadIdx.x == 0) blocksums[blockIdx.x] = total;
}

// one workgroup: exclusive scan of blocksums[0..nb) in place, blocksums[nb] = total
__global__ __launch_bounds__(kScanThreads) void scan_blocksums_kernel(int32_t* __restrict__ bs, int64_t nb) {
  __shared__ int32_t s_wave[kScanThreads / 64];
  int32_t carry = 0;
  for (int64_t c = 0; c < nb; c += kScanTile) {
    const int64_t base = c + threadIdx.x * kScanItems;
    int32_t v[kScanItems], s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      v[i] = base + i < nb ? bs[base + i] : 0;
      s += v[i];
    }
    int32_t total;
    const int32_t incl = block_incl_scan(s, s_wave, &total);
    int32_t run = carry + incl - s;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      if (base + i < nb) bs[base + i] = run;
      run += v[i];
    }
    carry += total;
  }
  if (threadIdx.x == 0) bs[nb] = carry;
}

__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(const int32_t* in, int32_t* out, int64_t n,
                                                                  const int32_t* __restrict__ bs, int64_t nb) {
  __shared__ int32_t s_wave[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int32_t v[kScanItems], s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    v[i] = base + i < n ? in[base + i] : 0;
    s += v[i];
  }
  int32_t total;
  const int32_t incl = block_incl_scan(s, s_wave, &total);
  int32_t run = bs[blockIdx.x] + incl - s;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = bs[nb];
}

__global__ void fill_i32_kernel(int32_t* p, int32_t value, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

int64_t scan_blocksums_len(int64_t n) { return ceil_div(std::max<int64_t>(n, 1), kScanTile) + 1; }

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* blocksums, hipStream_t s) {
  if (n == 0) return launch_fill_i32(out, 0, 1, s);
  const int64_t nb = ceil_div(n, kScanTile);
  hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, blocksums);
  hipLaunchKernelGGL(scan_blocksums_kernel, dim3(1), dim3(kScanThreads), 0, s, blocksums, nb);
  hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, out, n, blocksums, nb);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Single-pass exclusive scan with decoupled look-back.  Tiles take tickets in
// launch order, so every tile a workgroup waits for has already started and
// finishes without waiting on later ones.  A tile publishes its aggregate,
// then its inclusive prefix, as one 64-bit word (flag << 32 | value).  The
// first wave reads the words of up to 64 earlier tiles per poll and adds the
// values up to the nearest inclusive prefix, polling again while any word in
// that range is still empty.  The wait is bounded: after kSpinLimit such
// polls the tile reports an error instead of spinning on.
// ---------------------------------------------------------------------------
namespace {
constexpr uint32_t kFlagAggregate = 1, kFlagPrefix = 2;
constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ void publish(uint64_t* st, uint32_t flag, int32_t v) {
  __hip_atomic_store(st, ((uint64_t)flag << 32) | (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

__global__ __launch_bounds__(kScanThreads) void scan_lookback_kernel(const int32_t* __restrict__ in,
                                                                     int32_t* __restrict__ out, int64_t n,
                                                                     uint64_t* __restrict__ tile_status,
                                                                     int32_t* __restrict__ ticket,
                                                                     int32_t* __restrict__ err,
                                                                     int32_t* __restrict__ status_dev) {
  __shared__ int32_t s_wave[kScanThreads / 64];
  __shared__ int32_t s_tile, s_prefix;
  if (threadIdx.x == 0) s_tile = atomicAdd(ticket, 1);
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t base = tile * kScanTile + threadIdx.x * kScanItems;
  int32_t v[kScanItems], s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    v[i] = base + i < n ? in[base + i] : 0;
    s += v[i];
  }
  int32_t total;
  const int32_t incl = block_incl_scan(s, s_wave, &total);
  if (threadIdx.x < 64) {  // the first wave walks back over up to 64 earlier tiles per poll
    const int lane = threadIdx.x;
    int32_t prefix = 0;
    if (tile == 0) {
      if (lane == 0) publish(&tile_status[0], kFlagPrefix, total);
    } else {
      if (lane == 0) publish(&tile_status[tile], kFlagAggregate, total);
      int64_t j = tile - 1;  // lane l reads tile j - l
      int spins = 0;
      while (true) {
        const int64_t t = j - lane;
        const uint64_t w = t >= 0 ? __hip_atomic_load(&tile_status[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : (uint64_t)kFlagPrefix << 32;
        const uint32_t flag = (uint32_t)(w >> 32);
        const uint64_t pmask = __ballot(flag == kFlagPrefix), zmask = __ballot(flag == 0);
        const int first_p = pmask ? __ffsll((unsigned long long)pmask) - 1 : 64;  // nearest inclusive prefix
        const uint64_t need = first_p >= 63 ? ~0ull : (2ull << first_p) - 1;        // lanes 0 .. first_p
        if (zmask & need) {  // a tile up to that prefix has not published yet
          if (++spins > kSpinLimit) {
            if (lane == 0) {
              err[0] = 1;
              if (status_dev) *status_dev = GATTN_ERR_HIP;
            }
            break;
          }
          continue;
        }
        int32_t agg = lane <= first_p ? (int32_t)(uint32_t)w : 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) agg += __shfl_xor(agg, o, 64);
        prefix += agg;
        if (first_p < 64) break;
        j -= 64;
      }
      if (lane == 0) publish(&tile_status[tile], kFlagPrefix, prefix + total);
    }
    if (lane == 0) s_prefix = prefix;
  }
  __syncthreads();
  int32_t run = s_prefix + incl - s;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (base <= n && n <= base + kScanItems) out[n] = run;  // the thread holding the end writes the total
}

int64_t scan_tiles(int64_t n) { return ceil_div(std::max<int64_t>(n, 1), kScanTile); }

hipError_t launch_scan_lookback(const int32_t* in, int32_t* out, int64_t n, uint64_t* tile_status, int32_t* ticket,
                                int32_t* err, int32_t* status_dev, hipStream_t s) {
  hipLaunchKernelGGL(scan_lookback_kernel, dim3((unsigned)scan_tiles(n)), dim3(kScanThreads), 0, s, in, out, n,
                     tile_status, ticket, err, status_dev);
  return hipGetLastError();
}

}  // namespace gattn
