// build_csr.hip -- COO -> destination-grouped CSR in canonical order.
//
// The destination-grouped index is the CSC of the connection matrix
// G[src, dst] in the gattn-triton article ("Using the CSC index for fast
// edge lookup"): a pointer vector of N+1 entries, the source of every
// grouped edge and a map from grouped position to edge id.  The pages do not
// fix the order inside a destination; we sort it by (source, edge id), which
// makes the result unique although the scatter below uses atomics.
//
// Steps: count in-degrees (atomics) and flag bad indices -> exclusive scan ->
// scatter 64-bit keys (src << 32 | edge id) with per-destination atomic
// cursors -> sort every destination's keys: bitonic across the lanes of one
// wave for <= 64 keys, bitonic in LDS for <= 8192 keys, and for longer rows
// LDS-sorted chunks ranked against each other by binary search.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

namespace {

constexpr int kRowCap = 8192;  // keys per LDS sort (64 KiB)

struct CsrWs {
  int32_t* flags;      // [0] bad index seen, [1] number of long rows
  int32_t* counts;     // [n]
  int32_t* blocksums;  // scan scratch
  uint64_t* keys;      // [nnz]
  int32_t* long_rows;  // [n]
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

CsrWs carve(void* ws, int32_t n, int64_t nnz) {
  uint8_t* p = (uint8_t*)ws;
  CsrWs w;
  w.flags = (int32_t*)p;
  p += 256;
  w.counts = (int32_t*)p;
  p += align256(sizeof(int32_t) * std::max<int64_t>(n, 1));
  w.blocksums = (int32_t*)p;
  p += align256(sizeof(int32_t) * scan_blocksums_len(n));
  w.keys = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
  w.long_rows = (int32_t*)p;
  return w;
}

__global__ void count_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t nnz,
                             int32_t n, int32_t* __restrict__ counts, int32_t* __restrict__ flags) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if ((uint32_t)s >= (uint32_t)n || (uint32_t)d >= (uint32_t)n) {
      flags[0] = 1;
      continue;
    }
    atomicAdd(&counts[d], 1);
  }
}

__global__ void scatter_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t nnz,
                               int32_t n, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ cursor,
                               uint64_t* __restrict__ keys) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if ((uint32_t)s >= (uint32_t)n || (uint32_t)d >= (uint32_t)n) continue;
    const int32_t p = row_ptr[d] + atomicAdd(&cursor[d], 1);
    keys[p] = ((uint64_t)(uint32_t)s << 32) | (uint64_t)(uint32_t)e;
  }
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src_lane) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)x, src_lane, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(x >> 32), src_lane, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void emit(int32_t* col_idx, int32_t* edge_perm, int64_t p, uint64_t key) {
  col_idx[p] = (int32_t)(key >> 32);
  if (edge_perm) edge_perm[p] = (int32_t)(uint32_t)key;
}

// one wave per destination; rows longer than 64 are deferred to long_rows
__global__ __launch_bounds__(256) void sort_short_rows_kernel(int32_t n, const int32_t* __restrict__ row_ptr,
                                                              const uint64_t* __restrict__ keys,
                                                              int32_t* __restrict__ col_idx,
                                                              int32_t* __restrict__ edge_perm,
                                                              int32_t* __restrict__ flags,
                                                              int32_t* __restrict__ long_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int32_t st = row_ptr[r], d = row_ptr[r + 1] - st;
  if (d > 64) {
    if (lane == 0) long_rows[atomicAdd(&flags[1], 1)] = (int32_t)r;
    return;
  }
  if (d <= 0) return;
  uint64_t key = lane < d ? keys[st + lane] : ~0ull;
  int P = 1;
  while (P < d) P <<= 1;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      const int partner = (j == (k >> 1)) ? (lane ^ (k - 1)) : (lane ^ j);
      const uint64_t other = shfl_u64(key, partner);
      key = lane < partner ? (other < key ? other : key) : (other > key ? other : key);
    }
  }
  if (lane < d) emit(col_idx, edge_perm, st + lane, key);
}

// LDS bitonic sort of s[0..P), P a power of two <= kRowCap; all comparators
// ascending (the first step of each merge compares mirrored positions)
__device__ void lds_bitonic(uint64_t* s, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int partner = (j == (k >> 1)) ? (i ^ (k - 1)) : (i ^ j);
        if (partner > i) {
          const uint64_t x = s[i], y = s[partner];
          if (y < x) {
            s[i] = y;
            s[partner] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void sort_long_rows_kernel(const int32_t* __restrict__ row_ptr,
                                                             uint64_t* __restrict__ keys,
                                                             int32_t* __restrict__ col_idx,
                                                             int32_t* __restrict__ edge_perm,
                                                             const int32_t* __restrict__ flags,
                                                             const int32_t* __restrict__ long_rows) {
  __shared__ uint64_t s[kRowCap];
  const int count = flags[1];
  for (int li = blockIdx.x; li < count; li += gridDim.x) {
    const int32_t r = long_rows[li];
    const int32_t st = row_ptr[r], d = row_ptr[r + 1] - st;
    const int nchunks = (d + kRowCap - 1) / kRowCap;
    for (int c = 0; c < nchunks; ++c) {
      const int cs = c * kRowCap, cl = min(kRowCap, d - cs);
      int P = 1;
      while (P < cl) P <<= 1;
      for (int i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < cl ? keys[st + cs + i] : ~0ull;
      __syncthreads();
      lds_bitonic(s, P);
      if (nchunks == 1) {
        for (int i = threadIdx.x; i < cl; i += blockDim.x) emit(col_idx, edge_perm, st + i, s[i]);
      } else {
        for (int i = threadIdx.x; i < cl; i += blockDim.x) keys[st + cs + i] = s[i];
      }
      __syncthreads();
    }
    if (nchunks > 1) {
      // rank of a key = its index in its own sorted chunk + keys below it in the others
      for (int i = threadIdx.x; i < d; i += blockDim.x) {
        const uint64_t key = keys[st + i];
        const int own = i / kRowCap;
        int rank = i - own * kRowCap;
        for (int c = 0; c < nchunks; ++c) {
          if (c == own) continue;
          int lo = c * kRowCap, hi = min(lo + kRowCap, d);
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (keys[st + mid] < key) lo = mid + 1; else hi = mid;
          }
          rank += lo - c * kRowCap;
        }
        emit(col_idx, edge_perm, st + rank, key);
      }
      __syncthreads();
    }
  }
}

__global__ void write_status_kernel(const int32_t* flags, int32_t* status_dev) {
  *status_dev = flags[0] ? GATTN_ERR_BAD_GRAPH : GATTN_OK;
}

}  // namespace

size_t build_csr_workspace_bytes(int32_t n, int64_t nnz) {
  return 256 + align256(sizeof(int32_t) * std::max<int64_t>(n, 1)) +
         align256(sizeof(int32_t) * scan_blocksums_len(n)) + align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1)) +
         align256(sizeof(int32_t) * std::max<int64_t>(n, 1));
}

hipError_t launch_build_csr(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst, int32_t* row_ptr,
                            int32_t* col_idx, int32_t* edge_perm, void* ws, int32_t* status_dev, hipStream_t s) {
  CsrWs w = carve(ws, n, nnz);
  hipError_t err;
  if ((err = launch_fill_i32(w.flags, 0, 2, s)) != hipSuccess) return err;
  if ((err = launch_fill_i32(w.counts, 0, n, s)) != hipSuccess) return err;
  const unsigned eblocks = (unsigned)std::min<int64_t>(std::max<int64_t>(ceil_div(nnz, 256), 1), 16384);
  if (nnz > 0) {
    hipLaunchKernelGGL(count_kernel, dim3(eblocks), dim3(256), 0, s, src, dst, nnz, n, w.counts, w.flags);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = launch_scan(w.counts, row_ptr, n, w.blocksums, s)) != hipSuccess) return err;
  if (nnz > 0 && n > 0) {
    if ((err = launch_fill_i32(w.counts, 0, n, s)) != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(eblocks), dim3(256), 0, s, src, dst, nnz, n, row_ptr, w.counts, w.keys);
    hipLaunchKernelGGL(sort_short_rows_kernel, dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, s, n, row_ptr,
                       w.keys, col_idx, edge_perm, w.flags, w.long_rows);
    const unsigned lblocks = (unsigned)std::min<int64_t>(std::max<int64_t>(nnz / 65, 1), 2048);
    hipLaunchKernelGGL(sort_long_rows_kernel, dim3(lblocks), dim3(256), 0, s, row_ptr, w.keys, col_idx, edge_perm,
                       w.flags, w.long_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (status_dev) {
    hipLaunchKernelGGL(write_status_kernel, dim3(1), dim3(1), 0, s, w.flags, status_dev);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace gattn
