// build_csr.hip -- COO -> destination-grouped CSR in canonical order.
//
// The destination-grouped index is the CSC of the connection matrix
// G[src, dst] in the gattn-triton article ("Using the CSC index for fast
// edge lookup"): a pointer vector of N+1 entries, the source of every
// grouped edge and a map from grouped position to edge id.  The pages do not
// fix the order inside a destination; we sort it by (source, edge id), which
// makes the result unique although the scatter below uses atomics.
//
// Counting build (edge lists below 2^18; build_csr_radix.hip serves the
// larger ones with the same result).  Five launches: clear the scratch -> count in-degrees (atomics) and flag bad
// indices -> single-pass exclusive scan -> scatter 64-bit keys (src << 32 |
// edge id), each destination counting its in-degree back down for positions
// -> sort every destination's keys (bitonic across the lanes of one wave, four
// 16-key rows per wave when they fit; rows above 64 keys by the workgroup in
// LDS, beyond 2048 keys as LDS-sorted chunks merged pairwise through a second
// buffer).
#include "common.hpp"
#include "internal.hpp"
#include "merge_runs.hpp"

#include <stdlib.h>
#include <string.h>

namespace gattn {

namespace {

constexpr int kRowCap = 2048;  // keys per LDS sort (16 KiB)
static_assert(kRowCap == kMergeTile, "the LDS sort buffer stages the merge tiles");
constexpr int64_t kRadixMinEdges = 1 << 18;

// flag words at the head of the workspace
enum { kBad = 0, kScanErr = 2, kTicket = 3 };

struct CsrWs {
  int32_t* flags;         // [64]
  int32_t* counts;        // [n]
  uint64_t* tile_status;  // [scan_tiles(n)]
  uint64_t* keys;         // [nnz]
  uint64_t* tmp;          // [nnz] merge buffer of the sort of long rows
  int64_t clear_ints;     // flags + counts + tile_status, cleared in one launch
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

CsrWs carve(void* ws, int32_t n, int64_t nnz) {
  uint8_t* p = (uint8_t*)ws;
  CsrWs w;
  w.flags = (int32_t*)p;
  p += 256;
  w.counts = (int32_t*)p;
  p += align256(sizeof(int32_t) * std::max<int64_t>(n, 1));
  w.tile_status = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * scan_tiles(n));
  w.clear_ints = (p - (uint8_t*)ws) / 4;
  w.keys = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
  w.tmp = (uint64_t*)p;
  return w;
}

__global__ void init_kernel(int32_t* __restrict__ p, int64_t n, int32_t* __restrict__ status_dev) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
  if (status_dev && blockIdx.x == 0 && threadIdx.x == 0) *status_dev = GATTN_OK;
}

__global__ void count_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t nnz,
                             int32_t n, int32_t* __restrict__ counts, int32_t* __restrict__ flags,
                             int32_t* __restrict__ status_dev) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if ((uint32_t)s >= (uint32_t)n || (uint32_t)d >= (uint32_t)n) {
      flags[kBad] = 1;
      if (status_dev) *status_dev = GATTN_ERR_BAD_GRAPH;
      continue;
    }
    atomicAdd(&counts[d], 1);
  }
}

// position = row start + (remaining count - 1); counts end at zero
__global__ void scatter_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t nnz,
                               int32_t n, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ counts,
                               uint64_t* __restrict__ keys) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if ((uint32_t)s >= (uint32_t)n || (uint32_t)d >= (uint32_t)n) continue;
    const int32_t p = row_ptr[d] + atomicSub(&counts[d], 1) - 1;
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

// ascending bitonic sort of aligned groups of P lanes (P a power of two <= 64);
// the first compare of each merge pairs mirrored positions, so every
// comparator keeps the minimum at the lower lane
__device__ __forceinline__ uint64_t lane_bitonic(uint64_t key, int lane, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      const int partner = (j == (k >> 1)) ? (lane ^ (k - 1)) : (lane ^ j);
      const uint64_t other = shfl_u64(key, partner);
      key = lane < partner ? (other < key ? other : key) : (other > key ? other : key);
    }
  }
  return key;
}

// LDS bitonic sort of s[0..P), P a power of two <= kRowCap
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

// A workgroup sorts groups of 16 destinations (grid-stride).  Each wave takes four: side by side in
// 16-lane segments when all have <= 16 in-edges, else one after the other
// across the wave (<= 64).  Longer rows are listed in LDS and sorted by the
// whole workgroup afterwards: in LDS up to kRowCap keys, beyond that as
// LDS-sorted chunks written back and merged pairwise (runs of kRowCap,
// 2 kRowCap, ...) between the key array and `tmp`.
// a row's [start, start + degree) clamped to [0, nnz): a damaged row_ptr cannot
// send a read or write outside the key and output arrays
__device__ __forceinline__ void row_range(const int32_t* row_ptr, int64_t r, int32_t nnz, int32_t& st, int32_t& d) {
  const int32_t a = min(max(row_ptr[r], 0), nnz);
  const int32_t b = min(max(row_ptr[r + 1], a), nnz);
  st = a;
  d = b - a;
}

__global__ __launch_bounds__(256) void sort_rows_kernel(int32_t n, int32_t nnz, const int32_t* __restrict__ row_ptr,
                                                        uint64_t* __restrict__ keys, uint64_t* __restrict__ tmp,
                                                        int32_t* __restrict__ col_idx, int32_t* __restrict__ edge_perm,
                                                        const int32_t* __restrict__ run_flag) {
  if (run_flag && *run_flag == 0) return;  // rows already in order (radix build, sorted sources)
  __shared__ uint64_t s[kRowCap];
  __shared__ int32_t s_co[kMergeThreads + 1];
  __shared__ int32_t s_long[16];
  __shared__ int32_t s_nlong;
  const int lane = threadIdx.x & 63;
  const int64_t groups = ((int64_t)n + 15) / 16;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    if (threadIdx.x == 0) s_nlong = 0;
    __syncthreads();
    const int64_t r0 = (grp * 4 + (threadIdx.x >> 6)) * 4;
    if (r0 < n) {
      const int nr = (int)min<int64_t>(4, n - r0);
      int st[4], d[4], dmax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[i] = 0;
        d[i] = 0;
        if (i < nr) row_range(row_ptr, r0 + i, nnz, st[i], d[i]);
        dmax = max(dmax, d[i]);
      }
      if (dmax <= 16) {
        const int i = lane >> 4, t = lane & 15;
        const int64_t p = (int64_t)st[i] + t;
        uint64_t key = t < d[i] ? keys[p] : ~0ull;
        key = lane_bitonic(key, lane, 16);
        if (t < d[i]) emit(col_idx, edge_perm, p, key);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (d[i] <= 1) {
            if (d[i] == 1 && lane == 0) emit(col_idx, edge_perm, st[i], keys[st[i]]);
            continue;
          }
          if (d[i] > 64) {
            if (lane == 0) s_long[atomicAdd(&s_nlong, 1)] = (int32_t)(r0 + i);
            continue;
          }
          int P = 2;
          while (P < d[i]) P <<= 1;
          uint64_t key = lane < d[i] ? keys[st[i] + lane] : ~0ull;
          key = lane_bitonic(key, lane, P);
          if (lane < d[i]) emit(col_idx, edge_perm, st[i] + lane, key);
        }
      }
    }
    __syncthreads();
    const int nlong = s_nlong;
    for (int li = 0; li < nlong; ++li) {
      const int32_t r = s_long[li];
      int32_t st, d;
      row_range(row_ptr, r, nnz, st, d);
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
        // pairwise merges of the sorted chunks between the keys and tmp
        const uint64_t* sorted = merge_sorted_runs(keys + st, tmp + st, d, kRowCap, s, s_co);
        for (int i = threadIdx.x; i < d; i += blockDim.x) emit(col_idx, edge_perm, st + i, sorted[i]);
        __syncthreads();
      }
    }
    __syncthreads();  // s_long / s_nlong are reused by the next group
  }
}

}  // namespace

hipError_t launch_sort_rows(int32_t n, int64_t nnz, const int32_t* row_ptr, uint64_t* keys, uint64_t* tmp,
                            int32_t* col_idx, int32_t* edge_perm, const int32_t* run_flag, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(sort_rows_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(n, 16), 8192)), dim3(256), 0, s, n, (int32_t)nnz, row_ptr, keys,
                       tmp, col_idx, edge_perm, run_flag);
  return hipGetLastError();
}

// The counting build serves small edge lists, the radix build large ones;
// GATTN_CSR_PATH=atomic|radix in the environment overrides the choice.
bool csr_use_radix(int32_t n, int64_t nnz) {
  if (n < 1 || nnz < 1) return false;
  if (const char* e = getenv("GATTN_CSR_PATH")) {
    if (!strcmp(e, "radix")) return true;
    if (!strcmp(e, "atomic")) return false;
  }
  return nnz >= kRadixMinEdges;
}

size_t build_csr_workspace_bytes(int32_t n, int64_t nnz) {
  if (csr_use_radix(n, nnz)) return build_csr_radix_workspace_bytes(n, nnz);
  return 256 + align256(sizeof(int32_t) * std::max<int64_t>(n, 1)) + align256(sizeof(uint64_t) * scan_tiles(n)) +
         2 * align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
}

hipError_t launch_build_csr(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst, int32_t* row_ptr,
                            int32_t* col_idx, int32_t* edge_perm, void* ws, int32_t* status_dev, hipStream_t s) {
  if (csr_use_radix(n, nnz))
    return launch_build_csr_radix(n, nnz, src, dst, row_ptr, col_idx, edge_perm, ws, status_dev, s);
  CsrWs w = carve(ws, n, nnz);
  const unsigned cblocks = (unsigned)std::min<int64_t>(ceil_div(w.clear_ints, 256), 2048);
  hipLaunchKernelGGL(init_kernel, dim3(cblocks), dim3(256), 0, s, w.flags, w.clear_ints, status_dev);
  const unsigned eblocks = (unsigned)std::min<int64_t>(std::max<int64_t>(ceil_div(nnz, 256), 1), 16384);
  if (nnz > 0)
    hipLaunchKernelGGL(count_kernel, dim3(eblocks), dim3(256), 0, s, src, dst, nnz, n, w.counts, w.flags, status_dev);
  hipError_t err = launch_scan_lookback(w.counts, row_ptr, n, w.tile_status, &w.flags[kTicket], &w.flags[kScanErr],
                                        status_dev, s);
  if (err != hipSuccess) return err;
  if (nnz > 0 && n > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(eblocks), dim3(256), 0, s, src, dst, nnz, n, row_ptr, w.counts, w.keys);
    return launch_sort_rows(n, nnz, row_ptr, w.keys, w.tmp, col_idx, edge_perm, nullptr, s);
  }
  return hipGetLastError();
}

}  // namespace gattn
