// merge_runs.hpp -- a workgroup-wide stable merge of two sorted runs of
// 64-bit keys in global memory (keys of the first run go first on ties), used
// to sort rows and windows longer than one LDS sort: LDS-sorted chunks are
// merged pairwise, runs doubling, between two buffers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gattn {

constexpr int kMergeTile = 2048;     // output keys per LDS tile (the caller's LDS buffer holds them)
constexpr int kMergeThreads = 256;   // the workgroup size the helpers assume

// Elements of A among the first k outputs of the stable merge of sorted A [la]
// and B [lb]: the merge-path co-rank, by binary search.
__device__ __forceinline__ int merge_co_rank(const uint64_t* A, int la, const uint64_t* B, int lb, int k) {
  int lo = max(0, k - lb), hi = min(k, la);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A[mid] <= B[k - mid - 1]) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// out[0 .. la + lb) = stable merge of sorted A and B, by the whole workgroup:
// output tiles of kMergeTile keys, whose A and B parts are staged in the LDS
// buffer s [kMergeTile], each thread then merging kMergeTile / kMergeThreads
// consecutive outputs of the tile from LDS.  The co-ranks at the tile
// boundaries are found in parallel, one per thread, for batches of up to
// kMergeThreads tiles (s_co [kMergeThreads + 1]).  Ends with a barrier.
__device__ inline void merge_runs(const uint64_t* A, int la, const uint64_t* B, int lb, uint64_t* out, uint64_t* s,
                                  int32_t* s_co) {
  const int total = la + lb;
  constexpr int kPer = kMergeTile / kMergeThreads;
  const int tiles = (total + kMergeTile - 1) / kMergeTile;
  for (int t0 = 0; t0 < tiles; t0 += kMergeThreads) {
    const int nt = min(kMergeThreads, tiles - t0);
    for (int b = threadIdx.x; b <= nt; b += blockDim.x)
      s_co[b] = merge_co_rank(A, la, B, lb, (int)min((int64_t)(t0 + b) * kMergeTile, (int64_t)total));
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const int o0 = (t0 + tt) * kMergeTile, o1 = min(o0 + kMergeTile, total);
      const int i0 = s_co[tt], i1 = s_co[tt + 1];
      const int na = i1 - i0, nb = (o1 - o0) - na;
      for (int i = threadIdx.x; i < na; i += blockDim.x) s[i] = A[i0 + i];
      for (int i = threadIdx.x; i < nb; i += blockDim.x) s[na + i] = B[(o0 - i0) + i];
      __syncthreads();
      const int k0 = min((int)threadIdx.x * kPer, o1 - o0), k1 = min(k0 + kPer, o1 - o0);
      if (k0 < k1) {
        int ia = merge_co_rank(s, na, s + na, nb, k0), ib = k0 - ia;
        for (int k = k0; k < k1; ++k) {
          const bool take_a = ib >= nb || (ia < na && s[ia] <= s[na + ib]);
          out[o0 + k] = take_a ? s[ia++] : s[na + ib++];
        }
      }
      __syncthreads();
    }
  }
}

// Sorts data[0 .. len) given as sorted runs of `run` keys: pairwise merges
// between data and tmp, runs doubling; returns the buffer that holds the
// sorted keys (data or tmp).
__device__ inline uint64_t* merge_sorted_runs(uint64_t* data, uint64_t* tmp, int len, int run, uint64_t* s,
                                              int32_t* s_co) {
  uint64_t* from = data;
  uint64_t* to = tmp;
  for (int64_t R = run; R < len; R *= 2) {  // 64-bit: rows of up to 2^31 - 1 keys double R past 2^30
    for (int64_t a0 = 0; a0 < len; a0 += 2 * R) {
      const int a1 = (int)min(a0 + R, (int64_t)len), b1 = (int)min(a0 + 2 * R, (int64_t)len);
      merge_runs(from + a0, a1 - a0, from + a1, b1 - a1, to + a0, s, s_co);
    }
    uint64_t* t = from;
    from = to;
    to = t;
  }
  return from;
}

}  // namespace gattn
