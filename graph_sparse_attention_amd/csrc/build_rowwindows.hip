// build_rowwindows.hip -- CSR -> 16-row windows of compacted, 16-wide,
// bit-masked column tiles (Fused3S, Figure 1: a row window is compacted to
// the columns it uses and stored as tensor-core-sized blocks with a binary
// mask).  Tiles are 16 x 16 here to match the 16x16 MFMA output of gfx950.
//
// One workgroup per window.  The window's edges become 64-bit keys
// (src << 4 | row-in-window); after sorting them, distinct sources are the
// positions where src changes, a repeated key is a repeated (dst, src) pair,
// and the running count of distinct sources gives each key its column.
// Keys of windows up to 8192 edges are sorted in LDS; longer windows sort
// 8192-key chunks in LDS and rank the chunks against each other by binary
// search in the workspace.  The output does not depend on the order of the
// sources inside a CSR row.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

namespace {

constexpr int kCap = 8192;
constexpr int kThreads = 256;

struct RwWs {
  int32_t* flags;   // [0]: bit 0 bad graph, bit 1 duplicate edge
  int32_t* counts;  // [W] padded column count per window
  int32_t* blocksums;
  uint64_t* keys_a;  // [nnz] long-window scratch
  uint64_t* keys_b;  // [nnz] long-window sorted keys
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

RwWs carve(void* ws, int32_t n, int64_t nnz) {
  const int64_t W = ceil_div(n, 16);
  uint8_t* p = (uint8_t*)ws;
  RwWs w;
  w.flags = (int32_t*)p;
  p += 256;
  w.counts = (int32_t*)p;
  p += align256(sizeof(int32_t) * std::max<int64_t>(W, 1));
  w.blocksums = (int32_t*)p;
  p += align256(sizeof(int32_t) * scan_blocksums_len(W));
  w.keys_a = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
  w.keys_b = (uint64_t*)p;
  return w;
}

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
  for (int w = 0; w < kThreads / 64; ++w) {
    const int32_t v = s_wave[w];
    if (w < wave) off += v;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return x + off;
}

struct WindowView {
  const uint64_t* keys;  // sorted keys (LDS or workspace)
  int32_t len;
};

// Sorted (src << 4 | r) keys of window w.  Sets flag bits for bad indices.
__device__ WindowView sorted_window(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                    const int32_t* __restrict__ col_idx, int32_t w, uint64_t* s_keys,
                                    const RwWs& ws, int32_t* s_flag) {
  const int32_t r0 = 16 * w, r1 = min(r0 + 16, n);
  const int32_t nnz_i = (int32_t)nnz;
  const int32_t st = min(max(row_ptr[r0], 0), nnz_i);
  const int32_t en = max(st, min(max(row_ptr[r1], 0), nnz_i));
  const int32_t len = en - st;
  if (threadIdx.x == 0) {
    int bad = 0;
    for (int32_t r = r0; r < r1; ++r)
      if (row_ptr[r + 1] < row_ptr[r]) bad = 1;
    if (row_ptr[r0] < 0 || row_ptr[r1] > nnz) bad = 1;
    if (w == 0 && row_ptr[0] != 0) bad = 1;
    if (r1 == n && row_ptr[n] != nnz) bad = 1;
    if (bad) atomicOr(s_flag, 1);
  }
  // key of CSR position p: its source and its row inside the window
  auto key_at = [&](int32_t p, int32_t& bad) -> uint64_t {
    int32_t lo = r0, hi = r1 - 1;  // last row r with row_ptr[r] <= p
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (row_ptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    int32_t s = col_idx[p];
    if ((uint32_t)s >= (uint32_t)n) {
      bad = 1;
      s = 0;
    }
    return ((uint64_t)(uint32_t)s << 4) | (uint64_t)(lo - r0);
  };
  int32_t bad = 0;
  WindowView v;
  v.len = len;
  if (len <= kCap) {
    int P = 1;
    while (P < len) P <<= 1;
    for (int i = threadIdx.x; i < P; i += blockDim.x) s_keys[i] = i < len ? key_at(st + i, bad) : ~0ull;
    if (bad) atomicOr(s_flag, 1);
    __syncthreads();
    lds_bitonic(s_keys, P);
    v.keys = s_keys;
    return v;
  }
  uint64_t* a = ws.keys_a + st;
  uint64_t* b = ws.keys_b + st;
  const int nchunks = (len + kCap - 1) / kCap;
  for (int c = 0; c < nchunks; ++c) {
    const int cs = c * kCap, cl = min(kCap, len - cs);
    int P = 1;
    while (P < cl) P <<= 1;
    for (int i = threadIdx.x; i < P; i += blockDim.x) s_keys[i] = i < cl ? key_at(st + cs + i, bad) : ~0ull;
    __syncthreads();
    lds_bitonic(s_keys, P);
    for (int i = threadIdx.x; i < cl; i += blockDim.x) a[cs + i] = s_keys[i];
    __syncthreads();
  }
  if (bad) atomicOr(s_flag, 1);
  // rank = index inside own chunk + keys below it in other chunks (ties: the
  // lower chunk counts first, so equal keys still land on distinct ranks)
  for (int i = threadIdx.x; i < len; i += blockDim.x) {
    const uint64_t key = a[i];
    const int own = i / kCap;
    int rank = i - own * kCap;
    for (int c = 0; c < nchunks; ++c) {
      if (c == own) continue;
      int lo = c * kCap, hi = min(lo + kCap, len);
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (c < own ? a[mid] <= key : a[mid] < key) lo = mid + 1; else hi = mid;
      }
      rank += lo - c * kCap;
    }
    b[rank] = key;
  }
  __syncthreads();
  v.keys = b;
  return v;
}

__global__ __launch_bounds__(kThreads) void rw_count_kernel(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col_idx, RwWs ws) {
  __shared__ uint64_t s_keys[kCap];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int32_t s_flag;
  const int32_t w = blockIdx.x;
  if (threadIdx.x == 0) s_flag = 0;
  __syncthreads();
  const WindowView v = sorted_window(n, nnz, row_ptr, col_idx, w, s_keys, ws, &s_flag);
  int32_t distinct = 0, dup = 0;
  for (int i = threadIdx.x; i < v.len; i += blockDim.x) {
    const uint64_t k = v.keys[i];
    if (i == 0 || (k >> 4) != (v.keys[i - 1] >> 4)) ++distinct;
    if (i > 0 && k == v.keys[i - 1]) dup = 1;
  }
  if (dup) atomicOr(&s_flag, 2);
  int32_t total;
  block_incl_scan(distinct, s_wave, &total);
  if (threadIdx.x == 0) {
    ws.counts[w] = 16 * ((total + 15) / 16);
    if (s_flag) atomicOr(ws.flags, s_flag);
  }
}

__global__ __launch_bounds__(kThreads) void rw_fill_kernel(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ col_idx,
                                                           const int32_t* __restrict__ win_col_ptr,
                                                           int32_t* __restrict__ win_cols, uint32_t* __restrict__ mask_words,
                                                           int64_t capacity, RwWs ws) {
  __shared__ uint64_t s_keys[kCap];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int32_t s_flag;
  const int32_t w = blockIdx.x;
  if (threadIdx.x == 0) s_flag = 0;
  const int64_t base = min<int64_t>(max(win_col_ptr[w], 0), capacity) & ~int64_t(15);
  const int64_t stop = min<int64_t>(max<int64_t>(win_col_ptr[w + 1], base), capacity) & ~int64_t(15);
  const int32_t padded = (int32_t)(stop - base);
  // clear this window's masks (16-bit entries, two per word) and pad its columns
  for (int64_t i = threadIdx.x; i < padded / 2; i += blockDim.x) mask_words[base / 2 + i] = 0u;
  __syncthreads();
  const WindowView v = sorted_window(n, nnz, row_ptr, col_idx, w, s_keys, ws, &s_flag);
  int32_t carry = 0;
  for (int c = 0; c < v.len; c += kThreads) {
    const int i = c + threadIdx.x;
    uint64_t k = 0;
    int32_t f = 0;
    if (i < v.len) {
      k = v.keys[i];
      f = (i == 0 || (k >> 4) != (v.keys[i - 1] >> 4)) ? 1 : 0;
    }
    int32_t total;
    const int32_t incl = block_incl_scan(f, s_wave, &total);
    if (i < v.len) {
      const int32_t t = carry + incl - 1;  // column of this key's source
      if (t >= 0 && t < padded) {
        if (f) win_cols[base + t] = (int32_t)(k >> 4);
        const int64_t entry = base + (int64_t)(t >> 4) * 16 + (int64_t)(k & 15);  // [tile][row]
        atomicOr(&mask_words[entry >> 1], (1u << (t & 15)) << (16 * (entry & 1)));
      }
    }
    carry += total;
  }
  for (int32_t t = carry + threadIdx.x; t < padded; t += blockDim.x) win_cols[base + t] = -1;
}

__global__ void rw_status_kernel(const int32_t* flags, int32_t* status) {
  const int32_t f = flags[0];
  *status = (f & 1) ? GATTN_ERR_BAD_GRAPH : (f & 2) ? GATTN_ERR_DUPLICATE_EDGE : GATTN_OK;
}

}  // namespace

size_t rowwindows_workspace_bytes(int32_t n, int64_t nnz) {
  const int64_t W = ceil_div(n, 16);
  return 256 + align256(sizeof(int32_t) * std::max<int64_t>(W, 1)) + align256(sizeof(int32_t) * scan_blocksums_len(W)) +
         2 * align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
}

hipError_t launch_rowwindows_count(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                   int32_t* win_col_ptr, void* wsp, int32_t* status_dev, hipStream_t s) {
  RwWs ws = carve(wsp, n, nnz);
  const int64_t W = ceil_div(n, 16);
  hipError_t err;
  if ((err = launch_fill_i32(ws.flags, 0, 1, s)) != hipSuccess) return err;
  if (W > 0) {
    hipLaunchKernelGGL(rw_count_kernel, dim3((unsigned)W), dim3(kThreads), 0, s, n, nnz, row_ptr, col_idx, ws);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = launch_scan(ws.counts, win_col_ptr, W, ws.blocksums, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(rw_status_kernel, dim3(1), dim3(1), 0, s, ws.flags, status_dev);
  return hipGetLastError();
}

hipError_t launch_rowwindows_fill(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                  const int32_t* win_col_ptr, int32_t* win_cols, uint16_t* tile_mask,
                                  int64_t capacity, void* wsp, hipStream_t s) {
  RwWs ws = carve(wsp, n, nnz);
  const int64_t W = ceil_div(n, 16);
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(rw_fill_kernel, dim3((unsigned)W), dim3(kThreads), 0, s, n, nnz, row_ptr, col_idx, win_col_ptr,
                     win_cols, (uint32_t*)tile_mask, capacity, ws);
  return hipGetLastError();
}

// Per-window dispatch flag of a hybrid plan: -1 when window w goes to the MFMA
// path (it has columns and nnz_w >= min_density * 16 * cols_w, compared in
// double), else its edge count nnz_w (>= 0), which sizes the gather share.
__global__ __launch_bounds__(kThreads) void hybrid_flags_kernel(int32_t n, const int32_t* __restrict__ row_ptr,
                                                                 const int32_t* __restrict__ win_col_ptr, int32_t W,
                                                                 float min_density, int32_t* __restrict__ flags) {
  const int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (w >= W) return;
  const int32_t r0 = (int32_t)(16 * w), r1 = (int32_t)min<int64_t>(16 * w + 16, n);
  const int32_t edges = max(row_ptr[r1] - row_ptr[r0], 0);
  const int32_t cols = max(win_col_ptr[w + 1] - win_col_ptr[w], 0);
  const bool dense = cols > 0 && (double)edges >= (double)min_density * 16.0 * (double)cols;
  flags[w] = dense ? -1 : edges;
}

hipError_t launch_hybrid_flags(int32_t n, const int32_t* row_ptr, const int32_t* win_col_ptr, int32_t num_windows,
                               float min_density, int32_t* flags, hipStream_t s) {
  if (num_windows == 0) return hipSuccess;
  hipLaunchKernelGGL(hybrid_flags_kernel, dim3((unsigned)ceil_div(num_windows, kThreads)), dim3(kThreads), 0, s, n,
                     row_ptr, win_col_ptr, num_windows, min_density, flags);
  return hipGetLastError();
}

}  // namespace gattn
