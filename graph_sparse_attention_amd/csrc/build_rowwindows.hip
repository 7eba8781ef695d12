// build_rowwindows.hip -- CSR -> 16-row windows of compacted, 16-wide,
// bit-masked column tiles (Fused3S, Figure 1: a row window is compacted to
// the columns it uses and stored as tensor-core-sized blocks with a binary
// mask).  Tiles are 16 x 16 here to match the 16x16 MFMA output of gfx950.
//
// One workgroup per window.  The window's edges become 64-bit keys
// (src << 4 | row-in-window); after sorting them, distinct sources are the
// positions where src changes, a repeated key is a repeated (dst, src) pair,
// and the running count of distinct sources gives each key its column.
// A window whose sources span fewer than 4096 values (every window of a batch
// of small graphs) skips the sort: a bitmap of its sources in LDS gives the
// ascending distinct sources and, by popcounts, each edge's column; a bitmap
// per row finds repeated edges.  Otherwise the counting pass sorts the window
// once and leaves the sorted keys in the workspace for the fill pass.  Windows up to 2048 edges
// sort in registers (bitonic: shuffles, in-thread swaps, three rounds through
// 16 KiB of LDS, so several windows share a CU); longer ones sort 2048-key
// chunks that way and merge them pairwise (stable merges through both key
// arrays of the workspace).  The output does not depend on the order of the
// sources inside a CSR row.
#include "common.hpp"
#include "internal.hpp"
#include "merge_runs.hpp"

namespace gattn {

namespace {

constexpr int kCap = 2048;      // keys per LDS sort
constexpr int kMaskCap = 2048;  // padded columns whose masks are assembled in LDS
constexpr int kThreads = 256;
static_assert(kCap == kMergeTile && kThreads == kMergeThreads, "merge tiles staged in the sort buffer");
constexpr int kSpanBits = 4096; // a window whose sources span fewer values takes the bitmap
constexpr int kSpanWords = kSpanBits / 32;

// flag words at the head of the workspace: [0] bit 0 bad graph, bit 1
// duplicate edge; [1] status of call 1; [2] the scan's wait ran out; [3] ticket
enum { kFlags = 0, kStatus = 1, kScanErr = 2, kTicket = 3 };

struct RwWs {
  int32_t* flags;        // [64]
  int32_t* counts;       // [W] padded column count per window
  uint64_t* tile_status; // [scan_tiles(W)]
  uint64_t* keys_a;      // [nnz] long-window chunks
  uint64_t* keys_b;      // [nnz] every window's sorted keys, at its CSR offset
  int64_t clear_ints;    // flags + tile status
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

RwWs carve(void* ws, int32_t n, int64_t nnz) {
  const int64_t W = ceil_div(n, 16);
  uint8_t* p = (uint8_t*)ws;
  RwWs w;
  w.flags = (int32_t*)p;
  p += 256;
  w.tile_status = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * scan_tiles(W));
  w.clear_ints = (p - (uint8_t*)ws) / 4;
  w.counts = (int32_t*)p;
  p += align256(sizeof(int32_t) * std::max<int64_t>(W, 1));
  w.keys_a = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
  w.keys_b = (uint64_t*)p;
  return w;
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

// The window's CSR range [st, st + len) from row_ptr clamped to [0, nnz]
// (a malformed row_ptr cannot send an access out of bounds); s_rp[r] =
// clamped row_ptr[r0 + r] for r <= rows.  Flags a malformed row_ptr.
__device__ void window_range(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr, int32_t w, int32_t* s_rp,
                             int32_t* s_flag, int32_t& st, int32_t& len) {
  const int32_t r0 = 16 * w, rows = min(16, n - r0);
  const int32_t nnz_i = (int32_t)nnz;
  const int t = threadIdx.x;
  if (t <= rows) {
    const int32_t v = row_ptr[r0 + t];
    s_rp[t] = min(max(v, 0), nnz_i);
    bool bad = v < 0 || v > nnz_i;
    if (r0 + t == 0 && v != 0) bad = true;
    if (r0 + t == n && v != nnz_i) bad = true;
    if (bad) atomicOr(s_flag, 1);
  }
  __syncthreads();
  if (t < rows && s_rp[t + 1] < s_rp[t]) atomicOr(s_flag, 1);
  st = s_rp[0];
  len = max(s_rp[rows] - st, 0);
  // a decreasing row_ptr must not make rows overlap: clamp to a running max
  __syncthreads();
  if (t == 0)
    for (int r = 1; r <= rows; ++r) s_rp[r] = max(s_rp[r], s_rp[r - 1]);
  __syncthreads();
}

// key of CSR position p (st <= p < st + len): its source and its row inside the window
__device__ __forceinline__ uint64_t window_key(int32_t n, const int32_t* __restrict__ col_idx, const int32_t* s_rp,
                                               int rows, int32_t p, bool& bad) {
  int lo = 0, hi = rows - 1;  // last row r with s_rp[r] <= p
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_rp[mid] <= p) lo = mid; else hi = mid - 1;
  }
  int32_t s = col_idx[p];
  if ((uint32_t)s >= (uint32_t)n) {
    bad = true;
    s = 0;
  }
  return ((uint64_t)(uint32_t)s << 4) | (uint64_t)lo;
}

// source and row-in-window of CSR position p (a bad source counts as 0)
__device__ __forceinline__ int32_t window_edge(int32_t n, const int32_t* __restrict__ col_idx, const int32_t* s_rp,
                                               int rows, int32_t p, int& row, bool& bad) {
  int lo = 0, hi = rows - 1;  // last row r with s_rp[r] <= p
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_rp[mid] <= p) lo = mid; else hi = mid - 1;
  }
  row = lo;
  int32_t s = col_idx[p];
  if ((uint32_t)s >= (uint32_t)n) {
    bad = true;
    s = 0;
  }
  return s;
}

// smallest and largest source of the window's edges (bad sources count as 0)
__device__ void window_span(int32_t n, const int32_t* __restrict__ col_idx, int32_t st, int32_t len, int32_t* s_red,
                            int32_t& smin, int32_t& smax) {
  int32_t mn = INT32_MAX, mx = -1;
  for (int i = threadIdx.x; i < len; i += kThreads) {
    int32_t s = col_idx[st + i];
    if ((uint32_t)s >= (uint32_t)n) s = 0;
    mn = min(mn, s);
    mx = max(mx, s);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    mn = min(mn, __shfl_xor(mn, o, 64));
    mx = max(mx, __shfl_xor(mx, o, 64));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_red[wave] = mn;
    s_red[kThreads / 64 + wave] = mx;
  }
  __syncthreads();
  smin = s_red[0];
  smax = s_red[kThreads / 64];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    smin = min(smin, s_red[w]);
    smax = max(smax, s_red[kThreads / 64 + w]);
  }
  __syncthreads();
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, mask, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

// compare-exchange of registers r and r + M of every thread (stage j = 64 M)
template <int R, int M>
__device__ __forceinline__ void exchange_regs(uint64_t (&x)[R], int base, int k) {
  if constexpr (M < R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r & M) continue;
      const bool up = ((base + 64 * r) & k) == 0;
      const uint64_t a = x[r], b = x[r | M];
      const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
      x[r] = up ? lo : hi;
      x[r | M] = up ? hi : lo;
    }
  }
}

// Ascending bitonic sort of the workgroup's 256 R keys, R per thread: thread
// (wave w, lane l) holds elements w * 64R + 64 r + l in x[r].  Stages whose
// partner is less than 64 away swap across lanes (shuffles), those less than
// 64 R away inside the thread, the rest across waves through s (256 R keys of
// LDS): three LDS rounds for any R, the other stages without a barrier.
template <int R>
__device__ void block_sort(uint64_t (&x)[R], uint64_t* s) {
  constexpr int P = kThreads * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = wave * 64 * R + lane;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      if (j < 64) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = base + 64 * r;
          const uint64_t y = shfl_xor_u64(x[r], j);
          const bool keep_min = ((i & j) == 0) == ((i & k) == 0);
          x[r] = keep_min ? (y < x[r] ? y : x[r]) : (y > x[r] ? y : x[r]);
        }
      } else if (j < 64 * R) {
        if (j == 64) exchange_regs<R, 1>(x, base, k);
        else if (j == 128) exchange_regs<R, 2>(x, base, k);
        else exchange_regs<R, 4>(x, base, k);
      } else {
        __syncthreads();  // the previous LDS round has been read
#pragma unroll
        for (int r = 0; r < R; ++r) s[base + 64 * r] = x[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = base + 64 * r;
          const uint64_t y = s[i ^ j];
          const bool keep_min = ((i & j) == 0) == ((i & k) == 0);
          x[r] = keep_min ? (y < x[r] ? y : x[r]) : (y > x[r] ? y : x[r]);
        }
      }
    }
  }
}

// Sort the keys of window positions [p0, p0 + cnt) (cnt <= kCap) into s[0..cnt):
// the smallest R with 256 R >= cnt, padding keys ~0 sort last.
template <int R>
__device__ void sort_positions(int32_t n, const int32_t* __restrict__ col_idx, const int32_t* s_rp, int rows, int32_t p0,
                               int cnt, uint64_t* s, bool& bad) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = wave * 64 * R + lane;
  uint64_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = base + 64 * r;
    x[r] = i < cnt ? window_key(n, col_idx, s_rp, rows, p0 + i, bad) : ~0ull;
  }
  block_sort<R>(x, s);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) s[base + 64 * r] = x[r];
  __syncthreads();
}

__device__ void sort_window_chunk(int32_t n, const int32_t* __restrict__ col_idx, const int32_t* s_rp, int rows,
                                  int32_t p0, int cnt, uint64_t* s, bool& bad) {
  if (cnt <= kThreads) sort_positions<1>(n, col_idx, s_rp, rows, p0, cnt, s, bad);
  else if (cnt <= 2 * kThreads) sort_positions<2>(n, col_idx, s_rp, rows, p0, cnt, s, bad);
  else if (cnt <= 4 * kThreads) sort_positions<4>(n, col_idx, s_rp, rows, p0, cnt, s, bad);
  else sort_positions<8>(n, col_idx, s_rp, rows, p0, cnt, s, bad);
}

__global__ __launch_bounds__(kThreads) void rw_count_kernel(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col_idx, RwWs ws) {
  __shared__ uint64_t s_keys[kCap];  // sort keys, or the bitmaps of a narrow window
  __shared__ int32_t s_co[kMergeThreads + 1];
  __shared__ int32_t s_rp[17];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int32_t s_red[2 * (kThreads / 64)];
  __shared__ int32_t s_flag;
  const int32_t w = blockIdx.x;
  const int rows = min(16, n - 16 * w);
  if (threadIdx.x == 0) s_flag = 0;
  __syncthreads();
  int32_t st, len;
  window_range(n, nnz, row_ptr, w, s_rp, &s_flag, st, len);
  int32_t smin, smax;
  window_span(n, col_idx, st, len, s_red, smin, smax);
  bool bad = false;
  int32_t distinct = 0, dup = 0;
  if (len > 0 && smax - smin < kSpanBits) {
    // narrow window: one bit per source (distinct sources) and one per (row,
    // source) (a second hit is a repeated edge), no sort and no stored keys
    uint32_t* bits = reinterpret_cast<uint32_t*>(s_keys);  // [kSpanWords]
    uint32_t* rowbits = bits + kSpanWords;                  // [16][kSpanWords]
    for (int i = threadIdx.x; i < 17 * kSpanWords; i += kThreads) bits[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < len; i += kThreads) {
      int row;
      const int32_t b = window_edge(n, col_idx, s_rp, rows, st + i, row, bad) - smin;
      const uint32_t bit = 1u << (b & 31);
      if (atomicOr(&rowbits[row * kSpanWords + (b >> 5)], bit) & bit) dup = 1;
      atomicOr(&bits[b >> 5], bit);
    }
    __syncthreads();
    if (threadIdx.x < kSpanWords) distinct = __popc(bits[threadIdx.x]);
  } else {
    uint64_t* b = ws.keys_b + st;
    if (len <= kCap) {
      sort_window_chunk(n, col_idx, s_rp, rows, st, len, s_keys, bad);
      for (int i = threadIdx.x; i < len; i += kThreads) b[i] = s_keys[i];
    } else {
      uint64_t* a = ws.keys_a + st;
      const int nchunks = (len + kCap - 1) / kCap;
      for (int c = 0; c < nchunks; ++c) {
        const int cs = c * kCap, cl = min(kCap, len - cs);
        sort_window_chunk(n, col_idx, s_rp, rows, st + cs, cl, s_keys, bad);
        for (int i = threadIdx.x; i < cl; i += kThreads) a[cs + i] = s_keys[i];
        __syncthreads();
      }
      // pairwise stable merges of the sorted chunks between the two key
      // arrays (equal keys, i.e. repeated edges, stay adjacent); the result
      // must end in keys_b
      const uint64_t* sorted = merge_sorted_runs(a, b, len, kCap, s_keys, s_co);
      if (sorted != b) {
        for (int i = threadIdx.x; i < len; i += kThreads) b[i] = sorted[i];
        __syncthreads();
      }
    }
    // distinct sources and repeated keys, from the sorted keys: LDS when they
    // fit, else the workspace (two loops, so that no generic pointer can point
    // into LDS: a flat access there is not what these loads should be)
    auto scan_keys = [&](auto keys) {
      for (int i = threadIdx.x; i < len; i += kThreads) {
        const uint64_t k = keys(i);
        const uint64_t prev = i > 0 ? keys(i - 1) : ~k;
        if (i == 0 || (k >> 4) != (prev >> 4)) ++distinct;
        if (i > 0 && k == prev) dup = 1;
      }
    };
    if (len <= kCap) scan_keys([&](int i) { return s_keys[i]; });
    else scan_keys([&](int i) { return b[i]; });
  }
  if (bad) atomicOr(&s_flag, 1);
  if (dup) atomicOr(&s_flag, 2);
  int32_t total;
  block_incl_scan(distinct, s_wave, &total);
  if (threadIdx.x == 0) {
    ws.counts[w] = 16 * ((total + 15) / 16);
    if (s_flag) atomicOr(&ws.flags[kFlags], s_flag);
  }
}

// columns and masks of window w: from the source bitmap of a narrow window,
// else from the keys the counting pass sorted
__global__ __launch_bounds__(kThreads) void rw_fill_kernel(int32_t n, int64_t nnz, const int32_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ col_idx,
                                                           const int32_t* __restrict__ win_col_ptr,
                                                           int32_t* __restrict__ win_cols, uint32_t* __restrict__ mask_words,
                                                           int64_t capacity, RwWs ws) {
  __shared__ uint32_t s_mask[kMaskCap / 2];  // kMaskCap / 16 tiles x 16 rows x 16 bits, two per word
  __shared__ uint32_t s_bits[kSpanWords];
  __shared__ int32_t s_woff[kSpanWords];     // distinct sources in the words before
  __shared__ int32_t s_rp[17];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int32_t s_red[2 * (kThreads / 64)];
  __shared__ int32_t s_flag;
  const int32_t w = blockIdx.x;
  const int rows = min(16, n - 16 * w);
  if (threadIdx.x == 0) s_flag = 0;
  const int64_t base = min<int64_t>(max(win_col_ptr[w], 0), capacity) & ~int64_t(15);
  const int64_t stop = min<int64_t>(max<int64_t>(win_col_ptr[w + 1], base), capacity) & ~int64_t(15);
  const int32_t padded = (int32_t)(stop - base);
  const bool lds_mask = padded <= kMaskCap;
  const int32_t words = padded / 2;  // 16 rows x 16 bits per tile = 8 words
  if (lds_mask) {
    for (int i = threadIdx.x; i < words; i += kThreads) s_mask[i] = 0u;
  } else {
    for (int64_t i = threadIdx.x; i < words; i += kThreads) mask_words[base / 2 + i] = 0u;
  }
  for (int i = threadIdx.x; i < kSpanWords; i += kThreads) s_bits[i] = 0u;
  __syncthreads();
  int32_t st, len;
  window_range(n, nnz, row_ptr, w, s_rp, &s_flag, st, len);
  int32_t smin, smax;
  window_span(n, col_idx, st, len, s_red, smin, smax);
  auto set_mask = [&](int32_t t, int row) {  // column t of row `row`
    const int32_t entry = (t >> 4) * 16 + row;  // [tile][row] inside the window
    const uint32_t bit = (1u << (t & 15)) << (16 * (entry & 1));
    if (lds_mask) atomicOr(&s_mask[entry >> 1], bit);
    else atomicOr(&mask_words[base / 2 + (entry >> 1)], bit);
  };
  int32_t carry = 0;
  if (len > 0 && smax - smin < kSpanBits) {
    bool bad = false;
    for (int i = threadIdx.x; i < len; i += kThreads) {
      int row;
      const int32_t b = window_edge(n, col_idx, s_rp, rows, st + i, row, bad) - smin;
      atomicOr(&s_bits[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    const int32_t pc = threadIdx.x < kSpanWords ? __popc(s_bits[threadIdx.x]) : 0;
    int32_t total;
    const int32_t incl = block_incl_scan(pc, s_wave, &total);
    if (threadIdx.x < kSpanWords) s_woff[threadIdx.x] = incl - pc;
    __syncthreads();
    auto column = [&](int32_t b) {  // rank of source smin + b among the window's sources
      return s_woff[b >> 5] + __popc(s_bits[b >> 5] & ((1u << (b & 31)) - 1u));
    };
    for (int32_t b = threadIdx.x; b <= smax - smin; b += kThreads)
      if ((s_bits[b >> 5] >> (b & 31)) & 1u) {
        const int32_t t = column(b);
        if (t < padded) win_cols[base + t] = smin + b;
      }
    for (int i = threadIdx.x; i < len; i += kThreads) {
      int row;
      const int32_t b = window_edge(n, col_idx, s_rp, rows, st + i, row, bad) - smin;
      const int32_t t = column(b);
      if (t < padded) set_mask(t, row);
    }
    carry = total;
  } else {
    const uint64_t* keys = ws.keys_b + st;
    for (int c = 0; c < len; c += kThreads) {
      const int i = c + threadIdx.x;
      uint64_t k = 0;
      int32_t f = 0;
      if (i < len) {
        k = keys[i];
        f = (i == 0 || (k >> 4) != (keys[i - 1] >> 4)) ? 1 : 0;
      }
      int32_t total;
      const int32_t incl = block_incl_scan(f, s_wave, &total);
      if (i < len) {
        const int32_t t = carry + incl - 1;  // column of this key's source
        if (t >= 0 && t < padded) {
          if (f) win_cols[base + t] = (int32_t)(k >> 4);
          set_mask(t, (int)(k & 15));
        }
      }
      carry += total;
    }
  }
  for (int32_t t = carry + threadIdx.x; t < padded; t += kThreads) win_cols[base + t] = -1;
  if (lds_mask) {
    __syncthreads();
    for (int i = threadIdx.x; i < words; i += kThreads) mask_words[base / 2 + i] = s_mask[i];
  }
}

__global__ void rw_status_kernel(const int32_t* flags, int32_t* status) {
  const int32_t f = flags[kFlags];
  *status = flags[kScanErr] ? GATTN_ERR_HIP
            : (f & 1)       ? GATTN_ERR_BAD_GRAPH
            : (f & 2)       ? GATTN_ERR_DUPLICATE_EDGE
                            : GATTN_OK;
}

}  // namespace

size_t rowwindows_workspace_bytes(int32_t n, int64_t nnz) {
  const int64_t W = ceil_div(n, 16);
  return 256 + align256(sizeof(uint64_t) * scan_tiles(W)) + align256(sizeof(int32_t) * std::max<int64_t>(W, 1)) +
         2 * align256(sizeof(uint64_t) * std::max<int64_t>(nnz, 1));
}

hipError_t launch_rowwindows_count(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                   int32_t* win_col_ptr, void* wsp, int32_t* status_dev, hipStream_t s) {
  RwWs ws = carve(wsp, n, nnz);
  const int64_t W = ceil_div(n, 16);
  hipError_t err;
  if ((err = launch_fill_i32(ws.flags, 0, ws.clear_ints, s)) != hipSuccess) return err;
  if (W > 0) {
    hipLaunchKernelGGL(rw_count_kernel, dim3((unsigned)W), dim3(kThreads), 0, s, n, nnz, row_ptr, col_idx, ws);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = launch_scan_lookback(ws.counts, win_col_ptr, W, ws.tile_status, &ws.flags[kTicket], &ws.flags[kScanErr],
                                  nullptr, s)) != hipSuccess)
    return err;
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
