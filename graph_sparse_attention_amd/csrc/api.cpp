// api.cpp -- the C ABI of libgattn: argument checks, path choice, launches.
// Every argument error is detected here, before anything is enqueued.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "gattn.h"
#include "internal.hpp"

using namespace gattn;

// the Python binding mirrors these layouts with ctypes
static_assert(sizeof(gattn_forward_args) == 184, "gattn_forward_args layout");
static_assert(sizeof(gattn_hybrid) == 32, "gattn_hybrid layout");
static_assert(sizeof(gattn_aggregate_args) == 104, "gattn_aggregate_args layout");
static_assert(sizeof(gattn_rowwindows) == 40, "gattn_rowwindows layout");
static_assert(kStaticScratchBytes == GATTN_NOALLOC_SCRATCH_BYTES, "scratch size of gattn_forward_noalloc");

namespace {

// AUTO: nnz / (256 * tiles) at or above -> MFMA.  Measured crossover of the
// two kernels: uniformly random sparse rows (tiles 1/16 full) run no faster
// on the matrix cores and a power-law graph with hub rows (whose windows
// hold up to 2000 columns for one wave) slower, while a batch whose tiles
// are 12% full (half complete digraphs, half sparse blocks) runs 1.6x faster
// there.
constexpr double kMfmaMinDensity = 0.09;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

gattn_status from_hip(hipError_t e) { return e == hipSuccess ? GATTN_OK : GATTN_ERR_HIP; }

size_t elem_size(gattn_dtype t) { return t == GATTN_F32 ? 4 : 2; }

// The integer a C caller stored in an enum field.  Loading an enum object
// whose value lies outside the enum's range is undefined in C++, so every
// enum that crosses the ABI is validated through its bits.
template <typename E>
int32_t raw_enum(const E& e) {
  static_assert(sizeof(E) == sizeof(int32_t), "ABI enums are 32-bit");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

gattn_status check_forward(const gattn_forward_args* a, bool launch) {
  if (!a || a->struct_size != sizeof(gattn_forward_args)) return GATTN_ERR_INVALID_VALUE;
  if (a->num_nodes < 0 || a->num_heads < 1 || a->nnz < 0 || a->nnz > INT32_MAX) return GATTN_ERR_INVALID_VALUE;
  if (raw_enum(a->dtype) < GATTN_F32 || raw_enum(a->dtype) > GATTN_BF16) return GATTN_ERR_INVALID_VALUE;
  if (raw_enum(a->mode) < GATTN_SOFTMAX_STANDARD || raw_enum(a->mode) > GATTN_SOFTMAX_CLIPPED)
    return GATTN_ERR_INVALID_VALUE;
  if (raw_enum(a->path) < GATTN_PATH_AUTO || raw_enum(a->path) > GATTN_PATH_HYBRID) return GATTN_ERR_INVALID_VALUE;
  if (a->flags & ~GATTN_FLAG_VALIDATE) return GATTN_ERR_INVALID_VALUE;
  if (!(a->scale > 0.f) || !(a->scale < INFINITY)) return GATTN_ERR_INVALID_VALUE;
  if (a->mode == GATTN_SOFTMAX_CLIPPED) {
    if (!(a->clip_lo <= a->clip_hi) || !(a->eps >= 0.f) || !(a->eps < INFINITY)) return GATTN_ERR_INVALID_VALUE;
  }
  // the edge update exists in the clipped mode with an edge projection only
  if (a->e_out && (a->mode != GATTN_SOFTMAX_CLIPPED || !a->e)) return GATTN_ERR_INVALID_VALUE;
  if (a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128) return GATTN_ERR_UNSUPPORTED;
  if ((int64_t)a->num_heads * a->head_dim > (int64_t)1 << 20) return GATTN_ERR_UNSUPPORTED;
  if (a->num_nodes == 0) return GATTN_OK;
  if (!a->row_ptr || !a->q || !a->k || !a->v || (launch && !a->out)) return GATTN_ERR_INVALID_VALUE;
  if (a->nnz > 0 && !a->col_idx) return GATTN_ERR_INVALID_VALUE;
  if (!aligned(a->row_ptr, 4) || !aligned(a->col_idx, 4) || !aligned(a->edge_ids, 4)) return GATTN_ERR_INVALID_VALUE;
  const void* t[] = {a->q, a->k, a->v, a->e, a->out, a->e_out};
  for (const void* p : t)
    if (!aligned(p, 16)) return GATTN_ERR_INVALID_VALUE;
  const int64_t hd = (int64_t)a->num_heads * a->head_dim;
  for (int64_t st : {a->q_stride, a->kv_stride})
    if (st != 0 && (st < hd || st % 8 != 0 || st > ((int64_t)1 << 24))) return GATTN_ERR_INVALID_VALUE;
  const size_t es = elem_size(a->dtype);
  const size_t node_bytes = (size_t)a->num_nodes * hd * es;
  // bytes a strided [N, H, D] view spans: from row 0 to the end of row N - 1
  auto span = [&](int64_t st) { return ((size_t)(a->num_nodes - 1) * (size_t)(st ? st : hd) + (size_t)hd) * es; };
  const size_t q_bytes = span(a->q_stride), kv_bytes = span(a->kv_stride);
  const size_t edge_bytes = (size_t)a->nnz * a->num_heads * a->head_dim * elem_size(a->dtype);
  if (overlap(a->out, node_bytes, a->q, q_bytes) || overlap(a->out, node_bytes, a->k, kv_bytes) ||
      overlap(a->out, node_bytes, a->v, kv_bytes) || overlap(a->out, node_bytes, a->e, edge_bytes))
    return GATTN_ERR_INVALID_VALUE;
  if (a->e_out && a->nnz > 0) {
    const size_t ib = (size_t)a->nnz * 4;
    if (overlap(a->e_out, edge_bytes, a->q, q_bytes) || overlap(a->e_out, edge_bytes, a->k, kv_bytes) ||
        overlap(a->e_out, edge_bytes, a->v, kv_bytes) || overlap(a->e_out, edge_bytes, a->e, edge_bytes) ||
        overlap(a->e_out, edge_bytes, a->out, node_bytes) || overlap(a->e_out, edge_bytes, a->row_ptr, 4 * ((size_t)a->num_nodes + 1)) ||
        overlap(a->e_out, edge_bytes, a->col_idx, ib) || overlap(a->e_out, edge_bytes, a->edge_ids, ib))
      return GATTN_ERR_INVALID_VALUE;
  }
  if (a->workspace) {
    const size_t wb = a->workspace_bytes;
    if (!aligned(a->workspace, 256)) return GATTN_ERR_INVALID_VALUE;
    if (overlap(a->workspace, wb, a->q, q_bytes) || overlap(a->workspace, wb, a->k, kv_bytes) ||
        overlap(a->workspace, wb, a->v, kv_bytes) || overlap(a->workspace, wb, a->e, edge_bytes) ||
        overlap(a->workspace, wb, a->out, node_bytes) || overlap(a->workspace, wb, a->e_out, edge_bytes) ||
        overlap(a->workspace, wb, a->row_ptr, 4 * ((size_t)a->num_nodes + 1)) ||
        overlap(a->workspace, wb, a->col_idx, (size_t)a->nnz * 4) ||
        overlap(a->workspace, wb, a->edge_ids, (size_t)a->nnz * 4))
      return GATTN_ERR_INVALID_VALUE;
  }
  return GATTN_OK;
}

gattn_status check_aggregate(const gattn_aggregate_args* a, bool launch) {
  if (!a || a->struct_size != sizeof(gattn_aggregate_args)) return GATTN_ERR_INVALID_VALUE;
  if (a->num_nodes < 0 || a->num_heads < 1 || a->nnz < 0 || a->nnz > INT32_MAX) return GATTN_ERR_INVALID_VALUE;
  if (raw_enum(a->dtype) < GATTN_F32 || raw_enum(a->dtype) > GATTN_BF16) return GATTN_ERR_INVALID_VALUE;
  if (a->normalize != 0 && a->normalize != 1) return GATTN_ERR_INVALID_VALUE;
  if (!(a->eps >= 0.f) || !(a->eps < INFINITY)) return GATTN_ERR_INVALID_VALUE;
  if (a->flags & ~GATTN_FLAG_VALIDATE) return GATTN_ERR_INVALID_VALUE;
  if (a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128) return GATTN_ERR_UNSUPPORTED;
  if ((int64_t)a->num_heads * a->head_dim > (int64_t)1 << 20) return GATTN_ERR_UNSUPPORTED;
  if (a->num_nodes == 0) return GATTN_OK;
  if (!a->row_ptr || !a->x || (launch && !a->out)) return GATTN_ERR_INVALID_VALUE;
  if (a->nnz > 0 && (!a->col_idx || !a->w)) return GATTN_ERR_INVALID_VALUE;
  if (!aligned(a->row_ptr, 4) || !aligned(a->col_idx, 4) || !aligned(a->edge_ids, 4) || !aligned(a->w, 4))
    return GATTN_ERR_INVALID_VALUE;
  if (!aligned(a->x, 16) || !aligned(a->out, 16)) return GATTN_ERR_INVALID_VALUE;
  const size_t node_bytes = (size_t)a->num_nodes * a->num_heads * a->head_dim * elem_size(a->dtype);
  if (overlap(a->out, node_bytes, a->x, node_bytes) ||
      overlap(a->out, node_bytes, a->w, (size_t)a->nnz * a->num_heads * 4) ||
      overlap(a->out, node_bytes, a->row_ptr, 4 * ((size_t)a->num_nodes + 1)) ||
      overlap(a->out, node_bytes, a->col_idx, (size_t)a->nnz * 4) ||
      overlap(a->out, node_bytes, a->edge_ids, (size_t)a->nnz * 4))
    return GATTN_ERR_INVALID_VALUE;
  if (a->workspace) {
    const size_t wb = a->workspace_bytes;
    if (!aligned(a->workspace, 256)) return GATTN_ERR_INVALID_VALUE;
    if (overlap(a->workspace, wb, a->x, node_bytes) || overlap(a->workspace, wb, a->out, node_bytes) ||
        overlap(a->workspace, wb, a->w, (size_t)a->nnz * a->num_heads * 4) ||
        overlap(a->workspace, wb, a->row_ptr, 4 * ((size_t)a->num_nodes + 1)) ||
        overlap(a->workspace, wb, a->col_idx, (size_t)a->nnz * 4) ||
        overlap(a->workspace, wb, a->edge_ids, (size_t)a->nnz * 4))
      return GATTN_ERR_INVALID_VALUE;
  }
  return GATTN_OK;
}

gattn_status check_rw(const gattn_forward_args* a) {
  const gattn_rowwindows* rw = a->rw;
  if (!rw) return GATTN_ERR_INVALID_VALUE;
  if ((int64_t)rw->num_windows != ((int64_t)a->num_nodes + 15) / 16 || rw->num_cols < 0 || rw->num_cols % 16) return GATTN_ERR_INVALID_VALUE;
  if (!rw->win_col_ptr || (rw->num_cols > 0 && (!rw->win_cols || !rw->tile_mask))) return GATTN_ERR_INVALID_VALUE;
  if (!aligned(rw->win_col_ptr, 4) || !aligned(rw->win_cols, 4) || !aligned(rw->tile_mask, 4))
    return GATTN_ERR_INVALID_VALUE;
  return GATTN_OK;
}

// A hybrid plan: counts within the graph's windows and rows, ranges no
// larger than the gather path can stage, arrays present when counts are not 0.
gattn_status check_hybrid(const gattn_forward_args* a) {
  const gattn_hybrid* hy = a->hybrid;
  if (!hy) return GATTN_ERR_INVALID_VALUE;
  const int32_t W = (int32_t)(((int64_t)a->num_nodes + 15) / 16);
  if (hy->num_dense < 0 || hy->num_dense > W || hy->num_ranges < 0 || hy->num_ranges > a->num_nodes)
    return GATTN_ERR_INVALID_VALUE;
  if ((hy->num_dense > 0 && !hy->dense_windows) || (hy->num_ranges > 0 && !hy->ranges)) return GATTN_ERR_INVALID_VALUE;
  if (!aligned(hy->dense_windows, 4) || !aligned(hy->ranges, 4)) return GATTN_ERR_INVALID_VALUE;
  if (hy->num_ranges > 0 && (hy->range_rows < 1 || hy->range_rows > gather_max_range_rows(*a)))
    return GATTN_ERR_INVALID_VALUE;
  return GATTN_OK;
}

gattn_status resolve(const gattn_forward_args* a, gattn_path* out) {
  const bool mf = mfma_supported(*a);
  if (a->path == GATTN_PATH_GATHER) { *out = GATTN_PATH_GATHER; return GATTN_OK; }
  if (a->path == GATTN_PATH_HYBRID || (a->path == GATTN_PATH_AUTO && a->hybrid && mf)) {
    if (!mf) return GATTN_ERR_UNSUPPORTED;
    gattn_status st = check_rw(a);
    if (st == GATTN_OK) st = check_hybrid(a);
    if (st != GATTN_OK) return st;
    *out = GATTN_PATH_HYBRID;
    return GATTN_OK;
  }
  if (a->path == GATTN_PATH_MFMA) {
    if (!mf) return GATTN_ERR_UNSUPPORTED;
    gattn_status st = check_rw(a);
    if (st != GATTN_OK) return st;
    *out = GATTN_PATH_MFMA;
    return GATTN_OK;
  }
  *out = GATTN_PATH_GATHER;
  if (mf && a->rw && check_rw(a) == GATTN_OK && a->rw->num_cols > 0) {
    const double density = (double)a->nnz / (16.0 * (double)a->rw->num_cols);
    if (density >= kMfmaMinDensity) *out = GATTN_PATH_MFMA;
  }
  return GATTN_OK;
}

// GATTN_FLAG_VALIDATE: row pointers, column indices and the edge-id map
// (nullable; values in [0, nnz)) checked on the device; with `permutation`
// each id must also occur once, which is checked on the host (a copy of the
// ids; only the edge update, whose rows two positions must not share, asks).
gattn_status validate_graph(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                            const int32_t* ids, bool permutation, hipStream_t s) {
  bool ok = false;
  if (validate_on_device(n, nnz, row_ptr, col_idx, ids, s, &ok) != hipSuccess) return GATTN_ERR_HIP;
  if (!ok) return GATTN_ERR_BAD_GRAPH;
  if (permutation && ids && nnz > 0) {
    std::vector<int32_t> id((size_t)nnz);
    if (hipMemcpyAsync(id.data(), ids, id.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess) return GATTN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GATTN_ERR_HIP;
    std::vector<uint8_t> seen(id.size(), 0);
    for (int32_t r : id) {  // in range: checked above
      if (seen[r]) return GATTN_ERR_BAD_GRAPH;
      seen[r] = 1;
    }
  }
  return GATTN_OK;
}

}  // namespace

extern "C" {

int gattn_abi_version(void) { return GATTN_ABI_VERSION; }

const char* gattn_status_string(gattn_status status) {
  switch (raw_enum(status)) {
    case GATTN_OK: return "ok";
    case GATTN_ERR_INVALID_VALUE: return "invalid argument";
    case GATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GATTN_ERR_BAD_GRAPH: return "malformed graph (index out of range or bad row pointer)";
    case GATTN_ERR_DUPLICATE_EDGE: return "repeated (destination, source) pair";
    case GATTN_ERR_BUFFER_TOO_SMALL: return "buffer or workspace too small";
    case GATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

gattn_status gattn_build_csr_workspace(int32_t num_nodes, int64_t nnz, size_t* bytes) {
  if (!bytes || num_nodes < 0 || nnz < 0 || nnz > INT32_MAX) return GATTN_ERR_INVALID_VALUE;
  *bytes = build_csr_workspace_bytes(num_nodes, nnz);
  return GATTN_OK;
}

gattn_status gattn_build_csr(int32_t num_nodes, int64_t nnz, const int32_t* src, const int32_t* dst, int32_t* row_ptr,
                             int32_t* col_idx, int32_t* edge_perm, void* workspace, size_t workspace_bytes,
                             int32_t* status_dev, hipStream_t stream) {
  try {
    if (num_nodes < 0 || nnz < 0 || nnz > INT32_MAX || !row_ptr) return GATTN_ERR_INVALID_VALUE;
    if (nnz > 0 && (!src || !dst || !col_idx)) return GATTN_ERR_INVALID_VALUE;
    if (!workspace || !aligned(workspace, 256)) return GATTN_ERR_INVALID_VALUE;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) ||
        !aligned(edge_perm, 4) || !aligned(status_dev, 4))
      return GATTN_ERR_INVALID_VALUE;
    if (workspace_bytes < build_csr_workspace_bytes(num_nodes, nnz)) return GATTN_ERR_BUFFER_TOO_SMALL;
    gattn_status st = from_hip(launch_build_csr(num_nodes, nnz, src, dst, row_ptr, col_idx, edge_perm, workspace,
                                                status_dev, stream));
    if (st != GATTN_OK || status_dev) return st;
    // workspace head: [0] a bad index was seen, [2] the scan's bounded wait ran out
    int32_t flags[3] = {0, 0, 0};
    if (hipMemcpyAsync(flags, workspace, sizeof(flags), hipMemcpyDeviceToHost, stream) != hipSuccess) return GATTN_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GATTN_ERR_HIP;
    if (flags[0]) return GATTN_ERR_BAD_GRAPH;
    return flags[2] ? GATTN_ERR_HIP : GATTN_OK;
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_build_rowwindows_workspace(int32_t num_nodes, int64_t nnz, size_t* bytes) {
  if (!bytes || num_nodes < 0 || nnz < 0 || nnz > INT32_MAX) return GATTN_ERR_INVALID_VALUE;
  *bytes = rowwindows_workspace_bytes(num_nodes, nnz);
  return GATTN_OK;
}

gattn_status gattn_build_rowwindows(int32_t num_nodes, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                    int32_t* win_col_ptr, int32_t* win_cols, uint16_t* tile_mask, int64_t* num_cols,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (num_nodes < 0 || nnz < 0 || nnz > INT32_MAX || !row_ptr || !win_col_ptr || !num_cols)
      return GATTN_ERR_INVALID_VALUE;
    if (nnz > 0 && !col_idx) return GATTN_ERR_INVALID_VALUE;
    if (!workspace || !aligned(workspace, 256)) return GATTN_ERR_INVALID_VALUE;
    if (!aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(win_col_ptr, 4) || !aligned(win_cols, 4) ||
        !aligned(tile_mask, 4))
      return GATTN_ERR_INVALID_VALUE;
    if (workspace_bytes < rowwindows_workspace_bytes(num_nodes, nnz)) return GATTN_ERR_BUFFER_TOO_SMALL;
    const int64_t W = ((int64_t)num_nodes + 15) / 16;
    // win_col_ptr is int32: its total, at most nnz + 15 W, must fit
    if (nnz + 15 * W > INT32_MAX) return GATTN_ERR_UNSUPPORTED;
    if (!win_cols) {
      // call 1: sizes and checks; the status lives in the workspace's first 256 bytes
      int32_t* status_dev = (int32_t*)workspace + 1;
      hipError_t e = launch_rowwindows_count(num_nodes, nnz, row_ptr, col_idx, win_col_ptr, workspace, status_dev, stream);
      if (e != hipSuccess) return GATTN_ERR_HIP;
      int32_t host[2] = {0, 0};
      if (hipMemcpyAsync(&host[0], win_col_ptr + W, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return GATTN_ERR_HIP;
      if (hipMemcpyAsync(&host[1], status_dev, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return GATTN_ERR_HIP;
      if (hipStreamSynchronize(stream) != hipSuccess) return GATTN_ERR_HIP;
      if (host[1] != GATTN_OK) return (gattn_status)host[1];
      *num_cols = host[0];
      return GATTN_OK;
    }
    // call 2
    if (!tile_mask || *num_cols < 0 || *num_cols % 16) return GATTN_ERR_INVALID_VALUE;
    int32_t total = 0;
    if (hipMemcpyAsync(&total, win_col_ptr + W, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return GATTN_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GATTN_ERR_HIP;
    if (total < 0 || total > *num_cols) return GATTN_ERR_BUFFER_TOO_SMALL;
    return from_hip(launch_rowwindows_fill(num_nodes, nnz, row_ptr, col_idx, win_col_ptr, win_cols, tile_mask,
                                           *num_cols, workspace, stream));
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_forward_path(const gattn_forward_args* args, gattn_path* path) {
  if (!path) return GATTN_ERR_INVALID_VALUE;
  gattn_status st = check_forward(args, false);
  if (st != GATTN_OK) return st;
  return resolve(args, path);
}

gattn_status gattn_build_hybrid(const gattn_forward_args* args, float min_density, int32_t* dense_windows,
                                int32_t* ranges, gattn_hybrid* plan, hipStream_t stream) {
  try {
    if (!plan) return GATTN_ERR_INVALID_VALUE;
    gattn_status st = check_forward(args, false);
    if (st != GATTN_OK) return st;
    if (!mfma_supported(*args)) return GATTN_ERR_UNSUPPORTED;
    if ((st = check_rw(args)) != GATTN_OK) return st;
    if (!(min_density >= 0.f) || !(min_density < INFINITY)) return GATTN_ERR_INVALID_VALUE;
    const int32_t n = args->num_nodes, W = (int32_t)(((int64_t)n + 15) / 16);
    if (n > 0 && (!dense_windows || !ranges)) return GATTN_ERR_INVALID_VALUE;
    if (!aligned(dense_windows, 4) || !aligned(ranges, 4)) return GATTN_ERR_INVALID_VALUE;
    *plan = gattn_hybrid{0, 0, 1, dense_windows, ranges};
    if (n == 0) return GATTN_OK;
    // one flag per window on the device (into dense_windows), read back
    if (hipError_t e = launch_hybrid_flags(n, args->row_ptr, args->rw->win_col_ptr, W, min_density, dense_windows,
                                           stream);
        e != hipSuccess)
      return GATTN_ERR_HIP;
    std::vector<int32_t> flags((size_t)W);
    if (hipMemcpyAsync(flags.data(), dense_windows, flags.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return GATTN_ERR_HIP;
    // the dense list, and the sparse rows cut into ranges of consecutive rows
    std::vector<int32_t> dense, rng;
    int32_t sparse_rows = 0;
    int64_t sparse_nnz = 0;
    for (int32_t w = 0; w < W; ++w) {
      if (flags[w] < 0) {
        dense.push_back(w);
      } else {
        sparse_rows += std::min(16, n - 16 * w);
        sparse_nnz += flags[w];
      }
    }
    const int32_t R = sparse_rows > 0 ? std::max(1, std::min(hybrid_rows_per_range(*args, sparse_rows, sparse_nnz),
                                                             gather_max_range_rows(*args)))
                                      : 1;
    int32_t start = -1, count = 0;
    for (int32_t w = 0; w <= W; ++w) {
      const bool sparse = w < W && flags[w] >= 0;
      for (int32_t r = 16 * w; sparse && r < std::min(16 * w + 16, n); ++r) {
        if (count > 0 && (start + count != r || count == R)) {
          rng.push_back(start);
          rng.push_back(count);
          count = 0;
        }
        if (count == 0) start = r;
        ++count;
      }
      if (!sparse && count > 0) {
        rng.push_back(start);
        rng.push_back(count);
        count = 0;
      }
    }
    if (!dense.empty() && hipMemcpyAsync(dense_windows, dense.data(), dense.size() * 4, hipMemcpyHostToDevice,
                                         stream) != hipSuccess)
      return GATTN_ERR_HIP;
    if (!rng.empty() &&
        hipMemcpyAsync(ranges, rng.data(), rng.size() * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
      return GATTN_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GATTN_ERR_HIP;
    *plan = gattn_hybrid{(int32_t)dense.size(), (int32_t)(rng.size() / 2), R, dense_windows, ranges};
    return GATTN_OK;
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_forward_workspace(const gattn_forward_args* args, size_t* bytes) {
  try {
    if (!bytes) return GATTN_ERR_INVALID_VALUE;
    gattn_status st = check_forward(args, false);
    if (st != GATTN_OK) return st;
    *bytes = forward_gather_workspace_bytes(*args);
    return GATTN_OK;
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_aggregate_workspace(const gattn_aggregate_args* args, size_t* bytes) {
  try {
    if (!bytes) return GATTN_ERR_INVALID_VALUE;
    gattn_status st = check_aggregate(args, false);
    if (st != GATTN_OK) return st;
    *bytes = aggregate_workspace_bytes(*args);
    return GATTN_OK;
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_forward(const gattn_forward_args* args, hipStream_t stream) {
  try {
    gattn_status st = check_forward(args, true);
    if (st != GATTN_OK) return st;
    gattn_path path;
    if ((st = resolve(args, &path)) != GATTN_OK) return st;
    if (args->num_nodes == 0) return GATTN_OK;
    if (args->flags & GATTN_FLAG_VALIDATE) {
      const int32_t* ids = args->e ? args->edge_ids : nullptr;  // read only with an edge tensor
      if ((st = validate_graph(args->num_nodes, args->nnz, args->row_ptr, args->col_idx, ids, args->e_out != nullptr,
                               stream)) != GATTN_OK)
        return st;
    }
    if (path == GATTN_PATH_MFMA) return from_hip(launch_forward_mfma(*args, nullptr, 0, stream));
    if (path == GATTN_PATH_HYBRID) {
      const gattn_hybrid* hy = args->hybrid;
      if ((st = from_hip(launch_forward_mfma(*args, hy->dense_windows, hy->num_dense, stream))) != GATTN_OK) return st;
      return from_hip(launch_forward_gather_ranges(*args, hy->ranges, hy->num_ranges, hy->range_rows, stream));
    }
    if (args->workspace && args->workspace_bytes < forward_gather_workspace_bytes(*args))
      return GATTN_ERR_BUFFER_TOO_SMALL;
    return from_hip(launch_forward_gather(*args, stream));
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_forward_noalloc(const gattn_forward_args* args, hipStream_t stream) {
  try {
    gattn_status st = check_forward(args, true);
    if (st != GATTN_OK) return st;
    // the scratch is the library's; validation would copy to the host
    if (args->workspace || args->workspace_bytes || (args->flags & GATTN_FLAG_VALIDATE))
      return GATTN_ERR_INVALID_VALUE;
    gattn_path path;
    if ((st = resolve(args, &path)) != GATTN_OK) return st;
    if (args->num_nodes == 0) return GATTN_OK;
    if (path == GATTN_PATH_MFMA) return from_hip(launch_forward_mfma(*args, nullptr, 0, stream));
    if (path == GATTN_PATH_HYBRID) {
      const gattn_hybrid* hy = args->hybrid;
      if ((st = from_hip(launch_forward_mfma(*args, hy->dense_windows, hy->num_dense, stream))) != GATTN_OK) return st;
      return from_hip(launch_forward_gather_ranges(*args, hy->ranges, hy->num_ranges, hy->range_rows, stream));
    }
    const size_t need = forward_gather_workspace_bytes(*args);
    if (need > kStaticScratchBytes) return GATTN_ERR_BUFFER_TOO_SMALL;
    void* scratch = nullptr;
    if (static_scratch(&scratch) != hipSuccess) return GATTN_ERR_HIP;
    gattn_forward_args a = *args;
    a.workspace = scratch;
    a.workspace_bytes = kStaticScratchBytes;
    return from_hip(launch_forward_gather(a, stream));
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

gattn_status gattn_aggregate(const gattn_aggregate_args* args, hipStream_t stream) {
  try {
    gattn_status st = check_aggregate(args, true);
    if (st != GATTN_OK) return st;
    if (args->num_nodes == 0) return GATTN_OK;
    if (args->flags & GATTN_FLAG_VALIDATE) {
      if ((st = validate_graph(args->num_nodes, args->nnz, args->row_ptr, args->col_idx, args->edge_ids, false,
                               stream)) != GATTN_OK)
        return st;
    }
    if (args->workspace && args->workspace_bytes < aggregate_workspace_bytes(*args)) return GATTN_ERR_BUFFER_TOO_SMALL;
    return from_hip(launch_aggregate_gather(*args, stream));
  } catch (...) {
    return GATTN_ERR_HIP;
  }
}

}  // extern "C"
