// internal.hpp -- host-side launchers shared between api.cpp and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "gattn.h"

namespace gattn {

// Exclusive prefix sum of in[0..n) into out[0..n]; out[n] = total.  in may
// equal out.  `blocksums` needs scan_blocksums_len(n) ints.
int64_t scan_blocksums_len(int64_t n);
hipError_t launch_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* blocksums, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);

// Single-pass exclusive scan (out[n] = total).  tile_status [scan_tiles(n)]
// and *ticket must be zero on entry; a bounded wait that runs out sets
// err[0] = 1 and, if given, *status_dev = GATTN_ERR_HIP.
int64_t scan_tiles(int64_t n);
hipError_t launch_scan_lookback(const int32_t* in, int32_t* out, int64_t n, uint64_t* tile_status, int32_t* ticket,
                                int32_t* err, int32_t* status_dev, hipStream_t s);

// CSR build ------------------------------------------------------------------
size_t build_csr_workspace_bytes(int32_t n, int64_t nnz);
hipError_t launch_build_csr(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst,
                            int32_t* row_ptr, int32_t* col_idx, int32_t* edge_perm,
                            void* ws, int32_t* status_dev, hipStream_t s);
// stable radix-sort build for large edge lists (n >= 1, nnz >= 1); same result
size_t build_csr_radix_workspace_bytes(int32_t n, int64_t nnz);
hipError_t launch_build_csr_radix(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst,
                                  int32_t* row_ptr, int32_t* col_idx, int32_t* edge_perm,
                                  void* ws, int32_t* status_dev, hipStream_t s);
// sort each row's 64-bit (source << 32 | edge id) keys into col_idx / edge_perm;
// run_flag (nullable): the launch does nothing when *run_flag == 0
hipError_t launch_sort_rows(int32_t n, int64_t nnz, const int32_t* row_ptr, uint64_t* keys, uint64_t* tmp,
                            int32_t* col_idx, int32_t* edge_perm, const int32_t* run_flag, hipStream_t s);

// Row windows -----------------------------------------------------------------
size_t rowwindows_workspace_bytes(int32_t n, int64_t nnz);
// phase 1: win_col_ptr and status (status_dev: GATTN_OK / BAD_GRAPH / DUPLICATE_EDGE)
hipError_t launch_rowwindows_count(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                   int32_t* win_col_ptr, void* ws, int32_t* status_dev, hipStream_t s);
hipError_t launch_rowwindows_fill(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                  const int32_t* win_col_ptr, int32_t* win_cols, uint16_t* tile_mask,
                                  int64_t capacity, void* ws, hipStream_t s);

// Forward -------------------------------------------------------------------
hipError_t launch_forward_gather(const gattn_forward_args& a, hipStream_t s);
// GATTN_FLAG_VALIDATE's range checks of row_ptr, col_idx and the edge-id map
// (nullable) on the device; synchronizes the stream, *ok tells the result.
hipError_t validate_on_device(int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                              const int32_t* ids, hipStream_t s, bool* ok);
// windows: nullable list of the windows to run (count num_windows); else all
hipError_t launch_forward_mfma(const gattn_forward_args& a, const int32_t* windows, int32_t num_windows, hipStream_t s);
// gather over given (first row, row count) ranges of at most range_rows rows
// (range_rows <= hybrid_rows_per_range for the same geometry)
hipError_t launch_forward_gather_ranges(const gattn_forward_args& a, const int32_t* ranges, int32_t num_ranges,
                                        int32_t range_rows, hipStream_t s);
// most rows one gather range may hold (their Q rows must fit in LDS)
int32_t gather_max_range_rows(const gattn_forward_args& a);
// rows per gather range of a hybrid plan whose gather share has `rows` rows and `nnz` edges
int32_t hybrid_rows_per_range(const gattn_forward_args& a, int32_t rows, int64_t nnz);
// flags[w] = -1 when window w goes to the MFMA path, else its edge count (see gattn_build_hybrid)
hipError_t launch_hybrid_flags(int32_t n, const int32_t* row_ptr, const int32_t* win_col_ptr, int32_t num_windows,
                               float min_density, int32_t* flags, hipStream_t s);
hipError_t launch_aggregate_gather(const gattn_aggregate_args& a, hipStream_t s);
// bytes of the workspace that selects the balanced partition (0 for N = 0)
size_t forward_gather_workspace_bytes(const gattn_forward_args& a);
size_t aggregate_workspace_bytes(const gattn_aggregate_args& a);
// applicability of the MFMA row-window path (no launch)
bool mfma_supported(const gattn_forward_args& a);

// The fixed scratch array of gattn_forward_noalloc (one per GPU, alive until
// the process ends) and its device address on the current device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gattn
