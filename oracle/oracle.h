/* oracle.h -- CPU oracle for fused graph sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously correct fp64
 * restatement of what the HIP library computes.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never calls it.  It shares no code, header, table or constant with
 * the library.
 *
 * Graph convention: an edge j -> i has source j and destination i.  The
 * destination-grouped index is a pointer vector of N+1 entries plus one
 * source per edge (the CSC of the connection matrix G[src, dst] in the
 * gattn-triton article's "Using the CSC index for fast edge lookup"
 * section; row_ptr / col_idx in the POPCORNBENCH problem statement).
 */
#ifndef GSA_ORACLE_H
#define GSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_INVALID = 1,     /* bad sizes / null pointers                       */
  ORC_BAD_GRAPH = 2,   /* index out of range, row_ptr not a valid pointer */
  ORC_DUPLICATE = 3,   /* a (dst, src) pair repeats (row windows only)    */
  ORC_NOMEM = 4
};

/* COO -> destination-grouped CSR in canonical order (dst, src, edge id).
 * row_ptr [n+1], col_idx [nnz], edge_perm [nnz] (original edge id of the
 * entry at each CSR position). */
int orc_build_csr(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst,
                  int32_t* row_ptr, int32_t* col_idx, int32_t* edge_perm);

/* Row windows of 16 rows, column tiles of 16 (Fused3S, Figure 1 caption:
 * row windows compacted, then cut into tensor-core blocks with a binary
 * mask).  Pass 1 fills win_col_ptr [ceil(n/16)+1]. */
int orc_rowwindow_sizes(int32_t n, const int32_t* row_ptr, const int32_t* col_idx,
                        int32_t* win_col_ptr);
/* Pass 2 fills win_cols [win_col_ptr[W]] and tile_mask [win_col_ptr[W]/16][16]. */
int orc_build_rowwindows(int32_t n, const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* win_col_ptr, int32_t* win_cols, uint16_t* tile_mask);

/* Fused 3S forward, fp64.  q, k, v: [n, h, d]; e: [nnz, h, d] or NULL,
 * row edge_ids[p] for CSR position p (edge_ids NULL: row p).  clipped = 0:
 * standard softmax; 1: RTMScore clipped exp normalised by (sum + eps).
 * rows: destinations to compute (NULL = all n, in order); out / mag:
 * [nrows, h, d]; mag = sum_p alpha_p |v_p| (nullable); alpha: [nnz, h] by
 * CSR position (nullable; only positions of computed rows are written);
 * e_out: [nnz, h, d] (nullable, clipped mode with e only), the RTMScore
 * edge update clamp(scale q k) e, stored at the same row as e.  threads:
 * OpenMP threads over destinations (results do not depend on it). */
int orc_forward(int32_t n, int32_t h, int32_t d, int64_t nnz,
                const int32_t* row_ptr, const int32_t* col_idx,
                const double* q, const double* k, const double* v, const double* e,
                const int32_t* edge_ids,
                int clipped, double scale, double lo, double hi, double eps,
                const int32_t* rows, int64_t nrows,
                double* out, double* mag, double* alpha, double* e_out, int threads);

/* Weighted aggregation (the POPCORNBENCH CSR problem; with normalize = 1 the
 * gattn-triton article's scatter add divided by the summed scores + eps):
 * out[i, h, :] = sum_p w[id(p), h] x[col_idx[p], h, :]  (/ (sum_p w + eps)),
 * id(p) = edge_ids ? edge_ids[p] : p.  x: [n, h, d]; w: [nnz, h]. */
int orc_aggregate(int32_t n, int32_t h, int32_t d, int64_t nnz,
                  const int32_t* row_ptr, const int32_t* col_idx,
                  const double* x, const double* w, const int32_t* edge_ids,
                  int normalize, double eps, double* out, int threads);

#ifdef __cplusplus
}
#endif
#endif
