/* oracle.c -- CPU oracle for fused graph sparse attention (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Everything here
 * is the plain definition, written out as loops; no blocking, fusion or
 * online rescaling.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int cmp_u64(const void* a, const void* b) {
  uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return (x > y) - (x < y);
}
static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Destination-grouped CSR (gattn-triton article, "Using the CSC index for
 * fast edge lookup": edges grouped by destination, a pointer vector whose
 * entry i counts the edges before destination i, one source per edge, and a
 * map from grouped position to original edge id).  The pages leave the order
 * inside a destination open; the canonical order here is (src, edge id). */
int orc_build_csr(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst,
                  int32_t* row_ptr, int32_t* col_idx, int32_t* edge_perm) {
  if (n < 0 || nnz < 0 || nnz > INT32_MAX || !row_ptr) return ORC_INVALID;
  if (nnz > 0 && (!src || !dst || !col_idx)) return ORC_INVALID;
  for (int64_t e = 0; e < nnz; ++e)
    if (src[e] < 0 || src[e] >= n || dst[e] < 0 || dst[e] >= n) return ORC_BAD_GRAPH;

  /* histogram of destinations, exclusive prefix sum */
  for (int32_t i = 0; i <= n; ++i) row_ptr[i] = 0;
  for (int64_t e = 0; e < nnz; ++e) row_ptr[dst[e] + 1] += 1;
  for (int32_t i = 0; i < n; ++i) row_ptr[i + 1] += row_ptr[i];

  /* place edges in id order, then sort each destination's entries by
   * (src, edge id) packed into one unsigned 64-bit key */
  uint64_t* key = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(nnz > 0 ? nnz : 1));
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!key || !fill) { free(key); free(fill); return ORC_NOMEM; }
  for (int32_t i = 0; i < n; ++i) fill[i] = row_ptr[i];
  for (int64_t e = 0; e < nnz; ++e) {
    int32_t p = fill[dst[e]]++;
    key[p] = ((uint64_t)(uint32_t)src[e] << 32) | (uint64_t)(uint32_t)e;
  }
  for (int32_t i = 0; i < n; ++i)
    qsort(key + row_ptr[i], (size_t)(row_ptr[i + 1] - row_ptr[i]), sizeof(uint64_t), cmp_u64);
  for (int64_t p = 0; p < nnz; ++p) {
    col_idx[p] = (int32_t)(key[p] >> 32);
    if (edge_perm) edge_perm[p] = (int32_t)(key[p] & 0xffffffffu);
  }
  free(key);
  free(fill);
  return ORC_OK;
}

static int check_csr(int32_t n, const int32_t* row_ptr, const int32_t* col_idx) {
  if (row_ptr[0] != 0) return ORC_BAD_GRAPH;
  for (int32_t i = 0; i < n; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return ORC_BAD_GRAPH;
  for (int64_t p = 0; p < row_ptr[n]; ++p)
    if (col_idx[p] < 0 || col_idx[p] >= n) return ORC_BAD_GRAPH;
  return ORC_OK;
}

/* Sorted distinct sources of the window's rows into buf; returns the count,
 * or -1 when a row repeats a source (a binary mask cannot hold it). */
static int64_t window_sources(int32_t n, const int32_t* row_ptr, const int32_t* col_idx,
                              int32_t w, int32_t* buf, int32_t* rowbuf) {
  int32_t r0 = 16 * w, r1 = r0 + 16 < n ? r0 + 16 : n;
  for (int32_t r = r0; r < r1; ++r) {
    int32_t b = row_ptr[r], len = row_ptr[r + 1] - b;
    memcpy(rowbuf, col_idx + b, sizeof(int32_t) * (size_t)len);
    qsort(rowbuf, (size_t)len, sizeof(int32_t), cmp_i32);
    for (int32_t t = 1; t < len; ++t)
      if (rowbuf[t] == rowbuf[t - 1]) return -1;
  }
  int32_t b = row_ptr[r0], len = row_ptr[r1] - b;
  memcpy(buf, col_idx + b, sizeof(int32_t) * (size_t)len);
  qsort(buf, (size_t)len, sizeof(int32_t), cmp_i32);
  int64_t u = 0;
  for (int32_t t = 0; t < len; ++t)
    if (t == 0 || buf[t] != buf[t - 1]) buf[u++] = buf[t];
  return u;
}

static int32_t max_window_edges(int32_t n, const int32_t* row_ptr) {
  int32_t m = 1;
  for (int32_t r0 = 0; r0 < n; r0 += 16) {
    int32_t r1 = r0 + 16 < n ? r0 + 16 : n;
    if (row_ptr[r1] - row_ptr[r0] > m) m = row_ptr[r1] - row_ptr[r0];
  }
  return m;
}

/* Fused3S, Figure 1 caption: a row window is compacted to its distinct
 * columns, which are cut into fixed-width blocks with a binary mask.  Here
 * a window is 16 consecutive rows; its ascending distinct sources are padded
 * to a multiple of 16 with -1. */
int orc_rowwindow_sizes(int32_t n, const int32_t* row_ptr, const int32_t* col_idx,
                        int32_t* win_col_ptr) {
  if (n < 0 || !row_ptr || !win_col_ptr) return ORC_INVALID;
  int rc = check_csr(n, row_ptr, col_idx);
  if (rc) return rc;
  int32_t W = (n + 15) / 16;
  int32_t cap = max_window_edges(n, row_ptr);
  int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  int32_t* rowbuf = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  if (!buf || !rowbuf) { free(buf); free(rowbuf); return ORC_NOMEM; }
  int64_t total = 0;
  win_col_ptr[0] = 0;
  for (int32_t w = 0; w < W; ++w) {
    int64_t u = window_sources(n, row_ptr, col_idx, w, buf, rowbuf);
    if (u < 0) { free(buf); free(rowbuf); return ORC_DUPLICATE; }
    total += 16 * ((u + 15) / 16);
    if (total > INT32_MAX) { free(buf); free(rowbuf); return ORC_INVALID; }
    win_col_ptr[w + 1] = (int32_t)total;
  }
  free(buf);
  free(rowbuf);
  return ORC_OK;
}

int orc_build_rowwindows(int32_t n, const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* win_col_ptr, int32_t* win_cols, uint16_t* tile_mask) {
  if (n < 0 || !row_ptr || !win_col_ptr) return ORC_INVALID;
  int rc = check_csr(n, row_ptr, col_idx);
  if (rc) return rc;
  int32_t W = (n + 15) / 16;
  int32_t cap = max_window_edges(n, row_ptr);
  int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  int32_t* rowbuf = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  if (!buf || !rowbuf) { free(buf); free(rowbuf); return ORC_NOMEM; }
  for (int32_t w = 0; w < W; ++w) {
    int64_t u = window_sources(n, row_ptr, col_idx, w, buf, rowbuf);
    if (u < 0) { free(buf); free(rowbuf); return ORC_DUPLICATE; }
    int32_t base = win_col_ptr[w], len = win_col_ptr[w + 1] - base;
    if (len != 16 * ((u + 15) / 16)) { free(buf); free(rowbuf); return ORC_INVALID; }
    for (int32_t t = 0; t < len; ++t) win_cols[base + t] = t < u ? buf[t] : -1;
    for (int32_t t = 0; t < len; ++t) tile_mask[(int64_t)base + t] = 0; /* len/16 tiles x 16 rows */
    int32_t r0 = 16 * w, r1 = r0 + 16 < n ? r0 + 16 : n;
    for (int32_t r = r0; r < r1; ++r) {
      for (int32_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
        int32_t* hit = (int32_t*)bsearch(&col_idx[p], buf, (size_t)u, sizeof(int32_t), cmp_i32);
        int32_t t = (int32_t)(hit - buf);
        int64_t tile = base / 16 + t / 16;
        tile_mask[tile * 16 + (r - r0)] |= (uint16_t)(1u << (t % 16));
      }
    }
  }
  free(buf);
  free(rowbuf);
  return ORC_OK;
}

static double clampd(double x, double lo, double hi) { return x < lo ? lo : (x > hi ? hi : x); }

/* One destination, one head.
 *
 * Logit of edge p = (j -> i):
 *   standard: scale * sum_d q[i,d] k[j,d] (* e[p,d] when E is given)
 *             -- the SDDMM of the Fused3S abstract;
 *   clipped:  t_d = clamp(scale * q[i,d] k[j,d], lo, hi) (* e[p,d]),
 *             logit = clamp(sum_d t_d, lo, hi)
 *             -- gattn-triton article, "Fusing the full graph attention":
 *             the scaled q*k product is clamped elementwise, multiplied by
 *             the edge projection, summed over the feature axis and clamped
 *             again before the exponential.
 * Weights:
 *   standard: w_p = exp(logit_p - max), Z = sum w_p (max-subtracted softmax,
 *             Fused3S abstract); clipped: w_p = exp(logit_p), Z = sum w_p +
 *             eps (article, "Background": alpha = s / (sum s + epsilon)).
 * Output: o = sum_p (w_p / Z) v[j_p]  (article "Background"; SpMM of 3S).
 * A destination without in-edges gets exactly 0 (zero-initialised output of
 * the POPCORNBENCH CSR aggregation; 0/(0+eps) in the clipped form). */
static void one_slice(int32_t i, int32_t hh, int32_t h, int32_t d, const int32_t* row_ptr,
                      const int32_t* col_idx, const double* q, const double* k, const double* v,
                      const double* e, const int32_t* edge_ids, int clipped, double scale, double lo,
                      double hi, double eps, double* o, double* mg, double* alpha, double* e_out,
                      double* logit) {
  int32_t b = row_ptr[i], deg = row_ptr[i + 1] - b;
  for (int32_t c = 0; c < d; ++c) { o[c] = 0.0; if (mg) mg[c] = 0.0; }
  if (deg == 0) return;
  const double* qi = q + ((int64_t)i * h + hh) * d;
  for (int32_t t = 0; t < deg; ++t) {
    int64_t p = b + t;
    const double* kj = k + ((int64_t)col_idx[p] * h + hh) * d;
    const int64_t row = edge_ids ? (int64_t)edge_ids[p] : p;
    const double* ep = e ? e + (row * h + hh) * d : NULL;
    double s = 0.0;
    if (!clipped) {
      for (int32_t c = 0; c < d; ++c) s += qi[c] * kj[c] * (ep ? ep[c] : 1.0);
      logit[t] = scale * s;
    } else {
      for (int32_t c = 0; c < d; ++c) {
        double x = clampd(scale * qi[c] * kj[c], lo, hi);
        if (ep) x *= ep[c];
        if (e_out) e_out[(row * h + hh) * d + c] = x;   /* the edge update before the sum */
        s += x;
      }
      logit[t] = clampd(s, lo, hi);
    }
  }
  double m = 0.0, z = 0.0;
  if (!clipped) {
    m = logit[0];
    for (int32_t t = 1; t < deg; ++t) if (logit[t] > m) m = logit[t];
  }
  for (int32_t t = 0; t < deg; ++t) { logit[t] = exp(logit[t] - m); z += logit[t]; }
  if (clipped) z += eps;
  for (int32_t t = 0; t < deg; ++t) {
    int64_t p = b + t;
    double a = logit[t] / z;
    if (alpha) alpha[p * h + hh] = a;
    const double* vj = v + ((int64_t)col_idx[p] * h + hh) * d;
    for (int32_t c = 0; c < d; ++c) {
      o[c] += a * vj[c];
      if (mg) mg[c] += a * fabs(vj[c]);
    }
  }
}

int orc_forward(int32_t n, int32_t h, int32_t d, int64_t nnz,
                const int32_t* row_ptr, const int32_t* col_idx,
                const double* q, const double* k, const double* v, const double* e,
                const int32_t* edge_ids,
                int clipped, double scale, double lo, double hi, double eps,
                const int32_t* rows, int64_t nrows,
                double* out, double* mag, double* alpha, double* e_out, int threads) {
  if (n < 0 || h < 1 || d < 1 || nnz < 0 || !row_ptr || !out || nrows < 0) return ORC_INVALID;
  if (e_out && (!clipped || !e)) return ORC_INVALID;
  for (int64_t p = 0; edge_ids && p < nnz; ++p)
    if (edge_ids[p] < 0 || edge_ids[p] >= nnz) return ORC_INVALID;
  if (n > 0 && (!q || !k || !v)) return ORC_INVALID;
  if (row_ptr[n] != nnz) return ORC_BAD_GRAPH;
  int rc = check_csr(n, row_ptr, col_idx);
  if (rc) return rc;
  if (!rows && nrows != n) return ORC_INVALID;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= n) return ORC_INVALID;
  int32_t maxdeg = 1;
  for (int32_t i = 0; i < n; ++i)
    if (row_ptr[i + 1] - row_ptr[i] > maxdeg) maxdeg = row_ptr[i + 1] - row_ptr[i];
  int failed = 0;
#ifdef _OPENMP
  if (threads < 1) threads = 1;
#pragma omp parallel num_threads(threads)
#endif
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)maxdeg);
    if (!logit) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
    for (int64_t r = 0; r < nrows; ++r) {
      if (!logit) continue;
      int32_t i = rows ? rows[r] : (int32_t)r;
      for (int32_t hh = 0; hh < h; ++hh)
        one_slice(i, hh, h, d, row_ptr, col_idx, q, k, v, e, edge_ids, clipped, scale, lo, hi, eps,
                  out + (r * h + hh) * d, mag ? mag + (r * h + hh) * d : NULL, alpha, e_out, logit);
    }
    free(logit);
  }
  return failed ? ORC_NOMEM : ORC_OK;
}

/* Weighted aggregation over the in-edges of each destination: the
 * POPCORNBENCH CSR problem (out[dst] = sum of w * node features of the
 * sources, zero for no in-edges) and, with normalize, the gattn-triton
 * article's scatter add of value vectors and scores followed by
 * numerator / (denominator + epsilon). */
int orc_aggregate(int32_t n, int32_t h, int32_t d, int64_t nnz,
                  const int32_t* row_ptr, const int32_t* col_idx,
                  const double* x, const double* w, const int32_t* edge_ids,
                  int normalize, double eps, double* out, int threads) {
  if (n < 0 || h < 1 || d < 1 || nnz < 0 || !row_ptr || !out) return ORC_INVALID;
  if (n > 0 && (!x || (nnz > 0 && !w))) return ORC_INVALID;
  if (row_ptr[n] != nnz) return ORC_BAD_GRAPH;
  int rc = check_csr(n, row_ptr, col_idx);
  if (rc) return rc;
  for (int64_t p = 0; edge_ids && p < nnz; ++p)
    if (edge_ids[p] < 0 || edge_ids[p] >= nnz) return ORC_INVALID;
#ifdef _OPENMP
  if (threads < 1) threads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(threads)
#endif
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t hh = 0; hh < h; ++hh) {
      double* o = out + ((int64_t)i * h + hh) * d;
      double z = 0.0;
      for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int32_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
        const int64_t wrow = edge_ids ? (int64_t)edge_ids[p] : p;
        const double wp = w[wrow * h + hh];
        const double* xj = x + ((int64_t)col_idx[p] * h + hh) * d;
        for (int32_t c = 0; c < d; ++c) o[c] += wp * xj[c];
        z += wp;
      }
      if (normalize && row_ptr[i + 1] > row_ptr[i])
        for (int32_t c = 0; c < d; ++c) o[c] /= (z + eps);
    }
  }
  return ORC_OK;
}
