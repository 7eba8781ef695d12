/* sanitize_driver.c -- the host code under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_sanitizers.py on
 * the CPU; nothing here touches a GPU).
 *
 * Part 1 drives the C ABI of libgattn, built for the host only, through
 * every argument check, size query and planner, with pointers that are
 * aligned but never dereferenced; where every check passes and a call would
 * reach the device, it must return GATTN_ERR_HIP (no device here).
 * Part 2 runs the oracle on small graphs through every entry point and
 * option, checking results that do not depend on rounding (integer outputs,
 * weights that sum to 1 or S/(S+eps), exact zeros, a single in-edge giving
 * its source row, thread count not changing a bit).
 * Any memory error or undefined behaviour aborts the run with a report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gattn.h"
#include "oracle.h"

static int failures = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);  \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

/* aligned addresses, 1 TB apart so that no two tensors of the shapes below
 * overlap, and never dereferenced (the calls return first) */
#define FAKE(i) ((void*)(uintptr_t)((1ull << 44) + ((uint64_t)(i) << 40)))

static gattn_forward_args fwd(void) {
  gattn_forward_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = sizeof a;
  a.num_nodes = 100;
  a.num_heads = 8;
  a.head_dim = 64;
  a.nnz = 1000;
  a.row_ptr = (const int32_t*)FAKE(1);
  a.col_idx = (const int32_t*)FAKE(2);
  a.q = FAKE(3);
  a.k = FAKE(4);
  a.v = FAKE(5);
  a.out = FAKE(6);
  a.dtype = GATTN_F16;
  a.mode = GATTN_SOFTMAX_STANDARD;
  a.scale = 0.125f;
  a.clip_lo = -5.f;
  a.clip_hi = 5.f;
  a.eps = 1e-6f;
  a.path = GATTN_PATH_GATHER;
  return a;
}

static gattn_aggregate_args agg(void) {
  gattn_aggregate_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = sizeof a;
  a.num_nodes = 100;
  a.num_heads = 2;
  a.head_dim = 32;
  a.nnz = 500;
  a.row_ptr = (const int32_t*)FAKE(1);
  a.col_idx = (const int32_t*)FAKE(2);
  a.x = FAKE(3);
  a.w = (const float*)FAKE(4);
  a.out = FAKE(5);
  a.dtype = GATTN_BF16;
  a.eps = 1e-6f;
  return a;
}

static void abi_checks(void) {
  CHECK(gattn_abi_version() == GATTN_ABI_VERSION);
  for (int s = 0; s <= 7; ++s) CHECK(gattn_status_string((gattn_status)s) != NULL);

  /* CSR build */
  size_t bytes = 0;
  CHECK(gattn_build_csr_workspace(10, 100, NULL) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_csr_workspace(-1, 100, &bytes) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_csr_workspace(10, (int64_t)1 << 31, &bytes) == GATTN_ERR_INVALID_VALUE);
  const int64_t sizes[][2] = {{0, 0}, {1, 0}, {320, 4457}, {12197, 121970}, {169343, 622503},
                              {2450000, 101119663}, {1 << 20, 1 << 18}, {7, (1 << 18) - 1}};
  for (unsigned i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) {
    CHECK(gattn_build_csr_workspace((int32_t)sizes[i][0], sizes[i][1], &bytes) == GATTN_OK);
    CHECK(bytes % 256 == 0 || bytes < 256);
  }
  CHECK(gattn_build_csr_workspace(1000, 5000, &bytes) == GATTN_OK);
  CHECK(gattn_build_csr(1000, 5000, FAKE(1), FAKE(2), FAKE(3), FAKE(4), FAKE(5), FAKE(6), bytes - 1, NULL, 0) ==
        GATTN_ERR_BUFFER_TOO_SMALL);
  CHECK(gattn_build_csr(1000, 5000, FAKE(1), FAKE(2), NULL, FAKE(4), NULL, FAKE(6), bytes, NULL, 0) ==
        GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_csr(1000, 5000, (const int32_t*)((char*)FAKE(1) + 2), FAKE(2), FAKE(3), FAKE(4), NULL, FAKE(6),
                        bytes, NULL, 0) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_csr(1000, 5000, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, (char*)FAKE(6) + 128, bytes, NULL,
                        0) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_csr(1000, 5000, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, FAKE(6), bytes, NULL, 0) ==
        GATTN_ERR_HIP);

  /* row windows */
  CHECK(gattn_build_rowwindows_workspace(100, 1000, &bytes) == GATTN_OK);
  int64_t ncols = 0;
  CHECK(gattn_build_rowwindows(100, 1000, FAKE(1), FAKE(2), FAKE(3), NULL, NULL, &ncols, FAKE(4), bytes - 1, 0) ==
        GATTN_ERR_BUFFER_TOO_SMALL);
  CHECK(gattn_build_rowwindows(100, 1000, FAKE(1), FAKE(2), FAKE(3), NULL, NULL, NULL, FAKE(4), bytes, 0) ==
        GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_rowwindows_workspace(INT32_MAX, INT32_MAX - 10, &bytes) == GATTN_OK);
  CHECK(gattn_build_rowwindows(INT32_MAX, INT32_MAX - 10, FAKE(1), FAKE(2), FAKE(3), NULL, NULL, &ncols, FAKE(4),
                               bytes, 0) == GATTN_ERR_UNSUPPORTED);

  /* forward: one mutation per case */
  gattn_forward_args a = fwd();
  gattn_path path;
  CHECK(gattn_forward_path(&a, &path) == GATTN_OK && path == GATTN_PATH_GATHER);
  CHECK(gattn_forward_path(&a, NULL) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_forward(NULL, 0) == GATTN_ERR_INVALID_VALUE);
  a.struct_size -= 8;
  CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.num_heads = 0;                 CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.nnz = -1;                      CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.dtype = (gattn_dtype)7;        CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.mode = (gattn_mode)3;          CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.path = (gattn_path)9;          CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.flags = 2;                     CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.scale = 0.f;                   CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.scale = NAN;                   CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.scale = INFINITY;              CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.mode = GATTN_SOFTMAX_CLIPPED; a.clip_lo = 6.f;  CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.mode = GATTN_SOFTMAX_CLIPPED; a.eps = -1.f;     CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.e_out = FAKE(7);               CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.head_dim = 48;                 CHECK(gattn_forward(&a, 0) == GATTN_ERR_UNSUPPORTED);
  a = fwd(); a.num_heads = 1 << 15;           CHECK(gattn_forward(&a, 0) == GATTN_ERR_UNSUPPORTED);
  a = fwd(); a.q = NULL;                      CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.out = NULL;                    CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.k = (char*)FAKE(4) + 8;        CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.col_idx = (const int32_t*)((char*)FAKE(2) + 2); CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.out = (void*)a.q;                   CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.out = (char*)a.v + 4096;       CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.workspace = (char*)FAKE(8) + 16; a.workspace_bytes = 1 << 20;
  CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);
  a = fwd(); a.path = GATTN_PATH_MFMA;        CHECK(gattn_forward(&a, 0) == GATTN_ERR_INVALID_VALUE);  /* no rw */
  a = fwd(); a.dtype = GATTN_F32; a.path = GATTN_PATH_MFMA; CHECK(gattn_forward(&a, 0) == GATTN_ERR_UNSUPPORTED);
  a = fwd(); a.num_nodes = 0;                 CHECK(gattn_forward(&a, 0) == GATTN_OK);
  a = fwd();                                  CHECK(gattn_forward(&a, 0) == GATTN_ERR_HIP);

  /* row windows on the forward: the path choice and its checks */
  gattn_rowwindows rw = {7, 16 * 8, (const int32_t*)FAKE(9), (const int32_t*)FAKE(10), (const uint16_t*)FAKE(11)};
  a = fwd(); a.path = GATTN_PATH_AUTO; a.rw = &rw;
  CHECK(gattn_forward_path(&a, &path) == GATTN_OK && path == GATTN_PATH_MFMA);
  rw.num_cols = 16 * 1000;
  CHECK(gattn_forward_path(&a, &path) == GATTN_OK && path == GATTN_PATH_GATHER);  /* too sparse */
  rw.num_cols = 17;
  a.path = GATTN_PATH_MFMA;
  CHECK(gattn_forward_path(&a, &path) == GATTN_ERR_INVALID_VALUE);
  rw.num_cols = 16 * 8;
  rw.num_windows = 6;
  CHECK(gattn_forward_path(&a, &path) == GATTN_ERR_INVALID_VALUE);
  rw.num_windows = 7;
  gattn_hybrid hy = {3, 2, 8, (const int32_t*)FAKE(12), (const int32_t*)FAKE(13)};
  a.path = GATTN_PATH_HYBRID;
  a.hybrid = &hy;
  CHECK(gattn_forward_path(&a, &path) == GATTN_OK && path == GATTN_PATH_HYBRID);
  hy.num_dense = 8;
  CHECK(gattn_forward_path(&a, &path) == GATTN_ERR_INVALID_VALUE);
  hy.num_dense = 3;
  hy.range_rows = 1 << 20;
  CHECK(gattn_forward_path(&a, &path) == GATTN_ERR_INVALID_VALUE);
  hy.range_rows = 8;
  gattn_hybrid plan;
  a = fwd(); a.rw = &rw;
  CHECK(gattn_build_hybrid(&a, -1.f, FAKE(12), FAKE(13), &plan, 0) == GATTN_ERR_INVALID_VALUE);
  CHECK(gattn_build_hybrid(&a, 0.1f, FAKE(12), FAKE(13), NULL, 0) == GATTN_ERR_INVALID_VALUE);
  a.e = FAKE(14);
  CHECK(gattn_build_hybrid(&a, 0.1f, FAKE(12), FAKE(13), &plan, 0) == GATTN_ERR_UNSUPPORTED);

  /* workspace planners over many shapes (host arithmetic only) */
  const gattn_dtype dts[] = {GATTN_F32, GATTN_F16, GATTN_BF16};
  const int hds[][2] = {{1, 16}, {8, 16}, {3, 32}, {1, 64}, {8, 64}, {2, 128}, {5, 128}};
  const int64_t graphs[][2] = {{1, 0}, {1, 1}, {320, 4457}, {12197, 121970}, {169343, 622503},
                               {2450000, 101119663}, {5, 40000}, {40000, 5}};
  for (unsigned t = 0; t < 3; ++t)
    for (unsigned i = 0; i < sizeof hds / sizeof hds[0]; ++i)
      for (unsigned j = 0; j < sizeof graphs / sizeof graphs[0]; ++j)
        for (int mode = 0; mode < 2; ++mode)
          for (int with_e = 0; with_e < 2; ++with_e) {
            a = fwd();
            a.dtype = dts[t];
            a.num_heads = hds[i][0];
            a.head_dim = hds[i][1];
            a.num_nodes = (int32_t)graphs[j][0];
            a.nnz = graphs[j][1];
            a.mode = (gattn_mode)mode;
            a.e = with_e ? FAKE(14) : NULL;
            a.e_out = with_e && mode == 1 ? FAKE(15) : NULL;
            size_t wb = 0;
            CHECK(gattn_forward_workspace(&a, &wb) == GATTN_OK);
            CHECK(wb >= 256 && wb % 256 == 0);
            gattn_aggregate_args g = agg();
            g.dtype = dts[t];
            g.num_heads = hds[i][0];
            g.head_dim = hds[i][1];
            g.num_nodes = (int32_t)graphs[j][0];
            g.nnz = graphs[j][1];
            CHECK(gattn_aggregate_workspace(&g, &wb) == GATTN_OK);
            CHECK(wb >= 256 && wb % 256 == 0);
          }

  /* aggregation */
  gattn_aggregate_args g = agg();
  CHECK(gattn_aggregate(NULL, 0) == GATTN_ERR_INVALID_VALUE);
  g.normalize = 2;                        CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_INVALID_VALUE);
  g = agg(); g.eps = -1.f;                CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_INVALID_VALUE);
  g = agg(); g.w = NULL;                  CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_INVALID_VALUE);
  g = agg(); g.out = (void*)g.x;               CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_INVALID_VALUE);
  g = agg(); g.head_dim = 8;              CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_UNSUPPORTED);
  g = agg(); g.workspace = FAKE(8); g.workspace_bytes = 256;
  CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_BUFFER_TOO_SMALL);
  g = agg();                              CHECK(gattn_aggregate(&g, 0) == GATTN_ERR_HIP);
}

/* ------------------------------------------------------------------------ */

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static double unif(void) { return (rnd() + 0.5) / 4294967296.0 * 4.0 - 2.0; }

static void oracle_checks(void) {
  enum { N = 41, H = 2, D = 8, MMAX = 400 };
  int32_t src[MMAX], dst[MMAX];
  int32_t m = 0;
  /* node i gets i % 13 distinct sources (so some rows are empty, one has one
   * in-edge); the edge list is in no particular order */
  for (int32_t i = 0; i < N; ++i)
    for (int32_t t = 0; t < i % 13; ++t) {
      src[m] = (i * 7 + t * 5 + 3) % N;
      dst[m] = i;
      ++m;
    }
  for (int32_t e = m - 1; e > 0; --e) {
    int32_t j = (int32_t)(rnd() % (uint32_t)(e + 1)), ts = src[e], td = dst[e];
    src[e] = src[j]; dst[e] = dst[j]; src[j] = ts; dst[j] = td;
  }
  int32_t rp[N + 1], ci[MMAX], pe[MMAX];
  CHECK(orc_build_csr(N, m, src, dst, rp, ci, pe) == ORC_OK);
  CHECK(rp[0] == 0 && rp[N] == m);
  for (int32_t i = 0; i < N; ++i) {
    CHECK(rp[i + 1] - rp[i] == i % 13);
    for (int32_t p = rp[i]; p < rp[i + 1]; ++p) {
      CHECK(dst[pe[p]] == i && src[pe[p]] == ci[p]);
      if (p > rp[i]) CHECK(ci[p - 1] < ci[p]);
    }
  }
  int32_t bad[2] = {0, N};
  CHECK(orc_build_csr(N, 2, bad, bad, rp, ci, pe) == ORC_BAD_GRAPH);
  CHECK(orc_build_csr(N, m, src, dst, rp, ci, pe) == ORC_OK);

  /* row windows: every (row, column) bit decodes back to an edge */
  const int32_t W = (N + 15) / 16;
  int32_t wcp[W + 1];
  CHECK(orc_rowwindow_sizes(N, rp, ci, wcp) == ORC_OK);
  int32_t* cols = (int32_t*)malloc(sizeof(int32_t) * (size_t)(wcp[W] + 1));
  uint16_t* mask = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(wcp[W] + 1));
  CHECK(orc_build_rowwindows(N, rp, ci, wcp, cols, mask) == ORC_OK);
  int64_t bits = 0;
  for (int32_t w = 0; w < W; ++w)
    for (int32_t c = wcp[w]; c < wcp[w + 1]; ++c)
      for (int r = 0; r < 16; ++r)
        if (mask[(c / 16) * 16 + r] >> (c % 16) & 1) {
          ++bits;
          int32_t row = 16 * w + r, found = 0;
          for (int32_t p = rp[row]; p < rp[row + 1]; ++p) found |= ci[p] == cols[c];
          CHECK(found);
        }
  CHECK(bits == m);
  free(cols);
  free(mask);

  double q[N * H * D], k[N * H * D], v[N * H * D], e[MMAX * H * D], w[MMAX * H];
  for (int i = 0; i < N * H * D; ++i) { q[i] = 2.0 * unif(); k[i] = unif(); v[i] = unif(); }
  for (int i = 0; i < m * H * D; ++i) e[i] = unif();
  for (int i = 0; i < m * H; ++i) w[i] = exp(unif());
  static double out[N * H * D], out2[N * H * D], mag[N * H * D], alpha[MMAX * H], eo[MMAX * H * D];
  int32_t rows[5] = {40, 0, 13, 14, 7};
  static double sub[5 * H * D];
  for (int clipped = 0; clipped < 2; ++clipped)
    for (int with_e = 0; with_e < 2; ++with_e)
      for (int with_ids = 0; with_ids < 2; ++with_ids) {
        const double* ep = with_e ? e : NULL;
        const int32_t* ids = with_e && with_ids ? pe : NULL;
        double* eop = clipped && with_e ? eo : NULL;
        CHECK(orc_forward(N, H, D, m, rp, ci, q, k, v, ep, ids, clipped, 0.35, -5, 5, 1e-6, NULL, N, out, mag,
                          alpha, eop, 1) == ORC_OK);
        CHECK(orc_forward(N, H, D, m, rp, ci, q, k, v, ep, ids, clipped, 0.35, -5, 5, 1e-6, NULL, N, out2, NULL,
                          NULL, NULL, 4) == ORC_OK);
        CHECK(memcmp(out, out2, sizeof out) == 0);
        CHECK(orc_forward(N, H, D, m, rp, ci, q, k, v, ep, ids, clipped, 0.35, -5, 5, 1e-6, rows, 5, sub, NULL,
                          NULL, NULL, 2) == ORC_OK);
        for (int r = 0; r < 5; ++r)
          CHECK(memcmp(sub + r * H * D, out + rows[r] * H * D, sizeof(double) * H * D) == 0);
        for (int32_t i = 0; i < N; ++i)
          for (int h = 0; h < H; ++h) {
            double sa = 0.0;
            for (int32_t p = rp[i]; p < rp[i + 1]; ++p) sa += alpha[p * H + h];
            const int32_t deg = rp[i + 1] - rp[i];
            if (deg == 0) {
              for (int c = 0; c < D; ++c) CHECK(out[(i * H + h) * D + c] == 0.0 && mag[(i * H + h) * D + c] == 0.0);
            } else if (!clipped) {
              CHECK(fabs(sa - 1.0) < 1e-12);
            } else {
              CHECK(sa < 1.0 && sa > 0.99);
            }
            for (int c = 0; c < D; ++c) CHECK(mag[(i * H + h) * D + c] + 1e-12 >= fabs(out[(i * H + h) * D + c]));
            if (deg == 1 && !clipped)
              for (int c = 0; c < D; ++c) CHECK(out[(i * H + h) * D + c] == v[(ci[rp[i]] * H + h) * D + c]);
          }
      }
  CHECK(orc_forward(N, H, D, m, rp, ci, q, k, v, NULL, NULL, 0, 0.35, -5, 5, 1e-6, NULL, N, out, NULL, NULL, eo,
                    1) == ORC_INVALID);
  int32_t bad_rows[1] = {N};
  CHECK(orc_forward(N, H, D, m, rp, ci, q, k, v, NULL, NULL, 0, 0.35, -5, 5, 1e-6, bad_rows, 1, out, NULL, NULL,
                    NULL, 1) == ORC_INVALID);

  for (int normalize = 0; normalize < 2; ++normalize)
    for (int with_ids = 0; with_ids < 2; ++with_ids) {
      CHECK(orc_aggregate(N, H, D, m, rp, ci, v, w, with_ids ? pe : NULL, normalize, 1e-6, out, 3) == ORC_OK);
      for (int32_t i = 0; i < N; ++i)
        if (rp[i + 1] == rp[i])
          for (int c = 0; c < H * D; ++c) CHECK(out[i * H * D + c] == 0.0);
    }
  int32_t rp_bad[N + 1];
  memcpy(rp_bad, rp, sizeof rp_bad);
  rp_bad[N] = m + 1;
  CHECK(orc_aggregate(N, H, D, m, rp_bad, ci, v, w, NULL, 0, 1e-6, out, 1) == ORC_BAD_GRAPH);
}

int main(void) {
  abi_checks();
  oracle_checks();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("sanitized host code: all checks passed\n");
  return 0;
}
