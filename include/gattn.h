/* gattn.h -- fused graph sparse attention on AMD Instinct MI355X (gfx950).
 *
 * One C ABI, three operations:
 *
 *   gattn_build_csr        COO edge list -> destination-grouped CSR.
 *                          The gattn-triton article ("Using the CSC index for
 *                          fast edge lookup") groups edges by destination with
 *                          an N+1 pointer vector, one source per edge and a map
 *                          from grouped position to edge id; the POPCORNBENCH
 *                          problem calls the same arrays row_ptr / col_idx.
 *   gattn_build_rowwindows CSR -> 16-row windows of compacted columns cut into
 *                          16x16 tiles with per-row bit masks (Fused3S,
 *                          Figure 1: row windows compacted and stored as
 *                          tensor-core blocks with a binary mask).
 *   gattn_forward          fused SDDMM -> per-destination softmax -> SpMM
 *                          (Fused3S abstract: the "3S" pattern) with no edge
 *                          tensor written to memory; both softmax forms:
 *                          standard max-subtracted (Fused3S abstract) and the
 *                          RTMScore clipped form (gattn-triton article,
 *                          "Background" and "Fusing the full graph attention").
 *
 * Conventions shared by every call
 *   - An edge j -> i has source j and destination i.  The CSR groups edges by
 *     destination: the in-edges of node i occupy positions
 *     [row_ptr[i], row_ptr[i+1]) and col_idx[p] is the source of position p.
 *   - Pointers are DEVICE pointers unless marked [host].  Every buffer is owned
 *     by the caller and must stay alive until the stream has passed the call.
 *     The library keeps no pointer after a call returns and allocates no
 *     device memory: scratch space is the caller's `workspace`.
 *   - All work is enqueued on `stream` (a hipStream_t; 0 = the null stream).
 *     Calls that must report a data-dependent result to the host say so and
 *     synchronize that stream.
 *   - Argument errors are detected on the host and returned before anything
 *     is enqueued.  Errors of the HIP runtime (no device, launch failure)
 *     return GATTN_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Integer outputs (CSR, row windows) are unique functions of the input:
 *     identical bits on every run.  gattn_forward accumulates with no atomics:
 *     each destination's edges are folded in a fixed order (with a workspace,
 *     the partial states of a row cut across workgroups are merged in part
 *     order), so it too is bit-reproducible.
 */
#ifndef GATTN_H
#define GATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GATTN_ABI_VERSION 5

#ifndef GATTN_API
#define GATTN_API __attribute__((visibility("default")))
#endif

typedef enum {
  GATTN_OK = 0,
  GATTN_ERR_INVALID_VALUE = 1,    /* null required pointer, negative size, bad enum, misaligned
                                     tensor (q/k/v/e/out need 16-byte alignment), clip_lo > clip_hi,
                                     eps < 0, scale not > 0, struct_size mismatch                 */
  GATTN_ERR_UNSUPPORTED = 2,      /* head_dim not in {16,32,64,128}; H*D above 2^20; MFMA path
                                     asked for fp32, an edge tensor, the clipped softmax or
                                     head_dim 16                                                   */
  GATTN_ERR_BAD_GRAPH = 3,        /* an index outside [0, N); row_ptr[0] != 0, decreasing, or
                                     row_ptr[N] != nnz                                             */
  GATTN_ERR_DUPLICATE_EDGE = 4,   /* gattn_build_rowwindows: a (dst, src) pair repeats, which a
                                     bit mask cannot represent                                     */
  GATTN_ERR_BUFFER_TOO_SMALL = 5, /* workspace or output capacity below what the size query
                                     returned                                                      */
  GATTN_ERR_HIP = 6               /* a HIP runtime call failed                                     */
} gattn_status;

typedef enum { GATTN_F32 = 0, GATTN_F16 = 1, GATTN_BF16 = 2 } gattn_dtype;

typedef enum {
  /* alpha_p = exp(l_p - max) / sum exp(l - max); l_p = scale * sum_d q k (e).   */
  GATTN_SOFTMAX_STANDARD = 0,
  /* RTMScore: t_d = clamp(scale * q_d k_d, lo, hi) (* e_d); l = clamp(sum t, lo, hi);
     s = exp(l); alpha = s / (sum s + eps).  Elementwise clamp before the edge
     projection and a second clamp of the sum, in the order of the article's code. */
  GATTN_SOFTMAX_CLIPPED = 1
} gattn_mode;

typedef enum {
  GATTN_PATH_AUTO = 0,
  GATTN_PATH_GATHER = 1,
  GATTN_PATH_MFMA = 2,
  GATTN_PATH_HYBRID = 3  /* per row window: dense windows on the MFMA path, the rest gathered */
} gattn_path;

#define GATTN_FLAG_VALIDATE 1u /* gattn_forward / gattn_aggregate: check row_ptr, col_idx and
                                  edge_ids on the device first (BAD_GRAPH; synchronizes the
                                  stream; allocates nothing)                                   */

/* ------------------------------------------------------------------------ */
GATTN_API int gattn_abi_version(void);
GATTN_API const char* gattn_status_string(gattn_status s);

/* ------------------------------------------------------------------------
 * gattn_build_csr: COO -> CSR by destination in canonical order
 *   (destination, source, edge id), so the result is unique.
 *
 *   num_nodes >= 0, 0 <= nnz < 2^31.
 *   src, dst    [nnz] int32, COO source / destination of edge e (edge id = e).
 *   row_ptr     [num_nodes+1] int32 out.
 *   col_idx     [nnz] int32 out: source of each CSR position.
 *   edge_perm   [nnz] int32 out, nullable: edge id of each CSR position (use it
 *               to bring per-edge tensors such as E into CSR order).
 *   workspace   device scratch of at least gattn_build_csr_workspace() bytes,
 *               256-byte aligned (about 16 bytes per edge below 2^18 edges, 25
 *               above, where a radix sort replaces per-edge atomics; the two
 *               builds give the same bits; GATTN_CSR_PATH=atomic|radix in the
 *               environment forces one of them, for tests and measurement, and
 *               must not change between the size query and the call).
 *   status_dev  nullable device int32.  NULL: the call synchronizes `stream` and
 *               returns GATTN_ERR_BAD_GRAPH when any src/dst lies outside
 *               [0, num_nodes).  Non-NULL: the call stays asynchronous and the
 *               device writes GATTN_OK or GATTN_ERR_BAD_GRAPH there (or
 *               GATTN_ERR_HIP if the prefix sum's bounded wait ran out, which
 *               only a broken device can cause).  Outputs are unspecified
 *               unless the status is GATTN_OK.
 * ------------------------------------------------------------------------ */
GATTN_API gattn_status gattn_build_csr_workspace(int32_t num_nodes, int64_t nnz, size_t* bytes /*[host]*/);
GATTN_API gattn_status gattn_build_csr(int32_t num_nodes, int64_t nnz, const int32_t* src, const int32_t* dst,
                             int32_t* row_ptr, int32_t* col_idx, int32_t* edge_perm,
                             void* workspace, size_t workspace_bytes, int32_t* status_dev,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * gattn_build_rowwindows: CSR (any order inside a row) -> row windows.
 *   Window w covers rows [16w, min(16w+16, N)).  U_w = ascending distinct
 *   sources of those rows, padded with -1 to a multiple of 16.
 *     win_col_ptr[w+1] = win_col_ptr[w] + 16 * ceil(|U_w| / 16)
 *     win_cols[win_col_ptr[w] + t] = U_w[t] or -1
 *     tile T = win_col_ptr[w]/16 + t covers columns 16t..16t+15 of window w;
 *     tile_mask[16*T + r] bit c (LSB = column 0) is set iff row 16w+r has an
 *     edge from U_w[16t + c].  Rows >= N and padding columns have no bits.
 *
 *   Two calls.  Call 1 (win_cols == NULL): fills win_col_ptr [ceil(N/16)+1],
 *   checks the graph (BAD_GRAPH, DUPLICATE_EDGE), synchronizes `stream` and
 *   stores the total column count in *num_cols [host].  Call 2: *num_cols [host]
 *   holds the capacity of win_cols [num_cols] and tile_mask [num_cols] (uint16,
 *   i.e. num_cols/16 tiles x 16 rows); it needs win_col_ptr and the workspace
 *   from call 1 unchanged (call 1 leaves every window's sorted keys there),
 *   returns BUFFER_TOO_SMALL when the capacity is below win_col_ptr[W] (read
 *   back with one small synchronous copy), then enqueues the fill.
 *   workspace: at least gattn_build_rowwindows_workspace() bytes (256-B aligned).
 *   UNSUPPORTED when nnz + 15 * ceil(N/16) exceeds 2^31 - 1 (the int32
 *   win_col_ptr could not hold every padded column count).
 * ------------------------------------------------------------------------ */
GATTN_API gattn_status gattn_build_rowwindows_workspace(int32_t num_nodes, int64_t nnz, size_t* bytes /*[host]*/);
GATTN_API gattn_status gattn_build_rowwindows(int32_t num_nodes, int64_t nnz, const int32_t* row_ptr,
                                    const int32_t* col_idx, int32_t* win_col_ptr, int32_t* win_cols,
                                    uint16_t* tile_mask, int64_t* num_cols /*[host]*/,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * gattn_forward
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t num_windows;         /* ceil(num_nodes / 16)                         */
  int64_t num_cols;            /* win_col_ptr[num_windows]                     */
  const int32_t* win_col_ptr;  /* [num_windows + 1]                            */
  const int32_t* win_cols;     /* [num_cols]                                   */
  const uint16_t* tile_mask;   /* [num_cols] = [num_cols/16][16]               */
} gattn_rowwindows;

/* Per-window dispatch plan (from gattn_build_hybrid): which row windows run
 * on the MFMA path and which destination ranges the gather path takes.  The
 * windows and ranges together cover every row exactly once.                */
typedef struct {
  int32_t num_dense;             /* windows on the MFMA path                            */
  int32_t num_ranges;            /* gather workgroups                                   */
  int32_t range_rows;            /* most rows in one range                              */
  const int32_t* dense_windows;  /* [num_dense] ascending window ids (device)           */
  const int32_t* ranges;         /* [2 * num_ranges] (first row, row count) (device)    */
} gattn_hybrid;

typedef struct {
  uint32_t struct_size;        /* sizeof(gattn_forward_args)                         */
  int32_t num_nodes;           /* N >= 0                                             */
  int32_t num_heads;           /* H >= 1                                             */
  int32_t head_dim;            /* D in {16, 32, 64, 128}                             */
  int64_t nnz;                 /* edges; row_ptr[N] must equal it                    */
  const int32_t* row_ptr;      /* [N+1] CSR by destination                           */
  const int32_t* col_idx;      /* [nnz] source per position, any order inside a row  */
  const void* q;               /* [N, H, D] `dtype`, 16-byte aligned; rows q_stride apart */
  const void* k;               /* [N, H, D], rows kv_stride apart                    */
  const void* v;               /* [N, H, D], rows kv_stride apart                    */
  const void* e;               /* nullable; [nnz, H, D] by CSR position (or edge_ids) */
  void* out;                   /* [N, H, D] `dtype`; must not alias the inputs       */
  gattn_dtype dtype;           /* of q, k, v, e and out; arithmetic is fp32          */
  gattn_mode mode;
  float scale;                 /* > 0; usually 1/sqrt(D)                             */
  float clip_lo, clip_hi;      /* clipped mode (RTMScore: -5, 5)                     */
  float eps;                   /* clipped mode denominator term, >= 0                */
  gattn_path path;             /* AUTO: HYBRID when `hybrid` is given and the MFMA
                                  path applies, else MFMA when rw is given and dense
                                  enough, else GATHER                                  */
  const gattn_rowwindows* rw;  /* [host] struct of device arrays; MFMA / HYBRID paths */
  uint32_t flags;              /* GATTN_FLAG_*                                       */
  /* Edge-id indirection (the article's map from CSC position to edge id):
     nullable [nnz] int32; when set, the per-edge rows of e and e_out are
     e[edge_ids[p]] for CSR position p (pass gattn_build_csr's edge_perm to keep
     E in the caller's original edge order).  Values must lie in [0, nnz), and
     form a permutation when e_out is given (two positions writing one row
     race).  GATTN_FLAG_VALIDATE checks both (GATTN_ERR_BAD_GRAPH; the range on
     the device, the permutation with a host copy of the ids);
     unchecked, an out-of-range id is clamped into range (no fault, the
     result is unspecified).  Read only when e is given.                       */
  const int32_t* edge_ids;
  /* RTMScore edge update (the article's e_out): nullable [nnz, H, D] `dtype`,
     clipped mode with e only; row r = edge_ids ? edge_ids[p] : p receives
     clamp(scale * q[dst] * k[src], clip_lo, clip_hi) * e[r], the product before
     the feature sum.  Must not alias any input or out.                         */
  void* e_out;
  /* Optional workspace (gather path): when given, workgroups take equal shares
     of the edges (a merge path over row ends and edges) and a destination with
     more in-edges than about half a share is cut into edge-parallel parts
     whose partial softmax states are merged in order (Fused3S Figure 2's
     node- versus edge-parallel split).  Without it, workgroups take equal
     numbers of destinations.  Size from gattn_forward_workspace; 256-byte
     aligned; any contents on entry (flags are tagged with a random per-call
     token, and every flag a call raises is lowered again before it ends, so
     a call captured in a HIP graph may be replayed); must not alias any
     other argument; one workspace must not serve two calls that run at the
     same time.  Ignored on the MFMA path.                                      */
  void* workspace;
  size_t workspace_bytes;
  /* Per-window plan for the HYBRID path: [host] struct of device arrays built
     by gattn_build_hybrid for this graph, these row windows and this geometry
     (H, D, dtype, mode, e).  Nullable; required by GATTN_PATH_HYBRID.          */
  const gattn_hybrid* hybrid;
  /* Row strides, in elements, of q and of k / v (k and v share one): 0 means
     num_heads * head_dim (rows packed).  Otherwise at least that and a
     multiple of 8 elements (16 bytes), so that q, k and v may be views into a
     fused projection's output; k and v interleaved in one [N, 2, H, D] buffer
     (kv_stride = 2 H D) put an edge's K and V rows side by side, which random
     row gathers read faster.  At most 2^24; GATTN_ERR_INVALID_VALUE for a
     stride outside these rules.  Overlap checks take the strided spans
     ((N - 1) * stride + H * D elements).  The MFMA path needs each span under
     2^31 bytes (GATTN_ERR_UNSUPPORTED when it is forced; AUTO then gathers).
     out, e and e_out are always packed.                                        */
  int64_t q_stride;
  int64_t kv_stride;
} gattn_forward_args;

/* out[i, h, :] = sum_p alpha_p(h) v[col_idx[p], h, :] over the in-edges p of i;
 * a node without in-edges gets exactly 0 (0 / (0 + eps) in the clipped form).
 * Rounding: fp32 accumulation; the fp16/bf16 output is rounded to nearest even.
 * Without GATTN_FLAG_VALIDATE the graph is not checked; indices are clamped
 * into range so that a bad graph gives wrong numbers, never a fault.        */
GATTN_API gattn_status gattn_forward(const gattn_forward_args* args /*[host]*/, hipStream_t stream);

/* ------------------------------------------------------------------------
 * gattn_forward_noalloc: gattn_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  On the gather path it runs the balanced partition
 * (as gattn_forward with a workspace, same kernels, same bits) with its
 * workspace in a scratch array inside the library: one array of
 * GATTN_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends.  The MFMA and hybrid
 * paths use no scratch and run as in gattn_forward.
 *   args: as for gattn_forward, with workspace NULL and workspace_bytes 0
 *         (GATTN_ERR_INVALID_VALUE otherwise) and without GATTN_FLAG_VALIDATE
 *         (which copies to the host; GATTN_ERR_INVALID_VALUE).  The caller
 *         still provides every input and `out`.
 *   GATTN_ERR_BUFFER_TOO_SMALL when the problem's balanced-partition
 *         workspace (gattn_forward_workspace) exceeds the array; use
 *         gattn_forward with a workspace, or without one, instead.
 * Calls no allocating routine.  Every call on one GPU uses that GPU's array,
 * which keeps what the last call left (nothing in it needs clearing: its
 * flags are tagged per call and lowered again before a call ends).  Two calls
 * whose executions overlap on one GPU (different streams, or host threads)
 * race on the array and give wrong results: order them on one stream.
 * ------------------------------------------------------------------------ */
#define GATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
GATTN_API gattn_status gattn_forward_noalloc(const gattn_forward_args* args /*[host]*/, hipStream_t stream);

/* The path gattn_forward would take for these arguments (no work enqueued; `out` may be NULL). */
GATTN_API gattn_status gattn_forward_path(const gattn_forward_args* args /*[host]*/, gattn_path* path /*[host]*/);

/* ------------------------------------------------------------------------
 * gattn_build_hybrid: per-window dispatch between the MFMA row-window path and
 * the gather path.  Fused3S (Figure 1) compacts every row window into dense
 * tensor-core blocks; a window whose blocks are mostly empty wastes the
 * matrix-core work and reloads K / V rows for few edges, so this plan keeps
 * the row windows only where they are dense (the per-window choice is this
 * library's, not the page's).  Window w (rows 16w .. 16w+15) goes to the MFMA path when it
 * has columns and its tile density nnz_w / (16 * cols_w) >= min_density
 * (nnz_w = edges of its rows, cols_w = win_col_ptr[w+1] - win_col_ptr[w]);
 * the rows of the other windows are cut into gather ranges of consecutive
 * rows, sized like the gather path's workgroups for the sparse part.
 *   args: the forward arguments the plan is for (graph, sizes, dtype, mode,
 *         e, rw); `out`, `hybrid` and the tensors' contents are not read.
 *         The MFMA path must apply (fp16 / bf16, standard mode, no e).
 *   min_density >= 0; 0 sends every window with columns to the MFMA path,
 *         a value above 1 sends every window to the gather path (the Python
 *         binding's default, 0.125, was the fastest on a mixed batch).
 *   dense_windows: device int32 [ceil(N/16)] out; ranges: device int32 [2N]
 *         out (capacities that hold any plan).
 *   plan: [host] out; its pointers are dense_windows and ranges.
 * Synchronizes `stream` (the lists are built on the host from one flag per
 * window); a once-per-graph preprocessing step like the row windows.
 * ------------------------------------------------------------------------ */
GATTN_API gattn_status gattn_build_hybrid(const gattn_forward_args* args /*[host]*/, float min_density,
                                          int32_t* dense_windows, int32_t* ranges, gattn_hybrid* plan /*[host]*/,
                                          hipStream_t stream);

/* Workspace bytes for the balanced gather partition of these arguments (sizes,
 * dtype, mode, whether e and e_out are given; pointers are not read).  0 when
 * there is nothing to compute.  Depends on the current device's CU count. */
GATTN_API gattn_status gattn_forward_workspace(const gattn_forward_args* args /*[host]*/, size_t* bytes /*[host]*/);

/* ------------------------------------------------------------------------
 * gattn_aggregate: weighted aggregation over the CSR with given per-edge
 * weights (no logits, no softmax) -- the POPCORNBENCH CSR problem
 *   out[i, h, :] = sum_p w[r(p), h] * x[col_idx[p], h, :],  r(p) = edge_ids ? edge_ids[p] : p,
 * and, with normalize = 1, the gattn-triton article's scatter add of scaled
 * values and scores followed by numerator / (denominator + eps)
 *   out[i, h, :] = (sum_p w x) / (sum_p w + eps).
 * A destination without in-edges gets exactly 0.  Same kernels, balance and
 * determinism as the gather path of gattn_forward.
 * ------------------------------------------------------------------------ */
typedef struct {
  uint32_t struct_size;        /* sizeof(gattn_aggregate_args)                       */
  int32_t num_nodes;           /* N >= 0                                             */
  int32_t num_heads;           /* H >= 1                                             */
  int32_t head_dim;            /* D in {16, 32, 64, 128}                             */
  int64_t nnz;
  const int32_t* row_ptr;      /* [N+1] CSR by destination                           */
  const int32_t* col_idx;      /* [nnz]                                              */
  const void* x;               /* [N, H, D] `dtype`, 16-byte aligned                 */
  const float* w;              /* [nnz, H] fp32 weights                              */
  const int32_t* edge_ids;     /* nullable [nnz]: row of w for CSR position p, in
                                  [0, nnz) (checked with GATTN_FLAG_VALIDATE, else
                                  clamped)                                          */
  void* out;                   /* [N, H, D] `dtype`; must not alias the inputs       */
  gattn_dtype dtype;
  int32_t normalize;           /* 0: weighted sum; 1: divided by (sum of w + eps)    */
  float eps;                   /* >= 0                                               */
  uint32_t flags;              /* GATTN_FLAG_VALIDATE                                */
  void* workspace;             /* optional; as in gattn_forward_args                 */
  size_t workspace_bytes;
} gattn_aggregate_args;

GATTN_API gattn_status gattn_aggregate(const gattn_aggregate_args* args /*[host]*/, hipStream_t stream);

/* Workspace bytes for the balanced partition of gattn_aggregate (sizes, dtype;
 * `out` may be NULL and no pointer is read). */
GATTN_API gattn_status gattn_aggregate_workspace(const gattn_aggregate_args* args /*[host]*/, size_t* bytes /*[host]*/);

#ifdef __cplusplus
}
#endif
#endif /* GATTN_H */
