// gather_kernel.hpp -- wave64 gather kernel of the fused graph attention
// (included by forward_gather.hip, which instantiates the node partition,
// and forward_gather_split.hip, which instantiates the balanced one).
//
// What it computes (gattn-triton article, "Background" and "Fusing the full
// graph attention"; Fused3S abstract): for every destination i and head h,
// a logit per in-edge from q_i and k_j (times e_ij when an edge projection
// is given), a softmax over the in-edges of i -- standard max-subtracted, or
// the RTMScore form exp(clip) / (sum + eps) -- and o_i = sum_j alpha_ij v_j.
// No per-edge tensor is written, except the RTMScore edge update when asked
// for (the article's fused kernel stores clip(scale q k) * e per edge).
// The same kernel, without logits, is the weighted CSR aggregation of the
// POPCORNBENCH problem and of the article's scatter add (third mode below).
// Per-edge rows (E, the edge update, aggregation weights) are addressed by
// CSR position, or through an edge-id map (the article's CSC edge ids).
//
// Mapping on CDNA4.
//  * A "slot" is a group of G lanes (G = 2..64, a power of two) that holds one
//    edge's [HB heads x D] slice of a K / V / E row, 16 bytes per lane, so a
//    slot's loads are one contiguous, coalesced run.  A wave holds 64/G slots,
//    a 256-thread workgroup NS = 4*64/G slots.  The logit of a head is summed
//    over its D/VEC lanes with DPP inside a 16-lane row.
//  * A workgroup owns a contiguous range of destinations (node-parallel as in
//    the article's one-program-per-node kernels and Fused3S Figure 2, top) for
//    one block of heads.  It first stages the destinations' row pointers and
//    Q rows in LDS (one coalesced pass).  Its edges are then cut into NS equal
//    contiguous pieces (a merge path over the CSR): each slot walks its piece
//    U edges at a time (U = 4 with an edge tensor or a low average degree,
//    else 8), loading the next step's column indices and E rows (edge ids two
//    steps ahead) while it computes, and keeps the online-softmax state
//    (m, l) and the fp32 accumulator in registers.  A destination that is cut
//    by a piece boundary leaves partial (m, l, acc) records in LDS; the slot
//    holding its last edge merges them in slot order.  Deterministic, no
//    atomics.  The destination range is either equal-sized (node partition)
//    or read from a table of (first row, row count) pairs (the gather share
//    of a per-window hybrid plan).
//  * Consecutive workgroups are mapped onto one XCD so that destinations of
//    one batched graph, whose sources are nearby, share an L2.
//  * With a workspace, workgroups instead take equal ranges of the merged
//    sequence of row ends and edges (a merge path over the whole CSR), found
//    by a 64-lane search of row_ptr at the start; one round of resident
//    workgroups, each staging up to 24 KB of Q rows.  A light row belongs whole to
//    the workgroup holding its first item; a heavy row is cut at the range
//    boundaries (edge-parallel parts, Fused3S Figure 2's node- vs edge-parallel
//    split).  Each part leaves its (m, l, acc) in the workspace and raises a
//    flag tagged with this launch's token; a part that then finds every flag of
//    the row raised merges the parts in order, writes the row and lowers the
//    row's flags again.  Several parts may merge; they write identical bits.
//    The random token guards against whatever a new workspace holds; lowering
//    the flags makes a repeated token (a HIP graph replays its launch
//    arguments) safe.  No cache flush is needed: the parts and flags are
//    written and read with device-coherent (agent-scope) accesses, each wait
//    ordering them.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

#ifndef GATTN_GATHER_Q_LDS_BYTES
#define GATTN_GATHER_Q_LDS_BYTES 12288  // Q rows staged per workgroup
#endif
#ifndef GATTN_GATHER_Q_LDS_BYTES_SPLIT
// The same for the balanced partition: 207 rows of 128 B, the most that
// keeps four workgroups of its 16-bit, 64-wide instantiations on a CU (160 KB
// of LDS).  A range of many low-degree rows that outgrows the staged rows
// runs the edge loop that reads Q from global memory, whose waits are coarser.
#define GATTN_GATHER_Q_LDS_BYTES_SPLIT 26560
#endif
#ifndef GATTN_GATHER_EDGES_PER_SLOT
#define GATTN_GATHER_EDGES_PER_SLOT 3   // target edges per slot, in units of U
#endif
#ifndef GATTN_GATHER_U
#define GATTN_GATHER_U 8                // edges per step without an edge tensor
#endif
#ifndef GATTN_GATHER_U_LOW
#define GATTN_GATHER_U_LOW 4            // the same for graphs of low average degree
#endif
#ifndef GATTN_GATHER_LOW_DEGREE
#define GATTN_GATHER_LOW_DEGREE 8.0     // average in-degree below which U_LOW is used
#endif
#ifndef GATTN_GATHER_U_E
#define GATTN_GATHER_U_E 4              // edges per step with an edge tensor
#endif
#ifndef GATTN_GATHER_E_STREAMING
#define GATTN_GATHER_E_STREAMING 1      // non-temporal loads for the edge tensor
#endif
#ifndef GATTN_GATHER_MIN_WAVES
#define GATTN_GATHER_MIN_WAVES 1        // waves per SIMD the register budget must allow
#endif
#ifndef GATTN_XCD_REMAP
#define GATTN_XCD_REMAP 1
#endif

namespace gattn {

constexpr int kGatherThreads = 256;
constexpr int kMaxNodesPerWg = 1024;
constexpr int kQLdsBytes = GATTN_GATHER_Q_LDS_BYTES;
constexpr int kQLdsBytesSplit = GATTN_GATHER_Q_LDS_BYTES_SPLIT;
constexpr int kModeAggregate = 2;  // given per-edge weights instead of logits and softmax

// How workgroups divide the CSR (the kernel's PART parameter).
constexpr int kPartNode = 0;    // equal numbers of destinations
constexpr int kPartSplit = 1;   // equal ranges of row ends + edges; heavy rows cut across workgroups

struct GatherArgs {
  const int32_t* __restrict__ row_ptr;
  const int32_t* __restrict__ col_idx;
  const uint8_t* __restrict__ q;
  const uint8_t* __restrict__ k;
  const uint8_t* __restrict__ v;
  const uint8_t* __restrict__ e;
  uint8_t* __restrict__ out;
  int64_t nnz;
  int64_t q_stride, kv_stride;  // row strides (elements) of q and of k / v
  int32_t n, H, HB, log2G, npw;
  float scale;  // standard: scale * log2(e); clipped: scale
  float lo, hi, eps;
  const int32_t* __restrict__ ids;  // nullable: row of e / e_out / w for CSR position p
  uint8_t* __restrict__ e_out;      // clipped mode with e: the per-edge update
  const float* __restrict__ w;      // aggregate mode: [nnz, H] weights
  int32_t normalize;                // aggregate mode: divide by (sum of w + eps)
  // balanced partition with cut heavy rows (ws_flags != nullptr)
  uint64_t* ws_flags;               // [2][head blocks][B] launch tokens (kind 0: first row, 1: last row)
  float* ws_ml;                     // [2][head blocks][B][G][2] partial m, l
  float* ws_acc;                    // [2][head blocks][B][G][VEC] partial accumulators
  int64_t items_per_wg;             // C: width of a workgroup's range of (row ends + edges)
  int64_t total_items;              // N + nnz
  int32_t light_max;                // rows with deg + 1 <= light_max are never cut
  int32_t num_wg;                   // B: workgroups per head block
  uint64_t token;                   // this launch's flag value
  // node partition: nullable [2 * grid] (first row, row count) of each
  // workgroup (the gather share of a per-window hybrid plan); rows <= npw
  const int32_t* __restrict__ ranges;
};

// First item of row r in the merged sequence (row r's edges, then its end).
__device__ __forceinline__ int64_t first_item(const GatherArgs& a, int64_t r) {
  return r + min(max(a.row_ptr[r], 0), (int)a.nnz);
}

struct Cut {
  int row, edge;
  int cont;  // the range starts inside `row`: its edges before `edge` belong to earlier workgroups
};

// Start of the range that begins at item x, computed by one whole wave: r0 is
// the last row with first_item(r0) <= x.  Two round trips in the usual case:
// 64 samples 128 rows apart around the proportional guess bracket r0 within
// 128 rows (graphs whose cumulative degree stays within 4096 rows of its
// average slope), then those 128 rows, two per lane, give r0 and, from the
// same loads, its first and last edge.  Otherwise a 64-way search over the
// side the samples point to.  A light row straddling x was taken by the
// workgroup holding its first item, so the range starts at the next row; a
// heavy row is cut at x.
__device__ inline Cut locate(const GatherArgs& a, int64_t x, int lane) {
  const int n = a.n, nnz = (int)a.nnz;
  if (x >= a.total_items) return Cut{n, nnz, 0};
  auto cut_at = [&](int r0, int rs, int re) -> Cut {
    if (r0 + (int64_t)rs == x) return Cut{r0, rs, 0};
    const int64_t e = x - r0;
    if (re - rs + 1 > a.light_max && e > rs && e < re) return Cut{r0, (int)e, 1};
    return Cut{r0 + 1, re, 0};
  };
  constexpr int64_t S = 128;
  int64_t lo = 0, hi = n;  // r0 lies in [lo, hi]
  {
    const int64_t g = x * n / a.total_items;
    const int64_t base = min(max(g - 32 * S, (int64_t)0), max((int64_t)n - 63 * S, (int64_t)0));
    const int64_t fa = first_item(a, min(base + (int64_t)lane * S, (int64_t)n));
    const int k = __popcll(__ballot(fa <= x));
    if (k == 0) {
      hi = max(base - 1, (int64_t)0);
    } else if (k == 64) {
      lo = base + 63 * S;
    } else {
      // r0 in [p, p + S); row p + S is lane k's sample (past n: first_item(n) = N + nnz > x)
      const int64_t p = base + (int64_t)(k - 1) * S;
      const int64_t fnext = __shfl(fa, k, 64);
      const int64_t f0 = first_item(a, min(p + lane, (int64_t)n));
      const int64_t f1 = first_item(a, min(p + 64 + lane, (int64_t)n));
      const int c = __popcll(__ballot(f0 <= x)) + __popcll(__ballot(f1 <= x));  // >= 1: row p qualifies
      const int64_t r0 = p + c - 1;
      if (r0 >= n) return Cut{n, nnz, 0};  // only reachable for a malformed row_ptr
      const int64_t fr = c <= 64 ? __shfl(f0, c - 1, 64) : __shfl(f1, c - 65, 64);
      const int64_t fn = c < 64 ? __shfl(f0, c, 64) : (c < 128 ? __shfl(f1, c - 64, 64) : fnext);
      return cut_at((int)r0, (int)(fr - r0), (int)(fn - (r0 + 1)));
    }
  }
  while (hi > lo) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t pos = lo + (int64_t)(lane + 1) * step;
    const int k = __popcll(__ballot(pos <= hi && first_item(a, pos) <= x));
    lo += k * step;
    hi = min(hi, lo + step - 1);
  }
  const int r0 = (int)lo;
  if (r0 >= n) return Cut{n, nnz, 0};
  return cut_at(r0, min(max(a.row_ptr[r0], 0), nnz), min(max(a.row_ptr[r0 + 1], 0), nnz));
}

template <typename T, int D, int MODE, bool HAS_E, bool EOUT>
struct EdgeMath {
  static constexpr int VEC = Elem<T>::kVec;
  static constexpr int LPH = D / VEC;

  // one edge: logit, online softmax update, accumulate v (aggregate mode: the
  // given weight wt instead of a softmax weight); EOUT: xo = the edge update
  static __device__ __forceinline__ void step(const GatherArgs& a, const float* qf, u32x4 kr, u32x4 er,
                                              u32x4 vr, float wt, float& m, float& l, float* acc, u32x4& xo) {
    float kf[VEC], vf[VEC], ef[VEC];
    Conv<T>::widen(kr, kf);
    Conv<T>::widen(vr, vf);
    if constexpr (HAS_E) Conv<T>::widen(er, ef);
    float s = 0.f;
    if constexpr (MODE == GATTN_SOFTMAX_STANDARD) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) s += HAS_E ? qf[i] * kf[i] * ef[i] : qf[i] * kf[i];
      s = group_sum<LPH>(s);
      const float lg = s * a.scale;  // log2 domain
      const float mn = fmaxf(m, lg);
      // exp2(0) is exactly 1: keep the running max's own weight and an unchanged
      // max's rescale exact (the hardware exp2 is a 1-ulp approximation)
      const float corr = m == mn ? 1.f : fast_exp2(m - mn);
      const float p = lg == mn ? 1.f : fast_exp2(lg - mn);
      l = l * corr + p;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * corr + p * vf[i];
      m = mn;
    } else if constexpr (MODE == kModeAggregate) {
      l += wt;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += wt * vf[i];
    } else {
      float xs[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        float t = fminf(fmaxf(a.scale * qf[i] * kf[i], a.lo), a.hi);
        xs[i] = HAS_E ? t * ef[i] : t;
        s += xs[i];
      }
      if constexpr (EOUT) xo = Conv<T>::narrow(xs);
      s = group_sum<LPH>(s);
      const float lg = fminf(fmaxf(s, a.lo), a.hi);
      const float p = fast_exp2(lg * kLog2e);
      l += p;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += p * vf[i];
    }
  }

  static __device__ __forceinline__ void store(const GatherArgs& a, uint8_t* dst, float l, const float* acc) {
    float inv;
    if constexpr (MODE == GATTN_SOFTMAX_STANDARD) inv = 1.0f / l;
    else if constexpr (MODE == kModeAggregate) inv = a.normalize ? 1.0f / (l + a.eps) : 1.0f;
    else inv = 1.0f / (l + a.eps);
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = acc[i] * inv;
    st16(dst, Conv<T>::narrow(o));
  }

  // fold partial state (m2, l2, acc2) into (m, l, acc), in that order
  static __device__ __forceinline__ void fold(float& m, float& l, float* acc, float m2, float l2, const float* acc2) {
    if constexpr (MODE == GATTN_SOFTMAX_STANDARD) {
      const float mn = fmaxf(m, m2);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float c1 = fast_exp2(m - mu), c2 = fast_exp2(m2 - mu);
      l = l * c1 + l2 * c2;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * c1 + acc2[i] * c2;
      m = mn;
    } else {
      l += l2;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += acc2[i];
    }
  }
};

template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int U, int PART>
__global__ __launch_bounds__(kGatherThreads, GATTN_GATHER_MIN_WAVES) void gather_kernel(GatherArgs a) {
  using M = EdgeMath<T, D, MODE, HAS_E, EOUT>;
  constexpr int VEC = Elem<T>::kVec;
  constexpr int LPH = D / VEC;
  constexpr int ESZ = sizeof(T);
  constexpr bool AGG = MODE == kModeAggregate;
  constexpr bool ROWS = HAS_E || AGG;  // per-edge rows are read

  // Partial (m, l, acc) records of destinations cut by piece boundaries:
  // [0] the first destination of a piece (started in an earlier piece),
  // written during the edge loop; [1] the last one (continues into a later
  // piece), written only after it, into the Q staging buffer, which no slot
  // reads by then.  Sharing that buffer keeps a workgroup's LDS at about
  // 26 KB for 16-bit types (6 workgroups per CU) instead of 37 KB (4).
  constexpr int kRec1Bytes = kGatherThreads * (VEC + 2) * (int)sizeof(float);
  constexpr int kQLds = PART == kPartSplit ? kQLdsBytesSplit : kQLdsBytes;
  static_assert(AGG || kRec1Bytes <= kQLds, "records [1] must fit the Q staging buffer");
  __shared__ int32_t s_rp[kMaxNodesPerWg + 1];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[AGG ? kRec1Bytes : kQLds];
  __shared__ float s_pm0[kGatherThreads];
  __shared__ float s_pl0[kGatherThreads];
  __shared__ float s_pacc0[kGatherThreads * VEC];
  float* const s_pacc1 = reinterpret_cast<float*>(s_q);
  float* const s_pm1 = s_pacc1 + kGatherThreads * VEC;
  float* const s_pl1 = s_pm1 + kGatherThreads;
  __shared__ int32_t s_cut[6];  // (row, edge, cont) where the range starts and where it ends

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = 1 << a.log2G;
  const int spw = 64 >> a.log2G;
  const int NS = 4 * spw;
  const int slot = wave * spw + (lane >> a.log2G);
  const int lig = lane & (G - 1);
  const int rec = slot * G + lig;
  const int hh = lig / LPH, dch = lig % LPH;
  const int hb = blockIdx.y;
  const int head = hb * a.HB + hh;
  const bool active = hh < a.HB && head < a.H;
  const int64_t rowstride = (int64_t)a.H * D;
  const int64_t eoff = (int64_t)head * D + dch * VEC;
  const int nmax = a.n - 1;
  const int heads_here = min(a.HB, a.H - hb * a.HB);
  const int chunks = heads_here * LPH;                 // 16-byte chunks of this head block per node
  const int qrow = a.HB * D * ESZ;                     // LDS bytes per staged Q row

  const int blk = GATTN_XCD_REMAP ? (int)xcd_contiguous_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int nnz_i = (int)a.nnz;
  constexpr bool split = PART == kPartSplit;  // ranges of row ends + edges, cut heavy rows
  int n0, nn;
  bool cont_first = false, cont_last = false;
  if constexpr (split) {
    if (wave < 2) {
      const Cut c = locate(a, (int64_t)(blk + wave) * a.items_per_wg, lane);
      if (lane == 0) {
        s_cut[wave * 3] = c.row;
        s_cut[wave * 3 + 1] = c.edge;
        s_cut[wave * 3 + 2] = c.cont;
      }
    }
    __syncthreads();
    // workgroup-uniform: keep them in scalar registers
    n0 = __builtin_amdgcn_readfirstlane(s_cut[0]);
    cont_first = __builtin_amdgcn_readfirstlane(s_cut[2]) != 0;
    cont_last = __builtin_amdgcn_readfirstlane(s_cut[5]) != 0;
    const int row_end = cont_last ? __builtin_amdgcn_readfirstlane(s_cut[3]) : __builtin_amdgcn_readfirstlane(s_cut[3]) - 1;
    nn = max(0, min(row_end - n0 + 1, kMaxNodesPerWg));
  } else {
    if (a.ranges) {
      n0 = min(max(a.ranges[2 * blk], 0), a.n);
      nn = min(max(a.ranges[2 * blk + 1], 0), min(a.npw, a.n - n0));
    } else {
      n0 = blk * a.npw;
      nn = min(a.npw, a.n - n0);
    }
  }
  const int qcap = AGG ? 0 : kQLds / qrow;  // rows whose Q is staged in LDS
  auto rp_val = [&](int t, int v) {
    v = min(max(v, 0), nnz_i);
    if (split && t == nn) v = s_cut[4];
    if (split && t == 0) v = s_cut[1];
    return v;
  };

  // The workgroup's edges [E0, E1) are cut into NS equal contiguous pieces
  // (phase 1); the bounds come from the global row pointers (the same values
  // phase 0 stages), so that the first step's loads can be issued before it.
  const int E0 = __builtin_amdgcn_readfirstlane(rp_val(0, a.row_ptr[n0]));
  const int E1 = max(E0, (int)__builtin_amdgcn_readfirstlane(rp_val(nn, a.row_ptr[n0 + nn])));
  const int C = max((E1 - E0 + NS - 1) / NS, 1);
  const int ps = min(E0 + slot * C, E1);
  const int pe = min(ps + C, E1);
  const int plast = max(pe - 1, 0);

  // Addresses: a row of K / V / E / the edge update is rowbytes long (< 4 MB),
  // and this lane's 16 bytes sit at lane_b inside it (0 for idle lanes, whose
  // loads are issued like the others and never used).
  const uint32_t rowbytes = (uint32_t)(rowstride * ESZ);
  const uint32_t kv_rowbytes = (uint32_t)(a.kv_stride * ESZ);  // K and V rows may be strided
  const uint64_t lane_b = active ? (uint64_t)eoff * ESZ : 0;
  const int hw = active ? head : 0;
  auto row_ptr16 = [&](const uint8_t* base, int row) -> const uint8_t* {
    return base + lane_b + (uint64_t)(uint32_t)row * rowbytes;
  };
  auto kv_ptr16 = [&](const uint8_t* base, int row) -> const uint8_t* {
    return base + lane_b + (uint64_t)(uint32_t)row * kv_rowbytes;
  };
  auto load_e = [&](int row) -> u32x4 {
    const uint8_t* ptr = row_ptr16(a.e, row);
    return GATTN_GATHER_E_STREAMING ? ld16_stream(ptr) : ld16(ptr);
  };
  auto raw_row = [&](int p) -> int { return a.ids ? a.ids[p] : p; };
  auto fix_row = [&](int r) -> int { return a.ids ? min(max(r, 0), nnz_i - 1) : r; };

  // The edge loop's prefetch registers: column indices, per-edge rows (edge
  // ids two steps ahead) and edge tensor rows / weights of the next step.
  int cN[U], rN[U], rNN[U];
  u32x4 eN[U];
  float wN[U];
  // The first step's loads.  Each side of the (uniform) branch on the edge-id
  // map issues its own edge row loads: after a join, a use of rows that one
  // side loaded would make the other side wait for every load in flight
  // (the Q rows included), since the wait counts are per wave and in order.
  auto prefetch_first = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = min(ps + u, plast);
      cN[u] = a.col_idx[p];
      rN[u] = p;
      rNN[u] = min(ps + U + u, plast);
      eN[u] = u32x4{0u, 0u, 0u, 0u};
      wN[u] = 0.f;
    }
    if constexpr (ROWS) {
      auto edge_rows = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (HAS_E) eN[u] = load_e(rN[u]);
          if constexpr (AGG) wN[u] = a.w[(int64_t)rN[u] * a.H + hw];
        }
      };
      if (a.ids) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          rN[u] = a.ids[rN[u]];
          rNN[u] = a.ids[rNN[u]];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) rN[u] = fix_row(rN[u]);
        edge_rows();
      } else {
        edge_rows();
      }
    }
  };

  // ---- phase 0: row pointers and Q rows into LDS (one coalesced pass); a
  // range that starts or ends inside a row starts or ends at the cut edge.
  // The first batch of both is loaded before anything is stored, so that the
  // two loads are in flight together.
  constexpr int kQB = 4;  // Q chunks per thread in the first batch
  const int qn = AGG ? 0 : min(nn, qcap) * chunks;
  auto q_src = [&](int t) {
    const int li = t / chunks, c = t - li * chunks;
    return a.q + ((int64_t)(n0 + li) * a.q_stride + (int64_t)hb * a.HB * D + c * VEC) * ESZ;
  };
  auto q_dst = [&](int t) {
    const int li = t / chunks, c = t - li * chunks;
    return reinterpret_cast<u32x4*>(s_q + li * qrow + c * 16);
  };
  {
    // addresses clamped into range: no branch around a load, so no merge of
    // its register that would wait for it before the next load is issued
    const int r0 = a.row_ptr[n0 + min(tid, nn)];
    u32x4 qv[kQB];
#pragma unroll
    for (int j = 0; j < kQB; ++j) qv[j] = qn > 0 ? ld16(q_src(min(tid + j * kGatherThreads, qn - 1))) : u32x4{0u, 0u, 0u, 0u};
    if (tid <= nn) s_rp[tid] = rp_val(tid, r0);
#pragma unroll
    for (int j = 0; j < kQB; ++j)
      if (tid + j * kGatherThreads < qn) *q_dst(tid + j * kGatherThreads) = qv[j];
    // the first step's column indices and edge rows, in flight from here on
    // (issued after the stores above: a wait for Q placed after the branches
    // of this call would also wait for them)
    if (nnz_i > 0) prefetch_first();
  }
  for (int t = tid + kGatherThreads; t <= nn; t += kGatherThreads) s_rp[t] = rp_val(t, a.row_ptr[n0 + t]);
  for (int t = tid + kQB * kGatherThreads; t < qn; t += kGatherThreads) *q_dst(t) = ld16(q_src(t));
  __syncthreads();

  for (int t = tid; t < nn * chunks; t += kGatherThreads) {
    const int li = t / chunks, c = t - li * chunks;
    if (s_rp[li + 1] - s_rp[li] <= 0)
      st16(a.out + ((int64_t)(n0 + li) * rowstride + (int64_t)hb * a.HB * D + c * VEC) * ESZ, u32x4{0u, 0u, 0u, 0u});
  }

  // ---- phase 1: equal contiguous pieces of the workgroup's edges
  int node = 0, nstart = 0, nend = 0;
  bool first_rec = false;   // this slot holds a record [0]
  int rec0_node = -1;
  if (ps < pe) {
    int lo = 0, hi = nn - 1;  // last local node with s_rp[node] <= ps
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_rp[mid] <= ps) lo = mid; else hi = mid - 1;
    }
    node = lo;
    nstart = s_rp[node];
    nend = s_rp[node + 1];
    while (nend <= ps && node < nn - 1) {  // only reachable for malformed pointers
      ++node;
      nstart = nend;
      nend = s_rp[node + 1];
    }
  }
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  float qf[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) qf[i] = 0.f;
  // Q of local destination nd: from LDS when staged there; the value is
  // widened inside each branch so that no wait for the global load is left
  // pending where the branches join
  auto load_q = [&](int nd) {
    if constexpr (!AGG) {
      if (!active) return;
      if (nd < qcap) {
        Conv<T>::widen(*reinterpret_cast<const u32x4*>(s_q + nd * qrow + lig * 16), qf);
      } else {
        Conv<T>::widen(ld16(a.q + ((int64_t)(n0 + nd) * a.q_stride + eoff) * ESZ), qf);
      }
    }
  };
  if (ps < pe) load_q(node);


  // a row cut across workgroups always leaves records (merged in phase 3).
  // A destination that continues past the piece is its last one, so inside
  // the loop (after_loop false) only records [0] arise; a [1] there could
  // only come from a malformed row_ptr and is dropped (the result of such a
  // graph is unspecified) rather than written over Q rows still in use.
  auto flush = [&](bool after_loop) {
    const bool started_before = nstart < ps || (split && node == 0 && cont_first);
    const bool continues = nend > pe || (split && node == nn - 1 && cont_last);
    if (!started_before && !continues) {
      if (active) M::store(a, a.out + ((int64_t)(n0 + node) * rowstride + eoff) * ESZ, l, acc);
    } else if (started_before) {
      s_pm0[rec] = m;
      s_pl0[rec] = l;
#pragma unroll
      for (int i = 0; i < VEC; ++i) s_pacc0[rec * VEC + i] = acc[i];
      first_rec = true;
      rec0_node = node;
    } else if (after_loop) {
      s_pm1[rec] = m;
      s_pl1[rec] = l;
#pragma unroll
      for (int i = 0; i < VEC; ++i) s_pacc1[rec * VEC + i] = acc[i];
    }
  };

  // The edge loop.  Every load is issued without a branch around it: a
  // position past the slot's piece is clamped to its last edge (or to
  // position 0 for a slot without edges) and its rows are never used.  So the
  // compiler's in-order wait counts stay exact and a step waits for its own
  // K / V rows only, not for the column indices and edge rows of the next
  // step, which are in flight while it computes (edge ids, which the edge
  // rows depend on, run two steps ahead).  Divergent lanes run both sides of
  // a branch, so a global load on either side would make every later use
  // wait for all loads in flight: the choice below is workgroup-uniform.
  //  Q_LDS: every destination's Q row is staged in LDS.
  auto edge_loop = [&](auto q_lds) {
    constexpr bool Q_LDS = decltype(q_lds)::value;
    auto get_q = [&](int nd) {
      if constexpr (Q_LDS && !AGG) {
        if (active) Conv<T>::widen(*reinterpret_cast<const u32x4*>(s_q + nd * qrow + lig * 16), qf);
      } else {
        load_q(nd);
      }
    };
    for (int base = ps; base < pe; base += U) {
      int cols[U], rows[U];
      u32x4 er[U], kr[U], vr[U];
      float wt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cols[u] = min(max(cN[u], 0), nmax);
        rows[u] = rN[u];
        er[u] = eN[u];
        wt[u] = wN[u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (!AGG) kr[u] = ld16(kv_ptr16(a.k, cols[u]));
        vr[u] = ld16(kv_ptr16(a.v, cols[u]));
      }
      // the next step's indices and edge rows, in flight while this one computes
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cN[u] = a.col_idx[min(base + U + u, plast)];
        if constexpr (ROWS) {
          rN[u] = fix_row(rNN[u]);
          rNN[u] = raw_row(min(base + 2 * U + u, plast));
        }
        if constexpr (HAS_E) eN[u] = load_e(rN[u]);
        if constexpr (AGG) wN[u] = a.w[(int64_t)rN[u] * a.H + hw];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = base + u;
        if (p >= pe) break;
        if (p >= nend) {
          flush(false);
          while (node < nn - 1) {  // next destination with edges (monotone pointers: one step + empties)
            ++node;
            nstart = nend;
            nend = s_rp[node + 1];
            if (nend > p) break;
          }
          m = -INFINITY;
          l = 0.f;
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
          get_q(node);
        }
        u32x4 xo;
        M::step(a, qf, kr[u], er[u], vr[u], wt[u], m, l, acc, xo);
        if constexpr (EOUT)
          if (active) st16(const_cast<uint8_t*>(row_ptr16(a.e_out, rows[u])), xo);
      }
    }
  };
  if (nnz_i > 0) {
    if constexpr (split) {
      if (nn <= qcap) edge_loop(std::true_type{});
      else edge_loop(std::false_type{});
    } else {
      edge_loop(std::true_type{});  // the node partition stages every Q row
    }
  }
  __syncthreads();  // no slot reads the Q rows any more: records [1] may take their place
  if (ps < pe) flush(true);
  __syncthreads();

  // ---- phase 2: the slot holding a cut destination's last edge merges its pieces
  const bool xwg_first = split && cont_first && nn > 0;
  const bool xwg_last = split && cont_last && nn > 0 && !(nn == 1 && cont_first);
  if (first_rec && s_rp[rec0_node + 1] <= pe && !(rec0_node == 0 && xwg_first) && !(rec0_node == nn - 1 && xwg_last)) {
    const int first_slot = min(max((s_rp[rec0_node] - E0) / C, 0), slot);
    float mm = s_pm1[first_slot * G + lig], ll = s_pl1[first_slot * G + lig], aa[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) aa[i] = s_pacc1[(first_slot * G + lig) * VEC + i];
    for (int s = first_slot + 1; s <= slot; ++s) {
      float a2[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) a2[i] = s_pacc0[(s * G + lig) * VEC + i];
      M::fold(mm, ll, aa, s_pm0[s * G + lig], s_pl0[s * G + lig], a2);
    }
    if (active) M::store(a, a.out + ((int64_t)(n0 + rec0_node) * rowstride + eoff) * ESZ, ll, aa);
  }

  // ---- phase 3: rows cut across workgroups.  Wave 0 takes the first row, wave
  // 1 the last; its lanes 0..G-1 act as one slot.  The row's records in LDS
  // are merged in slot order into this workgroup's part, which is written to
  // the workspace with device-coherent stores; then the part's flag goes up,
  // and the flags of all parts are read: a part that finds them all raised
  // merges the parts in order and writes the row.  Of two parts the later to
  // raise its flag sees the other's (each waits until its stores are done
  // before reading), so some part merges; parts that merge write identical bits.
  if (split && lane < G && ((wave == 0 && xwg_first) || (wave == 1 && xwg_last))) {
    const int kind = wave, nd = kind == 0 ? 0 : nn - 1;
    const int s0 = min(max((s_rp[nd] - E0) / C, 0), NS - 1);
    const int t0 = min(max((max(s_rp[nd + 1], s_rp[nd] + 1) - 1 - E0) / C, s0), NS - 1);
    // the first row's records are all "started before"; the last row starts
    // inside slot s0's piece
    float pm, pl, pa[VEC];
    if (kind == 0) {
      pm = s_pm0[s0 * G + lig];
      pl = s_pl0[s0 * G + lig];
#pragma unroll
      for (int i = 0; i < VEC; ++i) pa[i] = s_pacc0[(s0 * G + lig) * VEC + i];
    } else {
      pm = s_pm1[s0 * G + lig];
      pl = s_pl1[s0 * G + lig];
#pragma unroll
      for (int i = 0; i < VEC; ++i) pa[i] = s_pacc1[(s0 * G + lig) * VEC + i];
    }
    for (int sl = s0 + 1; sl <= t0; ++sl) {
      float a2[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) a2[i] = s_pacc0[(sl * G + lig) * VEC + i];
      M::fold(pm, pl, pa, s_pm0[sl * G + lig], s_pl0[sl * G + lig], a2);
    }
    const int64_t HB_B = (int64_t)gridDim.y * a.num_wg, hb_B = (int64_t)hb * a.num_wg;
    auto part = [&](int k, int64_t bb) { return (int64_t)k * HB_B + hb_B + bb; };
    const int64_t row = n0 + nd;
    {
      const int64_t me = part(kind, blk) * G + lig;
      __hip_atomic_store(a.ws_ml + me * 2, pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ws_ml + me * 2 + 1, pl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        __hip_atomic_store(a.ws_acc + me * VEC + i, pa[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // the part is at the device coherence point before its flag
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lig == 0) __hip_atomic_store(a.ws_flags + part(kind, blk), a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // the flag is up before the other flags are read
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    {
      const int64_t rs = min(max(a.row_ptr[row], 0), nnz_i), re = min(max(a.row_ptr[row + 1], 0), nnz_i);
      const int64_t b0 = (row + rs) / a.items_per_wg, b1 = (row + re - 1) / a.items_per_wg;
      bool in = true;
      for (int64_t bb = b0 + lig; bb <= b1; bb += G)
        in = in && __hip_atomic_load(a.ws_flags + part(bb == b0 ? 1 : 0, bb), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == a.token;
      const uint64_t smask = G == 64 ? ~0ull : ((1ull << G) - 1);
      if (!(__ballot(!in) & smask)) {
        auto ld = [&](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        const int64_t q0 = part(1, b0) * G + lig;
        float mm = ld(a.ws_ml + q0 * 2), ll = ld(a.ws_ml + q0 * 2 + 1), aa[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) aa[i] = ld(a.ws_acc + q0 * VEC + i);
        for (int64_t bb = b0 + 1; bb <= b1; ++bb) {
          const int64_t qb = part(0, bb) * G + lig;
          float a2[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) a2[i] = ld(a.ws_acc + qb * VEC + i);
          M::fold(mm, ll, aa, ld(a.ws_ml + qb * 2), ld(a.ws_ml + qb * 2 + 1), a2);
        }
        if (active) M::store(a, a.out + (row * rowstride + eoff) * ESZ, ll, aa);
        // Lower the row's flags again.  Every flag a launch raises is back at
        // 0 when it ends, so a launch whose token repeats (a captured launch
        // replayed from a HIP graph keeps its arguments) never finds an
        // earlier launch's flags raised and never merges its stale parts.  A
        // part still reading the flags then sees a 0 and leaves the merge to
        // this one.
        for (int64_t bb = b0 + lig; bb <= b1; bb += G)
          __hip_atomic_store(a.ws_flags + part(bb == b0 ? 1 : 0, bb), (uint64_t)0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launch helpers, one set per partition kind (PART); the sets are compiled in
// separate translation units
// ---------------------------------------------------------------------------

// What a launch computes; the geometry is derived from it.
struct Problem {
  int32_t n, H, head_dim;
  int64_t nnz;
  gattn_dtype dtype;
  int mode;
  bool he, eout;
  bool low;  // low average degree: fewer edges per step (standard without E, aggregate)
};


namespace detail {

// Edges per step: U_E with an edge tensor, else U, or U_LOW for graphs of
// low average degree (standard mode and aggregation): with few edges per
// destination a shorter step keeps fewer registers and more waves resident.
inline int unroll_of(const Problem& p) {
  if (p.he) return GATTN_GATHER_U_E;
  return p.low && p.mode != GATTN_SOFTMAX_CLIPPED ? GATTN_GATHER_U_LOW : GATTN_GATHER_U;
}

template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int PART, int U>
constexpr auto kernel_of() { return gather_kernel<T, D, MODE, HAS_E, EOUT, U, PART>; }

// Workgroups of one instantiation that fit on a CU at once (queried once).
template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int PART, int U>
int resident_per_cu() {
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel_of<T, D, MODE, HAS_E, EOUT, PART, U>(),
                                                     kGatherThreads, 0) != hipSuccess)
      b = 1;
    return std::max(b, 1);
  }();
  return per_cu;
}

// Calls F::template run<T, D, MODE, HAS_E, EOUT, U>() for the instantiation
// of p.  The instantiations that exist: standard +-E, clipped +-E (+ edge
// update with E), aggregate; the standard mode without E and the aggregate
// also with the low-degree step.
template <typename F, typename T, int D>
auto by_variant(const Problem& p, const F& f) {
  constexpr int UE = GATTN_GATHER_U_E, UN = GATTN_GATHER_U, UL = GATTN_GATHER_U_LOW;
  const bool low = unroll_of(p) == UL && UL != UN;
  if (p.mode == kModeAggregate)
    return low ? f.template run<T, D, kModeAggregate, false, false, UL>()
               : f.template run<T, D, kModeAggregate, false, false, UN>();
  if (p.mode == GATTN_SOFTMAX_STANDARD) {
    if (p.he) return f.template run<T, D, GATTN_SOFTMAX_STANDARD, true, false, UE>();
    return low ? f.template run<T, D, GATTN_SOFTMAX_STANDARD, false, false, UL>()
               : f.template run<T, D, GATTN_SOFTMAX_STANDARD, false, false, UN>();
  }
  if (!p.he) return f.template run<T, D, GATTN_SOFTMAX_CLIPPED, false, false, UN>();
  return p.eout ? f.template run<T, D, GATTN_SOFTMAX_CLIPPED, true, true, UE>()
                : f.template run<T, D, GATTN_SOFTMAX_CLIPPED, true, false, UE>();
}

template <typename F, typename T>
auto by_dim(const Problem& p, const F& f) {
  switch (p.head_dim) {
    case 16: return by_variant<F, T, 16>(p, f);
    case 32: return by_variant<F, T, 32>(p, f);
    case 64: return by_variant<F, T, 64>(p, f);
    default: return by_variant<F, T, 128>(p, f);
  }
}

template <typename F>
auto dispatch(const Problem& p, const F& f) {
  switch (p.dtype) {
    case GATTN_F32: return by_dim<F, float>(p, f);
    case GATTN_F16: return by_dim<F, _Float16>(p, f);
    default: return by_dim<F, bf16_t>(p, f);
  }
}

template <int PART>
struct Resident {
  template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int U>
  int run() const { return resident_per_cu<T, D, MODE, HAS_E, EOUT, PART, U>(); }
};

template <int PART>
struct Launch {
  const GatherArgs& ga;
  dim3 grid;
  hipStream_t s;
  template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int U>
  hipError_t run() const {
    hipLaunchKernelGGL((kernel_of<T, D, MODE, HAS_E, EOUT, PART, U>()), grid, dim3(kGatherThreads), 0, s, ga);
    return hipGetLastError();
  }
};

// Defined in forward_gather.hip (kPartNode) and forward_gather_split.hip
// (kPartSplit).
template <int PART>
int resident_of(const Problem& p);
template <int PART>
hipError_t launch_kernels(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s);

template <> int resident_of<kPartNode>(const Problem& p);
template <> int resident_of<kPartSplit>(const Problem& p);
template <> hipError_t launch_kernels<kPartNode>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s);
template <> hipError_t launch_kernels<kPartSplit>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s);

template <int PART>
int resident_impl(const Problem& p) { return dispatch(p, Resident<PART>{}); }
template <int PART>
hipError_t launch_impl(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  return dispatch(p, Launch<PART>{ga, grid, s});
}

}  // namespace detail
}  // namespace gattn
