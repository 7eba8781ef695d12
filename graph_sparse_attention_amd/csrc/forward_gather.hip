// forward_gather.hip -- wave64 gather kernel of the fused graph attention.
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
//    U edges at a time, prefetching the next piece of column indices (and E
//    rows) while it computes, and keeps the online-softmax state (m, l) and
//    the fp32 accumulator in registers.  A destination that is cut by a piece
//    boundary leaves partial (m, l, acc) records in LDS; the slot holding its
//    last edge merges them in slot order.  Deterministic, no atomics.
//  * Consecutive workgroups are mapped onto one XCD so that destinations of
//    one batched graph, whose sources are nearby, share an L2.
#include "common.hpp"
#include "internal.hpp"

#ifndef GATTN_GATHER_Q_LDS_BYTES
#define GATTN_GATHER_Q_LDS_BYTES 12288  // Q rows staged per workgroup
#endif
#ifndef GATTN_GATHER_EDGES_PER_SLOT
#define GATTN_GATHER_EDGES_PER_SLOT 3   // target edges per slot, in units of U
#endif
#ifndef GATTN_GATHER_U
#define GATTN_GATHER_U 8                // edges per step without an edge tensor
#endif
#ifndef GATTN_GATHER_U_E
#define GATTN_GATHER_U_E 4              // edges per step with an edge tensor
#endif
#ifndef GATTN_GATHER_E_STREAMING
#define GATTN_GATHER_E_STREAMING 1      // non-temporal loads for the edge tensor
#endif
#ifndef GATTN_XCD_REMAP
#define GATTN_XCD_REMAP 1
#endif

namespace gattn {

constexpr int kGatherThreads = 256;
constexpr int kMaxNodesPerWg = 1024;
constexpr int kQLdsBytes = GATTN_GATHER_Q_LDS_BYTES;
constexpr int kModeAggregate = 2;  // given per-edge weights instead of logits and softmax

struct GatherArgs {
  const int32_t* __restrict__ row_ptr;
  const int32_t* __restrict__ col_idx;
  const uint8_t* __restrict__ q;
  const uint8_t* __restrict__ k;
  const uint8_t* __restrict__ v;
  const uint8_t* __restrict__ e;
  uint8_t* __restrict__ out;
  int64_t nnz;
  int32_t n, H, HB, log2G, npw;
  float scale;  // standard: scale * log2(e); clipped: scale
  float lo, hi, eps;
  const int32_t* __restrict__ ids;  // nullable: row of e / e_out / w for CSR position p
  uint8_t* __restrict__ e_out;      // clipped mode with e: the per-edge update
  const float* __restrict__ w;      // aggregate mode: [nnz, H] weights
  int32_t normalize;                // aggregate mode: divide by (sum of w + eps)
};

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

template <typename T, int D, int MODE, bool HAS_E, bool EOUT, int U>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
  using M = EdgeMath<T, D, MODE, HAS_E, EOUT>;
  constexpr int VEC = Elem<T>::kVec;
  constexpr int LPH = D / VEC;
  constexpr int ESZ = sizeof(T);
  constexpr bool AGG = MODE == kModeAggregate;
  constexpr bool ROWS = HAS_E || AGG;  // per-edge rows are read

  __shared__ int32_t s_rp[kMaxNodesPerWg + 1];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[AGG ? 16 : kQLdsBytes];
  // partial records: [0] first destination of a piece (started in an earlier
  // piece), [1] last destination of a piece (continues into a later one)
  __shared__ float s_pm[2][kGatherThreads];
  __shared__ float s_pl[2][kGatherThreads];
  __shared__ float s_pacc[2][kGatherThreads * VEC];

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
  const int n0 = blk * a.npw;
  const int nn = min(a.npw, a.n - n0);
  const int nnz_i = (int)a.nnz;

  // ---- phase 0: row pointers and Q rows into LDS (one coalesced pass)
  for (int t = tid; t <= nn; t += kGatherThreads) s_rp[t] = min(max(a.row_ptr[n0 + t], 0), nnz_i);
  if constexpr (!AGG) {
    for (int t = tid; t < nn * chunks; t += kGatherThreads) {
      const int li = t / chunks, c = t - li * chunks;
      *reinterpret_cast<u32x4*>(s_q + li * qrow + c * 16) =
          ld16(a.q + ((int64_t)(n0 + li) * rowstride + (int64_t)hb * a.HB * D + c * VEC) * ESZ);
    }
  }
  __syncthreads();
  for (int t = tid; t < nn * chunks; t += kGatherThreads) {
    const int li = t / chunks, c = t - li * chunks;
    if (s_rp[li + 1] - s_rp[li] <= 0)
      st16(a.out + ((int64_t)(n0 + li) * rowstride + (int64_t)hb * a.HB * D + c * VEC) * ESZ, u32x4{0u, 0u, 0u, 0u});
  }

  // ---- phase 1: equal contiguous pieces of the workgroup's edges
  const int E0 = s_rp[0];
  const int E1 = max(E0, s_rp[nn]);
  const int C = max((E1 - E0 + NS - 1) / NS, 1);
  const int ps = min(E0 + slot * C, E1);
  const int pe = min(ps + C, E1);
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
  if constexpr (!AGG)
    if (ps < pe && active) Conv<T>::widen(*reinterpret_cast<const u32x4*>(s_q + node * qrow + lig * 16), qf);

  // row of the per-edge tensors for CSR position p (clamped like the sources)
  auto edge_row = [&](int p) -> int { return a.ids ? min(max(a.ids[p], 0), nnz_i - 1) : p; };
  auto load_e = [&](int row) -> u32x4 {
    const uint8_t* ptr = a.e + ((int64_t)row * rowstride + eoff) * ESZ;
    return GATTN_GATHER_E_STREAMING ? ld16_stream(ptr) : ld16(ptr);
  };

  auto flush = [&]() {
    const bool started_before = nstart < ps;
    const bool continues = nend > pe;
    if (!started_before && !continues) {
      if (active) M::store(a, a.out + ((int64_t)(n0 + node) * rowstride + eoff) * ESZ, l, acc);
    } else {
      const int r = started_before ? 0 : 1;
      s_pm[r][rec] = m;
      s_pl[r][rec] = l;
#pragma unroll
      for (int i = 0; i < VEC; ++i) s_pacc[r][rec * VEC + i] = acc[i];
      if (started_before) {
        first_rec = true;
        rec0_node = node;
      }
    }
  };

  int colsN[U], rowN[U];
  u32x4 eN[U];
  float wN[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = ps + u;
    colsN[u] = p < pe ? a.col_idx[p] : 0;
    rowN[u] = 0;
    eN[u] = u32x4{0u, 0u, 0u, 0u};
    wN[u] = 0.f;
    if constexpr (ROWS)
      if (p < pe) rowN[u] = edge_row(p);
    if constexpr (HAS_E)
      if (p < pe && active) eN[u] = load_e(rowN[u]);
    if constexpr (AGG)
      if (p < pe && active) wN[u] = a.w[(int64_t)rowN[u] * a.H + head];
  }
  for (int base = ps; base < pe; base += U) {
    int cols[U], rows[U];
    u32x4 er[U], kr[U], vr[U];
    float wt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cols[u] = min(max(colsN[u], 0), nmax);
      rows[u] = rowN[u];
      er[u] = eN[u];
      wt[u] = wN[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (base + u < pe && active) {
        if constexpr (!AGG) kr[u] = ld16(a.k + ((int64_t)cols[u] * rowstride + eoff) * ESZ);
        vr[u] = ld16(a.v + ((int64_t)cols[u] * rowstride + eoff) * ESZ);
      }
    }
    // prefetch the next piece of indices (and edge rows) while this one computes
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + U + u;
      if (p < pe) {
        colsN[u] = a.col_idx[p];
        if constexpr (ROWS) rowN[u] = edge_row(p);
        if constexpr (HAS_E)
          if (active) eN[u] = load_e(rowN[u]);
        if constexpr (AGG)
          if (active) wN[u] = a.w[(int64_t)rowN[u] * a.H + head];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u;
      if (p >= pe) break;
      if (p >= nend) {
        flush();
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
        if (active) Conv<T>::widen(*reinterpret_cast<const u32x4*>(s_q + node * qrow + lig * 16), qf);
      }
      u32x4 xo;
      M::step(a, qf, kr[u], er[u], vr[u], wt[u], m, l, acc, xo);
      if constexpr (EOUT)
        if (active) st16(a.e_out + ((int64_t)rows[u] * rowstride + eoff) * ESZ, xo);
    }
  }
  if (ps < pe) flush();
  __syncthreads();

  // ---- phase 2: the slot holding a cut destination's last edge merges its pieces
  if (first_rec && s_rp[rec0_node + 1] <= pe) {
    const int first_slot = min(max((s_rp[rec0_node] - E0) / C, 0), slot);
    float mm = s_pm[1][first_slot * G + lig], ll = s_pl[1][first_slot * G + lig], aa[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) aa[i] = s_pacc[1][(first_slot * G + lig) * VEC + i];
    for (int s = first_slot + 1; s <= slot; ++s) {
      float a2[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) a2[i] = s_pacc[0][(s * G + lig) * VEC + i];
      M::fold(mm, ll, aa, s_pm[0][s * G + lig], s_pl[0][s * G + lig], a2);
    }
    if (active) M::store(a, a.out + ((int64_t)(n0 + rec0_node) * rowstride + eoff) * ESZ, ll, aa);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

template <int MODE, bool HAS_E>
constexpr int unroll() { return HAS_E ? GATTN_GATHER_U_E : GATTN_GATHER_U; }

template <typename T, int D, int MODE, bool HAS_E, bool EOUT>
constexpr auto kernel_of() { return gather_kernel<T, D, MODE, HAS_E, EOUT, unroll<MODE, HAS_E>()>; }

// Workgroups of one instantiation that fit on a CU at once (queried once).
template <typename T, int D, int MODE, bool HAS_E, bool EOUT>
int resident_per_cu() {
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel_of<T, D, MODE, HAS_E, EOUT>(), kGatherThreads, 0) !=
        hipSuccess)
      b = 1;
    return std::max(b, 1);
  }();
  return per_cu;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

struct Geometry {
  int npw_target, npw_cap, head_blocks;
};

// Destinations per workgroup: near the target, but rounded so that the grid is
// a whole number of "rounds" of co-resident workgroups (a last, partly filled
// round would leave most CUs idle while it runs).
template <typename T, int D, int MODE, bool HAS_E, bool EOUT>
hipError_t launch_typed(GatherArgs ga, const Geometry& geo, hipStream_t s) {
  const int64_t n = ga.n;
  const int64_t resident = (int64_t)resident_per_cu<T, D, MODE, HAS_E, EOUT>() * device_cus();
  const double wgs = (double)ceil_div(n, geo.npw_target) * geo.head_blocks;
  const int64_t rounds = std::max<int64_t>(1, (int64_t)std::llround(wgs / (double)resident));
  const int64_t per_round = std::max<int64_t>(1, resident / geo.head_blocks);
  int npw = (int)std::min<int64_t>(geo.npw_cap, std::max<int64_t>(1, ceil_div(n, rounds * per_round)));
  ga.npw = npw;
  dim3 grid((unsigned)ceil_div(n, npw), (unsigned)geo.head_blocks);
  hipLaunchKernelGGL((kernel_of<T, D, MODE, HAS_E, EOUT>()), grid, dim3(kGatherThreads), 0, s, ga);
  return hipGetLastError();
}

// the instantiations that exist: standard +-E, clipped +-E (+ edge update
// with E), aggregate
template <typename T, int D>
hipError_t launch_d(int mode, bool he, bool eout, const GatherArgs& ga, const Geometry& geo, hipStream_t s) {
  if (mode == kModeAggregate) return launch_typed<T, D, kModeAggregate, false, false>(ga, geo, s);
  if (mode == GATTN_SOFTMAX_STANDARD)
    return he ? launch_typed<T, D, GATTN_SOFTMAX_STANDARD, true, false>(ga, geo, s)
              : launch_typed<T, D, GATTN_SOFTMAX_STANDARD, false, false>(ga, geo, s);
  if (!he) return launch_typed<T, D, GATTN_SOFTMAX_CLIPPED, false, false>(ga, geo, s);
  return eout ? launch_typed<T, D, GATTN_SOFTMAX_CLIPPED, true, true>(ga, geo, s)
              : launch_typed<T, D, GATTN_SOFTMAX_CLIPPED, true, false>(ga, geo, s);
}

template <typename T>
hipError_t launch_t(int head_dim, int mode, bool he, bool eout, const GatherArgs& ga, const Geometry& geo,
                    hipStream_t s) {
  switch (head_dim) {
    case 16: return launch_d<T, 16>(mode, he, eout, ga, geo, s);
    case 32: return launch_d<T, 32>(mode, he, eout, ga, geo, s);
    case 64: return launch_d<T, 64>(mode, he, eout, ga, geo, s);
    default: return launch_d<T, 128>(mode, he, eout, ga, geo, s);
  }
}

// Heads per workgroup, slot width and destinations per workgroup, then launch.
// ga carries the pointers and scalars; the geometry fields are filled here.
hipError_t launch_gather(GatherArgs ga, int head_dim, gattn_dtype dtype, int mode, bool he, bool eout, hipStream_t s) {
  if (ga.n == 0) return hipSuccess;
  const int esz = dtype == GATTN_F32 ? 4 : 2;
  const int vec = 16 / esz;
  const int lph = head_dim / vec;
  const int hb = std::min(ga.H, 64 / lph);
  int g = 1;
  while (g < hb * lph) g <<= 1;
  int log2g = 0;
  while ((1 << log2g) < g) ++log2g;
  const int ns = 4 * (64 / g);
  const int u = he ? GATTN_GATHER_U_E : GATTN_GATHER_U;
  // about EDGES_PER_SLOT * U edges per slot, bounded by the LDS that stages Q
  // rows (the aggregate mode stages none)
  const int qrow = hb * head_dim * esz;
  Geometry geo;
  geo.npw_cap = mode == kModeAggregate ? kMaxNodesPerWg : std::max(1, std::min(kMaxNodesPerWg, kQLdsBytes / qrow));
  geo.head_blocks = (int)ceil_div(ga.H, hb);
  const double avg = (double)ga.nnz / ga.n;
  geo.npw_target = geo.npw_cap;
  if (avg > 0) {
    const double target = (double)ns * GATTN_GATHER_EDGES_PER_SLOT * u;
    geo.npw_target = (int)std::min<double>(geo.npw_cap, std::max(1.0, std::ceil(target / avg)));
  }
  ga.HB = hb;
  ga.log2G = log2g;
  ga.npw = 0;
  switch (dtype) {
    case GATTN_F32: return launch_t<float>(head_dim, mode, he, eout, ga, geo, s);
    case GATTN_F16: return launch_t<_Float16>(head_dim, mode, he, eout, ga, geo, s);
    default: return launch_t<bf16_t>(head_dim, mode, he, eout, ga, geo, s);
  }
}

}  // namespace

hipError_t launch_forward_gather(const gattn_forward_args& a, hipStream_t s) {
  GatherArgs ga = {};
  ga.row_ptr = a.row_ptr;
  ga.col_idx = a.col_idx;
  ga.q = (const uint8_t*)a.q;
  ga.k = (const uint8_t*)a.k;
  ga.v = (const uint8_t*)a.v;
  ga.e = (const uint8_t*)a.e;
  ga.out = (uint8_t*)a.out;
  ga.nnz = a.nnz;
  ga.n = a.num_nodes;
  ga.H = a.num_heads;
  ga.scale = a.mode == GATTN_SOFTMAX_STANDARD ? a.scale * kLog2e : a.scale;
  ga.lo = a.clip_lo;
  ga.hi = a.clip_hi;
  ga.eps = a.eps;
  ga.ids = a.e ? a.edge_ids : nullptr;
  ga.e_out = (uint8_t*)a.e_out;
  const bool eout = a.e_out != nullptr && a.e != nullptr && a.mode == GATTN_SOFTMAX_CLIPPED;
  return launch_gather(ga, a.head_dim, a.dtype, a.mode, a.e != nullptr, eout, s);
}

hipError_t launch_aggregate_gather(const gattn_aggregate_args& a, hipStream_t s) {
  GatherArgs ga = {};
  ga.row_ptr = a.row_ptr;
  ga.col_idx = a.col_idx;
  ga.v = (const uint8_t*)a.x;
  ga.out = (uint8_t*)a.out;
  ga.nnz = a.nnz;
  ga.n = a.num_nodes;
  ga.H = a.num_heads;
  ga.eps = a.eps;
  ga.ids = a.edge_ids;
  ga.w = a.w;
  ga.normalize = a.normalize;
  return launch_gather(ga, a.head_dim, a.dtype, kModeAggregate, false, false, s);
}

}  // namespace gattn
