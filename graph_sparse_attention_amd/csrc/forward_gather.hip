// forward_gather.hip -- wave64 gather kernel of the fused graph attention.
//
// What it computes (gattn-triton article, "Background" and "Fusing the full
// graph attention"; Fused3S abstract): for every destination i and head h,
// a logit per in-edge from q_i and k_j (times e_ij when an edge projection
// is given), a softmax over the in-edges of i -- standard max-subtracted, or
// the RTMScore form exp(clip) / (sum + eps) -- and o_i = sum_j alpha_ij v_j.
// No per-edge tensor is written.
//
// Mapping on CDNA4.
//  * A "slot" is a group of G lanes (G = 2..64, a power of two) that holds one
//    edge's [HB heads x D] slice of a K / V / E row, 16 bytes per lane, so a
//    slot's loads are one contiguous, coalesced run.  A wave holds 64/G slots,
//    a 256-thread workgroup NS = 4*64/G slots.  The logit of a head is summed
//    over its D/VEC lanes with DPP inside a 16-lane row.
//  * A workgroup owns a contiguous range of destinations (node-parallel as in
//    the article's one-program-per-node kernels and Fused3S Figure 2, top) for
//    one block of heads.  Its edges are cut into NS equal pieces; a slot
//    takes the destinations whose first edge falls in its piece and walks
//    their edges U at a time, keeping the online-softmax state (m, l) and the
//    fp32 accumulator in registers.  A destination with many more edges than
//    a piece is instead split over all slots, whose partial (m, l, acc) are
//    merged through LDS in slot order -- deterministic, no atomics.
//  * Consecutive workgroups are mapped onto one XCD so that destinations of
//    one batched graph, whose sources are nearby, share an L2.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

constexpr int kGatherThreads = 256;
constexpr int kMaxNodesPerWg = 1024;

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
};

template <typename T, int D, int MODE, bool HAS_E>
struct EdgeMath {
  static constexpr int VEC = Elem<T>::kVec;
  static constexpr int LPH = D / VEC;

  // one edge: logit, online softmax update, accumulate v
  static __device__ __forceinline__ void step(const GatherArgs& a, const float* qf, u32x4 kr, u32x4 er,
                                              u32x4 vr, float& m, float& l, float* acc) {
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
      const float corr = fast_exp2(m - mn);
      const float p = fast_exp2(lg - mn);
      l = l * corr + p;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * corr + p * vf[i];
      m = mn;
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        float t = fminf(fmaxf(a.scale * qf[i] * kf[i], a.lo), a.hi);
        s += HAS_E ? t * ef[i] : t;
      }
      s = group_sum<LPH>(s);
      const float lg = fminf(fmaxf(s, a.lo), a.hi);
      const float p = fast_exp2(lg * kLog2e);
      l += p;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += p * vf[i];
    }
  }

  static __device__ __forceinline__ void store(const GatherArgs& a, uint8_t* dst, float l, const float* acc) {
    const float den = (MODE == GATTN_SOFTMAX_STANDARD) ? l : l + a.eps;
    const float inv = 1.0f / den;
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = acc[i] * inv;
    st16(dst, Conv<T>::narrow(o));
  }
};

template <typename T, int D, int MODE, bool HAS_E, int U>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
  using M = EdgeMath<T, D, MODE, HAS_E>;
  constexpr int VEC = Elem<T>::kVec;
  constexpr int LPH = D / VEC;
  constexpr int ESZ = sizeof(T);

  __shared__ int32_t s_rp[kMaxNodesPerWg + 1];
  __shared__ int32_t s_big[kMaxNodesPerWg];
  __shared__ int32_t s_nbig;
  __shared__ float s_pm[kGatherThreads];
  __shared__ float s_pl[kGatherThreads];
  __shared__ float s_pacc[kGatherThreads * VEC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = 1 << a.log2G;
  const int spw = 64 >> a.log2G;
  const int NS = 4 * spw;
  const int slot = wave * spw + (lane >> a.log2G);
  const int lig = lane & (G - 1);
  const int hh = lig / LPH, dch = lig % LPH;
  const int hb = blockIdx.y;
  const int head = hb * a.HB + hh;
  const bool active = hh < a.HB && head < a.H;
  const int64_t rowstride = (int64_t)a.H * D;
  const int64_t eoff = (int64_t)head * D + dch * VEC;
  const int nmax = a.n - 1;

  const int blk = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int n0 = blk * a.npw;
  const int nn = min(a.npw, a.n - n0);
  const int nnz_i = (int)a.nnz;

  // ---- phase 0: pointer range into LDS; list heavy destinations; zero isolated ones
  for (int t = tid; t <= nn; t += kGatherThreads) s_rp[t] = min(max(a.row_ptr[n0 + t], 0), nnz_i);
  if (tid == 0) s_nbig = 0;
  __syncthreads();
  const int E0 = s_rp[0];
  const int E1 = max(E0, s_rp[nn]);
  const int C = (E1 - E0 + NS - 1) / NS;
  const int big = max(2 * C, 16);
  const int heads_here = min(a.HB, a.H - hb * a.HB);
  const int chunks = heads_here * LPH;  // 16-byte chunks of this head block per node
  for (int t = tid; t < nn * chunks; t += kGatherThreads) {
    const int li = t / chunks, c = t - li * chunks;
    if (s_rp[li + 1] - s_rp[li] <= 0) {
      uint8_t* dst = a.out + ((int64_t)(n0 + li) * rowstride + (int64_t)hb * a.HB * D + c * VEC) * ESZ;
      st16(dst, u32x4{0u, 0u, 0u, 0u});
    }
  }
  for (int t = tid; t < nn; t += kGatherThreads)
    if (s_rp[t + 1] - s_rp[t] > big) s_big[atomicAdd(&s_nbig, 1)] = t;
  __syncthreads();

  // ---- phase 1: each slot walks the light destinations that start in its piece
  auto lower = [&](int target) {
    int lo = 0, hi = nn;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_rp[mid] < target) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  const int a_s = slot == 0 ? 0 : lower(E0 + slot * C);
  const int a_e = slot == NS - 1 ? nn : lower(E0 + (slot + 1) * C);

  int node = a_s - 1, pos = 0, end = 0;
  auto advance = [&]() -> bool {
    for (;;) {
      ++node;
      if (node >= a_e) return false;
      pos = s_rp[node];
      end = s_rp[node + 1];
      if (end > pos && end - pos <= big) return true;
    }
  };
  bool have = advance();
  int cur = -1;
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  float qf[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) qf[i] = 0.f;

  while (have) {
    int cn[U], cp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (have) {
        cn[u] = node;
        cp[u] = pos;
        if (++pos >= end) have = advance();
      } else {
        cn[u] = -1;
        cp[u] = 0;
      }
    }
    u32x4 kr[U], vr[U], er[U], qr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = vr[u] = er[u] = qr[u] = u32x4{0u, 0u, 0u, 0u};
      if (cn[u] >= 0 && active) {
        const int j = min(max(a.col_idx[cp[u]], 0), nmax);
        kr[u] = ld16(a.k + ((int64_t)j * rowstride + eoff) * ESZ);
        vr[u] = ld16(a.v + ((int64_t)j * rowstride + eoff) * ESZ);
        if constexpr (HAS_E) er[u] = ld16_stream(a.e + ((int64_t)cp[u] * rowstride + eoff) * ESZ);
        if (u == 0 || cn[u] != cn[u - 1]) qr[u] = ld16(a.q + ((int64_t)(n0 + cn[u]) * rowstride + eoff) * ESZ);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (cn[u] < 0) break;
      if (cn[u] != cur) {
        if (cur >= 0 && active)
          M::store(a, a.out + ((int64_t)(n0 + cur) * rowstride + eoff) * ESZ, l, acc);
        cur = cn[u];
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
      }
      if (u == 0 || cn[u] != cn[u - 1]) Conv<T>::widen(qr[u], qf);
      M::step(a, qf, kr[u], er[u], vr[u], m, l, acc);
    }
  }
  if (cur >= 0 && active) M::store(a, a.out + ((int64_t)(n0 + cur) * rowstride + eoff) * ESZ, l, acc);

  // ---- phase 2: heavy destinations, split over all slots, merged in slot order
  const int nbig = s_nbig;
  for (int bi = 0; bi < nbig; ++bi) {
    const int li = s_big[bi];
    const int st = s_rp[li], en = s_rp[li + 1];
    const int cb = (en - st + NS - 1) / NS;
    const int ps = st + slot * cb, pe = min(ps + cb, en);
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    if (active) Conv<T>::widen(ld16(a.q + ((int64_t)(n0 + li) * rowstride + eoff) * ESZ), qf);
    for (int p = ps; p < pe; p += U) {
      u32x4 kr[U], vr[U], er[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = vr[u] = er[u] = u32x4{0u, 0u, 0u, 0u};
        if (p + u < pe && active) {
          const int j = min(max(a.col_idx[p + u], 0), nmax);
          kr[u] = ld16(a.k + ((int64_t)j * rowstride + eoff) * ESZ);
          vr[u] = ld16(a.v + ((int64_t)j * rowstride + eoff) * ESZ);
          if constexpr (HAS_E) er[u] = ld16_stream(a.e + ((int64_t)(p + u) * rowstride + eoff) * ESZ);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p + u >= pe) break;
        M::step(a, qf, kr[u], er[u], vr[u], m, l, acc);
      }
    }
    s_pm[slot * G + lig] = m;
    s_pl[slot * G + lig] = l;
#pragma unroll
    for (int i = 0; i < VEC; ++i) s_pacc[(slot * G + lig) * VEC + i] = acc[i];
    __syncthreads();
    if (tid < G) {
      const int hh2 = tid / LPH, dch2 = tid % LPH;
      const int head2 = hb * a.HB + hh2;
      if (hh2 < a.HB && head2 < a.H) {
        float mm = -INFINITY;
        if constexpr (MODE == GATTN_SOFTMAX_STANDARD)
          for (int s = 0; s < NS; ++s) mm = fmaxf(mm, s_pm[s * G + tid]);
        float L = 0.f, A[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) A[i] = 0.f;
        for (int s = 0; s < NS; ++s) {
          const float ls = s_pl[s * G + tid];
          if (ls == 0.f) continue;
          const float f = (MODE == GATTN_SOFTMAX_STANDARD) ? fast_exp2(s_pm[s * G + tid] - mm) : 1.f;
          L += ls * f;
#pragma unroll
          for (int i = 0; i < VEC; ++i) A[i] += s_pacc[(s * G + tid) * VEC + i] * f;
        }
        const int64_t eoff2 = (int64_t)head2 * D + dch2 * VEC;
        M::store(a, a.out + ((int64_t)(n0 + li) * rowstride + eoff2) * ESZ, L, A);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

template <typename T, int D, int MODE, bool HAS_E>
hipError_t launch_typed(const GatherArgs& ga, dim3 grid, hipStream_t s) {
  constexpr int U = (sizeof(T) == 4 || HAS_E) ? 4 : 8;
  hipLaunchKernelGGL((gather_kernel<T, D, MODE, HAS_E, U>), grid, dim3(kGatherThreads), 0, s, ga);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const gattn_forward_args& a, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  const bool he = a.e != nullptr;
  if (a.mode == GATTN_SOFTMAX_STANDARD)
    return he ? launch_typed<T, D, GATTN_SOFTMAX_STANDARD, true>(ga, grid, s)
              : launch_typed<T, D, GATTN_SOFTMAX_STANDARD, false>(ga, grid, s);
  return he ? launch_typed<T, D, GATTN_SOFTMAX_CLIPPED, true>(ga, grid, s)
            : launch_typed<T, D, GATTN_SOFTMAX_CLIPPED, false>(ga, grid, s);
}

template <typename T>
hipError_t launch_t(const gattn_forward_args& a, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  switch (a.head_dim) {
    case 16: return launch_d<T, 16>(a, ga, grid, s);
    case 32: return launch_d<T, 32>(a, ga, grid, s);
    case 64: return launch_d<T, 64>(a, ga, grid, s);
    default: return launch_d<T, 128>(a, ga, grid, s);
  }
}

}  // namespace

hipError_t launch_forward_gather(const gattn_forward_args& a, hipStream_t s) {
  if (a.num_nodes == 0) return hipSuccess;
  const int vec = a.dtype == GATTN_F32 ? 4 : 8;
  const int lph = a.head_dim / vec;
  const int hb = std::min(a.num_heads, 64 / lph);
  int g = 1;
  while (g < hb * lph) g <<= 1;
  int log2g = 0;
  while ((1 << log2g) < g) ++log2g;
  const int ns = 4 * (64 / g);
  const double avg = a.num_nodes > 0 ? (double)a.nnz / a.num_nodes : 0.0;
  const int u = (a.dtype == GATTN_F32 || a.e) ? 4 : 8;
  int npw = kMaxNodesPerWg;
  if (avg > 0) {
    const double target = ns * std::max(2.0 * u, 2.0 * avg);
    npw = (int)std::min<double>(kMaxNodesPerWg, std::max(1.0, std::ceil(target / avg)));
  }

  GatherArgs ga;
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
  ga.HB = hb;
  ga.log2G = log2g;
  ga.npw = npw;
  ga.scale = a.mode == GATTN_SOFTMAX_STANDARD ? a.scale * kLog2e : a.scale;
  ga.lo = a.clip_lo;
  ga.hi = a.clip_hi;
  ga.eps = a.eps;
  dim3 grid((unsigned)ceil_div(a.num_nodes, npw), (unsigned)ceil_div(a.num_heads, hb));
  switch (a.dtype) {
    case GATTN_F32: return launch_t<float>(a, ga, grid, s);
    case GATTN_F16: return launch_t<_Float16>(a, ga, grid, s);
    default: return launch_t<bf16_t>(a, ga, grid, s);
  }
}

}  // namespace gattn
