// forward_gather.hip -- host side of the gather path: geometry, partition
// plan, launch.  The kernel is in gather_kernel.hpp; this file instantiates
// it for the node partition, forward_gather_split.hip for the balanced one.
#include <atomic>
#include <chrono>
#include <random>

#include "gather_kernel.hpp"

namespace gattn {
namespace detail {
template <>
int resident_of<false>(const Problem& p) { return resident_impl<false>(p); }
template <>
hipError_t launch_kernels<false>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  return launch_impl<false>(p, ga, grid, s);
}
}  // namespace detail

namespace {

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

struct Plan {
  int hb, log2g, G, vec, head_blocks;
  int npw;                  // node partition: destinations per workgroup
  int64_t C, B;             // balanced partition: items per workgroup, workgroups per head block
  int light_max;
  size_t off_ml, off_acc, ws_bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Heads per workgroup, slot width, and the partition.  Both partitions aim at
// about EDGES_PER_SLOT * U edges per slot and round the grid to whole "rounds"
// of co-resident workgroups (a last, partly filled round would leave most CUs
// idle while it runs).  The node partition is bounded by the LDS that stages
// Q rows; the balanced one keeps its typical row count under that bound.
Plan make_plan(const Problem& p) {
  Plan g{};
  const int esz = p.dtype == GATTN_F32 ? 4 : 2;
  g.vec = 16 / esz;
  const int lph = p.head_dim / g.vec;
  g.hb = std::min(p.H, 64 / lph);
  g.G = 1;
  while (g.G < g.hb * lph) g.G <<= 1;
  g.log2g = 0;
  while ((1 << g.log2g) < g.G) ++g.log2g;
  g.head_blocks = (int)ceil_div(p.H, g.hb);
  const int ns = 4 * (64 / g.G);
  const int u = p.he ? GATTN_GATHER_U_E : GATTN_GATHER_U;
  const double target = (double)ns * GATTN_GATHER_EDGES_PER_SLOT * u;   // edges per workgroup
  const int qrow = g.hb * p.head_dim * esz;
  const int qcap = p.mode == kModeAggregate ? kMaxNodesPerWg : std::max(1, std::min(kMaxNodesPerWg, kQLdsBytes / qrow));
  if (p.n == 0) return g;
  const int64_t resident_all = (int64_t)detail::resident_of<false>(p) * device_cus();
  const int64_t per_round = std::max<int64_t>(1, resident_all / g.head_blocks);
  const int64_t resident_split = (int64_t)detail::resident_of<true>(p) * device_cus();
  const int64_t per_round_split = std::max<int64_t>(1, resident_split / g.head_blocks);

  // node partition
  const double avg = (double)p.nnz / p.n;
  int npw_target = qcap;
  if (avg > 0) npw_target = (int)std::min<double>(qcap, std::max(1.0, std::ceil(target / avg)));
  {
    const double wgs = (double)ceil_div(p.n, npw_target) * g.head_blocks;
    const int64_t rounds = std::max<int64_t>(1, (int64_t)std::llround(wgs / (double)resident_all));
    g.npw = (int)std::min<int64_t>(qcap, std::max<int64_t>(1, ceil_div(p.n, rounds * per_round)));
  }

  // balanced partition over T = N + nnz items
  const int64_t T = (int64_t)p.n + p.nnz;
  const int64_t cmax = kMaxNodesPerWg - 2;
  double c0 = p.nnz > 0 ? target * (double)T / (double)p.nnz : (double)cmax;
  c0 = std::min(c0, (double)qcap * (double)T / (double)p.n);   // typical rows per workgroup <= qcap
  int64_t C = std::min<int64_t>(cmax, std::max<int64_t>(8, (int64_t)c0));
  {
    const double wgs = (double)ceil_div(T, C) * g.head_blocks;
    const int64_t rounds = std::max<int64_t>(1, (int64_t)std::llround(wgs / (double)resident_split));
    C = std::min<int64_t>(cmax, std::max<int64_t>(8, ceil_div(T, rounds * per_round_split)));
  }
  g.C = C;
  g.B = ceil_div(T, C);
  g.light_max = (int)std::max<int64_t>(2, C / 2);
  const size_t parts = (size_t)2 * g.head_blocks * g.B;
  g.off_ml = align256(parts * sizeof(uint64_t));
  g.off_acc = g.off_ml + align256(parts * g.G * 2 * sizeof(float));
  g.ws_bytes = g.off_acc + align256(parts * g.G * g.vec * sizeof(float));
  return g;
}

// Flag value of one launch: distinct across launches of this process, and
// seeded at random so that stale flags of an earlier process (or any other
// contents of the workspace) match with probability 2^-64.
uint64_t next_token() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    uint64_t s = ((uint64_t)rd() << 32) ^ rd();
    s ^= (uint64_t)std::chrono::high_resolution_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull;
    return s;
  }()};
  uint64_t t = counter.fetch_add(0x9E3779B97F4A7C15ull, std::memory_order_relaxed);
  return t ? t : 1;
}

// ga carries the pointers and scalars; the geometry fields are filled here.
// A workspace (of at least the plan's size) selects the balanced partition.
hipError_t launch_gather(GatherArgs ga, const Problem& p, void* ws, hipStream_t s) {
  if (p.n == 0) return hipSuccess;
  const Plan g = make_plan(p);
  ga.HB = g.hb;
  ga.log2G = g.log2g;
  ga.npw = g.npw;
  ga.ws_flags = nullptr;
  dim3 grid((unsigned)ceil_div(p.n, g.npw), (unsigned)g.head_blocks);
  if (ws) {
    uint8_t* w = (uint8_t*)ws;
    ga.ws_flags = (uint64_t*)w;
    ga.ws_ml = (float*)(w + g.off_ml);
    ga.ws_acc = (float*)(w + g.off_acc);
    ga.items_per_wg = g.C;
    ga.total_items = (int64_t)p.n + p.nnz;
    ga.light_max = g.light_max;
    ga.num_wg = (int32_t)g.B;
    ga.token = next_token();
    grid.x = (unsigned)g.B;
  }
  return ws ? detail::launch_kernels<true>(p, ga, grid, s) : detail::launch_kernels<false>(p, ga, grid, s);
}

Problem forward_problem(const gattn_forward_args& a) {
  const bool he = a.e != nullptr;
  return Problem{a.num_nodes, a.num_heads, a.head_dim, a.nnz, a.dtype, a.mode, he,
                 a.e_out != nullptr && he && a.mode == GATTN_SOFTMAX_CLIPPED};
}

Problem aggregate_problem(const gattn_aggregate_args& a) {
  return Problem{a.num_nodes, a.num_heads, a.head_dim, a.nnz, a.dtype, kModeAggregate, false, false};
}

}  // namespace

size_t forward_gather_workspace_bytes(const gattn_forward_args& a) {
  return a.num_nodes == 0 ? 0 : make_plan(forward_problem(a)).ws_bytes;
}

size_t aggregate_workspace_bytes(const gattn_aggregate_args& a) {
  return a.num_nodes == 0 ? 0 : make_plan(aggregate_problem(a)).ws_bytes;
}

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
  return launch_gather(ga, forward_problem(a), a.workspace, s);
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
  return launch_gather(ga, aggregate_problem(a), a.workspace, s);
}

}  // namespace gattn
