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
int resident_of<kPartNode>(const Problem& p) { return resident_impl<kPartNode>(p); }
template <>
hipError_t launch_kernels<kPartNode>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  return launch_impl<kPartNode>(p, ga, grid, s);
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

// Heads per workgroup and slot width: a slot of G lanes (16 bytes each) holds
// one edge's slice of HB heads.
struct Geom {
  int hb, log2g, G, vec, head_blocks, ns, qrow;
};

Geom make_geom(const Problem& p, int hb_max) {
  Geom g{};
  const int esz = p.dtype == GATTN_F32 ? 4 : 2;
  g.vec = 16 / esz;
  const int lph = p.head_dim / g.vec;
  g.hb = std::max(1, std::min({p.H, 64 / lph, hb_max}));
  g.G = 1;
  while (g.G < g.hb * lph) g.G <<= 1;
  g.log2g = 0;
  while ((1 << g.log2g) < g.G) ++g.log2g;
  g.head_blocks = (int)ceil_div(p.H, g.hb);
  g.ns = 4 * (64 / g.G);
  g.qrow = g.hb * p.head_dim * esz;
  return g;
}

struct Plan {
  Geom geo;                 // node and balanced partitions
  int npw;                  // node partition: destinations per workgroup
  int64_t C, B;             // balanced partition: items per workgroup, workgroups per head block
  int light_max;
  size_t off_ml, off_acc, ws_bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Destinations per workgroup for an equal-count partition: about `target`
// edges each, at most `cap`, and the grid rounded to whole "rounds" of
// co-resident workgroups (a last, partly filled round would leave most CUs
// idle while it runs).  When the cap allows fewer rows than the rounded grid
// asks for, the grid takes one more round of smaller workgroups rather than a
// partly filled one.
int nodes_per_wg(const Problem& p, double target, int cap, int head_blocks, int64_t resident_all) {
  const int64_t per_round = std::max<int64_t>(1, resident_all / head_blocks);
  const double avg = (double)p.nnz / p.n;
  int npw_target = cap;
  if (avg > 0) npw_target = (int)std::min<double>(cap, std::max(1.0, std::ceil(target / avg)));
  const double wgs = (double)ceil_div(p.n, npw_target) * head_blocks;
  int64_t rounds = std::max<int64_t>(1, (int64_t)std::llround(wgs / (double)resident_all));
  rounds = std::max<int64_t>(rounds, ceil_div(ceil_div(p.n, cap), per_round));
  return (int)std::min<int64_t>(cap, std::max<int64_t>(1, ceil_div(p.n, rounds * per_round)));
}

// Both partitions aim at about EDGES_PER_SLOT * U edges per slot.  The node
// partition is bounded by the LDS that stages Q rows; the balanced one keeps
// its typical row count under that bound.
Plan make_plan(const Problem& p) {
  Plan g{};
  g.geo = make_geom(p, 64);
  if (p.n == 0) return g;
  const int u = detail::unroll_of(p);
  const int cus = device_cus();
  auto qcap_of = [&](const Geom& ge) {
    return p.mode == kModeAggregate ? kMaxNodesPerWg : std::max(1, std::min(kMaxNodesPerWg, kQLdsBytes / ge.qrow));
  };

  // node partition
  const int qcap = qcap_of(g.geo);
  const double target = (double)g.geo.ns * GATTN_GATHER_EDGES_PER_SLOT * u;  // edges per workgroup
  g.npw = nodes_per_wg(p, target, qcap, g.geo.head_blocks, (int64_t)detail::resident_of<kPartNode>(p) * cus);

  // balanced partition over T = N + nnz items: one round of resident
  // workgroups (every workgroup then finds its range while the memory system
  // is still idle; a second round would pay the search and staging round
  // trips again, each several times longer under full load), more only when
  // a workgroup's typical row count would exceed the rows whose Q it stages
  {
    const int64_t resident_split = (int64_t)detail::resident_of<kPartSplit>(p) * cus;
    const int64_t per_round = std::max<int64_t>(1, resident_split / g.geo.head_blocks);
    const int64_t T = (int64_t)p.n + p.nnz;
    const int64_t cmax = kMaxNodesPerWg - 2;
    const int qcap_s = p.mode == kModeAggregate
                           ? kMaxNodesPerWg
                           : std::max(1, std::min(kMaxNodesPerWg, kQLdsBytesSplit / g.geo.qrow));
    const double c_rows = (double)qcap_s * (double)T / (double)p.n;   // items of a typical qcap_s rows
    int64_t C = std::max<int64_t>(8, ceil_div(T, per_round));
    if ((double)C > c_rows) C = std::max<int64_t>(8, (int64_t)c_rows);
    C = std::min<int64_t>(C, cmax);
    const int64_t rounds = ceil_div(ceil_div(T, C), per_round);
    C = std::min<int64_t>(cmax, std::max<int64_t>(8, ceil_div(T, rounds * per_round)));
    g.C = C;
    g.B = ceil_div(T, C);
    g.light_max = (int)std::max<int64_t>(2, C / 2);
    const size_t parts = (size_t)2 * g.geo.head_blocks * g.B;
    g.off_ml = align256(parts * sizeof(uint64_t));
    g.off_acc = g.off_ml + align256(parts * g.geo.G * 2 * sizeof(float));
    g.ws_bytes = g.off_acc + align256(parts * g.geo.G * g.geo.vec * sizeof(float));
  }

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
// ranges (node partition): nullable (first row, row count) table of
// num_ranges workgroups of at most range_rows rows.
hipError_t launch_gather(GatherArgs ga, const Problem& p, int part, void* ws, hipStream_t s,
                         const int32_t* ranges = nullptr, int32_t num_ranges = 0, int32_t range_rows = 0) {
  if (p.n == 0) return hipSuccess;
  const Plan g = make_plan(p);
  const Geom& ge = g.geo;
  ga.HB = ge.hb;
  ga.log2G = ge.log2g;
  ga.ws_flags = nullptr;
  if (part == kPartSplit) {
    uint8_t* w = (uint8_t*)ws;
    ga.ws_flags = (uint64_t*)w;
    ga.ws_ml = (float*)(w + g.off_ml);
    ga.ws_acc = (float*)(w + g.off_acc);
    ga.items_per_wg = g.C;
    ga.total_items = (int64_t)p.n + p.nnz;
    ga.light_max = g.light_max;
    ga.num_wg = (int32_t)g.B;
    ga.token = next_token();
    return detail::launch_kernels<kPartSplit>(p, ga, dim3((unsigned)g.B, (unsigned)ge.head_blocks), s);
  }
  if (ranges) {
    if (num_ranges == 0) return hipSuccess;
    ga.ranges = ranges;
    ga.npw = range_rows;
    return detail::launch_kernels<kPartNode>(p, ga, dim3((unsigned)num_ranges, (unsigned)ge.head_blocks), s);
  }
  ga.npw = g.npw;
  return detail::launch_kernels<kPartNode>(p, ga, dim3((unsigned)ceil_div(p.n, ga.npw), (unsigned)ge.head_blocks), s);
}

bool low_degree(int32_t n, int64_t nnz) { return n > 0 && (double)nnz < GATTN_GATHER_LOW_DEGREE * (double)n; }

Problem forward_problem(const gattn_forward_args& a) {
  const bool he = a.e != nullptr;
  return Problem{a.num_nodes, a.num_heads, a.head_dim, a.nnz, a.dtype, a.mode, he,
                 a.e_out != nullptr && he && a.mode == GATTN_SOFTMAX_CLIPPED, low_degree(a.num_nodes, a.nnz)};
}

Problem aggregate_problem(const gattn_aggregate_args& a) {
  return Problem{a.num_nodes, a.num_heads, a.head_dim, a.nnz, a.dtype, kModeAggregate, false, false,
                 low_degree(a.num_nodes, a.nnz)};
}

// A workspace selects the balanced partition.
int pick_part(const void* ws) { return ws ? kPartSplit : kPartNode; }

}  // namespace

size_t forward_gather_workspace_bytes(const gattn_forward_args& a) {
  return a.num_nodes == 0 ? 0 : make_plan(forward_problem(a)).ws_bytes;
}

size_t aggregate_workspace_bytes(const gattn_aggregate_args& a) {
  return a.num_nodes == 0 ? 0 : make_plan(aggregate_problem(a)).ws_bytes;
}

namespace {
GatherArgs forward_gather_args(const gattn_forward_args& a) {
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
  const int64_t hd = (int64_t)a.num_heads * a.head_dim;
  ga.q_stride = a.q_stride ? a.q_stride : hd;
  ga.kv_stride = a.kv_stride ? a.kv_stride : hd;
  ga.scale = a.mode == GATTN_SOFTMAX_STANDARD ? a.scale * kLog2e : a.scale;
  ga.lo = a.clip_lo;
  ga.hi = a.clip_hi;
  ga.eps = a.eps;
  ga.ids = a.e ? a.edge_ids : nullptr;
  ga.e_out = (uint8_t*)a.e_out;
  return ga;
}
}  // namespace

hipError_t launch_forward_gather(const gattn_forward_args& a, hipStream_t s) {
  return launch_gather(forward_gather_args(a), forward_problem(a), pick_part(a.workspace), a.workspace, s);
}

int32_t gather_max_range_rows(const gattn_forward_args& a) {
  const Problem p = forward_problem(a);
  const Geom ge = make_geom(p, 64);
  return std::max(1, std::min(kMaxNodesPerWg, kQLdsBytes / ge.qrow));
}

int32_t hybrid_rows_per_range(const gattn_forward_args& a, int32_t rows, int64_t nnz) {
  Problem p = forward_problem(a);
  p.n = std::max(rows, 1);
  p.nnz = std::max<int64_t>(nnz, 0);
  return make_plan(p).npw;  // at most the rows whose Q rows fit in LDS
}

hipError_t launch_forward_gather_ranges(const gattn_forward_args& a, const int32_t* ranges, int32_t num_ranges,
                                        int32_t range_rows, hipStream_t s) {
  return launch_gather(forward_gather_args(a), forward_problem(a), kPartNode, nullptr, s, ranges, num_ranges,
                       range_rows);
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
  ga.q_stride = ga.kv_stride = (int64_t)a.num_heads * a.head_dim;
  ga.eps = a.eps;
  ga.ids = a.edge_ids;
  ga.w = a.w;
  ga.normalize = a.normalize;
  return launch_gather(ga, aggregate_problem(a), pick_part(a.workspace), a.workspace, s);
}

}  // namespace gattn
