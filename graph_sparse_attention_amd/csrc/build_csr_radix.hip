// build_csr_radix.hip -- COO -> destination-grouped CSR for large edge lists
// without per-edge global atomics.
//
// The result is the same canonical CSR as the counting build (edges of a
// destination in (source, edge id) order; the gattn-triton article, "Using
// the CSC index for fast edge lookup", groups edges by destination and keeps
// the edge-id map).  Here it comes from a stable least-significant-digit radix
// sort of the destinations, the edge's (source << 32 | edge id) riding along:
//
//   clear      flags, digit histograms, tile status words
//   histogram  digit counts of every pass in one read of src/dst (LDS
//              histograms, one global add per digit and workgroup); flags a
//              bad index and whether src is non-decreasing
//   pass x P   one launch per digit of at most 8 bits (9 where that saves a
//              pass; 512 buckets then).  A tile of 4096 keys (7168 from 2^23
//              edges) ranks its keys stably inside each wave (peer groups
//              matched through one LDS word per digit, one LDS counter per
//              digit and wave advanced by one atomic per group), learns the
//              global start of each digit from the histogram plus the tiles
//              before it (two-level decoupled look-back: the earlier tiles
//              of its group of 16, then the earlier groups, on 64-bit status
//              words per tile / group and digit, tiles taken in ticket
//              order), and writes its
//              keys, then its values, digit-run by digit-run through one LDS
//              buffer
//   row_ptr    from the boundaries of the sorted destinations
//   sort rows  only when src was not non-decreasing: the stable sort leaves
//              each destination's edges in edge-id order, which is (source,
//              edge id) order exactly when the sources never decrease.
//
// An invalid edge (either index outside [0, n)) takes key n, sorts behind
// every real edge and raises the bad-graph flag; outputs are then unspecified
// but every write stays inside its buffer.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRadixMax = 512;            // buckets per pass: digits of at most 9 bits
constexpr int kRankGroup = 4;   // items whose LDS atomics of the ranking are in flight together
// keys per thread: 16 (4096-key tiles) up to 2^23 edges, 28 (7168-key tiles)
// above, where longer digit runs write better and the extra tiles' latency
// matters less (28 x 12 bytes of keys and values per thread stay in registers)
constexpr int kItemsSmall = 16, kItemsLarge = 28;
constexpr int64_t kLargeEdges = 1 << 23;
constexpr int kLookback = 4;
constexpr int kGroup = 16;      // tiles per look-back group  // earlier tiles' status words read per look-back round (8 and 16 were no faster)
constexpr int kMaxPasses = 4;             // keys of at most 32 bits
constexpr int kHistBlocks = 2048;
constexpr int kHistItems = 16;             // edges per thread and round of the histogram
constexpr uint32_t kFlagAggregate = 1, kFlagPrefix = 2;
constexpr int kSpinLimit = 1 << 20;

// flag words at the head of the workspace: [0] bad index, [1] sources not
// non-decreasing, [2] a look-back wait ran out, [8 + p] tile ticket of pass p
enum { kBad = 0, kUnsorted = 1, kErr = 2, kTicket = 8 };

struct Digits {
  int passes;
  int shift[kMaxPasses];
  int bits[kMaxPasses];
};

// keys are 0..n (n marks an invalid edge): B = bit length of n, split as
// evenly as possible into ceil(B / 8) digits, lowest first -- or ceil(B / 9)
// digits of up to 9 bits (512 buckets) when that is one pass fewer (B = 17,
// 18, 25..27)
Digits digits_of(int32_t n) {
  const int B = 32 - __builtin_clz((uint32_t)n);
  Digits d{};
  d.passes = std::min((B + 7) / 8, (B + 8) / 9);
  int s = 0;
  for (int p = 0; p < d.passes; ++p) {
    d.bits[p] = B / d.passes + (p < B % d.passes ? 1 : 0);
    d.shift[p] = s;
    s += d.bits[p];
  }
  return d;
}

// buckets of the passes: 512 when some digit has 9 bits
int radix_of(const Digits& d) {
  for (int p = 0; p < d.passes; ++p)
    if (d.bits[p] > 8) return 512;
  return 256;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RadixWs {
  int32_t* flags;     // [64]
  uint32_t* hist;     // [kMaxPasses][kRadixMax]
  uint64_t* status;   // [passes][tiles][radix]
  uint64_t* gstatus;  // [passes][groups][radix]
  uint32_t* keys[2];  // [nnz] each
  uint64_t* vals[2];  // [nnz] each
  int64_t clear_ints; // flags + hist + status + gstatus, cleared in one launch
  int64_t tiles, groups;
};

int items_of(int64_t nnz) { return nnz >= kLargeEdges ? kItemsLarge : kItemsSmall; }
int64_t tiles_of(int64_t nnz) { return ceil_div(std::max<int64_t>(nnz, 1), (int64_t)kThreads * items_of(nnz)); }

RadixWs carve(void* ws, int32_t n, int64_t nnz) {
  const Digits dg = digits_of(n);
  uint8_t* p = (uint8_t*)ws;
  RadixWs w;
  w.tiles = tiles_of(nnz);
  w.flags = (int32_t*)p;
  p += 256;
  w.hist = (uint32_t*)p;
  p += align256(sizeof(uint32_t) * kMaxPasses * kRadixMax);
  w.status = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * dg.passes * w.tiles * radix_of(dg));
  w.groups = ceil_div(w.tiles, kGroup);
  w.gstatus = (uint64_t*)p;
  p += align256(sizeof(uint64_t) * dg.passes * w.groups * radix_of(dg));
  w.clear_ints = (p - (uint8_t*)ws) / 4;
  for (int b = 0; b < 2; ++b) {
    w.keys[b] = (uint32_t*)p;
    p += align256(sizeof(uint32_t) * nnz);
  }
  for (int b = 0; b < 2; ++b) {
    w.vals[b] = (uint64_t*)p;
    p += align256(sizeof(uint64_t) * nnz);
  }
  return w;
}

__global__ void radix_clear_kernel(int32_t* __restrict__ p, int64_t n, int32_t* __restrict__ status_dev) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
  if (status_dev && blockIdx.x == 0 && threadIdx.x == 0) *status_dev = GATTN_OK;
}

__device__ __forceinline__ uint32_t edge_key(int32_t s, int32_t d, int32_t n) {
  return ((uint32_t)s < (uint32_t)n && (uint32_t)d < (uint32_t)n) ? (uint32_t)d : (uint32_t)n;
}

__device__ __forceinline__ uint32_t digit(uint32_t key, int shift, int bits) {
  return (key >> shift) & ((1u << bits) - 1u);
}

// digit counts of every pass; the bad-index and source-order flags.  A round
// covers 16 x 256 consecutive edges (1024 per wave), the next round's loads
// are issued before this round is counted.
__device__ __forceinline__ void hist_load(const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                          int64_t wbase, int64_t last, int lane, int32_t* sv, int32_t* dv,
                                          int32_t& pv) {
#pragma unroll
  for (int k = 0; k < kHistItems; ++k) {
    const int64_t e = min(wbase + k * 64 + lane, last);
    sv[k] = src[e];
    dv[k] = dst[e];
  }
  pv = src[min(max(wbase - 1, (int64_t)0), last)];  // the edge before the wave's chunk
}

__global__ __launch_bounds__(kThreads) void radix_hist_kernel(const int32_t* __restrict__ src,
                                                              const int32_t* __restrict__ dst, int64_t nnz,
                                                              int32_t n, Digits dg, uint32_t* __restrict__ hist,
                                                              int32_t* __restrict__ flags,
                                                              int32_t* __restrict__ status_dev) {
  __shared__ uint32_t h[kMaxPasses * kRadixMax];
  for (int i = threadIdx.x; i < kMaxPasses * kRadixMax; i += kThreads) h[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t last = nnz - 1, stride = (int64_t)gridDim.x * (kThreads * kHistItems);
  bool bad = false, unsorted = false;
  int64_t e0 = (int64_t)blockIdx.x * (kThreads * kHistItems);
  int32_t sv[kHistItems], dv[kHistItems], pv;
  hist_load(src, dst, e0 + wave * (64 * kHistItems), last, lane, sv, dv, pv);
  for (; e0 < nnz; e0 += stride) {
    const int64_t wbase = e0 + wave * (64 * kHistItems);
    int32_t sn[kHistItems], dn[kHistItems], pn;
    hist_load(src, dst, wbase + stride, last, lane, sn, dn, pn);  // clamped: always in bounds
#pragma unroll
    for (int k = 0; k < kHistItems; ++k) {
      const int64_t e = wbase + k * 64 + lane;
      const int32_t up = __shfl_up(sv[k], 1, 64);
      const int32_t wrap = k > 0 ? __shfl(sv[k > 0 ? k - 1 : 0], 63, 64) : pv;
      const int32_t prev = lane == 0 ? wrap : up;
      if (e > last) continue;
      const uint32_t key = edge_key(sv[k], dv[k], n);
      bad |= key == (uint32_t)n;
      unsorted |= e > 0 && prev > sv[k];
      for (int p = 0; p < dg.passes; ++p) atomicAdd(&h[p * kRadixMax + digit(key, dg.shift[p], dg.bits[p])], 1u);
    }
#pragma unroll
    for (int k = 0; k < kHistItems; ++k) {
      sv[k] = sn[k];
      dv[k] = dn[k];
    }
    pv = pn;
  }
  if (bad) {
    flags[kBad] = 1;
    if (status_dev) *status_dev = GATTN_ERR_BAD_GRAPH;
  }
  if (unsorted) flags[kUnsorted] = 1;
  __syncthreads();
  for (int i = threadIdx.x; i < dg.passes * kRadixMax; i += kThreads) {
    const uint32_t v = h[i];
    if (v) atomicAdd(&hist[i], v);
  }
}

struct PassArgs {
  const int32_t* src;   // first pass: the COO arrays
  const int32_t* dst;
  const uint32_t* kin;  // later passes: keys / values of the previous pass
  const uint64_t* vin;
  uint32_t* kout;
  uint64_t* vout;
  int32_t* col_idx;     // last pass, sources non-decreasing: written directly
  int32_t* edge_perm;
  const uint32_t* hist;  // [radix] global digit counts of this pass
  uint64_t* status;      // [tiles][radix] tile aggregates
  uint64_t* gstatus;     // [groups][radix] group aggregates / inclusive prefixes
  int64_t tiles;
  int32_t* ticket;
  int32_t* flags;
  int32_t* status_dev;
  int64_t nnz;
  int32_t n;
  int shift, bits;
};

__device__ __forceinline__ void publish(uint64_t* st, uint32_t flag, uint32_t v) {
  __hip_atomic_store(st, ((uint64_t)flag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// exclusive scans of a and b over the workgroup in thread order
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t* ea, uint32_t* eb,
                                                 uint32_t (*s)[2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = a, y = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t xu = __shfl_up(x, o, 64), yu = __shfl_up(y, o, 64);
    if (lane >= o) {
      x += xu;
      y += yu;
    }
  }
  if (lane == 63) {
    s[wave][0] = x;
    s[wave][1] = y;
  }
  __syncthreads();
  uint32_t ox = 0, oy = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wave) {
      ox += s[w][0];
      oy += s[w][1];
    }
  *ea = ox + x - a;
  *eb = oy + y - b;
}

// One tile of one pass.  Key j of the tile (j = wave * 1024 + item * 64 +
// lane) keeps its order among equal digits: a wave ranks its items in item
// order, lanes in lane order, and waves follow each other.  Thread t owns
// the kRadix / 256 consecutive digits from t * kRadix / 256 on.
// The launch bound (2 waves per SIMD) holds the 7168-key tiles to 256
// registers (a few bytes of spill) instead of the ~270 that would leave one
// wave per SIMD.
template <int kItems, int kRadix, bool FIRST, bool LAST>
__global__ __launch_bounds__(kThreads, 2) void radix_pass_kernel(PassArgs a) {
  constexpr int kTile = kThreads * kItems;
  // two-level look-back for the 4096-key tiles (inputs of up to ~2^23 edges,
  // whose tiles mostly run at once); the 7168-key kernel keeps the one-level
  // walk, which needs fewer registers (it spills less at 256)
  constexpr bool kTwoLevel = kItems == kItemsSmall;
  constexpr int DPT = kRadix / kThreads;  // digits per thread
  __shared__ uint64_t s_vals[kTile];  // keys staged first (as 32-bit words), then values
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(s_vals);
  __shared__ uint32_t s_wcnt[kWaves][kRadix];  // per-wave digit counts, then per-wave offsets
  __shared__ uint32_t s_start[kRadix];         // tile-local start of each digit
  __shared__ uint32_t s_goff[kRadix];          // global position of tile-local index 0 of each digit
  __shared__ uint32_t s_scan[kWaves][2];
  __shared__ int32_t s_tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_tile = atomicAdd(a.ticket, 1);
  for (int i = tid; i < kWaves * kRadix; i += kThreads) (&s_wcnt[0][0])[i] = 0;
  // peer-group words, one per digit and wave, in the staging buffer (not
  // used before the tile is staged)
  static_assert(kWaves * kRadix <= kTile, "peer words must fit the staging buffer");
  for (int i = tid; i < kWaves * kRadix; i += kThreads) s_vals[i] = 0;
  uint64_t* const s_match = s_vals + wave * kRadix;
  uint32_t gcount[DPT];  // this thread's digits: global counts
#pragma unroll
  for (int j = 0; j < DPT; ++j) gcount[j] = a.hist[tid * DPT + j];
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t base = tile * kTile + wave * (kItems * 64) + lane;
  const int64_t last = a.nnz - 1;

  uint32_t key[kItems];
  uint64_t val[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int64_t i = base + k * 64;
    const int64_t ic = i < last ? i : last;  // clamped: every load in bounds, no branch
    if (FIRST) {
      const int32_t s = a.src[ic], d = a.dst[ic];
      key[k] = edge_key(s, d, a.n);
      val[k] = ((uint64_t)(uint32_t)s << 32) | (uint32_t)ic;
    } else {
      key[k] = a.kin[ic];
      val[k] = a.vin[ic];
    }
  }

  // stable rank inside the wave, item by item: the lanes holding one digit
  // in item k (its peer group) take the next positions of that digit in lane
  // order.  The group is found in LDS: each lane ORs its lane bit into the
  // wave's word for its digit, reads the word back and clears it (a wave's
  // LDS operations run in issue order, so the read sees every lane's bit and
  // the next item starts from zero).  The group's lowest lane then advances
  // the wave's counter of the digit by the group's size with an atomic add,
  // which sees the counts of all earlier items; the other lanes read the old
  // count from it.
  // kRankGroup items are in flight together.
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  const uint64_t lane_bit = 1ull << lane;
  uint32_t rank[kItems];
#pragma unroll
  for (int k0 = 0; k0 < kItems; k0 += kRankGroup) {
    constexpr int kg = kRankGroup;
    uint64_t peers[kg];
    uint32_t dgs[kg];
#pragma unroll
    for (int k = k0; k < k0 + kg && k < kItems; ++k) {
      const uint32_t dg = digit(key[k], a.shift, a.bits);
      dgs[k - k0] = dg;
      peers[k - k0] = 0;
      if (base + k * 64 <= last) {
        atomicOr(reinterpret_cast<unsigned long long*>(&s_match[dg]), (unsigned long long)lane_bit);
        peers[k - k0] = s_match[dg];
        s_match[dg] = 0;
      }
    }
    uint32_t old[kg];
#pragma unroll
    for (int k = k0; k < k0 + kg && k < kItems; ++k) {
      const uint64_t pm = peers[k - k0];
      const bool valid = pm != 0;  // a valid lane is its own peer
      const uint32_t leader = valid ? (uint32_t)__builtin_ctzll(pm) : (uint32_t)lane;
      // every lane takes part (the others add 0, which changes nothing), so
      // no branch holds the atomics back; only the leader's old value is used
      const uint32_t add = valid && leader == (uint32_t)lane ? (uint32_t)__popcll(pm) : 0u;
      old[k - k0] = atomicAdd(&s_wcnt[wave][dgs[k - k0]], add);
      rank[k] = (uint32_t)__popcll(pm & lanes_below) | (leader << 16);
    }
#pragma unroll
    for (int k = k0; k < k0 + kg && k < kItems; ++k)
      rank[k] = (rank[k] & 0xffffu) + (uint32_t)__shfl((int)old[k - k0], (int)(rank[k] >> 16), 64);
  }
  __syncthreads();

  // this thread's digits: tile counts, per-wave offsets, local starts
  uint32_t cnt[DPT], csum = 0, gsum = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int d = tid * DPT + j;
    cnt[j] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = s_wcnt[w][d];
      s_wcnt[w][d] = cnt[j];
      cnt[j] += c;
    }
    publish(a.status + tile * kRadix + d, !kTwoLevel && tile == 0 ? kFlagPrefix : kFlagAggregate, cnt[j]);
    csum += cnt[j];
    gsum += gcount[j];
  }
  uint32_t start0, gbase0;
  block_excl_scan2(csum, gsum, &start0, &gbase0, s_scan);
  uint32_t start[DPT], gbase[DPT];
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    start[j] = start0;
    gbase[j] = gbase0;
    start0 += cnt[j];
    gbase0 += gcount[j];
    s_start[tid * DPT + j] = start[j];
  }

  // Look-back for each of this thread's digits.  4096-key tiles, two levels:
  // tiles form groups of kGroup consecutive tickets; a tile sums the
  // aggregates of the earlier tiles of its group; the group's last tile
  // publishes the group's aggregate, and later its inclusive prefix; every
  // tile then walks back over the earlier groups' words, adding aggregates
  // until an inclusive prefix (group 0's always is one).  7168-key tiles, one
  // level: a walk back over the earlier tiles (tile 0's word is an inclusive
  // prefix), then the tile's own inclusive prefix.  Each walk reads kLookback
  // words per digit and round, the digits' walks side by side.  Every wait is
  // for a lower ticket, and an empty poll counts towards a bounded limit.
  int spins = 0;
  // adds st[pos .. lo] (stopping early at an inclusive prefix) to sum
  auto walk = [&](const uint64_t* st, int64_t pos0, int64_t lo, uint32_t* sum) {
    if (pos0 < lo) return;  // nothing before this tile (workgroup-uniform)
    int64_t pos[DPT];
    bool done[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      pos[j] = pos0;
      done[j] = pos0 < lo;
    }
    while (true) {
      uint64_t w[DPT][kLookback];
#pragma unroll
      for (int j = 0; j < DPT; ++j)
#pragma unroll
        for (int q = 0; q < kLookback; ++q) {
          const int64_t jj = pos[j] - q;
          const uint64_t x = __hip_atomic_load(st + (jj > lo ? jj : lo) * kRadix + tid * DPT + j,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          w[j][q] = (jj >= lo && !done[j]) ? x : ((uint64_t)kFlagPrefix << 32);  // past the range: an end of value 0
        }
      bool all = true, moved = false;
#pragma unroll
      for (int j = 0; j < DPT; ++j) {
        if (done[j]) continue;
        int used = 0;
#pragma unroll
        for (int q = 0; q < kLookback; ++q) {
          if (done[j] || used < q) break;
          const uint32_t flag = (uint32_t)(w[j][q] >> 32);
          if (flag == 0) break;
          sum[j] += (uint32_t)w[j][q];
          used = q + 1;
          done[j] = flag == kFlagPrefix;
        }
        pos[j] -= used;
        moved = moved || used > 0;
        all = all && done[j];
      }
      if (all) break;
      if (!moved && ++spins > kSpinLimit) {
        a.flags[kErr] = 1;
        if (a.status_dev) *a.status_dev = GATTN_ERR_HIP;
        break;
      }
    }
  };
  uint32_t prefix[DPT];
  if constexpr (kTwoLevel) {
    const int64_t grp = tile / kGroup, g0 = grp * kGroup;
    const bool group_last = tile == min(g0 + kGroup, a.tiles) - 1;
    uint32_t within[DPT], before[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) within[j] = before[j] = 0;
    walk(a.status, tile - 1, g0, within);
    if (group_last) {
#pragma unroll
      for (int j = 0; j < DPT; ++j)
        publish(a.gstatus + grp * kRadix + tid * DPT + j, grp == 0 ? kFlagPrefix : kFlagAggregate, within[j] + cnt[j]);
    }
    walk(a.gstatus, grp - 1, 0, before);
    if (group_last && grp > 0) {
#pragma unroll
      for (int j = 0; j < DPT; ++j)
        publish(a.gstatus + grp * kRadix + tid * DPT + j, kFlagPrefix, before[j] + within[j] + cnt[j]);
    }
#pragma unroll
    for (int j = 0; j < DPT; ++j) prefix[j] = before[j] + within[j];
  } else {
    // one level: back over the earlier tiles (tile 0 holds an inclusive
    // prefix), then this tile's own inclusive prefix
#pragma unroll
    for (int j = 0; j < DPT; ++j) prefix[j] = 0;
    walk(a.status, tile - 1, 0, prefix);
    if (tile > 0) {
#pragma unroll
      for (int j = 0; j < DPT; ++j) publish(a.status + tile * kRadix + tid * DPT + j, kFlagPrefix, prefix[j] + cnt[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < DPT; ++j) s_goff[tid * DPT + j] = gbase[j] + prefix[j] - start[j];  // modulo 2^32
  __syncthreads();

  // stage the tile in digit order, then write digit runs
  const int count = (int)min<int64_t>(kTile, a.nnz - tile * kTile);
  const bool direct = LAST && a.flags[kUnsorted] == 0;
  // keys, then values, through one LDS buffer (half the LDS of staging both)
  uint32_t lp[kItems], gpos[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const uint32_t dg = digit(key[k], a.shift, a.bits);
    lp[k] = s_start[dg] + s_wcnt[wave][dg] + rank[k];
    if (base + k * 64 <= last) s_keys[lp[k]] = key[k];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = tid + j * kThreads;
    gpos[j] = 0xffffffffu;
    if (i < count) {
      const uint32_t kk = s_keys[i];
      gpos[j] = s_goff[digit(kk, a.shift, a.bits)] + (uint32_t)i;
      if (gpos[j] < (uint32_t)a.nnz) a.kout[gpos[j]] = kk;  // else only after a failed look-back
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kItems; ++k)
    if (base + k * 64 <= last) s_vals[lp[k]] = val[k];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = tid + j * kThreads;
    const uint32_t g = gpos[j];
    if (i >= count || g >= (uint32_t)a.nnz) continue;
    const uint64_t vv = s_vals[i];
    if (direct) {
      a.col_idx[g] = (int32_t)(vv >> 32);
      if (a.edge_perm) a.edge_perm[g] = (int32_t)(uint32_t)vv;
    } else {
      a.vout[g] = vv;
    }
  }
}

// row_ptr[r] = first position whose key is >= r: position g writes the rows
// in (key[g-1], key[g]] (key[-1] = -1, key[nnz] = n).  A thread takes eight
// positions; short gaps are filled by their own lane, long ones (runs of
// empty rows) by the whole wave in turn.
__global__ __launch_bounds__(256) void radix_rowptr_kernel(const uint32_t* __restrict__ keys, int64_t nnz, int32_t n,
                                                           int32_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t b0 = (int64_t)blockIdx.x * blockDim.x * 8; b0 <= nnz; b0 += stride) {
    const int64_t g0 = b0 + threadIdx.x * 8;
    int64_t cur[8];
    if (g0 + 8 <= nnz) {
      const u32x4 x = ld16(keys + g0), y = ld16(keys + g0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cur[j] = x[j];
        cur[4 + j] = y[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) cur[j] = g0 + j < nnz ? (int64_t)keys[g0 + j] : (int64_t)n;
    }
    int64_t prev = (g0 == 0 || g0 > nnz) ? -1 : (int64_t)keys[g0 - 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t g = g0 + j;
      int64_t lo = 0, hi = -1;  // rows lo..hi start at g
      if (g <= nnz) {
        lo = prev + 1;
        hi = min<int64_t>(cur[j], n);
      }
      prev = cur[j];
      const bool longgap = hi - lo >= 32;
      if (!longgap)
        for (int64_t r = lo; r <= hi; ++r) row_ptr[r] = (int32_t)g;
      uint64_t todo = __ballot(longgap);
      while (todo) {
        const int l = __ffsll((unsigned long long)todo) - 1;
        todo &= todo - 1;
        const int64_t ra = __shfl(lo, l, 64), rb = __shfl(hi, l, 64), gg = __shfl(g, l, 64);
        for (int64_t r = ra + lane; r <= rb; r += 64) row_ptr[r] = (int32_t)gg;
      }
    }
  }
}

template <int kItems, int kRadix>
void launch_pass(bool first, bool lastp, dim3 grid, dim3 block, const PassArgs& a, hipStream_t s) {
  if (first && lastp) hipLaunchKernelGGL((radix_pass_kernel<kItems, kRadix, true, true>), grid, block, 0, s, a);
  else if (first) hipLaunchKernelGGL((radix_pass_kernel<kItems, kRadix, true, false>), grid, block, 0, s, a);
  else if (lastp) hipLaunchKernelGGL((radix_pass_kernel<kItems, kRadix, false, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((radix_pass_kernel<kItems, kRadix, false, false>), grid, block, 0, s, a);
}

}  // namespace

size_t build_csr_radix_workspace_bytes(int32_t n, int64_t nnz) {
  const Digits dg = digits_of(std::max(n, 1));
  const int64_t tiles = tiles_of(nnz);
  return 256 + align256(sizeof(uint32_t) * kMaxPasses * kRadixMax) +
         align256(sizeof(uint64_t) * dg.passes * tiles * radix_of(dg)) +
         align256(sizeof(uint64_t) * dg.passes * ceil_div(tiles, kGroup) * radix_of(dg)) +
         2 * align256(sizeof(uint32_t) * nnz) + 2 * align256(sizeof(uint64_t) * nnz);
}

hipError_t launch_build_csr_radix(int32_t n, int64_t nnz, const int32_t* src, const int32_t* dst, int32_t* row_ptr,
                                  int32_t* col_idx, int32_t* edge_perm, void* ws, int32_t* status_dev,
                                  hipStream_t s) {
  if (n < 1 || nnz < 1) return hipErrorInvalidValue;
  const Digits dg = digits_of(n);
  const int radix = radix_of(dg);
  RadixWs w = carve(ws, n, nnz);
  const unsigned cblocks = (unsigned)std::min<int64_t>(ceil_div(w.clear_ints, 256), 4096);
  hipLaunchKernelGGL(radix_clear_kernel, dim3(cblocks), dim3(256), 0, s, w.flags, w.clear_ints, status_dev);
  const unsigned hblocks = (unsigned)std::min<int64_t>(ceil_div(nnz, kThreads * kHistItems), kHistBlocks);
  hipLaunchKernelGGL(radix_hist_kernel, dim3(hblocks), dim3(kThreads), 0, s, src, dst, nnz, n, dg, w.hist, w.flags,
                     status_dev);
  int cur = 0;
  for (int p = 0; p < dg.passes; ++p) {
    PassArgs a{};
    a.src = src;
    a.dst = dst;
    a.kin = w.keys[cur];
    a.vin = w.vals[cur];
    a.kout = w.keys[cur ^ 1];
    a.vout = w.vals[cur ^ 1];
    a.col_idx = col_idx;
    a.edge_perm = edge_perm;
    a.hist = w.hist + p * kRadixMax;
    a.status = w.status + (int64_t)p * w.tiles * radix;
    a.gstatus = w.gstatus + (int64_t)p * w.groups * radix;
    a.tiles = w.tiles;
    a.ticket = &w.flags[kTicket + p];
    a.flags = w.flags;
    a.status_dev = status_dev;
    a.nnz = nnz;
    a.n = n;
    a.shift = dg.shift[p];
    a.bits = dg.bits[p];
    const bool first = p == 0, lastp = p == dg.passes - 1;
    const dim3 grid((unsigned)w.tiles), block(kThreads);
    if (items_of(nnz) == kItemsLarge) {
      if (radix == 512) launch_pass<kItemsLarge, 512>(first, lastp, grid, block, a, s);
      else launch_pass<kItemsLarge, 256>(first, lastp, grid, block, a, s);
    } else {
      if (radix == 512) launch_pass<kItemsSmall, 512>(first, lastp, grid, block, a, s);
      else launch_pass<kItemsSmall, 256>(first, lastp, grid, block, a, s);
    }
    cur ^= 1;
  }
  const unsigned rblocks = (unsigned)std::min<int64_t>(ceil_div(nnz + 1, 256 * 8), 4096);
  hipLaunchKernelGGL(radix_rowptr_kernel, dim3(rblocks), dim3(256), 0, s, w.keys[cur], nnz, n, row_ptr);
  // rows need sorting by source only when the sources were not non-decreasing
  return launch_sort_rows(n, nnz, row_ptr, w.vals[cur], w.vals[cur ^ 1], col_idx, edge_perm, &w.flags[kUnsorted], s);
}

}  // namespace gattn
