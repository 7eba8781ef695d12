// forward_mfma.hip -- row-window kernel of the fused graph attention on the
// matrix cores of gfx950 (fp16 / bf16 inputs, fp32 accumulation and softmax).
//
// Prior art: Fused3S (abstract; Figures 1-4) fuses SDDMM, online softmax and
// SpMM per row window on tensor cores, with a register remap between the
// SDDMM output and the SpMM input.  Here, per (16-row window, head), one
// wave64 walks the window's 16-column tiles:
//
//   S^T (16 src x 16 rows) = K_t (16 x D) . Q_w^T (D x 16)
//        v_mfma_f32_16x16x32_{f16,bf16}, D/32 steps.  Lane l holds
//        S[row l%16][src 4(l/16)+i], i = 0..3.
//   masked entries -> -inf; online softmax in fp32 against a per-row
//        reference max that moves only when a logit passes it by 2^8 (the
//        row max over a row's four 16-lane groups, by cross-row lane
//        swaps, runs only then); per-lane partial sums, reduced at the end
//   O^T (D x 16 rows) += V_t^T (D x 16 src) . P^T (16 src x 16 rows)
//        v_mfma_f32_16x16x16_{f16,bf16}, D/16 blocks.  The B operand P^T
//        needs lane l to hold P[row l%16][src 4(l/16)+i] -- exactly the S^T
//        accumulator layout, so P goes from the SDDMM accumulators to the
//        SpMM operand without leaving the registers (our counterpart of
//        Fused3S's register remapping).  K_t and V_t^T come from a per-wave
//        LDS copy of the tile's rows (V through gfx950's transposing read).
//   O^T accumulators keep row l%16 in lane l like the softmax state, so the
//   per-row rescale is a register multiply.
//
// S and P never leave the chip.  What bounds the work is the memory traffic
// and its latency, not the matrix cores: each K / V row is loaded once per
// window instead of once per edge, a window's column ids and masks once per
// window, and every load and store moves whole rows.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerWg = 4;
constexpr int kMetaCols = 256;  // column ids (and masks) a wave stages in LDS at a time

struct MfmaArgs {
  const int32_t* __restrict__ win_col_ptr;
  const int32_t* __restrict__ win_cols;
  const uint16_t* __restrict__ tile_mask;
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ out;
  const int32_t* __restrict__ windows;  // nullable: the grid's windows (a hybrid plan's dense ones)
  int64_t num_cols;
  int32_t n, H, W;
  int32_t nwb;        // windows in the grid (W, or the hybrid plan's dense ones)
  float scale_l2;     // scale * log2(e)
  uint32_t kv_bytes;  // bytes K (and V) span, at most 2^31
  uint32_t q_bytes;   // bytes Q spans, at most 2^31
  int64_t q_stride, kv_stride;  // row strides (elements) of Q and of K / V
};

template <bool BF16>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x4 mfma_pv(uint2 a, uint2 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row's four
// 16-lane groups) with the cross-row swaps of gfx950: called with the same
// value twice, each returns a lane's own value and its partner's (l ^ 32,
// then l ^ 16), in an order that may differ between lanes; max and a
// two-term sum do not depend on it, so all four lanes get the same result.
__device__ __forceinline__ float rows_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even into one packed register (one
// v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// Offset of a padding column's loads: past the end of K and V, which the host
// keeps at or below 2^31 bytes, so no offset wraps around.
constexpr uint32_t kPastEnd = 0x80000000u;

// Every global access moves whole rows: a tile's K and V rows, the window's
// Q rows and its output rows each go through per-wave LDS buffers, so one
// 64-lane instruction covers 512 / D whole rows instead of a 32- or 64-byte
// piece of each of sixteen rows (the operand layouts of the matrix cores);
// on 1024 complete digraphs of 20-40 nodes (8 heads, D = 64) this alone
// took the kernel from 41.7 to 33.3 us.  Two tiles in flight per wave: tile
// t + 1's rows are issued into the other pair of buffers (direct-to-LDS
// loads, no registers) before the wave waits for tile t's, so they load
// while tile t computes; the wait counts exactly the loads issued after
// tile t's.  K, V and Q are addressed through buffer resources: a padding
// column's (or a row past the end's) loads fall past the end, return zeros
// and reach no memory.
template <bool BF16, int D>
// The second launch bound (at least 2 waves per SIMD) makes the compiler pack
// the registers.
__global__ __launch_bounds__(kWavesPerWg * 64, 2) void mfma_kernel(MfmaArgs a) {
  constexpr int KS = D / 32;   // 16x16x32 steps for S^T
  constexpr int NB = D / 16;   // 16-wide d blocks for O^T
  constexpr int VB = KS * 1024;  // one tile's K (or V) rows in LDS: KS loads of 64 lanes x 16 bytes
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kWavesPerWg][2][VB];
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kWavesPerWg][2][VB];
  // a wave's window: column ids and masks of up to kMetaCols / 16 tiles at a time
  __shared__ int32_t s_col[kWavesPerWg][kMetaCols];
  __shared__ uint32_t s_msk[kWavesPerWg][kMetaCols / 2];  // two 16-bit masks per word

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // A workgroup's waves: heads h0 .. h0 + 3 of one window when there are at
  // least 4 heads (grid y = head group); with fewer, consecutive (window,
  // head) items, heads fastest, so that no wave of a workgroup sits idle.
  const int lin = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  int wb, h;
  if (a.H >= kWavesPerWg) {
    wb = lin;
    h = blockIdx.y * kWavesPerWg + wave;
  } else {
    const int item = __builtin_amdgcn_readfirstlane(lin * kWavesPerWg + wave);  // wave-uniform
    wb = item / a.H;
    h = item - wb * a.H;
  }
  if (h >= a.H || wb >= a.nwb) return;
  const int w = a.windows ? a.windows[wb] : wb;
  if (w < 0 || w >= a.W) return;
  const int r = lane & 15, g = lane >> 4;
  const int64_t rowstride = (int64_t)a.H * D;

  // The window's Q rows go whole into the wave's second V buffer (rows past
  // the end read as zeros), 2D bytes per row; the first chunk's wait covers
  // them, and the B operand of S^T (Q_w^T: lane holds Q[row r][d = 32s + 8g
  // .. +7]) is read from there before any tile loads into that buffer.
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per 64-lane load or store
  {
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.q, (short)0, (int)a.q_bytes, kBufferWord3);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int row = s * RPI + lane / CPR;
      const uint32_t off = (uint32_t)((((uint64_t)(16 * w + row) * a.q_stride + (uint64_t)h * D) * 2)) + 16 * (lane % CPR);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)&s_v[wave][1][s * 1024],
                                               16, off, 0, 0, 0);
    }
  }
  u32x4 qf[KS];

  const int64_t c0 = min<int64_t>(max(a.win_col_ptr[w], 0), a.num_cols) & ~int64_t(15);
  const int64_t c1 = min<int64_t>(max<int64_t>(a.win_col_ptr[w + 1], c0), a.num_cols) & ~int64_t(15);

  // Online softmax with a lazily moved reference.  Each row keeps a reference
  // max m (the same in its four lanes) and each lane a partial sum lp of the
  // weights of its own columns.  A tile's weights are exp2(x - m); m moves,
  // and O^T and lp are rescaled, only when a logit exceeds it by more than
  // 2^kLazy, which after a row's first tile is rare, so most tiles skip the
  // row-wide max and the rescale (a wave-wide vote decides).  The weights
  // stay at most 2^kLazy = 256, which fp16 and bf16 hold.  The logit that set
  // m gives x - m = 0 exactly and weight exp2(0) = 1 exactly (so does the
  // hardware's exp2), so a row with one edge returns that edge's v bit for bit.
  constexpr float kLazy = 8.f;
  float m = -INFINITY, lp = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A tile's K and V rows land in LDS row-major, 2D bytes per row, each
  // 64-lane load covering RPI whole rows (lane l: row l / CPR of the load,
  // 16-byte chunk slot l % CPR).  Slot p of row t holds chunk p ^ (t % CPR),
  // which spreads the column reads below over the LDS banks.
  // K and V descriptors as raw words (base, num_records, flags) for the
  // direct-to-LDS loads below
  const uint64_t kbase = (uint64_t)a.k, vbase = (uint64_t)a.v;
  const i32x4 dk = {(int)(uint32_t)kbase, (int)(uint32_t)(kbase >> 32) & 0xffff, (int)a.kv_bytes, kBufferWord3};
  const i32x4 dv = {(int)(uint32_t)vbase, (int)(uint32_t)(vbase >> 32) & 0xffff, (int)a.kv_bytes, kBufferWord3};
  // One 16-byte direct-to-LDS load per lane: lane l's bytes land at LDS
  // address lds + 16 l.  Written as asm because the compiler, which cannot
  // tell the two buffer pairs apart, would otherwise make every LDS read
  // wait for all such loads in flight (the next tile's included); every wait
  // for these loads is explicit instead (wait_vm).
  auto dma16 = [&](const i32x4& d, uint32_t voff, const void* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here, not preserved
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(d)
                 : "memory", "m0");
#pragma clang diagnostic pop
  };
  auto slot = [&](int row, int chunk) { return row * 2 * D + 16 * (chunk ^ (row % CPR)); };
  auto issue = [&](int32_t c, int b) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int row = s * RPI + lane / CPR;
      const int32_t col = s_col[wave][c + row];
      const uint32_t off = (uint32_t)col < (uint32_t)a.n
                               ? (uint32_t)(((uint64_t)col * a.kv_stride + (uint64_t)h * D) * 2) +
                                     16 * ((lane % CPR) ^ (row % CPR))
                               : kPastEnd;
      dma16(dk, off, &s_k[wave][b][s * 1024]);
      dma16(dv, off, &s_v[wave][b][s * 1024]);
    }
  };
  // Operands of tile buffer b.  K (A operand of S^T): lane (r, g) takes
  // K[source r][d = 32s + 8g .. +7], chunk 4s + g of row r.  V^T (A operand of
  // O^T, d block j): lane (i = lane % 16, q = lane / 16) takes V[source 4q +
  // t][d = 16j + i], t = 0..3, from one transposing LDS read, which hands
  // lane i of each 16-lane group element i % 4 of the 8 bytes addressed by
  // lane 4t + i / 4 of the group; so lane k of group q addresses V[source 4q
  // + k / 4][d = 16j + 4 (k % 4) .. +3], half of one 16-byte chunk.
  auto read_tile = [&](int b, u32x4* kf, uint2* va) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = *reinterpret_cast<const u32x4*>(&s_k[wave][b][slot(r, 4 * s + g)]);
    const int src = 4 * g + (r >> 2);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int d0 = 16 * j + 4 * (r & 3);
      const int byte = slot(src, d0 >> 3) + 2 * (d0 & 7);
      va[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (__attribute__((address_space(3))) i16x4*)(
                                                (__attribute__((address_space(3))) uint8_t*)&s_v[wave][b][0] + byte)));
    }
  };
  // one tile: S^T on the matrix cores, the online softmax over the tile's 16
  // sources per row, P^T straight from the accumulator registers, and O^T +=
  // V^T P^T
  auto compute = [&](const u32x4* kf, const uint2* va, uint32_t mask) {
#pragma clang fp contract(off)  // x - m stays a rounded logit minus m: exactly 0 where x set m
    const uint32_t bits = mask >> (4 * g);
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) st = mfma_qk<BF16>(kf[s], qf[s], st);
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (bits >> i & 1u) ? st[i] * a.scale_l2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    if (__builtin_amdgcn_ballot_w64(tmax > m + kLazy)) {  // wave-uniform
      const float rmax = rows_max(tmax);
      const float mn = rmax > m + kLazy ? rmax : m;
      const float corr = mn == m ? 1.f : fast_exp2(m - mn);  // m = -inf: nothing accumulated yet
      lp *= corr;
#pragma unroll
      for (int j = 0; j < NB; ++j) o[j] *= corr;
      m = mn;
    }
    const float mu = m == -INFINITY ? 0.f : m;  // a row without an edge so far: every x is -inf
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - mu);
    lp += (p[0] + p[1]) + (p[2] + p[3]);
    uint2 pb;
    pb.x = pack2<BF16>(p[0], p[1]);
    pb.y = pack2<BF16>(p[2], p[3]);
#pragma unroll
    for (int j = 0; j < NB; ++j) o[j] = mfma_pv<BF16>(va[j], pb, o[j]);
  };
  // wait until at most N direct-to-LDS loads of this wave are in flight (they
  // complete in order), with compiler fences so that no LDS access crosses it
  auto wait_vm = [&](auto n_) {
    constexpr int N = decltype(n_)::value;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  using kTile = std::integral_constant<int, 2 * KS>;
  using kNone = std::integral_constant<int, 0>;
  // the mask of row r of tile c / 16, c counted from the start of the staged chunk
  auto mask_of = [&](int32_t c) -> uint32_t { return reinterpret_cast<const uint16_t*>(s_msk[wave])[c + r]; };

  // The window's ids and masks go to LDS once per chunk of up to 16 tiles, 64
  // ids or 128 masks per direct-to-LDS load (lane l's 4 bytes land at 4 l),
  // instead of two loads per tile: the kernel is bound by the rate at which a
  // CU issues vector memory instructions, not by their bytes.
  for (int64_t cb = c0; cb < c1; cb += kMetaCols) {
    const int32_t n = (int32_t)min<int64_t>(kMetaCols, c1 - cb);
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.win_cols + cb), (short)0, n * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rm =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.tile_mask + cb), (short)0, n * 2, kBufferWord3);
    for (int i = 0; i < n; i += 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)&s_col[wave][i], 4,
                                               (uint32_t)(i + lane) * 4, 0, 0, 0);
    for (int i = 0; i < n; i += 128)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (__attribute__((address_space(3))) void*)&s_msk[wave][i / 2], 4,
                                               (uint32_t)(2 * i + 4 * lane), 0, 0, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (cb == c0) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[s] = *reinterpret_cast<const u32x4*>(&s_v[wave][1][r * 2 * D + 64 * s + 16 * g]);
    }
    uint32_t maskA = mask_of(0), maskB = 0;
    u32x4 kf[KS];
    uint2 va[NB];
    issue(0, 0);
    // tiles c (buffers 0) and c + 16 (buffers 1) per pass: a tile's rows load
    // while the one before it computes.  The branches are uniform across the wave.
    for (int32_t c = 0; c < n; c += 32) {
      if (c + 16 < n) {
        maskB = mask_of(c + 16);
        issue(c + 16, 1);
        wait_vm(kTile{});
      } else {
        wait_vm(kNone{});
      }
      read_tile(0, kf, va);
      compute(kf, va, maskA);
      if (c + 16 >= n) break;
      if (c + 32 < n) {
        maskA = mask_of(c + 32);
        issue(c + 32, 0);
        wait_vm(kTile{});
      } else {
        wait_vm(kNone{});
      }
      read_tile(1, kf, va);
      compute(kf, va, maskB);
    }
  }

  // O[row][d = 16j + 4g + i] = O^T[d][row] / l  (row without edges -> 0).
  // The rows go through the wave's V buffers (every load into them has been
  // waited for) so that each store instruction writes whole 2D-byte rows.
  const float l = rows_sum(lp);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // a window without columns still has its Q rows in flight
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  constexpr int RS = 2 * D + 16;  // padded row stride in LDS (bytes)
  static_assert(16 * RS <= 2 * VB, "the output rows fit the wave's V buffers");
  uint8_t* so = &s_v[wave][0][0];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    uint2 w2;
    w2.x = pack2<BF16>(o[j][0] * inv, o[j][1] * inv);
    w2.y = pack2<BF16>(o[j][2] * inv, o[j][3] * inv);
    *reinterpret_cast<uint2*>(so + r * RS + 2 * (16 * j + 4 * g)) = w2;
  }
#pragma unroll
  for (int q = 0; q < 16 / RPI; ++q) {
    const int row = q * RPI + lane / CPR, ch = lane % CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(so + row * RS + 16 * ch);
    const int nd = 16 * w + row;
    if (nd < a.n) st16(a.out + (int64_t)nd * rowstride + (int64_t)h * D + 8 * ch, x);
  }
}

template <bool BF16>
hipError_t launch_b(const gattn_forward_args& fa, const MfmaArgs& ma, int32_t blocks, hipStream_t s) {
  const dim3 grid = fa.num_heads >= kWavesPerWg
                       ? dim3((unsigned)blocks, (unsigned)ceil_div(fa.num_heads, kWavesPerWg))
                       : dim3((unsigned)ceil_div((int64_t)blocks * fa.num_heads, kWavesPerWg));
  dim3 block(kWavesPerWg * 64);
  switch (fa.head_dim) {
    case 32: hipLaunchKernelGGL((mfma_kernel<BF16, 32>), grid, block, 0, s, ma); break;
    case 64: hipLaunchKernelGGL((mfma_kernel<BF16, 64>), grid, block, 0, s, ma); break;
    default: hipLaunchKernelGGL((mfma_kernel<BF16, 128>), grid, block, 0, s, ma); break;
  }
  return hipGetLastError();
}

}  // namespace

namespace {
// bytes a 16-bit [N, H, D] view with row stride st (0: packed) spans
uint64_t span_bytes(const gattn_forward_args& a, int64_t st) {
  const uint64_t hd = (uint64_t)a.num_heads * a.head_dim;
  if (a.num_nodes <= 0) return 0;
  return ((uint64_t)(a.num_nodes - 1) * (st ? (uint64_t)st : hd) + hd) * 2;
}
}  // namespace

bool mfma_supported(const gattn_forward_args& a) {
  // K, V and Q are read through 32-bit buffer offsets, padding columns at 2^31
  return (a.dtype == GATTN_F16 || a.dtype == GATTN_BF16) && a.mode == GATTN_SOFTMAX_STANDARD && a.e == nullptr &&
         (a.head_dim == 32 || a.head_dim == 64 || a.head_dim == 128) &&
         span_bytes(a, a.kv_stride) <= ((uint64_t)1 << 31) && span_bytes(a, a.q_stride) <= ((uint64_t)1 << 31);
}

hipError_t launch_forward_mfma(const gattn_forward_args& fa, const int32_t* windows, int32_t num_windows,
                               hipStream_t s) {
  if (fa.num_nodes == 0 || (windows && num_windows == 0)) return hipSuccess;
  MfmaArgs ma;
  ma.windows = windows;
  ma.win_col_ptr = fa.rw->win_col_ptr;
  ma.win_cols = fa.rw->win_cols;
  ma.tile_mask = fa.rw->tile_mask;
  ma.q = (const uint16_t*)fa.q;
  ma.k = (const uint16_t*)fa.k;
  ma.v = (const uint16_t*)fa.v;
  ma.out = (uint16_t*)fa.out;
  ma.num_cols = fa.rw->num_cols;
  ma.n = fa.num_nodes;
  ma.H = fa.num_heads;
  ma.W = fa.rw->num_windows;
  ma.scale_l2 = fa.scale * kLog2e;
  ma.kv_bytes = (uint32_t)span_bytes(fa, fa.kv_stride);
  ma.q_bytes = (uint32_t)span_bytes(fa, fa.q_stride);
  const int64_t hd = (int64_t)fa.num_heads * fa.head_dim;
  ma.q_stride = fa.q_stride ? fa.q_stride : hd;
  ma.kv_stride = fa.kv_stride ? fa.kv_stride : hd;
  const int32_t blocks = windows ? num_windows : ma.W;
  ma.nwb = blocks;
  return fa.dtype == GATTN_BF16 ? launch_b<true>(fa, ma, blocks, s) : launch_b<false>(fa, ma, blocks, s);
}

}  // namespace gattn
