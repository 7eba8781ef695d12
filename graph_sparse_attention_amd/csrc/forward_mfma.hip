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
//   masked entries -> -inf; running row max / sum in fp32 (online softmax)
//   O^T (D x 16 rows) += V_t^T (D x 16 src) . P^T (16 src x 16 rows)
//        v_mfma_f32_16x16x16_{f16,bf16}, D/16 blocks.  The B operand P^T
//        needs lane l to hold P[row l%16][src 4(l/16)+i] -- exactly the S^T
//        accumulator layout, so P goes from the SDDMM accumulators to the
//        SpMM operand without leaving the registers (our counterpart of
//        Fused3S's register remapping).  V_t^T is read transposed from a
//        per-wave LDS copy of the tile's V rows.
//   O^T accumulators keep row l%16 in lane l like the softmax state, so the
//   per-row rescale is a register multiply.
//
// S and P never leave the chip.  The work is still bounded by HBM / L2: each
// K / V row is loaded once per window instead of once per edge.
#include "common.hpp"
#include "internal.hpp"

namespace gattn {

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerWg = 4;

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
  float scale_l2;  // scale * log2(e)
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

template <bool BF16>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (BF16) return (uint16_t)bf16_rne(x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <bool BF16, int D>
// The second launch bound (at least 2 waves per SIMD) makes the compiler pack
// the registers: 80 for D = 64 (6 waves per SIMD), 52 for D = 32, 112 for
// D = 128, without spills; with no bound it takes 96 for D = 64.
__global__ __launch_bounds__(kWavesPerWg * 64, 2) void mfma_kernel(MfmaArgs a) {
  constexpr int KS = D / 32;   // 16x16x32 steps for S^T
  constexpr int NB = D / 16;   // 16-wide d blocks for O^T
  constexpr int LDW = D + 8;   // LDS row pitch in 16-bit elements (breaks bank aliasing)
  __shared__ uint16_t s_v[kWavesPerWg][16 * LDW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wb = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int w = a.windows ? a.windows[wb] : wb;
  const int h = blockIdx.y * kWavesPerWg + wave;
  if (h >= a.H || w < 0 || w >= a.W) return;
  const int r = lane & 15, g = lane >> 4;
  const int node = 16 * w + r;
  const bool row_ok = node < a.n;
  const int64_t rowstride = (int64_t)a.H * D;
  uint16_t* sv = s_v[wave];

  // B operand of S^T: Q_w^T, lane holds Q[row r][d = 32s + 8g .. +7]
  u32x4 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = row_ok ? ld16(a.q + (int64_t)node * rowstride + (int64_t)h * D + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};

  const int64_t c0 = min<int64_t>(max(a.win_col_ptr[w], 0), a.num_cols) & ~int64_t(15);
  const int64_t c1 = min<int64_t>(max<int64_t>(a.win_col_ptr[w + 1], c0), a.num_cols) & ~int64_t(15);

  float m = -INFINITY, l = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads are issued with no branch around them (a padding column reads row
  // 0, whose V is zeroed before use).  One register set per tile: the
  // (window, head) waves of a CU hide each other's load latency, and a second
  // set for the next tile's rows would cost two waves per SIMD.
  auto load_kv = [&](int32_t col, u32x4* kk, u32x4* vv) {
    const int64_t src_off = (int64_t)((uint32_t)col < (uint32_t)a.n ? col : 0) * rowstride + (int64_t)h * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kk[s] = ld16(a.k + src_off + 32 * s + 8 * g);
      vv[s] = ld16(a.v + src_off + 32 * s + 8 * g);
    }
  };
  // tile at column c with rows (kf, vf), column id col and row mask `mask`
  auto tile = [&](u32x4* kf, u32x4* vf, int32_t col, uint32_t mask) {
    const uint32_t bits = mask >> (4 * g);
    if ((uint32_t)col >= (uint32_t)a.n) {  // padding column: no edge, V row zero
#pragma unroll
      for (int s = 0; s < KS; ++s) vf[s] = u32x4{0u, 0u, 0u, 0u};
    }

    // SDDMM on the matrix cores
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) st = mfma_qk<BF16>(kf[s], qf[s], st);

    // online softmax over this tile's 16 sources, per row r
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (bits >> i & 1u) ? st[i] * a.scale_l2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float corr = m == mn ? 1.f : fast_exp2(m - mu);  // exp2(0) kept exact
    float p[4], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = x[i] == mu ? 1.f : fast_exp2(x[i] - mu);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l = l * corr + psum;
    m = mn;
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] *= corr;

    // P^T operand straight from the accumulator registers
    uint2 pb;
    pb.x = (uint32_t)to_bits<BF16>(p[0]) | ((uint32_t)to_bits<BF16>(p[1]) << 16);
    pb.y = (uint32_t)to_bits<BF16>(p[2]) | ((uint32_t)to_bits<BF16>(p[3]) << 16);

    // V tile rows -> LDS, read back transposed as the A operand V^T
#pragma unroll
    for (int s = 0; s < KS; ++s) *reinterpret_cast<u32x4*>(sv + r * LDW + 32 * s + 8 * g) = vf[s];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint16_t* col0 = sv + (4 * g) * LDW + 16 * b + r;
      uint2 va;
      va.x = (uint32_t)col0[0] | ((uint32_t)col0[LDW] << 16);
      va.y = (uint32_t)col0[2 * LDW] | ((uint32_t)col0[3 * LDW] << 16);
      o[b] = mfma_pv<BF16>(va, pb, o[b]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (c0 < c1) {
    u32x4 kf[KS], vf[KS];
    for (int64_t c = c0; c < c1; c += 16) {
      const int32_t col = a.win_cols[c + r];
      const uint32_t mask = a.tile_mask[c + r];
      load_kv(col, kf, vf);
      tile(kf, vf, col, mask);
    }
  }

  // O[row r][d = 16b + 4g + i] = O^T[d][r] / l  (row without edges -> 0)
  if (row_ok) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint16_t* dst = a.out + (int64_t)node * rowstride + (int64_t)h * D + 4 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint2 w2;
      w2.x = (uint32_t)to_bits<BF16>(o[b][0] * inv) | ((uint32_t)to_bits<BF16>(o[b][1] * inv) << 16);
      w2.y = (uint32_t)to_bits<BF16>(o[b][2] * inv) | ((uint32_t)to_bits<BF16>(o[b][3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst + 16 * b) = w2;
    }
  }
}

template <bool BF16>
hipError_t launch_b(const gattn_forward_args& fa, const MfmaArgs& ma, int32_t blocks, hipStream_t s) {
  dim3 grid((unsigned)blocks, (unsigned)ceil_div(fa.num_heads, kWavesPerWg));
  dim3 block(kWavesPerWg * 64);
  switch (fa.head_dim) {
    case 32: hipLaunchKernelGGL((mfma_kernel<BF16, 32>), grid, block, 0, s, ma); break;
    case 64: hipLaunchKernelGGL((mfma_kernel<BF16, 64>), grid, block, 0, s, ma); break;
    default: hipLaunchKernelGGL((mfma_kernel<BF16, 128>), grid, block, 0, s, ma); break;
  }
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(const gattn_forward_args& a) {
  return (a.dtype == GATTN_F16 || a.dtype == GATTN_BF16) && a.mode == GATTN_SOFTMAX_STANDARD && a.e == nullptr &&
         (a.head_dim == 32 || a.head_dim == 64 || a.head_dim == 128);
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
  const int32_t blocks = windows ? num_windows : ma.W;
  return fa.dtype == GATTN_BF16 ? launch_b<true>(fa, ma, blocks, s) : launch_b<false>(fa, ma, blocks, s);
}

}  // namespace gattn
