// common.hpp -- device helpers shared by the gfx950 kernels of libgattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gattn.h"

namespace gattn {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage types: float, _Float16, and bf16 held as uint16_t bits.
struct bf16_t { uint16_t bits; };

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kVec = 4; static constexpr gattn_dtype kDtype = GATTN_F32; };
template <> struct Elem<_Float16> { static constexpr int kVec = 8; static constexpr gattn_dtype kDtype = GATTN_F16; };
template <> struct Elem<bf16_t> { static constexpr int kVec = 8; static constexpr gattn_dtype kDtype = GATTN_BF16; };

// ---- 16-byte loads / stores -------------------------------------------------
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format).
// The range check then makes each dword of a load that falls past the
// resource's size return zero without any memory access.
constexpr int32_t kBufferWord3 = 0x00020000;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }

// ---- widening to fp32 (exact) ----------------------------------------------
template <typename T> struct Conv;
template <> struct Conv<float> {
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
};
template <> struct Conv<_Float16> {
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = x[i];
      _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
      _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      f[2 * i] = (float)lo;
      f[2 * i + 1] = (float)hi;
    }
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {  // round to nearest even
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i]);
      uint16_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i + 1]);
      r[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return r;
  }
};
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
template <> struct Conv<bf16_t> {
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = x[i];
      f[2 * i] = __uint_as_float(w << 16);
      f[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = bf16_rne(f[2 * i]) | (bf16_rne(f[2 * i + 1]) << 16);
    return r;
  }
};

// ---- cross-lane sums over aligned groups of 2..32 lanes --------------------
// DPP inside a 16-lane row; ds_swizzle-free xor for 32.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32, "group");
  if constexpr (LANES >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LANES >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LANES >= 8) x += dpp<0x141>(x);   // row_half_mirror: other quad of the 8
  if constexpr (LANES >= 16) x += dpp<0x140>(x);  // row_mirror: other half of the 16
  if constexpr (LANES >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// blockIdx.x -> logical block so that consecutive logical blocks share an XCD
// (the dispatcher deals workgroups round-robin over the 8 XCDs).
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t nb) {
  const uint32_t x = b & 7u, i = b >> 3, q = nb >> 3, r = nb & 7u;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

}  // namespace gattn
