// Device-side helpers shared by the gfx950 KDA kernels (decode and prefill).
// gfx950 only: 64-wide wavefronts, MFMA 16x16 tiles, hardware bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "kda_launch.h"

// Statements that only a timing build (-DKDA_PHASE_STAMPS) compiles: per-phase
// s_memtime stamps of the long-running kernels.  Nothing in the product build.
#if defined(KDA_PHASE_STAMPS)
#define KDA_PHASE(...) __VA_ARGS__
#else
#define KDA_PHASE(...)
#endif

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// e^x through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round-to-nearest-even through the gfx950 conversion instruction
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 1 / (1 + e^{-x}) through the hardware exponential and reciprocal (0 and 1 at the
// extremes, no overflow trap).
__device__ __forceinline__ float sigmoid_hw(float x) {
  return __builtin_amdgcn_rcpf(1.f + exp_hw(-x));
}
// v of the lane selected by the DPP control CTRL (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xf, 0xf, false));
}
// Sum over aligned groups of `width` (16 or 32) lanes, every lane receiving the total:
// within each 16-lane row by DPP (neighbour swap, pair swap, half-row and row mirror:
// each step adds a lane whose partial covers the other half of the current block),
// then one cross-row exchange for width 32.
template <int width>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(width == 16 || width == 32, "row_sum over 16 or 32 lanes");
  x += dpp_mov<0xb1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4e>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  if constexpr (width == 32) x += __shfl_xor(x, 16, 32);
  return x;
}

// log(sigmoid(a)) = -log(1 + e^{-a}): a retention logit as a log-decay g (0 when
// e^{-a} is below fp32 resolution, -inf for a below about -88, so e^g is 1 or 0).
__device__ __forceinline__ float log_sigmoid_hw(float a) {
  return -__builtin_amdgcn_logf(1.f + exp_hw(-a)) * 0.6931471805599453f;
}
__device__ __forceinline__ f32x4 log_sigmoid4(f32x4 a) {
  return f32x4{log_sigmoid_hw(a[0]), log_sigmoid_hw(a[1]), log_sigmoid_hw(a[2]),
               log_sigmoid_hw(a[3])};
}

// Four consecutive elements of an fp32 or bf16 array, widened to fp32.
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace kda
