// Internal declarations and device helpers of the rf library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rf {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// bf16 <-> fp32. A bf16 is the top half of a binary32, so widening is a shift.
// Narrowing rounds to nearest, ties to even; NaN stays a quiet NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Streaming (non-temporal) 16-byte global accesses for data touched exactly once.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_load(const float4* p) {
  const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store(float4 x, float4* p) {
  nt_f32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
}
__device__ __forceinline__ void nt_store(uint4 x, uint4* p) {
  nt_u32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4*>(p));
}

// Hardware base-2 exponential (v_exp_f32). exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// Cross-lane moves inside a wavefront (64 lanes).
// DPP row = 16 lanes. quad_perm xor1 = 0xB1, xor2 = 0x4E, row_half_mirror =
// 0x141 (lane i of 8 <- lane 7-i), row_mirror = 0x140 (lane i of 16 <- 15-i).
// Each butterfly step leaves bit-identical sums in every participating lane.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N consecutive lanes (N in {2, 4, 8, 16}); all lanes of a group get the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group size");
  x += dpp_mov<0xB1>(x);
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);
  return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group size");
  x = fmaxf(x, dpp_mov<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Max / sum of a value over the lane pair (l, l ^ 32), via v_permlane32_swap:
// the two results hold the low half and the high half of x broadcast across
// the wavefront, so combining them symmetrically needs no LDS round trip.
__device__ __forceinline__ float pair_max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The (m, l) pair of a partial safe-softmax reduction, m in log2 units:
// (m_a, l_a) (+) (m_b, l_b) = (M, l_a 2^(m_a - M) + l_b 2^(m_b - M)), M = max.
// The identity is (-inf, 0); combining two identities stays the identity.
__device__ __forceinline__ void ml_combine(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  const float Mu = (M == kNegInf) ? 0.f : M;
  l = l * fast_exp2(m - Mu) + l2 * fast_exp2(m2 - Mu);
  m = M;
}
// Same monoid with m in natural units: only the (small) differences m - M are
// scaled by log2(e), so a large common offset costs no accuracy.
__device__ __forceinline__ void ml_combine_nat(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  const float Mu = (M == kNegInf) ? 0.f : M;
  l = l * fast_exp2((m - Mu) * kLog2e) + l2 * fast_exp2((m2 - Mu) * kLog2e);
  m = M;
}

}  // namespace rf

// The host-side launchers are declared in launch.h.
