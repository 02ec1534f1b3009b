// Log-sum-exp merge of normalised partial results (the merge of the
// multi-segment strategy, RedFuser page, 3. Contributions clés).
//
// The pairs (O_s, lse_s) form a commutative monoid (RedFuser Korean page,
// 2. 방법론, 가: decomposability, commutative monoid, distributivity), so the
// merge order is free:
//   M = max_s lse_s, w_s = e^{lse_s - M}, W = sum_s w_s,
//   O = sum_s w_s O_s / W,  LSE = M + ln W.
// A part whose lse is -inf is the identity: its weight is exactly zero and
// its O_s row is never read.
//
// Layout: one thread per (row, 4-float chunk of d) when d % 4 == 0 and the
// pointers are 16-byte aligned, else one thread per (row, element). Each
// thread rescans the row's S lse values (they stay in L1) — the data volume
// that matters is the S x d partial rows, read once.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

template <int VEC, bool OUT_BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ o_parts,
                                                        const float* __restrict__ lse_parts,
                                                        void* __restrict__ o, float* __restrict__ lse,
                                                        int64_t n_rows, int S, int d) {
  const int nchunk = d / VEC;
  const int64_t total = n_rows * nchunk;
  for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
  const int64_t row = idx / nchunk;
  const int c = int(idx % nchunk);
  const float* lp = lse_parts + row * S;

  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  float W = 0.f;
  if (M != kNegInf) {
    const float* op = o_parts + row * int64_t(S) * d + int64_t(c) * VEC;
    for (int s = 0; s < S; ++s) {
      const float ls = lp[s];
      if (ls == kNegInf) continue;  // identity part: weight 0, O_s not read
      const float w = fast_exp2((ls - M) * kLog2e);
      W += w;
      if constexpr (VEC == 4) {
        const float4 v = *reinterpret_cast<const float4*>(op + int64_t(s) * d);
        acc[0] += w * v.x; acc[1] += w * v.y; acc[2] += w * v.z; acc[3] += w * v.w;
      } else {
        acc[0] += w * op[int64_t(s) * d];
      }
    }
    const float inv = 1.f / W;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= inv;
  }
  const int64_t out = row * d + int64_t(c) * VEC;
  if constexpr (OUT_BF16) {
    uint16_t* ob = static_cast<uint16_t*>(o) + out;
    if constexpr (VEC == 4) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(ob) = pk;
    } else {
      ob[0] = uint16_t(f32_to_bf16_bits(acc[0]));
    }
  } else {
    float* of = static_cast<float*>(o) + out;
    if constexpr (VEC == 4) {
      *reinterpret_cast<float4*>(of) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      of[0] = acc[0];
    }
  }
  if (lse != nullptr && c == 0) lse[row] = (M == kNegInf) ? kNegInf : M + fast_log2(W) * kLn2;
  }
}

template <int VEC>
hipError_t launch(const float* o_parts, const float* lse_parts, void* o, float* lse, int64_t n_rows,
                  int S, int d, bool out_bf16, hipStream_t stream) {
  const int64_t n = n_rows * (d / VEC);
  int64_t blocks = (n + 255) / 256;
  if (blocks > (1LL << 22)) blocks = 1LL << 22;  // grid-stride beyond this
  if (out_bf16)
    hipLaunchKernelGGL((lse_merge_kernel<VEC, true>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       o_parts, lse_parts, o, lse, n_rows, S, d);
  else
    hipLaunchKernelGGL((lse_merge_kernel<VEC, false>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       o_parts, lse_parts, o, lse, n_rows, S, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                            int64_t n_rows, int num_splits, int d, int out_dtype, hipStream_t stream) {
  const bool out_bf16 = out_dtype == 1;
  const uintptr_t al = reinterpret_cast<uintptr_t>(o_parts) | reinterpret_cast<uintptr_t>(o);
  const bool vec_ok = d % 4 == 0 && (al % (out_bf16 ? 8 : 16)) == 0 &&
                      reinterpret_cast<uintptr_t>(o_parts) % 16 == 0;
  if (vec_ok) return launch<4>(o_parts, lse_parts, o, lse, n_rows, num_splits, d, out_bf16, stream);
  return launch<1>(o_parts, lse_parts, o, lse, n_rows, num_splits, d, out_bf16, stream);
}

}  // namespace rf
