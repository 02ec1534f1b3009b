// Split-KV decode: the multi-segment strategy (RedFuser page, 3. Contributions
// clés) for one query token per (b, h). The Lk cached keys are cut into S
// contiguous chunks; each chunk is reduced to a normalised partial (O_s, lse_s)
// in incremental form, and rf_lse_merge combines the partials.
//
// This path is bound by streaming K and V from HBM (about 1 flop per byte),
// so the kernel is organised around the loads, not around matrix cores: it
// is the row-wise kernel shape of the STOF page (Méthodologie 1: a query row
// per group of lanes, lane-level reductions, no inter-wave synchronisation in
// the loop).
//
// Work mapping (D = head dim, 64 or 128):
//   - one workgroup (4 waves) per unit (b, h, s); the waves take interleaved
//     blocks of KPI = 32 keys of the chunk;
//   - inside a wave, LPK = D/8 lanes share one key: each lane owns 8 consecutive
//     elements of d, so a wave's 16-byte loads cover KPW = 64/LPK whole keys
//     (4 contiguous 256-byte rows for D = 128): fully coalesced;
//   - each group of LPK lanes runs its own online (m, l, acc) over its keys;
//     q.k is a bf16 dot2 chain plus a DPP butterfly over the LPK lanes;
//   - at the end the KPW groups and the 4 waves meet in the (m, l, acc)
//     monoid, and the unit writes O_s = acc / l (fp32) and lse_s (natural log).
// Scores are kept in log2 units: t = (q . k) * scale * log2(e), p = 2^(t - m).
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int D, int U>
__global__ __launch_bounds__(256) void decode_partial_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             float* __restrict__ o_parts,
                                                             float* __restrict__ lse_parts, int64_t n_units,
                                                             int Lk, int S, int chunk, float scale_log2) {
  constexpr int LPK = D / 8;      // lanes per key
  constexpr int KPW = 64 / LPK;   // keys per wave per load step
  constexpr int KPI = KPW * U;    // keys per wave per iteration
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPK;  // which key of a load step
  const int ds = lane % LPK;   // this lane's 8-element slice of d

  for (int64_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int64_t bh = unit / S;
    const int s = int(unit % S);
    const int64_t lo = min(int64_t(s) * chunk, int64_t(Lk));
    const int64_t hi = min(lo + chunk, int64_t(Lk));

    const uint4 qv = *reinterpret_cast<const uint4*>(q + bh * D + 8 * ds);
    const uint16_t* kb = k + bh * int64_t(Lk) * D + 8 * ds;
    const uint16_t* vb = v + bh * int64_t(Lk) * D + 8 * ds;

    float m = kNegInf, l = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    for (int64_t base = lo + int64_t(wave) * KPI; base < hi; base += 4 * KPI) {
      uint4 kr[U], vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t key = base + u * KPW + sub;
        if (key < hi) {
          kr[u] = nt_load(reinterpret_cast<const uint4*>(kb + key * D));
          vr[u] = nt_load(reinterpret_cast<const uint4*>(vb + key * D));
        } else {
          kr[u] = make_uint4(0, 0, 0, 0);
          vr[u] = make_uint4(0, 0, 0, 0);
        }
      }
      float t[U];
      float bm = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dsum = dot2_bf16(kr[u].x, qv.x, 0.f);
        dsum = dot2_bf16(kr[u].y, qv.y, dsum);
        dsum = dot2_bf16(kr[u].z, qv.z, dsum);
        dsum = dot2_bf16(kr[u].w, qv.w, dsum);
        dsum = group_sum<LPK>(dsum);
        const int64_t key = base + u * KPW + sub;
        t[u] = (key < hi) ? dsum * scale_log2 : kNegInf;
        bm = fmaxf(bm, t[u]);
      }
      const float mn = fmaxf(m, bm);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m - mu);  // rescale of the running pair when the max moves
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(t[u] - mu);
        l += p;
        acc[0] += p * bf16_lo(vr[u].x);
        acc[1] += p * bf16_hi(vr[u].x);
        acc[2] += p * bf16_lo(vr[u].y);
        acc[3] += p * bf16_hi(vr[u].y);
        acc[4] += p * bf16_lo(vr[u].z);
        acc[5] += p * bf16_hi(vr[u].z);
        acc[6] += p * bf16_lo(vr[u].w);
        acc[7] += p * bf16_hi(vr[u].w);
      }
      m = mn;
    }

    // Merge the KPW key groups of this wave (lanes with equal ds).
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      const float m2 = shfl_xor(m, off);
      const float l2 = shfl_xor(l, off);
      const float M = fmaxf(m, m2);
      const float Mu = (M == kNegInf) ? 0.f : M;
      const float a = fast_exp2(m - Mu), b = fast_exp2(m2 - Mu);
      l = l * a + l2 * b;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + shfl_xor(acc[e], off) * b;
      m = M;
    }
    if (lane < LPK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][8 * ds + e] = acc[e];
      if (lane == 0) {
        s_m[wave] = m;
        s_l[wave] = l;
      }
    }
    __syncthreads();
    // Merge the 4 waves and write the normalised partial.
    if (threadIdx.x < D) {
      const int e = threadIdx.x;
      float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
      const float Mu = (M == kNegInf) ? 0.f : M;
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = fast_exp2(s_m[w] - Mu);
        L += a * s_l[w];
        O += a * s_acc[w][e];
      }
      const bool live = L > 0.f;
      o_parts[unit * D + e] = live ? O / L : 0.f;
      if (e == 0) lse_parts[unit] = live ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode_partials(const void* q, const void* k, const void* v, float* o_parts,
                                  float* lse_parts, int B, int H, int Lk, int d, float scale,
                                  int num_splits, hipStream_t stream) {
  const int64_t n_units = int64_t(B) * H * num_splits;
  const int chunk = Lk > 0 ? int((int64_t(Lk) + num_splits - 1) / num_splits) : 0;
  const float scale_log2 = float(double(scale) * 1.4426950408889634);
  const unsigned grid = unsigned(n_units < (1LL << 20) ? n_units : (1LL << 20));
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  if (d == 128) {
    hipLaunchKernelGGL((decode_partial_kernel<128, 8>), dim3(grid), dim3(256), 0, stream, qb, kb, vb, o_parts,
                       lse_parts, n_units, Lk, num_splits, chunk, scale_log2);
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<64, 4>), dim3(grid), dim3(256), 0, stream, qb, kb, vb, o_parts,
                       lse_parts, n_units, Lk, num_splits, chunk, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace rf
