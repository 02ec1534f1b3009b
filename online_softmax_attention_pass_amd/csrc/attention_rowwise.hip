// Row-wise masked attention: the row kernel of the STOF page (Méthodologie 1,
// dual-kernel strategy: for highly sparse masks and short sequences, Q is cut
// into rows, lanes of a warp reduce together and no synchronisation crosses
// warps), for bf16 with the same masks as the tile kernel: causal rule, tile
// kinds (0 empty, 1 full, other = partial) and, inside partial tiles, one
// 64-bit row word per tile row (bit j: key j of the tile is visible).
//
// One wavefront owns one query row and walks only the key tiles its mask row
// keeps, and inside a tile only the key groups with a visible key: a sparse
// row costs its visible keys, not whole 64 x 64 tiles. Lanes are laid out as
// in the split-KV decode kernel: D/8 lanes share a key (8 elements of d each,
// 16-byte coalesced loads), KPW = 64 / (D/8) keys per load step, U steps per
// iteration; each group of D/8 lanes keeps its own online (m, l, acc), and the
// groups meet in the (m, l, acc) monoid at the end. Scores are in log2 units.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kRowTile = 64;

__device__ __forceinline__ float dot2_bf16r(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int D, int U>
__global__ __launch_bounds__(256) void attention_rowwise_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float scale_log2, int causal,
    const uint8_t* __restrict__ tile_kind, const uint64_t* __restrict__ tile_bits, int64_t n_rows) {
  constexpr int LPK = D / 8;     // lanes per key
  constexpr int KPW = 64 / LPK;  // keys per load step
  constexpr int KPI = KPW * U;   // keys per iteration
  static_assert(kRowTile % KPI == 0, "iterations tile the 64-key tile");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPK;  // which key of a load step
  const int ds = lane % LPK;   // this lane's 8-element slice of d
  const int n_cols = (Lk + kRowTile - 1) / kRowTile;
  const int64_t off = int64_t(Lk) - Lq;  // bottom-right causal alignment

  for (int64_t row = int64_t(blockIdx.x) * 4 + wave; row < n_rows; row += int64_t(gridDim.x) * 4) {
    const int64_t bh = row / Lq;
    const int i = int(row % Lq);
    const uint4 qv = *reinterpret_cast<const uint4*>(q + row * D + 8 * ds);
    const uint16_t* kb = k + bh * int64_t(Lk) * D + 8 * ds;
    const uint16_t* vb = v + bh * int64_t(Lk) * D + 8 * ds;
    // last visible key of the row (causal rule and sequence end)
    int64_t last = causal ? int64_t(i) + off : int64_t(Lk) - 1;
    if (last > Lk - 1) last = Lk - 1;
    const int j_end = last < 0 ? 0 : int(last / kRowTile) + 1;
    const int64_t mrow = int64_t(i / kRowTile) * n_cols;

    float m = kNegInf, l = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    // The row's mask, 64 tiles per step: lane j reads tile J0 + j's kind and
    // this row's word of it, a ballot keeps the tiles with a visible key, and
    // the wave visits just those (the word comes back by readlane).
    for (int J0 = 0; J0 < j_end; J0 += 64) {
      const int Jl = J0 + lane;
      uint64_t wl = 0;
      if (Jl < j_end) {
        const uint8_t kind = tile_kind != nullptr ? tile_kind[mrow + Jl] : uint8_t(1);
        if (kind != 0)
          wl = (tile_bits != nullptr && kind != 1) ? tile_bits[(mrow + Jl) * kRowTile + (i % kRowTile)]
                                                   : ~uint64_t(0);
        if (int64_t(Jl) * kRowTile + kRowTile - 1 > last) {  // keys past the last visible one
          const int n = int(last - int64_t(Jl) * kRowTile) + 1;  // 1 .. 63 (Jl < j_end)
          wl &= (uint64_t(1) << n) - 1;
        }
      }
      uint64_t todo = __builtin_amdgcn_ballot_w64(wl != 0);
      while (todo != 0) {
        const int jl = __builtin_ctzll(todo);
        todo &= todo - 1;
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(wl), jl);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(wl >> 32), jl);
        const uint64_t word = (uint64_t(hi) << 32) | lo;
        const int k0 = (J0 + jl) * kRowTile;
        for (int kk = 0; kk < kRowTile; kk += KPI) {
          if (((word >> kk) & ((uint64_t(1) << KPI) - 1)) == 0) continue;  // no visible key in this group
          uint4 kr[U], vr[U];
          bool vis[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int t = kk + u * KPW + sub;
            vis[u] = (word >> t) & 1;
            const int64_t key = k0 + t;
            if (vis[u]) {
              kr[u] = nt_load(reinterpret_cast<const uint4*>(kb + key * D));
              vr[u] = nt_load(reinterpret_cast<const uint4*>(vb + key * D));
            } else {
              kr[u] = make_uint4(0, 0, 0, 0);
              vr[u] = make_uint4(0, 0, 0, 0);
            }
          }
          float ts[U];
          float bm = kNegInf;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float dsum = dot2_bf16r(kr[u].x, qv.x, 0.f);
            dsum = dot2_bf16r(kr[u].y, qv.y, dsum);
            dsum = dot2_bf16r(kr[u].z, qv.z, dsum);
            dsum = dot2_bf16r(kr[u].w, qv.w, dsum);
            dsum = group_sum<LPK>(dsum);
            ts[u] = vis[u] ? dsum * scale_log2 : kNegInf;
            bm = fmaxf(bm, ts[u]);
          }
          const float mn = fmaxf(m, bm);
          const float mu = (mn == kNegInf) ? 0.f : mn;
          const float alpha = fast_exp2(m - mu);
          l *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float p = fast_exp2(ts[u] - mu);
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
      }
    }
    // Merge the KPW key groups of the wave (lanes with equal ds).
#pragma unroll
    for (int sh = LPK; sh < 64; sh <<= 1) {
      const float m2 = shfl_xor(m, sh);
      const float l2 = shfl_xor(l, sh);
      const float M = fmaxf(m, m2);
      const float Mu = (M == kNegInf) ? 0.f : M;
      const float a = fast_exp2(m - Mu), b = fast_exp2(m2 - Mu);
      l = l * a + l2 * b;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + shfl_xor(acc[e], sh) * b;
      m = M;
    }
    const bool live = l > 0.f;
    const float inv = live ? 1.f / l : 0.f;
    if (sub == 0) {
      uint4 out;
      out.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      out.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      out.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
      out.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
      *reinterpret_cast<uint4*>(o + row * D + 8 * ds) = out;
      if (lse != nullptr && lane == 0) lse[row] = live ? (m + fast_log2(l)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_attention_rowwise(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int Lq, int Lk, int d, float scale, int causal, const uint8_t* tile_kind,
                                    const uint64_t* tile_bits, hipStream_t stream) {
  const int64_t n_rows = int64_t(B) * H * Lq;
  const int64_t blocks = (n_rows + 3) / 4;
  const unsigned grid = unsigned(blocks < (1 << 20) ? blocks : (1 << 20));
  const float scale_log2 = float(double(scale) * 1.4426950408889634);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(o);
  if (d == 128)
    hipLaunchKernelGGL((attention_rowwise_kernel<128, 4>), dim3(grid), dim3(256), 0, stream, qq, kk, vv, oo, lse, Lq,
                       Lk, scale_log2, causal, tile_kind, tile_bits, n_rows);
  else
    hipLaunchKernelGGL((attention_rowwise_kernel<64, 4>), dim3(grid), dim3(256), 0, stream, qq, kk, vv, oo, lse, Lq,
                       Lk, scale_log2, causal, tile_kind, tile_bits, n_rows);
  return hipGetLastError();
}

}  // namespace rf
