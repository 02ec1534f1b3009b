// Mixture-of-experts routing: per token, the softmax over its E expert logits
// and its k largest probabilities (RedFuser page, 1. Problématique: MoE routing
// is a cascaded reduction, max -> sum of exp -> normalise -> selection).
//
// One group of G lanes owns a token (G = 1 .. 64, a power of two, the fewest
// lanes that hold E logits at up to 16 per lane); lane g holds the logits of
// experts g, g + G, ... in registers, so each logit is read once.
// The group reduces (max, then sum of exp) and then takes k selection rounds:
// the largest remaining logit, and among equal ones the lowest expert index
// (the softmax is monotone, so this is the order of the probabilities). Weights are the probabilities of the chosen experts,
// optionally renormalised over them. All group exchanges are DPP / swizzle /
// permlane moves; every lane of a group ends each reduction with the same bits.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

constexpr int kMaxTopK = 32;

template <int CTRL>
__device__ __forceinline__ int dpp_int(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int swz16_int(int x) { return __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 0x1F); }
__device__ __forceinline__ float swz16(float x) { return __int_as_float(swz16_int(__float_as_int(x))); }

// Group partner values, level by level: xor 1, xor 2 (quad_perm), half-row
// mirror (lane i of 8 <- 7 - i), row mirror (i of 16 <- 15 - i), xor 16
// (swizzle), and the other half of the wavefront (permlane32 swap). After the
// levels below a group size, every lane of each sub-group holds the same
// value, so a mirror partner carries the other sub-group's result.
template <int LEVEL>
__device__ __forceinline__ float partner(float x) {
  if constexpr (LEVEL == 0) return dpp_mov<0xB1>(x);
  if constexpr (LEVEL == 1) return dpp_mov<0x4E>(x);
  if constexpr (LEVEL == 2) return dpp_mov<0x141>(x);
  if constexpr (LEVEL == 3) return dpp_mov<0x140>(x);
  if constexpr (LEVEL == 4) return swz16(x);
  if constexpr (LEVEL == 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
  return x;
}
template <int LEVEL>
__device__ __forceinline__ int partner_int(int x) {
  if constexpr (LEVEL == 0) return dpp_int<0xB1>(x);
  if constexpr (LEVEL == 1) return dpp_int<0x4E>(x);
  if constexpr (LEVEL == 2) return dpp_int<0x141>(x);
  if constexpr (LEVEL == 3) return dpp_int<0x140>(x);
  if constexpr (LEVEL == 4) return swz16_int(x);
  if constexpr (LEVEL == 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(uint32_t(x), uint32_t(x), false, false);
    return int((threadIdx.x & 32) ? r[0] : r[1]);
  }
  return x;
}

template <int G>
__device__ __forceinline__ float group_max_all(float x) {
  constexpr int LV = __builtin_ctz(G);
  if constexpr (LV > 0) x = fmaxf(x, partner<0>(x));
  if constexpr (LV > 1) x = fmaxf(x, partner<1>(x));
  if constexpr (LV > 2) x = fmaxf(x, partner<2>(x));
  if constexpr (LV > 3) x = fmaxf(x, partner<3>(x));
  if constexpr (LV > 4) x = fmaxf(x, partner<4>(x));
  if constexpr (LV > 5) x = fmaxf(x, partner<5>(x));
  return x;
}
// a + b is commutative in IEEE arithmetic, so both partners get the same bits.
template <int G>
__device__ __forceinline__ float group_sum_all(float x) {
  constexpr int LV = __builtin_ctz(G);
  if constexpr (LV > 0) x = x + partner<0>(x);
  if constexpr (LV > 1) x = x + partner<1>(x);
  if constexpr (LV > 2) x = x + partner<2>(x);
  if constexpr (LV > 3) x = x + partner<3>(x);
  if constexpr (LV > 4) x = x + partner<4>(x);
  if constexpr (LV > 5) x = x + partner<5>(x);
  return x;
}

// A logit's bits mapped so that unsigned order is float order (-0 and +0 map
// alike: v + 0 turns -0 into +0). No logit maps to 0, so 0 marks a retired
// or absent candidate.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t u = __float_as_uint(v + 0.f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t h) {
  return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}
template <int G>
__device__ __forceinline__ uint32_t group_umax(uint32_t a) {
  constexpr int LV = __builtin_ctz(G);
  if constexpr (LV > 0) a = max(a, uint32_t(partner_int<0>(int(a))));
  if constexpr (LV > 1) a = max(a, uint32_t(partner_int<1>(int(a))));
  if constexpr (LV > 2) a = max(a, uint32_t(partner_int<2>(int(a))));
  if constexpr (LV > 3) a = max(a, uint32_t(partner_int<3>(int(a))));
  if constexpr (LV > 4) a = max(a, uint32_t(partner_int<4>(int(a))));
  if constexpr (LV > 5) a = max(a, uint32_t(partner_int<5>(int(a))));
  return a;
}
template <int G>
__device__ __forceinline__ uint32_t group_umin(uint32_t a) {
  constexpr int LV = __builtin_ctz(G);
  if constexpr (LV > 0) a = min(a, uint32_t(partner_int<0>(int(a))));
  if constexpr (LV > 1) a = min(a, uint32_t(partner_int<1>(int(a))));
  if constexpr (LV > 2) a = min(a, uint32_t(partner_int<2>(int(a))));
  if constexpr (LV > 3) a = min(a, uint32_t(partner_int<3>(int(a))));
  if constexpr (LV > 4) a = min(a, uint32_t(partner_int<4>(int(a))));
  if constexpr (LV > 5) a = min(a, uint32_t(partner_int<5>(int(a))));
  return a;
}

template <typename T>
__device__ __forceinline__ float load_logit(const T* p);
template <>
__device__ __forceinline__ float load_logit<float>(const float* p) {
  return __builtin_nontemporal_load(p);
}
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(__builtin_nontemporal_load(p));
}

// G lanes per token, EPL logits per lane (E <= G * EPL), 256 threads per block.
template <typename T, int G, int EPL>
__global__ __launch_bounds__(256) void moe_route_kernel(const T* __restrict__ logits, int32_t* __restrict__ idx_out,
                                                        float* __restrict__ w_out, int64_t T_, int E, int k,
                                                        int renorm) {
  constexpr int TPB = 256 / G;  // tokens per block
  constexpr int KCAP = kMaxTopK < G * EPL ? kMaxTopK : G * EPL;
  constexpr int SLOTS = (KCAP + G - 1) / G;  // ranks kept per lane
  const int g = threadIdx.x % G;
  for (int64_t t0 = int64_t(blockIdx.x) * TPB; t0 < T_; t0 += int64_t(gridDim.x) * TPB) {
    const int64_t t = t0 + threadIdx.x / G;
    const bool live = t < T_;                   // uniform within a group
    const T* row = logits + (live ? t : 0) * int64_t(E);
    float x[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = g + G * j;
      x[j] = (live && e < E) ? load_logit(row + e) : kNegInf;
    }
    // softmax statistics of the token
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, x[j]);
    m = group_max_all<G>(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += fast_exp2((x[j] - m) * kLog2e);
    const float inv_l = 1.f / group_sum_all<G>(s);
    // k selection rounds. Each round takes the largest remaining logit (group
    // max of the ordered bits), then the lowest expert holding it (group min),
    // and retires that expert.
    uint32_t hk[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) hk[j] = (g + G * j < E) ? ordered_bits(x[j]) : 0u;
    float p_slot[SLOTS];
    int e_slot[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      p_slot[i] = 0.f;
      e_slot[i] = 0;
    }
    float psum = 0.f;
    for (int r = 0; r < k; ++r) {
      uint32_t mx = hk[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) mx = max(mx, hk[j]);
      mx = group_umax<G>(mx);
      uint32_t ei = 0xFFFFFFFFu;
#pragma unroll
      for (int j = EPL - 1; j >= 0; --j) ei = hk[j] == mx ? uint32_t(g + G * j) : ei;
      ei = group_umin<G>(ei);
#pragma unroll
      for (int j = 0; j < EPL; ++j) hk[j] = uint32_t(g + G * j) == ei ? 0u : hk[j];
      const int be = int(ei);
      const float p = fast_exp2((from_ordered_bits(mx) - m) * kLog2e) * inv_l;
      psum += p;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        const bool mine = r == g + G * i;
        p_slot[i] = mine ? p : p_slot[i];
        e_slot[i] = mine ? be : e_slot[i];
      }
    }
    const float scale = renorm ? 1.f / psum : 1.f;
    if (live) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        const int r = g + G * i;
        if (r < k) {
          idx_out[t * k + r] = e_slot[i];
          w_out[t * k + r] = p_slot[i] * scale;
        }
      }
    }
  }
}

// The same routing for 128 < E <= 256 (16 lanes per token, 16 logits per
// lane) and k <= 16, with two changes that cut the vector work of the
// selection by about half:
//   - a lane reads its logits as 16-byte vectors: lane g holds the VE
//     consecutive experts VE g .. VE g + VE - 1 of each 16 VE-expert block,
//     so e(j) = (j / VE) 16 VE + VE g + j % VE, still increasing in j;
//   - each lane sorts its own C best logits once (value, then lower expert
//     first). A round then compares only the lanes' heads: the group maximum
//     of the heads, the lowest expert holding it, and the winning lane moves
//     to its next entry. A lane whose list runs out while it still holds
//     logits not in it rebuilds the list from those (rare: it needs more than
//     C of the token's k largest). The rounds use selects, not branches, so
//     the lanes of a wave stay on one path. With C = 4 the routing of 256
//     experts ran about 8% faster than the rescanning rounds above; with
//     C = 3 the rebuilds cost more than the shorter lists saved.
// The choice is the same as the rounds above: the largest remaining logit,
// and among equal ones the lowest expert index.
template <typename T, int C>
__global__ __launch_bounds__(256) void moe_route_heads_kernel(const T* __restrict__ logits,
                                                              int32_t* __restrict__ idx_out,
                                                              float* __restrict__ w_out, int64_t T_, int E, int k,
                                                              int renorm) {
  constexpr int G = 16, EPL = 16, TPB = 256 / G;
  constexpr int VE = 16 / int(sizeof(T));  // experts per 16-byte vector
  constexpr int NV = EPL / VE;             // vectors per lane
  const int g = threadIdx.x % G;
  auto expert = [&](int j) { return (j / VE) * (16 * VE) + VE * g + j % VE; };
  for (int64_t t0 = int64_t(blockIdx.x) * TPB; t0 < T_; t0 += int64_t(gridDim.x) * TPB) {
    const int64_t t = t0 + threadIdx.x / G;
    const bool live = t < T_;                   // uniform within a group
    const T* row = logits + (live ? t : 0) * int64_t(E);
    uint4 raw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      // E is a multiple of VE, so a vector lies wholly inside the row or wholly
      // past it; one past it reads the row's first vector and is set aside.
      const int e0 = v * 16 * VE + VE * g;
      raw[v] = nt_load(reinterpret_cast<const uint4*>(row + (e0 < E ? e0 : 0)));
    }
    float x[EPL];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e0 = v * 16 * VE + VE * g;
      const bool in = live && e0 < E;
      const uint32_t wd[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
      for (int c = 0; c < VE; ++c) {
        float f;
        if constexpr (sizeof(T) == 4) f = __uint_as_float(wd[c]);
        else f = (c & 1) ? bf16_hi(wd[c / 2]) : bf16_lo(wd[c / 2]);
        x[v * VE + c] = in ? f : kNegInf;
      }
    }
    // softmax statistics of the token
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, x[j]);
    m = group_max_all<G>(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += fast_exp2((x[j] - m) * kLog2e);
    const float inv_l = 1.f / group_sum_all<G>(s);

    uint32_t hk[EPL];  // ordered bits; 0 = absent
#pragma unroll
    for (int j = 0; j < EPL; ++j) hk[j] = (live && expert(j) < E) ? ordered_bits(x[j]) : 0u;
    // This lane's C best (value descending, equal values in slot order), over
    // the slots not yet taken; n = how many of them it holds, more = whether
    // it holds further logits beyond them.
    uint32_t hv[C];
    int hj[C];
    int n = 0;
    bool more = false;
    uint32_t taken = 0;
    auto build = [&]() {
#pragma unroll
      for (int i = 0; i < C; ++i) {
        hv[i] = 0u;
        hj[i] = 0;
      }
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const uint32_t v = ((taken >> j) & 1u) ? 0u : hk[j];
        cnt += v != 0u;
        // insert after every entry it does not exceed
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
          const bool gt = v > hv[i];
          const bool gt_prev = i == 0 ? true : v > hv[i - 1];
          if (i > 0) {
            hv[i] = gt_prev ? hv[i - 1] : (gt ? v : hv[i]);
            hj[i] = gt_prev ? hj[i - 1] : (gt ? j : hj[i]);
          } else {
            hv[0] = gt ? v : hv[0];
            hj[0] = gt ? j : hj[0];
          }
        }
      }
      n = cnt < C ? cnt : C;
      more = cnt > C;
    };
    build();
    float p_mine = 0.f;
    int e_mine = 0;
    float psum = 0.f;
    for (int r = 0; r < k; ++r) {
      // selects only (no branch per lane): every lane computes every value
      const uint32_t mx = group_umax<G>(hv[0]);
      const uint32_t eh = uint32_t(expert(hj[0]));
      const bool top = n > 0 && hv[0] == mx;
      const uint32_t ei = group_umin<G>(top ? eh : 0xFFFFFFFFu);
      const bool win = top && eh == ei;
      const float p = fast_exp2((from_ordered_bits(mx) - m) * kLog2e) * inv_l;
      psum += p;
      p_mine = g == r ? p : p_mine;
      e_mine = g == r ? int(ei) : e_mine;
      taken |= win ? 1u << hj[0] : 0u;
#pragma unroll
      for (int i = 0; i + 1 < C; ++i) {
        hv[i] = win ? hv[i + 1] : hv[i];
        hj[i] = win ? hj[i + 1] : hj[i];
      }
      hv[C - 1] = win ? 0u : hv[C - 1];
      n -= win ? 1 : 0;
      const bool refill = win && n == 0 && more;
      if (__builtin_amdgcn_ballot_w64(refill)) {
        if (refill) build();
      }
    }
    const float scale = renorm ? 1.f / psum : 1.f;
    if (live && g < k) {
      idx_out[t * k + g] = e_mine;
      w_out[t * k + g] = p_mine * scale;
    }
  }
}

template <typename T, int G, int EPL>
hipError_t launch(const T* x, int32_t* idx, float* w, int64_t T_, int E, int k, int renorm, hipStream_t stream) {
  constexpr int TPB = 256 / G;
  const int64_t blocks = (T_ + TPB - 1) / TPB;
  const unsigned grid = unsigned(blocks < (1 << 20) ? blocks : (1 << 20));
  hipLaunchKernelGGL((moe_route_kernel<T, G, EPL>), dim3(grid), dim3(256), 0, stream, x, idx, w, T_, E, k, renorm);
  return hipGetLastError();
}

// Lanes per token: each lane holds up to 16 logits, so a token takes the fewest
// lanes (and cross-lane levels per selection round) that hold its E logits.
template <typename T>
hipError_t dispatch(const T* x, int32_t* idx, float* w, int64_t T_, int E, int k, int renorm, hipStream_t stream) {
  constexpr int VE = 16 / int(sizeof(T));
  if (E > 128 && E <= 256 && E % VE == 0 && k <= 16 && reinterpret_cast<uintptr_t>(x) % 16 == 0) {
    constexpr int TPB = 256 / 16;
    const int64_t blocks = (T_ + TPB - 1) / TPB;
    const unsigned grid = unsigned(blocks < (1 << 20) ? blocks : (1 << 20));
    hipLaunchKernelGGL((moe_route_heads_kernel<T, 4>), dim3(grid), dim3(256), 0, stream, x, idx, w, T_, E, k, renorm);
    return hipGetLastError();
  }
  if (E <= 1) return launch<T, 1, 1>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 2) return launch<T, 1, 2>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 4) return launch<T, 1, 4>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 8) return launch<T, 1, 8>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 16) return launch<T, 1, 16>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 32) return launch<T, 2, 16>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 64) return launch<T, 4, 16>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 128) return launch<T, 8, 16>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 256) return launch<T, 16, 16>(x, idx, w, T_, E, k, renorm, stream);
  if (E <= 512) return launch<T, 32, 16>(x, idx, w, T_, E, k, renorm, stream);
  return launch<T, 64, 16>(x, idx, w, T_, E, k, renorm, stream);
}

}  // namespace

hipError_t launch_moe_route(const void* logits, int32_t* idx, float* w, int64_t T_, int E, int k, int renorm,
                            int dtype, hipStream_t stream) {
  if (dtype == 0) return dispatch(static_cast<const float*>(logits), idx, w, T_, E, k, renorm, stream);
  return dispatch(static_cast<const uint16_t*>(logits), idx, w, T_, E, k, renorm, stream);
}

}  // namespace rf
