// fp32 attention forward with the online softmax (single-segment strategy,
// RedFuser page, 3. Contributions clés; online rescale as on the FLASHLIGHT
// page, Metodologia 3). Used for fp32 inputs with any head dim d <= 128.
//
// A workgroup of 256 lanes owns BM = 32 query rows of one (b, h) and sweeps
// the visible key tiles of BN = 32 keys. Lane (r, p) = (t / 8, t % 8) holds
// query row r: it scores keys p, p + 8, p + 16, p + 24 of the tile and
// accumulates output columns p, p + 8, ... of row r, so the running (m, l)
// of a row lives in the 8 lanes that share it. Masked key tiles are skipped
// before any load (STOF page, Énoncé du problème / Méthodologie 1: skip rather
// than compute and reset); only tiles that straddle the causal diagonal or
// the end of the keys are masked per element.
//
// This is a small-problem, fp32-exact path: scores and accumulators are fp32
// FMA chains; matrix cores are used by the bf16 path.
#include <stdint.h>

#include "rf_internal.h"

namespace rf {
namespace {

constexpr int kBM = 32, kBN = 32, kMaskTile = 64;

template <int DMAX>
__global__ __launch_bounds__(256) void attention_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, float* __restrict__ o,
                                                            float* __restrict__ lse, int H, int Lq, int Lk, int d,
                                                            float scale_log2, int causal,
                                                            const uint8_t* __restrict__ block_mask, int n_qt,
                                                            int64_t n_items) {
  constexpr int DP = DMAX + 1;  // padded row: lanes of one row hit distinct banks
  constexpr int NACC = DMAX / 8;
  __shared__ float Qs[kBM][DP];
  __shared__ float Ks[kBN][DP];
  __shared__ float Vs[kBN][DP];
  __shared__ float Ps[kBM][kBN + 1];

  const int t = threadIdx.x;
  const int r = t >> 3, p = t & 7;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int n_kt = (Lk + kBN - 1) / kBN;

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t bh = item / n_qt;
    const int qt = int(item % n_qt);
    const int q0 = qt * kBM;
    const float* qh = q + bh * int64_t(Lq) * d;
    const float* kh = k + bh * int64_t(Lk) * d;
    const float* vh = v + bh * int64_t(Lk) * d;

    __syncthreads();  // previous item's readers of Qs are done
    for (int i = t; i < kBM * DMAX; i += 256) {
      const int rr = i / DMAX, e = i % DMAX;
      Qs[rr][e] = (q0 + rr < Lq && e < d) ? qh[int64_t(q0 + rr) * d + e] : 0.f;
    }

    const int qi = q0 + r;  // this lane's query row
    float m = kNegInf, l = 0.f;
    float acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.f;

    // Last key any row of this tile may see under the causal rule.
    const int64_t causal_last = int64_t(min(q0 + kBM, Lq) - 1) + (Lk - Lq);
    for (int kt = 0; kt < n_kt; ++kt) {
      const int k0 = kt * kBN;
      if (causal && k0 > causal_last) break;  // every later tile is masked too
      if (block_mask != nullptr &&
          block_mask[int64_t(q0 / kMaskTile) * n_mask_cols + k0 / kMaskTile] == 0)
        continue;  // the whole tile is masked: skip it, no load
      __syncthreads();
      for (int i = t; i < kBN * DMAX; i += 256) {
        const int c = i / DMAX, e = i % DMAX;
        const bool in = (k0 + c < Lk) && e < d;
        Ks[c][e] = in ? kh[int64_t(k0 + c) * d + e] : 0.f;
        Vs[c][e] = in ? vh[int64_t(k0 + c) * d + e] : 0.f;
      }
      __syncthreads();

      float s[4];
      float bm = kNegInf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = p + 8 * j;
        float dot = 0.f;
        for (int e = 0; e < d; ++e) dot = fmaf(Qs[r][e], Ks[c][e], dot);
        const int kj = k0 + c;
        const bool vis = (kj < Lk) && (qi < Lq) && (!causal || int64_t(kj) <= int64_t(qi) + (Lk - Lq));
        s[j] = vis ? dot * scale_log2 : kNegInf;
        bm = fmaxf(bm, s[j]);
      }
      bm = group_max<8>(bm);
      const float mn = fmaxf(m, bm);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m - mu);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = fast_exp2(s[j] - mu);
        Ps[r][p + 8 * j] = pj;
        ps += pj;
      }
      ps = group_sum<8>(ps);
      l = l * alpha + ps;
      m = mn;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NACC; ++i) {
        const int e = p + 8 * i;
        float a = acc[i] * alpha;
        for (int c = 0; c < kBN; ++c) a = fmaf(Ps[r][c], Vs[c][e], a);
        acc[i] = a;
      }
    }

    if (qi < Lq) {
      const bool live = l > 0.f;
      const float inv = live ? 1.f / l : 0.f;
      float* orow = o + (bh * Lq + qi) * int64_t(d);
#pragma unroll
      for (int i = 0; i < NACC; ++i) {
        const int e = p + 8 * i;
        if (e < d) orow[e] = acc[i] * inv;
      }
      if (lse != nullptr && p == 0) lse[bh * Lq + qi] = live ? (m + fast_log2(l)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_attention_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                                int H, int Lq, int Lk, int d, float scale, int causal,
                                const uint8_t* block_mask, hipStream_t stream) {
  const int n_qt = (Lq + kBM - 1) / kBM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  const unsigned grid = unsigned(n_items < (1LL << 20) ? n_items : (1LL << 20));
  const float scale_log2 = float(double(scale) * 1.4426950408889634);
#define RF_ATT_F32(DM)                                                                                    \
  hipLaunchKernelGGL((attention_f32_kernel<DM>), dim3(grid), dim3(256), 0, stream, q, k, v, o, lse, H, Lq, \
                     Lk, d, scale_log2, causal, block_mask, n_qt, n_items)
  if (d <= 32)
    RF_ATT_F32(32);
  else if (d <= 64)
    RF_ATT_F32(64);
  else
    RF_ATT_F32(128);
#undef RF_ATT_F32
  return hipGetLastError();
}

}  // namespace rf
