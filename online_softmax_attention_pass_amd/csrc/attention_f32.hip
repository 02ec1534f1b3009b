// fp32 attention forward with the online softmax (single-segment strategy,
// RedFuser page, 3. Contributions clés; online rescale as on the FLASHLIGHT
// page, Metodologia 3). Used for fp32 inputs with any head dim d <= 128.
//
// A workgroup of 256 lanes owns BM = 16 query rows of one (b, h) and sweeps
// the visible key tiles of BN keys (64 for d <= 64, else 32). Lane
// (r, p) = (t / 16, t % 16) holds query row r: it scores keys p, p + 16, ...
// of the tile and accumulates the output columns
// [p * DMAX / 16, (p + 1) * DMAX / 16) of row r, so the running (m, l) of a
// row lives in the 16 lanes that share it. Masked key tiles are
// skipped before any load (STOF page, Énoncé du problème / Méthodologie 1:
// skip rather than compute and reset); only tiles that straddle the causal
// diagonal or the end of the keys are masked per element.
//
// This is a small-problem, fp32-exact path, shaped for latency: every dot
// product runs as four independent partial chains over 16-byte LDS reads
// (rows are zero-padded to DMAX so the loops have fixed trip counts), and P.V
// keeps one independent accumulator per output column. Matrix cores are used
// by the bf16 path.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

constexpr int kBM = 16, kMaskTile = 64;

template <int DMAX>
__global__ __launch_bounds__(256) void attention_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, float* __restrict__ o,
                                                            float* __restrict__ lse, int H, int Lq, int Lk, int d,
                                                            float scale_log2, int causal,
                                                            const uint8_t* __restrict__ block_mask,
                                                            const uint64_t* __restrict__ tile_bits, int n_qt,
                                                            int64_t n_items, int window,
                                                            const float* __restrict__ slopes, float softcap) {
  // Rows padded by 4 floats: 16-byte aligned, and the 16 key rows one
  // instruction reads start 4 banks apart.
  constexpr int DP = DMAX + 4;
  constexpr int NC = DMAX / 16;  // output columns per lane
  // Keys per step: 64 (one mask tile) while the tile's K and V fit the
  // register double buffer, so a short sequence takes half the dependent steps.
  constexpr int kBN = DMAX <= 64 ? 64 : 32;
  constexpr int NK = kBN / 16;  // keys scored per lane and step
  static_assert(DMAX % 16 == 0, "column split");
  static_assert(kMaskTile % kBN == 0, "a key tile lies in one mask tile");
  __shared__ __align__(16) float Qs[kBM][DP];
  __shared__ __align__(16) float Ks[kBN][DP];
  __shared__ __align__(16) float Vs[kBN][DP];
  __shared__ __align__(16) float Ps[kBM][kBN];

  const int t = threadIdx.x;
  const int r = t >> 4, p = t & 15;
  const int c0 = p * NC;  // first output column of this lane
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int n_kt = (Lk + kBN - 1) / kBN;

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t bh = item / n_qt;
    const int qt = int(item % n_qt);
    const int q0 = qt * kBM;
    const float* qh = q + bh * int64_t(Lq) * d;
    const float* kh = k + bh * int64_t(Lk) * d;
    const float* vh = v + bh * int64_t(Lk) * d;

    // Q of the tile's rows, in registers until the first barrier.
    float qreg[kBM * DMAX / 256];
#pragma unroll
    for (int j = 0; j < kBM * DMAX / 256; ++j) {
      const int i = t + 256 * j, rr = i / DMAX, e = i % DMAX;
      qreg[j] = (q0 + rr < Lq && e < d) ? qh[int64_t(q0 + rr) * d + e] : 0.f;
    }

    const int qi = q0 + r;  // this lane's query row
    // Score modifications: query position (bottom-right), the head's ALiBi
    // slope in log2 units, and the window's lowest key for this row.
    const int64_t qpos = int64_t(qi) + (Lk - Lq);
    const float sl2 = slopes != nullptr ? slopes[bh % H] * kLog2e : 0.f;
    const int64_t lo = window > 0 ? qpos - window + 1 : 0;
    const int64_t lo_first = int64_t(q0) + (Lk - Lq) - window + 1;  // lowest window key of the tile's rows
    float m = kNegInf, l = 0.f;
    float acc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] = 0.f;

    // Last key any row of this tile may see under the causal rule.
    const int64_t causal_last = int64_t(min(q0 + kBM, Lq) - 1) + (Lk - Lq);
    // Key tiles this workgroup visits, in order: not past the causal diagonal
    // of its last row, not wholly before every row's window, not masked out by
    // the block mask (skipped tiles are never loaded).
    auto visible = [&](int kt) {
      const int k0 = kt * kBN;
      if (window > 0 && int64_t(k0) + kBN - 1 < lo_first) return false;
      const int64_t tile = int64_t(q0 / kMaskTile) * n_mask_cols + k0 / kMaskTile;
      return block_mask == nullptr || block_mask[tile] != 0;
    };
    const int kt_stop = causal ? int(min(int64_t(n_kt), causal_last < 0 ? 0 : causal_last / kBN + 1)) : n_kt;
    auto next_tile = [&](int kt) {
      while (kt < kt_stop && !visible(kt)) ++kt;
      return kt;
    };
    // A tile's K, V (this thread's share) and this row's bitmap word, into
    // registers: the next tile's are issued before the current one is used.
    constexpr int PER = kBN * DMAX / 256;
    float kreg[PER], vreg[PER];
    uint64_t wreg = ~uint64_t(0);
    auto fetch = [&](int kt) {
      const int k0 = kt * kBN;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = t + 256 * j, c = i / DMAX, e = i % DMAX;
        const bool in = (k0 + c < Lk) && e < d;
        kreg[j] = in ? kh[int64_t(k0 + c) * d + e] : 0.f;
        vreg[j] = in ? vh[int64_t(k0 + c) * d + e] : 0.f;
      }
      const int64_t tile = int64_t(q0 / kMaskTile) * n_mask_cols + k0 / kMaskTile;
      const uint8_t kind = block_mask != nullptr ? block_mask[tile] : uint8_t(1);
      // A partial tile (kind other than 0 and 1, with bitmaps): bit (j mod 64)
      // of this row's word says whether key j is visible. The 16 rows of a
      // workgroup lie in one 64-row mask tile.
      wreg = ~uint64_t(0);
      if (tile_bits != nullptr && kind != 1 && qi < Lq) wreg = tile_bits[tile * kMaskTile + (qi % kMaskTile)];
    };
    int kt = next_tile(0);
    if (kt < kt_stop) fetch(kt);
    __syncthreads();  // previous item's readers of Qs are done
#pragma unroll
    for (int j = 0; j < kBM * DMAX / 256; ++j) {
      const int i = t + 256 * j;
      Qs[i / DMAX][i % DMAX] = qreg[j];
    }
    while (kt < kt_stop) {
      const int k0 = kt * kBN;
      const uint64_t word = wreg;
      __syncthreads();  // previous tile's readers of Ks, Vs are done
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = t + 256 * j;
        Ks[i / DMAX][i % DMAX] = kreg[j];
        Vs[i / DMAX][i % DMAX] = vreg[j];
      }
      __syncthreads();
      const int kt_next = next_tile(kt + 1);
      if (kt_next < kt_stop) fetch(kt_next);

      // Scores of keys p + 16 j: four partial sums each over 16-byte reads.
      float pk[NK][4];
#pragma unroll
      for (int j = 0; j < NK; ++j) pk[j][0] = pk[j][1] = pk[j][2] = pk[j][3] = 0.f;
#pragma unroll
      for (int e = 0; e < DMAX; e += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(&Qs[r][e]);
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          const float4 kv = *reinterpret_cast<const float4*>(&Ks[p + 16 * j][e]);
          pk[j][0] = fmaf(qv.x, kv.x, pk[j][0]);
          pk[j][1] = fmaf(qv.y, kv.y, pk[j][1]);
          pk[j][2] = fmaf(qv.z, kv.z, pk[j][2]);
          pk[j][3] = fmaf(qv.w, kv.w, pk[j][3]);
        }
      }
      float s[NK];
      float bm = kNegInf;
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int kj = k0 + p + 16 * j;
        const bool vis = (kj < Lk) && (qi < Lq) && (!causal || int64_t(kj) <= int64_t(qi) + (Lk - Lq)) &&
                         ((word >> (kj % kMaskTile)) & 1) && int64_t(kj) >= lo;
        // s = scale (q . k) in log2 units; the softcap cap tanh(s / cap) moves
        // to log2 units as (cap log2 e) tanh(t / (cap log2 e)); ALiBi adds
        // slope (j - p_i).
        float t2 = ((pk[j][0] + pk[j][1]) + (pk[j][2] + pk[j][3])) * scale_log2;
        if (softcap > 0.f) t2 = softcap * kLog2e * tanhf(t2 / (softcap * kLog2e));
        t2 = fmaf(sl2, float(int64_t(kj) - qpos), t2);
        s[j] = vis ? t2 : kNegInf;
        bm = fmaxf(bm, s[j]);
      }
      bm = group_max<16>(bm);
      const float mn = fmaxf(m, bm);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m - mu);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const float pj = fast_exp2(s[j] - mu);
        Ps[r][p + 16 * j] = pj;
        psum += pj;
      }
      l = l * alpha + group_sum<16>(psum);
      m = mn;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[i] *= alpha;
#pragma unroll 8
      for (int c = 0; c < kBN; ++c) {
        const float pc = Ps[r][c];
        if constexpr (NC % 4 == 0) {
#pragma unroll
          for (int i = 0; i < NC; i += 4) {
            const float4 vv = *reinterpret_cast<const float4*>(&Vs[c][c0 + i]);
            acc[i] = fmaf(pc, vv.x, acc[i]);
            acc[i + 1] = fmaf(pc, vv.y, acc[i + 1]);
            acc[i + 2] = fmaf(pc, vv.z, acc[i + 2]);
            acc[i + 3] = fmaf(pc, vv.w, acc[i + 3]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < NC; i += 2) {  // NC = 2: 8-byte aligned pairs
            const float2 vv = *reinterpret_cast<const float2*>(&Vs[c][c0 + i]);
            acc[i] = fmaf(pc, vv.x, acc[i]);
            acc[i + 1] = fmaf(pc, vv.y, acc[i + 1]);
          }
        }
      }
      kt = kt_next;
    }

    if (qi < Lq) {
      const bool live = l > 0.f;
      const float inv = live ? 1.f / l : 0.f;
      float* orow = o + (bh * Lq + qi) * int64_t(d);
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (c0 + i < d) orow[c0 + i] = acc[i] * inv;
      if (lse != nullptr && p == 0) lse[bh * Lq + qi] = live ? (m + fast_log2(l)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// Small problems (d <= 64, too few 16-row tiles to occupy the chip): one
// wavefront per query row. A workgroup's 4 waves are 4 consecutive rows of
// one (b, h) and share each 64-key tile of K and V through LDS. In the score
// step lane p takes key p of the tile (a d-long dot product against the
// row's q, read as a broadcast); the row max and sum are wave reductions; in
// the P.V step lane (g, c) accumulates output columns 4c .. 4c + 3 over key
// group g of the tile (64 / (d/4) keys per group), and the key groups are
// summed once, at the end. Per lane and tile this is about a quarter of the
// 16-row kernel's instructions, on four times as many workgroups: the
// single-head workload's 128 rows run as 32 workgroups instead of 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
  x = group_max<16>(x);
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return pair_max_halves(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16, 64);
  return pair_sum_halves(x);
}

constexpr int kRowsPerWg = 4;

template <int DMAX>
__global__ __launch_bounds__(256) void attention_f32_rows_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, int H, int Lq, int Lk, int d, float scale_log2, int causal,
    const uint8_t* __restrict__ block_mask, const uint64_t* __restrict__ tile_bits, int n_rt, int64_t n_items,
    int window, const float* __restrict__ slopes, float softcap) {
  constexpr int BN = 64;           // keys per tile: one mask tile
  constexpr int DP = DMAX + 4;     // padded LDS row: 16-byte aligned, rows 4 banks apart
  constexpr int CG = DMAX / 4;     // P.V column groups of 4
  constexpr int KG = 64 / CG;      // P.V key groups
  constexpr int KPG = BN / KG;     // keys per key group
  constexpr int PER = BN * DMAX / 256;  // K (and V) elements per thread and tile
  static_assert(DMAX == 32 || DMAX == 64, "row kernel widths");
  __shared__ __align__(16) float Ks[BN][DP];
  __shared__ __align__(16) float Vs[BN][DP];
  __shared__ __align__(16) float Qs[kRowsPerWg][DMAX];
  __shared__ __align__(16) float Ps[kRowsPerWg][BN];

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int cg = lane % CG, kg = lane / CG;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int n_kt = (Lk + BN - 1) / BN;

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t bh = item / n_rt;
    const int q0 = int(item % n_rt) * kRowsPerWg;
    const int qi = q0 + wave;  // this wave's query row
    const float* qh = q + bh * int64_t(Lq) * d;
    const float* kh = k + bh * int64_t(Lk) * d;
    const float* vh = v + bh * int64_t(Lk) * d;
    const int64_t qpos = int64_t(qi) + (Lk - Lq);
    const float sl2 = slopes != nullptr ? slopes[bh % H] * kLog2e : 0.f;
    const int64_t lo = window > 0 ? qpos - window + 1 : 0;
    const int64_t lo_first = int64_t(q0) + (Lk - Lq) - window + 1;
    const int64_t causal_last = int64_t(min(q0 + kRowsPerWg, Lq) - 1) + (Lk - Lq);
    const int kt_stop = causal ? int(min(int64_t(n_kt), causal_last < 0 ? 0 : causal_last / BN + 1)) : n_kt;
    auto visible = [&](int kt) {
      const int k0 = kt * BN;
      if (window > 0 && int64_t(k0) + BN - 1 < lo_first) return false;
      return block_mask == nullptr || block_mask[int64_t(q0 / kMaskTile) * n_mask_cols + kt] != 0;
    };
    auto next_tile = [&](int kt) {
      while (kt < kt_stop && !visible(kt)) ++kt;
      return kt;
    };
    float kreg[PER], vreg[PER];
    uint64_t wreg = ~uint64_t(0);
    auto fetch = [&](int kt) {
      const int k0 = kt * BN;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = t + 256 * j, c = i / DMAX, e = i % DMAX;
        const bool in = (k0 + c < Lk) && e < d;
        kreg[j] = in ? kh[int64_t(k0 + c) * d + e] : 0.f;
        vreg[j] = in ? vh[int64_t(k0 + c) * d + e] : 0.f;
      }
      const int64_t tile = int64_t(q0 / kMaskTile) * n_mask_cols + kt;
      const uint8_t kind = block_mask != nullptr ? block_mask[tile] : uint8_t(1);
      wreg = ~uint64_t(0);
      if (tile_bits != nullptr && kind != 1 && qi < Lq) wreg = tile_bits[tile * kMaskTile + (qi % kMaskTile)];
    };

    // q of this wave's row, zero past d and for rows past Lq
    const float qv = (lane < DMAX && lane < d && qi < Lq) ? qh[int64_t(qi) * d + lane] : 0.f;
    int kt = next_tile(0);
    if (kt < kt_stop) fetch(kt);
    __syncthreads();  // the previous item's readers of Qs are done
    if (lane < DMAX) Qs[wave][lane] = qv;

    float m = kNegInf, l = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    while (kt < kt_stop) {
      const int k0 = kt * BN;
      const uint64_t word = wreg;
      __syncthreads();  // the previous tile's readers of Ks, Vs are done
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = t + 256 * j;
        Ks[i / DMAX][i % DMAX] = kreg[j];
        Vs[i / DMAX][i % DMAX] = vreg[j];
      }
      __syncthreads();
      const int kt_next = next_tile(kt + 1);
      if (kt_next < kt_stop) fetch(kt_next);

      // score of key k0 + lane: four partial sums over 16-byte reads
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < DMAX; e += 4) {
        const float4 qq = *reinterpret_cast<const float4*>(&Qs[wave][e]);
        const float4 kk = *reinterpret_cast<const float4*>(&Ks[lane][e]);
        ps[0] = fmaf(qq.x, kk.x, ps[0]);
        ps[1] = fmaf(qq.y, kk.y, ps[1]);
        ps[2] = fmaf(qq.z, kk.z, ps[2]);
        ps[3] = fmaf(qq.w, kk.w, ps[3]);
      }
      const int kj = k0 + lane;
      const bool vis = (kj < Lk) && (qi < Lq) && (!causal || int64_t(kj) <= qpos) && ((word >> lane) & 1) &&
                       int64_t(kj) >= lo;
      float t2 = ((ps[0] + ps[1]) + (ps[2] + ps[3])) * scale_log2;
      if (softcap > 0.f) t2 = softcap * kLog2e * tanhf(t2 / (softcap * kLog2e));
      t2 = fmaf(sl2, float(int64_t(kj) - qpos), t2);
      const float sc = vis ? t2 : kNegInf;
      const float mn = fmaxf(m, wave_max(sc));
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m - mu);
      const float pj = fast_exp2(sc - mu);
      l = l * alpha + wave_sum(pj);
      m = mn;
      Ps[wave][lane] = pj;  // read back by this wave only (LDS operations of a wave stay in order)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
#pragma unroll
      for (int i = 0; i < KPG; i += 4) {
        const float4 pp = *reinterpret_cast<const float4*>(&Ps[wave][kg * KPG + i]);
        const float pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 vv = *reinterpret_cast<const float4*>(&Vs[kg * KPG + i + u][4 * cg]);
          acc[0] = fmaf(pv[u], vv.x, acc[0]);
          acc[1] = fmaf(pv[u], vv.y, acc[1]);
          acc[2] = fmaf(pv[u], vv.z, acc[2]);
          acc[3] = fmaf(pv[u], vv.w, acc[3]);
        }
      }
      kt = kt_next;
    }
    // sum the key groups (lanes cg, cg + CG, ...)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
    if (qi < Lq) {
      const bool live = l > 0.f;
      const float inv = live ? 1.f / l : 0.f;
      float* orow = o + (bh * Lq + qi) * int64_t(d);
      if (kg == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * cg + i < d) orow[4 * cg + i] = acc[i] * inv;
      }
      if (lse != nullptr && lane == 0) lse[bh * Lq + qi] = live ? (m + fast_log2(l)) * kLn2 : kNegInf;
    }
  }
}

// The row kernel takes a call when d <= 64 and the 16-row kernel would have
// fewer workgroups than this (two per CU): there, latency, not throughput,
// sets the time.
constexpr int64_t kRowKernelBelow = 512;

}  // namespace

hipError_t launch_attention_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                                int H, int Lq, int Lk, int d, float scale, int causal,
                                const uint8_t* block_mask, const uint64_t* tile_bits, hipStream_t stream,
                                int window, const float* alibi_slopes, float softcap) {
  const int n_qt = (Lq + kBM - 1) / kBM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  const unsigned grid = unsigned(n_items < (1LL << 20) ? n_items : (1LL << 20));
  const float scale_log2 = float(double(scale) * 1.4426950408889634);
  if (d <= 64 && n_items < kRowKernelBelow) {
    const int n_rt = (Lq + kRowsPerWg - 1) / kRowsPerWg;
    const int64_t n_row_items = int64_t(B) * H * n_rt;
    const unsigned rgrid = unsigned(n_row_items < (1LL << 20) ? n_row_items : (1LL << 20));
    if (d <= 32)
      hipLaunchKernelGGL((attention_f32_rows_kernel<32>), dim3(rgrid), dim3(256), 0, stream, q, k, v, o, lse, H, Lq,
                         Lk, d, scale_log2, causal, block_mask, tile_bits, n_rt, n_row_items, window, alibi_slopes,
                         softcap);
    else
      hipLaunchKernelGGL((attention_f32_rows_kernel<64>), dim3(rgrid), dim3(256), 0, stream, q, k, v, o, lse, H, Lq,
                         Lk, d, scale_log2, causal, block_mask, tile_bits, n_rt, n_row_items, window, alibi_slopes,
                         softcap);
    return hipGetLastError();
  }
#define RF_ATT_F32(DM)                                                                                    \
  hipLaunchKernelGGL((attention_f32_kernel<DM>), dim3(grid), dim3(256), 0, stream, q, k, v, o, lse, H, Lq, \
                     Lk, d, scale_log2, causal, block_mask, tile_bits, n_qt, n_items, window, alibi_slopes, \
                     softcap)
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
