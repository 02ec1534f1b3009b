// bf16 attention forward on gfx950 matrix cores, with the online softmax.
//
// What is computed (RedFuser page, 1. Problématique: safe softmax followed by
// a GEMM; FLASHLIGHT page, Metodologia 2–4: max() fused into QK^T and
// softmax(QK^T)V fused; STOF page, Méthodologie 1: block masks, masked tiles
// skipped): for every query row i,
//   O_i = sum_j P_ij V_j / sum_j P_ij,  P_ij = 2^(t_ij - m_i),
//   t_ij = scale * log2(e) * (q_i . k_j) over visible keys j,
// with the running max m_i and sum l_i rescaled by 2^(m_old - m_new) as each
// key tile arrives (single-segment strategy: one workgroup sweeps every
// visible key tile of its query tile; on-chip state is O(1) in Lk).
//
// Layout of the work (D = head dim, 64 or 128; NW waves of 32 query rows):
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K from LDS (row-major),
//     B = Q^T kept in registers for the whole sweep. In the 32x32 result each
//     lane holds ONE query row (column l % 32) and 16 keys, so the row max and
//     row sum are lane-local plus one exchange with lane l ^ 32, and the
//     running (m, l) and the output rescale need no cross-lane traffic.
//   - O^T += V^T P^T with the same instruction: B = P^T is exactly the S^T
//     accumulator rounded to bf16 (no data movement), because the order of
//     keys inside an MFMA K-step is free as long as A and B agree; V^T is
//     written to LDS transposed and key-permuted to match that order.
//   - K and V^T tiles of BN = 64 keys are double-buffered in LDS: the global
//     loads of tile n+1 are issued before the MFMAs of tile n, one barrier
//     per tile.
//   - Tiles above the causal diagonal or outside the block mask are never
//     loaded or computed; the element mask is applied only on tiles that
//     straddle the diagonal or the end of the keys.
//   - Work items (b, h, query tile) are laid out so that all query tiles of
//     a head run back to back on one XCD (its L2 serves the head's K/V to
//     every tile), heaviest causal tiles first.
#include <stdint.h>

#include "rf_internal.h"

namespace rf {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 64;        // keys per tile
constexpr int kMaskTile = 64;  // block-mask granularity

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Position of key kappa (0..15) inside a 16-key group of a V^T row: the MFMA
// K-slot that the S^T accumulator layout assigns to it (key quads 1 and 2 swap).
__device__ __forceinline__ int vt_quad_pos(int quad) { return ((quad & 1) << 1) | (quad >> 1); }

template <int D, int NW>
struct Smem {
  static constexpr int KROW = D + 8;      // padded K row (bf16): conflict-free 16-byte reads
  static constexpr int VROW = kBN + 8;    // padded V^T row (bf16)
  static constexpr int K_ELEMS = kBN * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * BUF_ELEMS * 2;
};

// Per-item description shared by all waves.
struct Item {
  int64_t bh;
  int q0;
};

template <int D, int NW>
__device__ __forceinline__ Item item_of(int64_t item, int n_qt, bool heavy_first) {
  Item it;
  it.bh = item / n_qt;
  const int r = int(item % n_qt);
  it.q0 = (heavy_first ? (n_qt - 1 - r) : r) * (32 * NW);
  return it;
}

// Is key tile kt visible to any of the workgroup's mask rows?
__device__ __forceinline__ bool tile_active(const uint8_t* __restrict__ mask, int n_mask_cols, int mr0, int mr1,
                                            int kt) {
  if (mask == nullptr) return true;
  const int mc = (kt * kBN) / kMaskTile;
  bool a = false;
  for (int mr = mr0; mr <= mr1; ++mr) a |= mask[int64_t(mr) * n_mask_cols + mc] != 0;
  return a;
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attention_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap) {
  using S = Smem<D, NW>;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KCH = D / 8;          // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;      // MFMA K-steps for S^T
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int K_LD = kBN * KCH / NT;  // K chunks per thread per tile
  constexpr int V_ITEMS = 16 * KCH;      // (key quad, d chunk) items per tile
  constexpr int V_LD = (V_ITEMS + NT - 1) / NT;
  static_assert(kBN * KCH % NT == 0, "K tile split");

  extern __shared__ __align__(16) uint16_t smem[];

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int off = Lk - Lq;  // bottom-right causal alignment: key j visible to row i iff j <= i + off
  const int n_kt = (Lk + kBN - 1) / kBN;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int64_t per_xcd = n_items / 8;

  for (int64_t g = blockIdx.x; g < n_items; g += gridDim.x) {
    // XCD-aware placement: consecutive workgroups land on consecutive XCDs, so
    // give each XCD a contiguous range of items (whole heads, tiles in order).
    const int64_t item = xcd_remap ? (g % 8) * per_xcd + g / 8 : g;
    const Item it = item_of<D, NW>(item, n_qt, causal != 0);
    const int q0 = it.q0;
    const int q0w = q0 + 32 * wave;
    const uint16_t* qh = q + it.bh * int64_t(Lq) * D;
    const uint16_t* kh = k + it.bh * int64_t(Lk) * D;
    const uint16_t* vh = v + it.bh * int64_t(Lk) * D;

    // Key tiles this workgroup may need: [0, kt_end), minus masked tiles.
    int64_t last_key = int64_t(min(q0 + BM, Lq) - 1) + (causal ? off : int64_t(Lk));
    if (last_key > Lk - 1) last_key = Lk - 1;
    const int kt_end = last_key < 0 ? 0 : int(last_key / kBN) + 1;
    const int mr0 = q0 / kMaskTile;
    const int mr1 = min(q0 + BM - 1, Lq - 1) / kMaskTile;
    const int mr_w = min(q0w, Lq - 1) / kMaskTile;
    auto next_tile = [&](int kt) {
      while (kt < kt_end && !tile_active(block_mask, n_mask_cols, mr0, mr1, kt)) ++kt;
      return kt;
    };

    // Q^T fragments (B operand of S^T): lane holds row q0w + l32, d = 16 ks + 8 h .. + 8.
    uint4 qf[KSTEPS];
    {
      const int qi = q0w + l32;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qi < Lq) x = *reinterpret_cast<const uint4*>(qh + int64_t(qi) * D + 16 * ks + 8 * h);
        if (q_mode == 1) { x.x ^= 0x80008000u; x.y ^= 0x80008000u; x.z ^= 0x80008000u; x.w ^= 0x80008000u; }
        if (q_mode == 2) x = make_uint4(0, 0, 0, 0);
        qf[ks] = x;
      }
    }

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_run = kNegInf;  // running max of this lane's query row (log2 units)
    float l_run = 0.f;      // this lane's share of the running sum (lane l ^ 32 holds the rest)

    // Global -> register staging of one K/V tile.
    uint4 kst[K_LD];
    uint4 vst[V_LD][4];
    auto load_tile = [&](int kt) {
      const int k0 = kt * kBN;
#pragma unroll
      for (int i = 0; i < K_LD; ++i) {
        const int idx = t + i * NT;
        const int row = idx / KCH, c = idx % KCH;
        kst[i] = (k0 + row < Lk) ? *reinterpret_cast<const uint4*>(kh + int64_t(k0 + row) * D + 8 * c)
                                 : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < V_LD; ++i) {
        const int idx = t + i * NT;
        if (idx < V_ITEMS) {
          const int quad = idx % 16, c = idx / 16;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * quad + j;
            vst[i][j] = (key < Lk) ? *reinterpret_cast<const uint4*>(vh + int64_t(key) * D + 8 * c)
                                   : make_uint4(0, 0, 0, 0);
          }
        }
      }
    };
    auto store_tile = [&](int buf) {
      uint16_t* ks_ = smem + buf * S::BUF_ELEMS;
      uint16_t* vs_ = ks_ + S::K_ELEMS;
#pragma unroll
      for (int i = 0; i < K_LD; ++i) {
        const int idx = t + i * NT;
        const int row = idx / KCH, c = idx % KCH;
        *reinterpret_cast<uint4*>(ks_ + row * S::KROW + 8 * c) = kst[i];
      }
#pragma unroll
      for (int i = 0; i < V_LD; ++i) {
        const int idx = t + i * NT;
        if (idx < V_ITEMS) {
          const int quad = idx % 16, c = idx / 16;
          const int pos = 16 * (quad >> 2) + 4 * vt_quad_pos(quad & 3);
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vst[i][0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vst[i][1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vst[i][2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vst[i][3]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint2 col;
            if (e & 1) {
              col.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
              col.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
            } else {
              col.x = (w0[w] & 0xffffu) | (w1[w] << 16);
              col.y = (w2[w] & 0xffffu) | (w3[w] << 16);
            }
            *reinterpret_cast<uint2*>(vs_ + (8 * c + e) * S::VROW + pos) = col;
          }
        }
      }
    };

    __syncthreads();  // the previous item's last readers of both buffers are done
    int kt = next_tile(0);
    int buf = 0;
    if (kt < kt_end) {
      load_tile(kt);
      store_tile(0);
    }
    __syncthreads();

    while (kt < kt_end) {
      const int kt_next = next_tile(kt + 1);
      if (kt_next < kt_end) load_tile(kt_next);  // in flight during this tile's math

      const int k0 = kt * kBN;
      const bool wave_visible =
          (!causal || int64_t(k0) <= int64_t(q0w) + 31 + off) && q0w < Lq &&
          (block_mask == nullptr || block_mask[int64_t(mr_w) * n_mask_cols + k0 / kMaskTile] != 0);
      if (wave_visible) {
        const uint16_t* ks_ = smem + buf * S::BUF_ELEMS;
        const uint16_t* vs_ = ks_ + S::K_ELEMS;
        // ---- S^T = K Q^T (two 32-key blocks) ----
        f32x16_t st[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) st[mb][r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4*>(ks_ + (32 * mb + l32) * S::KROW + 16 * ks + 8 * h);
            st[mb] = mfma32(as_bf16x8(a), as_bf16x8(qf[ks]), st[mb]);
          }
        }
        // ---- element mask, only where the tile straddles the diagonal or the key end ----
        const bool edge = (causal && int64_t(k0) + kBN - 1 > int64_t(q0w) + off) || (k0 + kBN > Lk);
        if (edge) {
          const int64_t lim = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
          const int64_t kmax = lim < Lk - 1 ? lim : int64_t(Lk) - 1;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
              if (key > kmax) st[mb][r] = kNegInf;
            }
        }
        // ---- online softmax update (log2 units) ----
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
        mx = fmaxf(mx, shfl_xor(mx, 32));  // lane l ^ 32 holds the other 32 keys of the row
        const float m_new = fmaxf(m_run, mx * c_log2);
        const float mu = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - mu);
        m_run = m_new;
        float psum = 0.f;
        uint32_t pk[2][8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(st[mb][r], c_log2, -mu));
            const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_log2, -mu));
            psum += p0 + p1;
            pk[mb][r >> 1] = cvt_pk_bf16(p0, p1);
          }
        l_run = l_run * alpha + psum;
        if (alpha != 1.f) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
        }
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int mb = ks >> 1, r0 = (ks & 1) * 4;
          const uint4 bp = make_uint4(pk[mb][r0], pk[mb][r0 + 1], pk[mb][r0 + 2], pk[mb][r0 + 3]);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint4 a = *reinterpret_cast<const uint4*>(vs_ + (32 * db + l32) * S::VROW + 16 * ks + 8 * h);
            acc_o[db] = mfma32(as_bf16x8(a), as_bf16x8(bp), acc_o[db]);
          }
        }
      }

      if (kt_next < kt_end) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      kt = kt_next;
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
    const float l_tot = l_run + shfl_xor(l_run, 32);
    const int qi = q0w + l32;
    if (qi < Lq) {
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_tot : 0.f;
      uint16_t* orow = o + (it.bh * Lq + qi) * int64_t(D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * db + 8 * r4 + 4 * h;
          uint2 pkt;
          pkt.x = cvt_pk_bf16(acc_o[db][4 * r4] * inv, acc_o[db][4 * r4 + 1] * inv);
          pkt.y = cvt_pk_bf16(acc_o[db][4 * r4 + 2] * inv, acc_o[db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d0) = pkt;
        }
      if (lse != nullptr && h == 0) lse[it.bh * Lq + qi] = live ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, int NW>
hipError_t launch_kernel(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                         int Lk, float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const int n_qt = (Lq + BM - 1) / BM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  int q_mode = 0;
  float c = float(double(scale) * 1.4426950408889634);
  if (scale < 0.f) {
    q_mode = 1;  // s * scale = ((-q) . k) * |scale|; negating bf16 is exact
    c = -c;
  } else if (scale == 0.f) {
    q_mode = 2;  // every score is exactly 0
    c = 1.f;
  }
  const int64_t cap = 1LL << 22;
  const unsigned grid = unsigned(n_items < cap ? n_items : cap);
  const int xcd_remap = (n_items % 8 == 0 && n_items <= cap) ? 1 : 0;
  const size_t shmem = Smem<D, NW>::BYTES;
  // One-time, thread-safe opt-in to more than 64 KiB of dynamic LDS for this instantiation.
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attention_bf16_kernel<D, NW>), hipFuncAttributeMaxDynamicSharedMemorySize,
      int(shmem));
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL((attention_bf16_kernel<D, NW>), dim3(grid), dim3(NW * 64), shmem, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                     block_mask, n_qt, n_items, xcd_remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Lq, int Lk, int d, float scale, int causal, const uint8_t* block_mask,
                                 hipStream_t stream) {
  if (d == 128) return launch_kernel<128, 4>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask, stream);
  return launch_kernel<64, 4>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask, stream);
}

}  // namespace rf
