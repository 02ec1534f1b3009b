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

// Launch shape per head dim: waves per workgroup (32 query rows each) and
// waves per SIMD the register allocation must allow.
#ifndef RF_ATT_NW_D128
#define RF_ATT_NW_D128 4
#endif
#ifndef RF_ATT_WPE_D128
#define RF_ATT_WPE_D128 2
#endif
#ifndef RF_ATT_NW_D64
#define RF_ATT_NW_D64 2
#endif
#ifndef RF_ATT_WPE_D64
#define RF_ATT_WPE_D64 2
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// Raw buffer access: loads outside [0, bytes) return zero, so ragged tiles
// need no predication.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte rows supplied by lanes i/4,
// i/4 + 4, i/4 + 8, i/4 + 12 of its group.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(uint2, v);
}

template <int D>
struct Smem {
  static constexpr int KROW = D + 8;      // K row stride (bf16): 16-byte pad, conflict-free b128 reads
  // V row stride (bf16): the pad shifts consecutive rows so the 4-row transposed reads
  // of a lane group hit distinct banks (64 bytes for D = 128; 32 bytes for D = 64, which
  // keeps four 2-wave workgroups within the 160 KiB of LDS).
  static constexpr int VROW = D + (D >= 128 ? 32 : 16);
  static constexpr int K_ELEMS = kBN * KROW;
  static constexpr int V_ELEMS = kBN * VROW;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * BUF_ELEMS * 2;
};

// Is key tile kt visible to any of the workgroup's mask rows?
__device__ __forceinline__ bool tile_active(const uint8_t* __restrict__ mask, int n_mask_cols, int mr0, int mr1,
                                            int kt) {
  if (mask == nullptr) return true;
  const int mc = (kt * kBN) / kMaskTile;
  bool a = false;
  for (int mr = mr0; mr <= mr1; ++mr) a |= mask[int64_t(mr) * n_mask_cols + mc] != 0;
  return a;
}

template <int D, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attention_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap) {
  using S = Smem<D>;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KCH = D / 8;            // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;        // MFMA K-steps for S^T
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int LD = kBN * KCH / NT;    // chunks per thread per tile, for K and for V
  static_assert(kBN * KCH % NT == 0, "tile split");

  extern __shared__ __align__(16) uint16_t smem[];

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t off = int64_t(Lk) - Lq;  // bottom-right causal alignment: key j visible to row i iff j <= i + off
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int64_t per_xcd = n_items / 8;
  const uint32_t head_bytes = uint32_t(Lk) * D * 2;

  // Per-thread parts of the tile addressing (constant over the sweep).
  uint32_t ld_goff[LD];
  int ld_soff[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int idx = t + i * NT;
    const int row = idx / KCH, c = idx % KCH;
    ld_goff[i] = uint32_t(row * D * 2 + 16 * c);
    ld_soff[i] = row * S::KROW + 8 * c;  // K offset; V uses row * VROW + 8 c
  }
  // Transposed V^T fragment addressing (see lds_read_tr16): this lane supplies
  // row 4 h + (lane % 16) / 4 (+ 8 for the second half) and column
  // 16 ((lane / 16) % 2) + 4 (lane % 4) of each 16-key, 32-column block.
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int64_t g = blockIdx.x; g < n_items; g += gridDim.x) {
    // XCD-aware placement: consecutive workgroups land on consecutive XCDs, so
    // give each XCD a contiguous range of items (whole heads, tiles in order).
    const int64_t item = xcd_remap ? (g % 8) * per_xcd + g / 8 : g;
    const int64_t bh = item / n_qt;
    const int qr = int(item % n_qt);
    const int q0 = (causal ? (n_qt - 1 - qr) : qr) * BM;  // heaviest causal tiles first
    const int q0w = q0 + 32 * wave;
    const uint16_t* qh = q + bh * int64_t(Lq) * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + bh * int64_t(Lk) * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + bh * int64_t(Lk) * D, head_bytes);

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
    float m_ref = kNegInf;  // running max of this lane's query row (log2 units)
    float l_run = 0.f;      // this lane's share of the running sum (lane l ^ 32 holds the rest)
    // Last visible key of this lane's row, relative to tile start k0 and to the
    // lane's key offset 4 h (the register pattern adds 32 mb + 8 (r/4) + r%4).
    const int64_t row_last = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
    const int row_lim = int(row_last < int64_t(Lk) - 1 ? (row_last < -1 ? -1 : row_last) : int64_t(Lk) - 1);

    uint4 kst[LD], vst[LD];
    auto load_tile = [&](int kt) {
      const uint32_t base = uint32_t(kt) * kBN * D * 2;
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        kst[i] = buf_load16(krs, base + ld_goff[i]);
        vst[i] = buf_load16(vrs, base + ld_goff[i]);
      }
    };
    auto store_tile = [&](int buf) {
      uint16_t* ks_ = smem + buf * S::BUF_ELEMS;
      uint16_t* vs_ = ks_ + S::K_ELEMS;
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        const int idx = t + i * NT;
        const int row = idx / KCH, c = idx % KCH;
        *reinterpret_cast<uint4*>(ks_ + ld_soff[i]) = kst[i];
        *reinterpret_cast<uint4*>(vs_ + row * S::VROW + 8 * c) = vst[i];
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
          const int lim = row_lim - k0 - 4 * h;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * mb + 8 * (r >> 2) + (r & 3) > lim) st[mb][r] = kNegInf;
        }
        // ---- online softmax update (log2 units) ----
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
        mx = pair_max_halves(mx);  // lane l ^ 32 holds the other 32 keys of the row
        // The reference is the exact running max, so the row's largest weight is
        // exactly 1 and carries no bf16 rounding into O. The accumulator is
        // rescaled only on tiles where some row's max moved (wave-uniform branch).
        const float mt = mx * c_log2;
        const bool move = mt > m_ref;
        if (__builtin_amdgcn_ballot_w64(move)) {
          const float alpha = move ? fast_exp2(m_ref - mt) : 1.f;
          if (move) m_ref = mt;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
        }
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        uint32_t pk[2][8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(st[mb][r], c_log2, -mu));
            const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_log2, -mu));
            l_run += p0 + p1;
            pk[mb][r >> 1] = cvt_pk_bf16(p0, p1);
          }
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int mb = ks >> 1, r0 = (ks & 1) * 4;
          const uint4 bp = make_uint4(pk[mb][r0], pk[mb][r0 + 1], pk[mb][r0 + 2], pk[mb][r0 + 3]);
          const uint16_t* vrow = vs_ + (16 * ks + tr_row) * S::VROW + tr_col;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint2 lo = lds_read_tr16(vrow + 32 * db);
            const uint2 hi = lds_read_tr16(vrow + 8 * S::VROW + 32 * db);
            acc_o[db] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(bp), acc_o[db]);
          }
        }
      }

      if (kt_next < kt_end) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      kt = kt_next;
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
    const float l_tot = pair_sum_halves(l_run);
    const int qi = q0w + l32;
    if (qi < Lq) {
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_tot : 0.f;
      uint16_t* orow = o + (bh * Lq + qi) * int64_t(D);
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
      if (lse != nullptr && h == 0) lse[bh * Lq + qi] = live ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, int NW, int WPE>
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
  const size_t shmem = Smem<D>::BYTES;
  // One-time, thread-safe opt-in to more than 64 KiB of dynamic LDS for this instantiation.
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attention_bf16_kernel<D, NW, WPE>), hipFuncAttributeMaxDynamicSharedMemorySize,
      int(shmem));
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL((attention_bf16_kernel<D, NW, WPE>), dim3(grid), dim3(NW * 64), shmem, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                     block_mask, n_qt, n_items, xcd_remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Lq, int Lk, int d, float scale, int causal, const uint8_t* block_mask,
                                 hipStream_t stream) {
  if (d == 128)
    return launch_kernel<128, RF_ATT_NW_D128, RF_ATT_WPE_D128>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                block_mask, stream);
  return launch_kernel<64, RF_ATT_NW_D64, RF_ATT_WPE_D64>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask,
                                                           stream);
}

}  // namespace rf
