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
//   - K and V tiles of BN = 64 keys go straight from HBM into double-buffered
//     LDS (buffer loads with an LDS destination), one barrier per tile.
//   - The default kernel runs each wave's stages one tile apart: the score
//     product of tile j+1 is issued between the exponentials of tile j, and
//     the P.V product of tile j between the row maxima of tile j+1, so the
//     matrix core and the vector ALU work side by side (K is therefore loaded
//     two tiles ahead, V one).
//   - Tiles above the causal diagonal or outside the block mask of the whole
//     workgroup are never loaded or computed; the element mask is applied
//     only on tiles that straddle the diagonal or the end of the keys, or
//     that one wave's mask row hides while another's needs them.
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
#ifndef RF_ATT_DMA
#define RF_ATT_DMA 1
#endif
#ifndef RF_ATT_SREAD_AHEAD
#define RF_ATT_SREAD_AHEAD 4
#endif
#ifndef RF_ATT_VREAD_AHEAD
#define RF_ATT_VREAD_AHEAD 2
#endif
#ifndef RF_ATT_SP
#define RF_ATT_SP 1
#endif
#ifndef RF_ATT_SPLITEXP
#define RF_ATT_SPLITEXP 1
#endif
#ifndef RF_ATT_SUMGUARD
#define RF_ATT_SUMGUARD 1
#endif
#if RF_ATT_SPLITEXP && !RF_ATT_SUMGUARD
#error "the split exponentials rely on the sum guard"
#endif
#ifndef RF_ATT_HEAD_GROUP
#define RF_ATT_HEAD_GROUP 2
#endif
#ifndef RF_ATT_SP_SCHED
#define RF_ATT_SP_SCHED 1
#endif
#ifndef RF_ATT_SP_VALU_B
#define RF_ATT_SP_VALU_B 2
#endif
#ifndef RF_ATT_BN_D128
#define RF_ATT_BN_D128 64
#endif
#ifndef RF_ATT_BN_D64
#define RF_ATT_BN_D64 64
#endif
#ifndef RF_ATT_PINGPONG_D128
#define RF_ATT_PINGPONG_D128 0
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

// Sum of the two bf16 halves of a packed pair, accumulated in fp32.
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

// Lazy rescale: a row's exponent reference moves only when a tile's max exceeds
// it by more than kRescaleSlack (log2 units), so almost every tile skips the
// accumulator rescale. The weights p = 2^(t - m_ref) then stay <= 2^8 but the
// largest is no longer exactly 1 in bf16, so O is normalised by the sum of the
// same rounded weights the MFMA consumed (O stays an exact convex combination of
// V rows), while the LSE uses the sum of the unrounded weights.
constexpr float kRescaleSlack = 8.f;
constexpr float kSlackSum = 256.f;  // 2^kRescaleSlack

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
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
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

// Barrier that publishes the workgroup's direct-to-LDS loads. Such a load
// counts as complete (vmcnt) only in the wave that issued it, and the
// compiler waits for it only before that same wave's own LDS reads; for the
// other waves to read the data after the barrier, every wave must wait for
// its own loads before it. Every barrier that hands a DMA-filled buffer to
// other waves goes through here.
__device__ __forceinline__ void publish_lds_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Compiler-level pin: keeps the prefetch loads issued above it from being sunk
// next to their use (which would turn the prefetch into a synchronous wait).
__device__ __forceinline__ void pin_memory_order() { asm volatile("" ::: "memory"); }

// Walks the key tiles a workgroup must visit, in order. Without a block mask it
// is every tile below kt_end. With one, the mask bytes of the next 64 tiles are
// read once per 64 tiles (one byte per lane) and turned into two wave-uniform
// 64-bit words by ballot: tiles active for any of the workgroup's mask rows, and
// tiles active for this wave's own mask row. The scan itself is scalar bit work.
struct TileWalker {
  const uint8_t* mask;
  int n_mask_cols, mr0, mr1, mr_w, kt_end;
  int bn;  // keys per tile (divides the 64-key mask tile)
  int base = -64;
  uint64_t wg_bits = 0, wv_bits = 0;
  // With element bitmaps: tiles this wave's mask row has as partial (a kind
  // other than 0 and 1), and tiles partial for any row of the workgroup.
  bool bits = false;
  uint64_t pv_bits = 0, pg_bits = 0;

  __device__ void refill(int b) {
    const int kt = b + int(threadIdx.x & 63);
    bool any = false, mine = false, part = false, anypart = false;
    if (kt < kt_end) {
      const int mc = kt * bn / kMaskTile;
      for (int mr = mr0; mr <= mr1; ++mr) {
        const uint8_t kind = mask[int64_t(mr) * n_mask_cols + mc];
        const bool a = kind != 0;
        const bool pa = bits && kind != 0 && kind != 1;
        any |= a;
        mine |= (mr == mr_w) && a;
        anypart |= pa;
        part |= (mr == mr_w) && pa;
      }
    }
    wg_bits = __builtin_amdgcn_ballot_w64(any);
    wv_bits = __builtin_amdgcn_ballot_w64(mine);
    if (bits) {
      pg_bits = __builtin_amdgcn_ballot_w64(anypart);
      pv_bits = __builtin_amdgcn_ballot_w64(part);
    }
    base = b;
  }
  // First tile >= kt that the workgroup must visit (kt_end if none); *mine says
  // whether this wave's mask row has it. With bitmaps, *part (bit 0: this
  // wave's row, bit 1: any row of the workgroup) says whether it is partial.
  __device__ int next(int kt, bool* mine, int* part = nullptr) {
    if (part != nullptr) *part = 0;
    if (mask == nullptr) {
      *mine = true;
      return kt < kt_end ? kt : kt_end;
    }
    while (kt < kt_end) {
      if (kt < base || kt >= base + 64) refill(kt & ~63);
      const uint64_t rest = wg_bits >> (kt - base);
      if (rest) {
        kt += int(__builtin_ctzll(rest));
        if (kt >= kt_end) break;
        *mine = (wv_bits >> (kt - base)) & 1;
        if (part != nullptr) *part = int((pv_bits >> (kt - base)) & 1) | (int((pg_bits >> (kt - base)) & 1) << 1);
        return kt;
      }
      kt = base + 64;
    }
    *mine = false;
    return kt_end;
  }
};

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
    TileWalker walk{block_mask, n_mask_cols, q0 / kMaskTile, min(q0 + BM - 1, Lq - 1) / kMaskTile,
                    min(q0w, Lq - 1) / kMaskTile, kt_end, kBN};

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
      // The Q fragments are complete before the sweep, so the loop's waits only
      // ever concern the tile prefetches.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_ref = kNegInf;  // exponent reference of this lane's query row (log2 units)
    float l_run = 0.f;      // this lane's share of the sum of weights (lane l ^ 32 holds the rest)
    float l_rnd = 0.f;      // the same sum over the bf16-rounded weights
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
    bool mine = false;
    int kt = walk.next(0, &mine);
    int buf = 0;
    if (kt < kt_end) {
      load_tile(kt);
      store_tile(0);
    }
    __syncthreads();

    while (kt < kt_end) {
      bool mine_next = false;
      const int kt_next = walk.next(kt + 1, &mine_next);

      const int k0 = kt * kBN;
      const bool wave_visible = (!causal || int64_t(k0) <= int64_t(q0w) + 31 + off) && q0w < Lq && mine;
      f32x16_t st[2];
      if (wave_visible) {
        const uint16_t* ks_ = smem + buf * S::BUF_ELEMS;
        // ---- S^T = K Q^T (two 32-key blocks) ----
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
      }
      // The next tile's loads go out after the score MFMAs and stay in flight
      // through the softmax and the P.V products.
      if (kt_next < kt_end) load_tile(kt_next);
      pin_memory_order();
      if (wave_visible) {
        const uint16_t* vs_ = smem + buf * S::BUF_ELEMS + S::K_ELEMS;
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
        const float mt = mx * c_log2;
        const bool move = mt > m_ref + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(move)) {  // wave-uniform: rare after the first tile
          const float alpha = move ? fast_exp2(m_ref - mt) : 1.f;
          if (move) m_ref = mt;
          l_run *= alpha;
          l_rnd *= alpha;
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
            const uint32_t pp = cvt_pk_bf16(p0, p1);
            l_run += p0 + p1;
            l_rnd = add_bf16_pair(pp, l_rnd);
            pk[mb][r >> 1] = pp;
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
      mine = mine_next;
    }

    // ---- epilogue: O = acc / sum(rounded weights), LSE = (m + log2 sum(weights)) ln 2 ----
    const float l_tot = pair_sum_halves(l_run);
    const float l_rtot = pair_sum_halves(l_rnd);
    const int qi = q0w + l32;
    if (qi < Lq) {
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_rtot : 0.f;
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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant. K and V tiles travel global -> LDS with buffer loads
// that write LDS themselves (no staging registers, no LDS store instructions).
// Such a load writes lane i's 16 bytes at (LDS base + 16 i), so a tile lands as
// unpadded rows; bank conflicts are avoided by XOR-swizzling the 16-byte chunks
// of each row instead: K chunk c of row r sits in slot c ^ (r mod KCH), which
// spreads the 16 rows that one 16-lane read touches over 16 slots; V chunk c of
// row r sits in slot c ^ s(r mod 4) (s = 4 for d = 128, 2 for d = 64), which
// spreads the 4 rows x 2 chunks of one transposed 16-lane read over 8 slots.
// The sweep is unrolled by two so the buffer being read and the buffer being
// filled are distinct LDS objects at compile time: reads never wait for the
// other buffer's loads, and the end-of-tile barrier (which waits for this
// wave's loads) publishes the next tile.
// ---------------------------------------------------------------------------
template <int D>
struct Swz {
  static constexpr int KCH = D / 8;
  static constexpr int VX = D >= 128 ? 4 : 2;
  __device__ static int k_slot(int row, int c) { return c ^ (row & (KCH - 1)); }
  __device__ static int v_slot(int row, int c) { return c ^ (VX * (row & 3)); }
};

// Issue one tile's worth of direct-to-LDS loads for K and V: this wave's n
// instructions, each writing 64 x 16 contiguous bytes of LDS. Device-only (the
// LDS address-space cast has no host meaning).
__device__ __forceinline__ void dma_tile(const uint16_t* khead, const uint16_t* vhead, uint32_t head_bytes,
                                         uint16_t* kdst, uint16_t* vdst, uint32_t base, const uint32_t* kv_off,
                                         const uint32_t* vv_off, int ins0, int n) {
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(khead, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vhead, head_bytes);
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const int ins = ins0 + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(kdst + ins * 512), 16,
                                             base + kv_off[j], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(vdst + ins * 512), 16,
                                             base + vv_off[j], 0, 0, 0);
  }
}

// One wave-wide direct-to-LDS load of 1 KiB of tile row bitmaps into bb
// (lane i writes bytes 16 i .. 16 i + 15); off is this lane's byte offset.
__device__ __forceinline__ void dma_bits(const uint64_t* bits, uint32_t bytes, uint64_t* bb, uint32_t off) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(bits, bytes);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(bb), 16, off, 0, 0, 0);
}

// One tensor's share of a tile: this wave's n direct-to-LDS instructions.
__device__ __forceinline__ void dma_one(const uint16_t* head, uint32_t head_bytes, uint16_t* dst, uint32_t base,
                                        const uint32_t* lane_off, int ins0, int n) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head, head_bytes);
#pragma unroll
  for (int j = 0; j < n; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (ins0 + j) * 512), 16,
                                             base + lane_off[j], 0, 0, 0);
}

template <int D, int NW, int WPE, int BN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attention_bf16_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap) {
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int MB = BN / 32;                 // 32-key blocks per tile
  constexpr int PVK = BN / 16;                // MFMA K-steps of the P.V product per tile
  constexpr int CHUNKS = BN * KCH;            // 16-byte chunks per K (or V) tile
  constexpr int INSTR = CHUNKS / 64;          // wave-wide DMA instructions per tile and tensor
  constexpr int IPW = INSTR / NW;             // ... per wave
  static_assert(INSTR % NW == 0, "tile split");
  static_assert(BN % 32 == 0 && BN <= kMaskTile, "tile size");
  using SW = Swz<D>;

  __shared__ __align__(16) uint16_t kb0[BN * D];
  __shared__ __align__(16) uint16_t kb1[BN * D];
  __shared__ __align__(16) uint16_t vb0[BN * D];
  __shared__ __align__(16) uint16_t vb1[BN * D];

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t off = int64_t(Lk) - Lq;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int64_t per_xcd = n_items / 8;
  const uint32_t head_bytes = uint32_t(Lk) * D * 2;

  // This lane's source chunk for each of its DMA instructions (same for K and V
  // up to the swizzle), relative to the tile start.
  uint32_t kv_off[IPW], vv_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int g = 64 * (wave * IPW + j) + lane;
    const int row = g / KCH, slot = g % KCH;
    // slot = swizzle(row, c) is an involution in c: c = swizzle(row, slot)
    kv_off[j] = uint32_t(row * D * 2 + 16 * SW::k_slot(row, slot));
    vv_off[j] = uint32_t(row * D * 2 + 16 * SW::v_slot(row, slot));
  }
  // Transposed V^T read addressing (see lds_read_tr16).
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_x = (lane >> 4) & 1, tr_y = lane & 3;

  for (int64_t gi = blockIdx.x; gi < n_items; gi += gridDim.x) {
    const int64_t item = xcd_remap ? (gi % 8) * per_xcd + gi / 8 : gi;
    const int64_t bh = item / n_qt;
    const int qr = int(item % n_qt);
    const int q0 = (causal ? (n_qt - 1 - qr) : qr) * BM;
    const int q0w = q0 + 32 * wave;
    const uint16_t* qh = q + bh * int64_t(Lq) * D;
    const uint16_t* khead = k + bh * int64_t(Lk) * D;
    const uint16_t* vhead = v + bh * int64_t(Lk) * D;

    int64_t last_key = int64_t(min(q0 + BM, Lq) - 1) + (causal ? off : int64_t(Lk));
    if (last_key > Lk - 1) last_key = Lk - 1;
    const int kt_end = last_key < 0 ? 0 : int(last_key / BN) + 1;
    // The walker works on 64-key mask columns; tiles of BN keys map to column kt * BN / 64.
    TileWalker walk{block_mask, n_mask_cols, q0 / kMaskTile, min(q0 + BM - 1, Lq - 1) / kMaskTile,
                    min(q0w, Lq - 1) / kMaskTile, kt_end, BN};

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
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_ref = kNegInf, l_run = 0.f, l_rnd = 0.f;
    const int64_t row_last = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
    const int row_lim = int(row_last < int64_t(Lk) - 1 ? (row_last < -1 ? -1 : row_last) : int64_t(Lk) - 1);


    auto compute = [&](const uint16_t* ks_, const uint16_t* vs_, int kt, bool mine) {
      const int k0 = kt * BN;
      const bool wave_visible = (!causal || int64_t(k0) <= int64_t(q0w) + 31 + off) && q0w < Lq && mine;
      if (!wave_visible) return;
      // Score MFMAs: the 32-key blocks (and, with one block, the even / odd K-steps)
      // accumulate in separate registers so consecutive MFMAs never depend on
      // each other.
      constexpr int NACC = MB >= 2 ? MB : 2;
      f32x16_t st[MB];
      f32x16_t sacc[NACC];
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[a][r] = 0.f;
      // All K fragments are read first and the MFMAs follow with a fixed read-ahead
      // (RF_ATT_SREAD_AHEAD reads in flight): LDS latency is several MFMA issue
      // slots, so a one-deep read / multiply alternation would stall every step.
      uint4 kfrag[KSTEPS * MB];
#pragma unroll
      for (int kstep = 0; kstep < KSTEPS; ++kstep)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = 32 * mb + l32;
          kfrag[kstep * MB + mb] =
              *reinterpret_cast<const uint4*>(ks_ + row * D + 8 * SW::k_slot(row, 2 * kstep + h));
        }
#pragma unroll
      for (int kstep = 0; kstep < KSTEPS; ++kstep)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int acc = MB >= 2 ? mb : (kstep & 1);
          sacc[acc] = mfma32(as_bf16x8(kfrag[kstep * MB + mb]), as_bf16x8(qf[kstep]), sacc[acc]);
        }
#if RF_ATT_SREAD_AHEAD > 0
      __builtin_amdgcn_sched_group_barrier(0x100, RF_ATT_SREAD_AHEAD, 0);
#pragma unroll
      for (int i = 0; i < KSTEPS * MB - RF_ATT_SREAD_AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, RF_ATT_SREAD_AHEAD, 0);
#endif
      if constexpr (MB >= 2) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) st[mb] = sacc[mb];
      } else {
        st[0] = sacc[0] + sacc[1];
      }
      const bool edge = (causal && int64_t(k0) + BN - 1 > int64_t(q0w) + off) || (k0 + BN > Lk);
      if (edge) {
        const int lim = row_lim - k0 - 4 * h;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mb + 8 * (r >> 2) + (r & 3) > lim) st[mb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
      mx = pair_max_halves(mx);
      const float mt = mx * c_log2;
      const bool move = mt > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float alpha = move ? fast_exp2(m_ref - mt) : 1.f;
        if (move) m_ref = mt;
        l_run *= alpha;
        l_rnd *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      }
      const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
      uint32_t pk[MB][8];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(st[mb][r], c_log2, -mu));
          const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_log2, -mu));
          const uint32_t pp = cvt_pk_bf16(p0, p1);
          l_run += p0 + p1;
          l_rnd = add_bf16_pair(pp, l_rnd);
          pk[mb][r >> 1] = pp;
        }
      // V^T fragments for the P.V products, product i = kstep * DB + db, read in a
      // rolling window of VAHEAD fragments ahead of the product that uses them.
      constexpr int NPV = PVK * DB;
      constexpr int VAHEAD = RF_ATT_VREAD_AHEAD > 0 ? RF_ATT_VREAD_AHEAD : 1;
      auto vread = [&](int i) {
        const int kstep = i / DB, db = i % DB;
        const int row_lo = 16 * kstep + tr_row, row_hi = row_lo + 8;
        const int c = 4 * db + 2 * tr_x + (tr_y >> 1);
        const uint2 lo = lds_read_tr16(vs_ + row_lo * D + 8 * SW::v_slot(row_lo, c) + 4 * (tr_y & 1));
        const uint2 hi = lds_read_tr16(vs_ + row_hi * D + 8 * SW::v_slot(row_hi, c) + 4 * (tr_y & 1));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 vfrag[VAHEAD];
#pragma unroll
      for (int i = 0; i < VAHEAD; ++i) vfrag[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int kstep = i / DB, db = i % DB;
        const int mb = kstep >> 1, r0 = (kstep & 1) * 4;
        const uint4 bp = make_uint4(pk[mb][r0], pk[mb][r0 + 1], pk[mb][r0 + 2], pk[mb][r0 + 3]);
        const uint4 a = vfrag[i % VAHEAD];
        if (i + VAHEAD < NPV) vfrag[i % VAHEAD] = vread(i + VAHEAD);
        acc_o[db] = mfma32(as_bf16x8(a), as_bf16x8(bp), acc_o[db]);
      }
#if RF_ATT_VREAD_AHEAD > 0
      // Same read-ahead for the two transposed V reads behind each P.V product.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * RF_ATT_VREAD_AHEAD, 1);
#pragma unroll
      for (int i = 0; i < PVK * DB - RF_ATT_VREAD_AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, RF_ATT_VREAD_AHEAD, 1);
#endif
    };

    __syncthreads();  // the previous item's readers of every buffer are done
    bool mine = false;
    int kt = walk.next(0, &mine);
    if (kt < kt_end) dma_tile(khead, vhead, head_bytes, kb0, vb0, uint32_t(kt) * BN * D * 2, kv_off, vv_off, wave * IPW, IPW);
    __syncthreads();  // waits for this wave's loads, then publishes tile 0
    while (kt < kt_end) {
      // even step: read buffers 0, fill buffers 1
      bool mine1 = false;
      const int kt1 = walk.next(kt + 1, &mine1);
      if (kt1 < kt_end) dma_tile(khead, vhead, head_bytes, kb1, vb1, uint32_t(kt1) * BN * D * 2, kv_off, vv_off, wave * IPW, IPW);
      compute(kb0, vb0, kt, mine);
      __syncthreads();
      if (kt1 >= kt_end) break;
      // odd step: read buffers 1, fill buffers 0
      bool mine2 = false;
      const int kt2 = walk.next(kt1 + 1, &mine2);
      if (kt2 < kt_end) dma_tile(khead, vhead, head_bytes, kb0, vb0, uint32_t(kt2) * BN * D * 2, kv_off, vv_off, wave * IPW, IPW);
      compute(kb1, vb1, kt1, mine1);
      __syncthreads();
      kt = kt2;
      mine = mine2;
    }

    const float l_tot = pair_sum_halves(l_run);
    const float l_rtot = pair_sum_halves(l_rnd);
    const int qi = q0w + l32;
    if (qi < Lq) {
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_rtot : 0.f;
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

// Work item of launch slot gi. With xcd_remap, consecutive slots (which the
// hardware deals round-robin to the 8 XCDs) map to 8 contiguous ranges of
// items, one per XCD, so that the query tiles of a head share one L2. Then
// each complete block of head_group heads x n_qt query tiles is dispatched
// query tile first, head second: the causal tiles of the block go heaviest
// first across its heads (longest-first list scheduling, which keeps the
// workgroups of an XCD finishing together), while only head_group heads' K/V
// are live in that L2 at a time. A last partial block keeps its order.
__device__ __forceinline__ int64_t work_item(int64_t gi, int64_t n_items, int64_t per_xcd, int xcd_remap, int n_qt,
                                             int head_group) {
  const int64_t flat = xcd_remap ? (gi % 8) * per_xcd + gi / 8 : gi;
  if (head_group <= 1) return flat;
  const int64_t bsz = int64_t(head_group) * n_qt;
  const int64_t b = flat / bsz, w = flat % bsz;
  if ((b + 1) * bsz > n_items) return flat;
  return (b * head_group + w % head_group) * n_qt + w / head_group;
}

// ---------------------------------------------------------------------------
// Software-pipelined variant of the direct-to-LDS kernel.
//
// Within one wave the three stages of a key tile (score product, softmax
// update, P.V product) depend on each other, so run back to back they leave
// the matrix core idle during the exponentials and the vector ALU idle during
// the products. Here every wave runs them one tile apart:
//
//   phase A of tile j :  S(j+1) = K(j+1) Q^T      while  P(j) = exp(S(j) - m)
//   phase B of tile j :  O^T   += V(j)^T P(j)^T   while  m <- max(m, rowmax S(j+1))
//
// so each phase pairs a run of MFMAs with independent vector work. The score
// product of the next tile needs its K one tile earlier than its V, so K is
// loaded two tiles ahead and V one tile ahead; both stay double-buffered and
// one barrier per tile both publishes the loads and frees the buffers:
//
//   after the barrier of tile j:  load K(j+2) -> the K buffer of tile j,
//                                 load V(j+1) -> the V buffer of tile j-1.
//
// The softmax state follows the same lazy rescale as the other kernels: the
// running reference m only moves (and O and the sums are only rescaled) when
// a tile's row maximum exceeds it by more than 2^kRescaleSlack. The rescale
// of O waits for the P.V product that precedes it in phase B.
// ---------------------------------------------------------------------------
//
// SPLIT: split-KV partials. Item = (head, split, query tile); split s visits
// key tiles [s kt_split, (s + 1) kt_split) only, and writes its output,
// normalised, in fp32 with its LSE into ws_o [head rows, n_splits, D] and
// ws_lse [head rows, n_splits] for a log-sum-exp merge. Used for decode with
// grouped queries, where the query heads sharing one key/value head are the
// rows of the query tile.
template <int D, int NW, int WPE, bool BITS, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attention_bf16_sp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap, int head_group,
    int64_t item_base, const uint64_t* __restrict__ tile_bits, uint32_t bits_bytes, int n_splits = 1,
    int kt_split = 0, float* __restrict__ ws_o = nullptr, float* __restrict__ ws_lse = nullptr) {
  constexpr int BN = 64;
  constexpr int BM = 32 * NW;
  constexpr int KCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int MB = BN / 32;
  constexpr int PVK = BN / 16;
  constexpr int NS = KSTEPS * MB;   // score MFMAs per tile
  constexpr int NPV = PVK * DB;     // P.V MFMAs per tile
  constexpr int CHUNKS = BN * KCH;
  constexpr int INSTR = CHUNKS / 64;
  constexpr int IPW = INSTR / NW;
  static_assert(INSTR % NW == 0, "tile split");
  using SW = Swz<D>;

  __shared__ __align__(16) uint16_t kb0[BN * D];
  __shared__ __align__(16) uint16_t kb1[BN * D];
  __shared__ __align__(16) uint16_t vb0[BN * D];
  __shared__ __align__(16) uint16_t vb1[BN * D];
  // Row bitmaps of the workgroup's 128 query rows for the tile in kb0 / kb1
  // (word 32 w + r belongs to wave w's row r), loaded with that tile's K.
  __shared__ __align__(16) uint64_t bb0[BITS ? 128 : 2];
  __shared__ __align__(16) uint64_t bb1[BITS ? 128 : 2];

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t off = int64_t(Lk) - Lq;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int64_t per_xcd = n_items / 8;
  const uint32_t head_bytes = uint32_t(Lk) * D * 2;

  uint32_t kv_off[IPW], vv_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int g = 64 * (wave * IPW + j) + lane;
    const int row = g / KCH, slot = g % KCH;
    kv_off[j] = uint32_t(row * D * 2 + 16 * SW::k_slot(row, slot));
    vv_off[j] = uint32_t(row * D * 2 + 16 * SW::v_slot(row, slot));
  }
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_x = (lane >> 4) & 1, tr_y = lane & 3;

  // One work item per workgroup: items [item_base, item_base + gridDim.x) of
  // this launch, permuted by work_item within the launch.
  {
    const int64_t item = item_base + work_item(blockIdx.x, n_items, per_xcd, xcd_remap, n_qt, head_group);
    const int64_t bhs = item / n_qt;
    const int64_t bh = SPLIT ? bhs / n_splits : bhs;
    const int split = SPLIT ? int(bhs % n_splits) : 0;
    const int qr = int(item % n_qt);
    const int q0 = (causal ? (n_qt - 1 - qr) : qr) * BM;
    const int q0w = q0 + 32 * wave;
    const uint16_t* qh = q + bh * int64_t(Lq) * D;
    const uint16_t* khead = k + bh * int64_t(Lk) * D;
    const uint16_t* vhead = v + bh * int64_t(Lk) * D;

    int64_t last_key = int64_t(min(q0 + BM, Lq) - 1) + (causal ? off : int64_t(Lk));
    if (last_key > Lk - 1) last_key = Lk - 1;
    const int kt_all = last_key < 0 ? 0 : int(last_key / BN) + 1;
    const int kt_begin = SPLIT ? split * kt_split : 0;
    const int kt_end = SPLIT ? min(kt_all, kt_begin + kt_split) : kt_all;
    TileWalker walk{block_mask, n_mask_cols, q0 / kMaskTile, min(q0 + BM - 1, Lq - 1) / kMaskTile,
                    min(q0w, Lq - 1) / kMaskTile, kt_end, BN};
    walk.bits = BITS;

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
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_ref = kNegInf, l_run = 0.f, l_rnd = 0.f;
    const int64_t row_last = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
    const int row_lim = int(row_last < int64_t(Lk) - 1 ? (row_last < -1 ? -1 : row_last) : int64_t(Lk) - 1);

    // ---- stage pieces (inlined into the phase bodies below) ----
    auto score_mfmas = [&](const uint16_t* ks_, f32x16_t (&sacc)[MB]) {
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[a][r] = 0.f;
      // K fragments in a rolling window of KAHEAD reads ahead of their product.
      constexpr int KAHEAD = RF_ATT_SREAD_AHEAD > 0 ? RF_ATT_SREAD_AHEAD : 1;
      auto kread = [&](int i) {
        const int kstep = i / MB, mb = i % MB;
        const int row = 32 * mb + l32;
        return *reinterpret_cast<const uint4*>(ks_ + row * D + 8 * SW::k_slot(row, 2 * kstep + h));
      };
      uint4 kfrag[KAHEAD];
#pragma unroll
      for (int i = 0; i < KAHEAD; ++i) kfrag[i] = kread(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int kstep = i / MB, mb = i % MB;
        const uint4 a = kfrag[i % KAHEAD];
        if (i + KAHEAD < NS) kfrag[i % KAHEAD] = kread(i + KAHEAD);
        sacc[mb] = mfma32(as_bf16x8(a), as_bf16x8(qf[kstep]), sacc[mb]);
      }
    };
    // P of a tile against the reference m_ref, with the tile's sums of P
    // (exact, and of P as rounded for the P.V product) added to lt, ltr.
    auto exp_tile = [&](const f32x16_t (&st)[MB], uint32_t (&pk)[MB][8], float& lt, float& ltr) {
      const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(st[mb][r], c_log2, -mu));
          const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_log2, -mu));
          const uint32_t pp = cvt_pk_bf16(p0, p1);
          lt += p0 + p1;
          ltr = add_bf16_pair(pp, ltr);
          pk[mb][r >> 1] = pp;
        }
    };
    // P.V MFMAs i0 .. i1 - 1 of the tile (i = kstep * DB + db; K-steps 0 and 1
    // use keys 0..31, i.e. the first half of P), V^T fragments read a window
    // ahead; hook(j) runs after the j-th of them (vector work to interleave).
    auto pv_range = [&](const uint16_t* vs_, const uint32_t (&pk)[MB][8], int i0, int i1, auto&& hook) {
      constexpr int VAHEAD = RF_ATT_VREAD_AHEAD > 0 ? RF_ATT_VREAD_AHEAD : 1;
      auto vread = [&](int i) {
        const int kstep = i / DB, db = i % DB;
        const int row_lo = 16 * kstep + tr_row, row_hi = row_lo + 8;
        const int c = 4 * db + 2 * tr_x + (tr_y >> 1);
        const uint2 lo = lds_read_tr16(vs_ + row_lo * D + 8 * SW::v_slot(row_lo, c) + 4 * (tr_y & 1));
        const uint2 hi = lds_read_tr16(vs_ + row_hi * D + 8 * SW::v_slot(row_hi, c) + 4 * (tr_y & 1));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 vfrag[VAHEAD];
#pragma unroll
      for (int i = 0; i < VAHEAD; ++i)
        if (i0 + i < i1) vfrag[i] = vread(i0 + i);
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const int kstep = i / DB, db = i % DB;
        const int mb = kstep >> 1, r0 = (kstep & 1) * 4;
        const uint4 bp = make_uint4(pk[mb][r0], pk[mb][r0 + 1], pk[mb][r0 + 2], pk[mb][r0 + 3]);
        const uint4 a = vfrag[(i - i0) % VAHEAD];
        if (i + VAHEAD < i1) vfrag[(i - i0) % VAHEAD] = vread(i + VAHEAD);
        acc_o[db] = mfma32(as_bf16x8(a), as_bf16x8(bp), acc_o[db]);
        hook(i - i0);
      }
    };
    auto pv_mfmas = [&](const uint16_t* vs_, const uint32_t (&pk)[MB][8]) {
      pv_range(vs_, pk, 0, NPV, [](int) {});
    };
    // Scores this wave must not see -> -inf: keys past the row's last key (causal
    // diagonal, sequence end), and the whole tile when the wave's block-mask row
    // skips it or the causal diagonal ends before it. A fully hidden tile then
    // contributes exp(-inf) = 0 everywhere.
    // This lane's row word of a tile's bitmaps (read early: it gates the mask).
    auto row_word = [&](int part, const uint64_t* bb) -> uint64_t {
      return (BITS && (part & 1)) ? bb[32 * wave + l32] : ~uint64_t(0);
    };
    auto mask_tile = [&](f32x16_t (&st)[MB], int kt, bool mine, int part, uint64_t word) {
      const int k0 = kt * BN;
      const bool bitmap = BITS && (part & 1);
      const bool edge =
          !mine || bitmap || (causal && int64_t(k0) + BN - 1 > int64_t(q0w) + off) || (k0 + BN > Lk);
      if (edge) {
        const int lim = mine ? row_lim - k0 - 4 * h : -BN;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mb + 8 * (r >> 2) + (r & 3) > lim) st[mb][r] = kNegInf;
        if (bitmap) {
          // Key 32 mb + 8 (r / 4) + 4 h + r % 4 of the tile is visible iff its
          // bit in this row's word is set.
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const uint32_t w = uint32_t(word >> (32 * mb)) >> (4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (((w >> (8 * (r >> 2) + (r & 3))) & 1u) == 0) st[mb][r] = kNegInf;
          }
        }
      }
    };
    // Row maximum of a tile; moves the reference when it is exceeded by more than
    // the slack and returns the factor for the state accumulated so far.
    auto tile_max = [&](const f32x16_t (&st)[MB], bool* moved) {
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
      mx = pair_max_halves(mx);
      const float mt = mx * c_log2;
      const bool move = mt > m_ref + kRescaleSlack;
      *moved = __builtin_amdgcn_ballot_w64(move) != 0;
      float alpha = 1.f;
      if (move) {
        alpha = fast_exp2(m_ref - mt);
        m_ref = mt;
      }
      return alpha;
    };
    auto rescale = [&](float alpha) {
      l_run *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
    };
    // Commit a tile's P. It was formed against m_ref without looking at the
    // tile's maximum: each lane's sum of its P bounds every one of them, so
    // while that sum stays within 2^kRescaleSlack (and the row has a
    // reference at all) the lazy-rescale bound holds and P is kept. Otherwise
    // the row maximum decides as in the lazy rescale: if it exceeds the
    // reference by more than the slack, the reference moves to it, the state
    // so far is rescaled and the tile's P is formed again.
    auto commit_tile = [&](const f32x16_t (&st)[MB], uint32_t (&pk)[MB][8], float lt, float ltr) {
      const bool suspect = !(lt <= kSlackSum) || m_ref == kNegInf;
      if (__builtin_amdgcn_ballot_w64(suspect)) {
        bool moved = false;
        const float alpha = tile_max(st, &moved);
        if (moved) {
          rescale(alpha);
          lt = 0.f;
          ltr = 0.f;
          exp_tile(st, pk, lt, ltr);
        }
      }
      l_run += lt;
      l_rnd += ltr;
    };

    // One score pair (keys 2r, 2r + 1 of 32-key block mb) of P against mu.
    auto exp_pair = [&](const f32x16_t (&st)[MB], uint32_t (&pk)[MB][8], int mb, int r, float mu, float& lt,
                        float& ltr) {
      const float p0 = fast_exp2(fmaf(st[mb][2 * r], c_log2, -mu));
      const float p1 = fast_exp2(fmaf(st[mb][2 * r + 1], c_log2, -mu));
      const uint32_t pp = cvt_pk_bf16(p0, p1);
      lt += p0 + p1;
      ltr = add_bf16_pair(pp, ltr);
      pk[mb][r] = pp;
    };
    // commit_tile for one 32-key half of the tile: the guard looks at this
    // half's sums, the reference follows the whole tile's maximum, and only
    // this half's P is formed again. Halves committed earlier are already in
    // O and the sums, and the rescale covers them.
    auto commit_half = [&](const f32x16_t (&st)[MB], uint32_t (&pk)[MB][8], int mb, float lt, float ltr) {
      const bool suspect = !(lt <= kSlackSum) || m_ref == kNegInf;
      if (__builtin_amdgcn_ballot_w64(suspect)) {
        bool moved = false;
        const float alpha = tile_max(st, &moved);
        if (moved) {
          rescale(alpha);
          lt = 0.f;
          ltr = 0.f;
          const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
          for (int r = 0; r < 8; ++r) exp_pair(st, pk, mb, r, mu, lt, ltr);
        }
      }
      l_run += lt;
      l_rnd += ltr;
    };
#if RF_ATT_SPLITEXP
    static_assert(MB == 2, "two halves per tile");
    // Steady-state step with the exponentials split across both phases:
    //   phase A : S(next) MFMAs     with the exponentials of keys 0..31
    //   phase B1: P.V keys 0..31    with the exponentials of keys 32..63
    //   phase B2: P.V keys 32..63
    auto step = [&](const uint16_t* ks_next, const uint16_t* vs_cur, f32x16_t (&s_cur)[MB],
                    f32x16_t (&s_next)[MB], int kt_next, bool mine_next, int part_next,
                    const uint64_t* bb_next) {
      uint32_t pk[MB][8];
      // d = 64 has registers to spare: read the word before phase A.
      const uint64_t word_next = D <= 64 ? row_word(part_next, bb_next) : 0;
      float lt0 = 0.f, ltr0 = 0.f, lt1 = 0.f, ltr1 = 0.f;
      {
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) s_next[a][r] = 0.f;
        constexpr int KAHEAD = RF_ATT_SREAD_AHEAD > 0 ? RF_ATT_SREAD_AHEAD : 1;
        auto kread = [&](int i) {
          const int kstep = i / MB, mb = i % MB;
          const int row = 32 * mb + l32;
          return *reinterpret_cast<const uint4*>(ks_next + row * D + 8 * SW::k_slot(row, 2 * kstep + h));
        };
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        uint4 kfrag[KAHEAD];
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) kfrag[i] = kread(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const int kstep = i / MB, mb = i % MB;
          const uint4 a = kfrag[i % KAHEAD];
          if (i + KAHEAD < NS) kfrag[i % KAHEAD] = kread(i + KAHEAD);
          s_next[mb] = mfma32(as_bf16x8(a), as_bf16x8(qf[kstep]), s_next[mb]);
#pragma unroll
          for (int r = i * 8 / NS; r < (i + 1) * 8 / NS; ++r) exp_pair(s_cur, pk, 0, r, mu, lt0, ltr0);
#if RF_ATT_SP_SCHED
          __builtin_amdgcn_sched_barrier(0);
#endif
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[0][i]));
      asm volatile("" ::"v"(lt0), "v"(ltr0));
      commit_half(s_cur, pk, 0, lt0, ltr0);
      mask_tile(s_next, kt_next, mine_next, part_next, D <= 64 ? word_next : row_word(part_next, bb_next));
      {
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        constexpr int NB1 = NPV / 2;
        pv_range(vs_cur, pk, 0, NB1, [&](int j) {
#pragma unroll
          for (int r = j * 8 / NB1; r < (j + 1) * 8 / NB1; ++r) exp_pair(s_cur, pk, 1, r, mu, lt1, ltr1);
#if RF_ATT_SP_SCHED
          __builtin_amdgcn_sched_barrier(0);
#endif
        });
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[1][i]));
      asm volatile("" ::"v"(lt1), "v"(ltr1));
      commit_half(s_cur, pk, 1, lt1, ltr1);
      pv_range(vs_cur, pk, NPV / 2, NPV, [](int) {});
    };
#else
    // One steady-state step: current tile (scores s_cur, V in vs_cur), next tile
    // (K in ks_next, scores into s_next).
    auto step = [&](const uint16_t* ks_next, const uint16_t* vs_cur, f32x16_t (&s_cur)[MB],
                    f32x16_t (&s_next)[MB], int kt_next, bool mine_next, int part_next,
                    const uint64_t* bb_next) {
      uint32_t pk[MB][8];
      // d = 64 has registers to spare: read the word before phase A.
      const uint64_t word_next = D <= 64 ? row_word(part_next, bb_next) : 0;
      float lt = 0.f, ltr = 0.f;
      // Phase A: score product of the next tile with the exponentials of this
      // one, written as NS chunks of one MFMA plus its share of the vector work
      // (fenced so the compiler keeps the interleave).
      {
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) s_next[a][r] = 0.f;
        constexpr int KAHEAD = RF_ATT_SREAD_AHEAD > 0 ? RF_ATT_SREAD_AHEAD : 1;
        constexpr int PAIRS = MB * 8;             // score pairs per lane and tile
        constexpr int PPC = (PAIRS + NS - 1) / NS;  // pairs per chunk
        auto kread = [&](int i) {
          const int kstep = i / MB, mb = i % MB;
          const int row = 32 * mb + l32;
          return *reinterpret_cast<const uint4*>(ks_next + row * D + 8 * SW::k_slot(row, 2 * kstep + h));
        };
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        uint4 kfrag[KAHEAD];
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) kfrag[i] = kread(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const int kstep = i / MB, mb = i % MB;
          const uint4 a = kfrag[i % KAHEAD];
          if (i + KAHEAD < NS) kfrag[i % KAHEAD] = kread(i + KAHEAD);
          s_next[mb] = mfma32(as_bf16x8(a), as_bf16x8(qf[kstep]), s_next[mb]);
#pragma unroll
          for (int j = 0; j < PPC; ++j) {
            const int pr = i * PPC + j;
            if (pr < PAIRS) {
              const int cb = pr / 8, r = 2 * (pr % 8);
              const float p0 = fast_exp2(fmaf(s_cur[cb][r], c_log2, -mu));
              const float p1 = fast_exp2(fmaf(s_cur[cb][r + 1], c_log2, -mu));
              const uint32_t pp = cvt_pk_bf16(p0, p1);
              lt += p0 + p1;
              ltr = add_bf16_pair(pp, ltr);
              pk[cb][r >> 1] = pp;
            }
          }
#if RF_ATT_SP_SCHED
          __builtin_amdgcn_sched_barrier(0);
#endif
        }
      }
      // Keep P and the sums in phase A: without these uses the compiler sinks
      // the exponentials past the mask branch, next to the P.V product.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[mb][i]));
      asm volatile("" ::"v"(lt), "v"(ltr));
#if RF_ATT_SUMGUARD
      commit_tile(s_cur, pk, lt, ltr);
      mask_tile(s_next, kt_next, mine_next, part_next, D <= 64 ? word_next : row_word(part_next, bb_next));
      // Phase B: P.V product of this tile.
      pv_mfmas(vs_cur, pk);
#else
      l_run += lt;
      l_rnd += ltr;
      mask_tile(s_next, kt_next, mine_next, part_next, D <= 64 ? word_next : row_word(part_next, bb_next));
      // Phase B: P.V product of this tile with the row maximum of the next one.
      pv_mfmas(vs_cur, pk);
      bool moved = false;
      const float alpha = tile_max(s_next, &moved);
#if RF_ATT_SP_SCHED
      {
        constexpr int VAHEAD = RF_ATT_VREAD_AHEAD > 0 ? RF_ATT_VREAD_AHEAD : 1;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VAHEAD, 1);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          if (i < NPV - VAHEAD) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
          __builtin_amdgcn_sched_group_barrier(0x002, RF_ATT_SP_VALU_B, 1);
        }
      }
#endif
      if (moved) rescale(alpha);
#endif
    };
#endif
    // The last tile: exponentials and P.V product only.
    auto finish = [&](const uint16_t* vs_cur, const f32x16_t (&s_cur)[MB]) {
      uint32_t pk[MB][8];
      float lt = 0.f, ltr = 0.f;
      exp_tile(s_cur, pk, lt, ltr);
#if RF_ATT_SUMGUARD
      commit_tile(s_cur, pk, lt, ltr);
#else
      l_run += lt;
      l_rnd += ltr;
#endif
      pv_mfmas(vs_cur, pk);
    };
    f32x16_t s0[MB], s1[MB];

    bool m0 = false, m1 = false, m2 = false;
    int p0 = 0, p1 = 0, p2 = 0;
    // Row bitmaps of tile kt into bb, when some row of the workgroup has it as
    // partial: one wave issues one 1 KiB direct-to-LDS load (lane i: 16 bytes =
    // rows 2 (i % 32), +1 of mask row q0 / 64 + i / 32).
    auto load_bits = [&](uint64_t* bb, int kt, int part) {
      if (BITS && (part & 2) && wave == 0) {
        const uint32_t mr = uint32_t(q0 / kMaskTile + (lane >> 5));
        const uint32_t off = ((mr * uint32_t(n_mask_cols) + uint32_t(kt)) * 64u + 2u * uint32_t(lane & 31)) * 8u;
        dma_bits(tile_bits, bits_bytes, bb, off);
      }
    };
    int t0 = walk.next(kt_begin, &m0, &p0);
    if (t0 < kt_end) {
      int t1 = walk.next(t0 + 1, &m1, &p1);
      dma_one(khead, head_bytes, kb0, uint32_t(t0) * BN * D * 2, kv_off, wave * IPW, IPW);
      dma_one(vhead, head_bytes, vb0, uint32_t(t0) * BN * D * 2, vv_off, wave * IPW, IPW);
      load_bits(bb0, t0, p0);
      if (t1 < kt_end) {
        dma_one(khead, head_bytes, kb1, uint32_t(t1) * BN * D * 2, kv_off, wave * IPW, IPW);
        load_bits(bb1, t1, p1);
      }
      publish_lds_loads();  // K(t0), K(t1), V(t0) resident
      score_mfmas(kb0, s0);
      mask_tile(s0, t0, m0, p0, row_word(p0, bb0));
      {
        bool moved = false;
        const float alpha = tile_max(s0, &moved);
        if (moved) rescale(alpha);
      }
      // Steady state, unrolled by two: in the even step the current tile's V is
      // in vb0 and the next tile's K in kb1; the odd step mirrors it. The loop
      // leaves with the last tile's scores in s0 and its V in vb0 or vb1.
      bool last_in_vb1 = false;
      while (true) {
        publish_lds_loads();  // loads of the previous step resident; kb0 and vb1 free
        if (t1 >= kt_end) break;
        int t2 = walk.next(t1 + 1, &m2, &p2);
        if (t2 < kt_end) {
          dma_one(khead, head_bytes, kb0, uint32_t(t2) * BN * D * 2, kv_off, wave * IPW, IPW);
          load_bits(bb0, t2, p2);
        }
        dma_one(vhead, head_bytes, vb1, uint32_t(t1) * BN * D * 2, vv_off, wave * IPW, IPW);
        step(kb1, vb0, s0, s1, t1, m1, p1, bb1);

        publish_lds_loads();  // this step's loads resident; kb1 and vb0 free
        if (t2 >= kt_end) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) s0[mb] = s1[mb];
          last_in_vb1 = true;
          break;
        }
        bool m3 = false;
        int p3 = 0;
        const int t3 = walk.next(t2 + 1, &m3, &p3);
        if (t3 < kt_end) {
          dma_one(khead, head_bytes, kb1, uint32_t(t3) * BN * D * 2, kv_off, wave * IPW, IPW);
          load_bits(bb1, t3, p3);
        }
        dma_one(vhead, head_bytes, vb0, uint32_t(t2) * BN * D * 2, vv_off, wave * IPW, IPW);
        step(kb0, vb1, s1, s0, t2, m2, p2, bb0);
        t1 = t3;
        m1 = m3;
        p1 = p3;
      }
      finish(last_in_vb1 ? vb1 : vb0, s0);
    }

    const float l_tot = pair_sum_halves(l_run);
    const float l_rtot = pair_sum_halves(l_rnd);
    const int qi = q0w + l32;
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_rtot : 0.f;
    if constexpr (SPLIT) {
      // fp32 partial: lane (row l32, half h) holds d = 32 db + 16 pp + 8 sel + 4 h + i
      // in acc_o[db][8 pp + 4 sel + i]; 16-byte stores of 4 consecutive d.
      if (qi < Lq) {
        const int64_t prow = (bh * Lq + qi) * n_splits + split;
        float* orow = ws_o + prow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float4 x = make_float4(acc_o[db][r] * inv, acc_o[db][r + 1] * inv, acc_o[db][r + 2] * inv,
                                         acc_o[db][r + 3] * inv);
            *reinterpret_cast<float4*>(orow + 32 * db + 2 * r + 4 * h) = x;
          }
        if (h == 0) ws_lse[prow] = live ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
      }
      return;
    }
    // Output: each wave's 32 rows are one contiguous block of O. Lanes l and
    // l + 32 hold alternate 8-byte pieces of a row; one v_permlane32_swap per
    // dword gives each lane a 16-byte run, which goes through this wave's own
    // slice of the (now idle) K buffers so that every store instruction writes
    // 1 KiB of consecutive bytes.
    {
      static_assert(NW * 32 <= 2 * BN, "output staging fits in the K buffers");
      constexpr int OCH = D / 8;  // 16-byte chunks per row
      uint16_t* stage = (wave < NW / 2 ? kb0 : kb1) + (wave % (NW / 2)) * 32 * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int ra = 8 * pp, rb = 8 * pp + 4;  // d = 32 db + 16 pp + 4 h (+ 8 for rb)
          const uint32_t ax = cvt_pk_bf16(acc_o[db][ra] * inv, acc_o[db][ra + 1] * inv);
          const uint32_t ay = cvt_pk_bf16(acc_o[db][ra + 2] * inv, acc_o[db][ra + 3] * inv);
          const uint32_t bx = cvt_pk_bf16(acc_o[db][rb] * inv, acc_o[db][rb + 1] * inv);
          const uint32_t by = cvt_pk_bf16(acc_o[db][rb + 2] * inv, acc_o[db][rb + 3] * inv);
          const auto sx = __builtin_amdgcn_permlane32_swap(ax, bx, false, false);
          const auto sy = __builtin_amdgcn_permlane32_swap(ay, by, false, false);
          const int c = 4 * db + 2 * pp + h;  // this lane now holds d = 8c .. 8c + 7
          *reinterpret_cast<uint4*>(stage + l32 * D + 8 * (c ^ (l32 & (OCH - 1)))) =
              make_uint4(sx[0], sy[0], sx[1], sy[1]);
        }
      uint16_t* obase = o + (bh * Lq + q0w) * int64_t(D);
#pragma unroll
      for (int i = 0; i < 32 * OCH / 64; ++i) {
        const int g = 64 * i + lane, row = g / OCH, c = g % OCH;
        const uint4 x = *reinterpret_cast<const uint4*>(stage + row * D + 8 * (c ^ (row & (OCH - 1))));
        if (q0w + row < Lq) *reinterpret_cast<uint4*>(obase + row * D + 8 * c) = x;
      }
    }
    if (lse != nullptr && h == 0 && qi < Lq) lse[bh * Lq + qi] = live ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong variant for long causal / dense sweeps (d = 128).
//
// Eight waves form two groups of four; each SIMD holds one wave of each group.
// A workgroup barrier splits every key tile into two phases, and the groups
// run one phase apart, so on every SIMD one wave issues matrix-core work while
// the other issues the softmax's vector work:
//
//   phase 2n   : group A  M(n) = { O += V(n-1)^T P(n-1)^T ; S(n) = K(n) Q^T }
//                group B  V(n-1) = softmax update of S(n-1) -> P(n-1)
//   phase 2n+1 : group A  V(n)
//                group B  M(n)
//                all      K(n+1), V(n) staged registers -> LDS; issue the
//                         global loads of K(n+2), V(n+1)
//
// K therefore runs one tile ahead of V: K(n) and V(n-1) are live during tile
// n, each double-buffered. Group A owns the even 32-row blocks of the 256-row
// query tile and group B the odd ones, so both see the same causal diagonal.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attention_bf16_pp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap) {
  using S = Smem<D>;
  constexpr int NT = 512;
  constexpr int BM = 256;
  constexpr int KCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int LD = kBN * KCH / NT;
  static_assert(kBN * KCH % NT == 0, "tile split");
  // LDS: two K buffers, then two V buffers.
  constexpr int KBUF = S::K_ELEMS, VBUF = S::V_ELEMS;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* const kbuf0 = smem;
  uint16_t* const vbuf0 = smem + 2 * KBUF;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const bool grpA = wave < 4;
  const int rowblk = 2 * (wave & 3) + (grpA ? 0 : 1);  // 32-row block inside the 256-row tile
  const int64_t off = int64_t(Lk) - Lq;
  const int n_mask_cols = (Lk + kMaskTile - 1) / kMaskTile;
  const int64_t per_xcd = n_items / 8;
  const uint32_t head_bytes = uint32_t(Lk) * D * 2;

  uint32_t ld_goff[LD];
  int ld_row[LD], ld_c[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int idx = t + i * NT;
    ld_row[i] = idx / KCH;
    ld_c[i] = idx % KCH;
    ld_goff[i] = uint32_t(ld_row[i] * D * 2 + 16 * ld_c[i]);
  }
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int64_t g = blockIdx.x; g < n_items; g += gridDim.x) {
    const int64_t item = xcd_remap ? (g % 8) * per_xcd + g / 8 : g;
    const int64_t bh = item / n_qt;
    const int qr = int(item % n_qt);
    const int q0 = (causal ? (n_qt - 1 - qr) : qr) * BM;
    const int q0w = q0 + 32 * rowblk;
    const uint16_t* qh = q + bh * int64_t(Lq) * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + bh * int64_t(Lk) * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + bh * int64_t(Lk) * D, head_bytes);

    int64_t last_key = int64_t(min(q0 + BM, Lq) - 1) + (causal ? off : int64_t(Lk));
    if (last_key > Lk - 1) last_key = Lk - 1;
    const int kt_end = last_key < 0 ? 0 : int(last_key / kBN) + 1;
    TileWalker walk{block_mask, n_mask_cols, q0 / kMaskTile, min(q0 + BM - 1, Lq - 1) / kMaskTile,
                    min(q0w, Lq - 1) / kMaskTile, kt_end, kBN};
    auto visible = [&](int kt, bool mine) {
      return (!causal || int64_t(kt) * kBN <= int64_t(q0w) + 31 + off) && q0w < Lq && mine;
    };

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
      // The Q fragments are complete before the sweep, so the loop's waits only
      // ever concern the tile prefetches.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_ref = kNegInf;
    float l_run = 0.f;
    const int64_t row_last = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
    const int row_lim = int(row_last < int64_t(Lk) - 1 ? (row_last < -1 ? -1 : row_last) : int64_t(Lk) - 1);

    f32x16_t st[2];
    uint32_t pk[2][8];
    uint4 kst[LD], vst[LD];
    auto load_k = [&](int kt) {
      const uint32_t base = uint32_t(kt) * kBN * D * 2;
#pragma unroll
      for (int i = 0; i < LD; ++i) kst[i] = buf_load16(krs, base + ld_goff[i]);
    };
    auto load_v = [&](int kt) {
      const uint32_t base = uint32_t(kt) * kBN * D * 2;
#pragma unroll
      for (int i = 0; i < LD; ++i) vst[i] = buf_load16(vrs, base + ld_goff[i]);
    };
    auto store_k = [&](int b) {
#pragma unroll
      for (int i = 0; i < LD; ++i)
        *reinterpret_cast<uint4*>(kbuf0 + b * KBUF + ld_row[i] * S::KROW + 8 * ld_c[i]) = kst[i];
    };
    auto store_v = [&](int b) {
#pragma unroll
      for (int i = 0; i < LD; ++i)
        *reinterpret_cast<uint4*>(vbuf0 + b * VBUF + ld_row[i] * S::VROW + 8 * ld_c[i]) = vst[i];
    };

    // Matrix-core block: O += V(prev)^T P(prev)^T, then S = K(cur) Q^T.
    auto mblock = [&](bool do_pv, int vb, bool do_s, int kb) {
      if (do_pv) {
        const uint16_t* vs_ = vbuf0 + vb * VBUF;
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
      if (do_s) {
        const uint16_t* ks_ = kbuf0 + kb * KBUF;
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
      }
    };
    // Vector block: online softmax update of S(kt) into P.
    auto vblock = [&](int kt) {
      const int k0 = kt * kBN;
      const bool edge = (causal && int64_t(k0) + kBN - 1 > int64_t(q0w) + off) || (k0 + kBN > Lk);
      if (edge) {
        const int lim = row_lim - k0 - 4 * h;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mb + 8 * (r >> 2) + (r & 3) > lim) st[mb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
      mx = pair_max_halves(mx);
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
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(st[mb][r], c_log2, -mu));
          const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_log2, -mu));
          l_run += p0 + p1;
          pk[mb][r >> 1] = cvt_pk_bf16(p0, p1);
        }
    };

    __syncthreads();  // the previous item's readers of every buffer are done
    // Prologue: K(t0) into K buffer 0; stage K(t1) and V(t0).
    bool m_cur = false, m_nxt = false;
    int t_cur = walk.next(0, &m_cur);
    int t_nxt = t_cur < kt_end ? walk.next(t_cur + 1, &m_nxt) : kt_end;
    if (t_cur < kt_end) {
      load_k(t_cur);
      store_k(0);
      load_v(t_cur);
      if (t_nxt < kt_end) load_k(t_nxt);
      pin_memory_order();
    }
    __syncthreads();

    // n-th active tile: t_cur. prev: the tile whose V / P are pending (t_prev).
    int t_prev = kt_end;  // none yet
    bool vis_prev = false;
    int n = 0;
    while (true) {
      const bool have_cur = t_cur < kt_end;
      const bool have_prev = t_prev < kt_end;
      if (!have_cur && !have_prev) break;
      const bool vis_cur = have_cur && visible(t_cur, m_cur);
      const int kb = n & 1, vb = (n - 1) & 1;
      // ---- phase 2n ----
      if (grpA) {
        mblock(have_prev && vis_prev, vb, vis_cur, kb);
      } else if (have_prev && vis_prev) {
        vblock(t_prev);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      // ---- phase 2n+1 ----
      if (grpA) {
        if (vis_cur) vblock(t_cur);
      } else {
        mblock(have_prev && vis_prev, vb, vis_cur, kb);
      }
      // K(next) and V(cur) go to LDS; then the next loads are issued.
      bool m_nn = false;
      const int t_nn = t_nxt < kt_end ? walk.next(t_nxt + 1, &m_nn) : kt_end;
      if (t_nxt < kt_end) store_k((n + 1) & 1);
      if (have_cur) store_v(n & 1);
      if (t_nxt < kt_end) load_v(t_nxt);
      if (t_nn < kt_end) load_k(t_nn);
      pin_memory_order();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      t_prev = t_cur;
      vis_prev = vis_cur;
      t_cur = t_nxt;
      m_cur = m_nxt;
      t_nxt = t_nn;
      m_nxt = m_nn;
      ++n;
    }
    // Group B's last softmax already ran in the final phase 2n (as vblock(t_prev)) and
    // its last P.V in the final phase 2n+1; group A finished its P.V in the final phase 2n.

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

template <int D>
hipError_t launch_pp(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                     int Lk, float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  constexpr int BM = 256;
  const int n_qt = (Lq + BM - 1) / BM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  int q_mode = 0;
  float c = float(double(scale) * 1.4426950408889634);
  if (scale < 0.f) {
    q_mode = 1;
    c = -c;
  } else if (scale == 0.f) {
    q_mode = 2;
    c = 1.f;
  }
  const int64_t cap = 1LL << 22;
  const unsigned grid = unsigned(n_items < cap ? n_items : cap);
  const int xcd_remap = (n_items % 8 == 0 && n_items <= cap) ? 1 : 0;
  const size_t shmem = Smem<D>::BYTES;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attention_bf16_pp_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
      int(shmem));
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL((attention_bf16_pp_kernel<D>), dim3(grid), dim3(512), shmem, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                     block_mask, n_qt, n_items, xcd_remap);
  return hipGetLastError();
}

// Score coefficient in log2 units. The kernels take it positive: a negative
// scale negates Q as it is loaded (q_mode 1), a zero scale zeroes it (q_mode 2).
inline float score_coef(float scale, int* q_mode) {
  float c = float(double(scale) * 1.4426950408889634);
  *q_mode = 0;
  if (scale < 0.f) {
    *q_mode = 1;
    c = -c;
  } else if (scale == 0.f) {
    *q_mode = 2;
    c = 1.f;
  }
  return c;
}

template <int D, int NW, int WPE, int BN, bool SP, bool BITS = false>
hipError_t launch_dma(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                      int Lk, float scale, int causal, const uint8_t* block_mask, hipStream_t stream,
                      const uint64_t* tile_bits = nullptr) {
  constexpr int BM = 32 * NW;
  const int n_qt = (Lq + BM - 1) / BM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  int q_mode = 0;
  const float c = score_coef(scale, &q_mode);
  const int64_t cap = 1LL << 22;
  const unsigned grid = unsigned(n_items < cap ? n_items : cap);
  const int xcd_remap = (n_items % 8 == 0 && n_items <= cap) ? 1 : 0;
  // Bytes of the row-bitmap array (validated below 2^32 at the boundary).
  const uint32_t bits_bytes =
      BITS ? uint32_t(int64_t((Lq + kMaskTile - 1) / kMaskTile) * ((Lk + kMaskTile - 1) / kMaskTile) * 512) : 0u;
  if constexpr (SP) {
    // One workgroup per item; more items than one grid allows go in chunks
    // (then without the XCD placement, which assumes the whole item range).
    for (int64_t base = 0; base < n_items; base += cap) {
      const int64_t n = n_items - base < cap ? n_items - base : cap;
      hipLaunchKernelGGL((attention_bf16_sp_kernel<D, NW, WPE, BITS>), dim3(unsigned(n)), dim3(NW * 64), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                         block_mask, n_qt, n, xcd_remap, (causal && xcd_remap) ? RF_ATT_HEAD_GROUP : 1, base,
                         tile_bits, bits_bytes);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else
    hipLaunchKernelGGL((attention_bf16_dma_kernel<D, NW, WPE, BN>), dim3(grid), dim3(NW * 64), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                       block_mask, n_qt, n_items, xcd_remap);
  return hipGetLastError();
}


// Split-KV partials (no mask): items (head, split, query tile), key tiles
// divided into n_splits contiguous ranges of ceil(n_tiles / n_splits) tiles.
template <int D, int NW, int WPE>
hipError_t launch_split(const void* q, const void* k, const void* v, float* ws_o, float* ws_lse, int n_heads, int Lq,
                        int Lk, float scale, int n_splits, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const int n_qt = (Lq + BM - 1) / BM;
  const int n_kt = (Lk + 63) / 64;
  const int kt_split = (n_kt + n_splits - 1) / n_splits;
  const int64_t n_items = int64_t(n_heads) * n_splits * n_qt;
  int q_mode = 0;
  const float c = score_coef(scale, &q_mode);
  const int64_t cap = 1LL << 22;
  const int xcd_remap = (n_items % 8 == 0 && n_items <= cap) ? 1 : 0;
  for (int64_t base = 0; base < n_items; base += cap) {
    const int64_t n = n_items - base < cap ? n_items - base : cap;
    hipLaunchKernelGGL((attention_bf16_sp_kernel<D, NW, WPE, false, true>), dim3(unsigned(n)), dim3(NW * 64), 0,
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), nullptr, nullptr, Lq, Lk, c, q_mode, 0, nullptr, n_qt, n,
                       xcd_remap, 1, base, nullptr, 0u, n_splits, kt_split, ws_o, ws_lse);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attention_bf16_split(const void* q, const void* k, const void* v, float* ws_o, float* ws_lse,
                                       int n_heads, int Lq, int Lk, int d, float scale, int n_splits,
                                       hipStream_t stream) {
  if (d == 128)
    return launch_split<128, RF_ATT_NW_D128, RF_ATT_WPE_D128>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale,
                                                               n_splits, stream);
  return launch_split<64, RF_ATT_NW_D64, RF_ATT_WPE_D64>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale, n_splits,
                                                          stream);
}

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Lq, int Lk, int d, float scale, int causal, const uint8_t* block_mask,
                                 const uint64_t* tile_bits, hipStream_t stream) {
  if (tile_bits != nullptr) {  // element bitmaps: the pipelined kernel only
    if (d == 128)
      return launch_dma<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, 64, true, true>(q, k, v, o, lse, B, H, Lq, Lk, scale,
                                                                             causal, block_mask, stream, tile_bits);
    return launch_dma<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, 64, true, true>(q, k, v, o, lse, B, H, Lq, Lk, scale,
                                                                        causal, block_mask, stream, tile_bits);
  }
#if RF_ATT_DMA
  if (d == 128)
    return launch_dma<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, RF_ATT_SP ? 64 : RF_ATT_BN_D128, bool(RF_ATT_SP)>(
        q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask, stream);
  return launch_dma<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, RF_ATT_SP ? 64 : RF_ATT_BN_D64, bool(RF_ATT_SP)>(
      q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask, stream);
#endif
  if (d == 128) {
#if RF_ATT_PINGPONG_D128
    return launch_pp<128>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask, stream);
#else
    return launch_kernel<128, RF_ATT_NW_D128, RF_ATT_WPE_D128>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                block_mask, stream);
#endif
  }
  return launch_kernel<64, RF_ATT_NW_D64, RF_ATT_WPE_D64>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask,
                                                           stream);
}

}  // namespace rf
