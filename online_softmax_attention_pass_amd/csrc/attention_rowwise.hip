// Row-wise masked attention: the row kernel of the STOF page (Méthodologie 1,
// dual-kernel strategy: for highly sparse masks and short sequences, Q is cut
// into rows, lanes of a warp reduce together and no synchronisation crosses
// warps), for bf16 with the same masks as the tile kernel: causal rule, tile
// kinds (0 empty, 1 full, other = partial) and, inside partial tiles, one
// 64-bit row word per tile row (bit j: key j of the tile is visible).
//
// One wavefront owns one query row and walks only the key tiles its mask row
// keeps; their visible keys, in order, are gathered into batches of KB keys,
// so a sparse row costs its visible keys, not whole 64 x 64 tiles. Lanes are
// laid out as in the split-KV decode kernel: D/8 lanes share a key (8 elements
// of d each, 16-byte coalesced loads), KPW = 64 / (D/8) keys per load step, U
// steps per batch; each group of D/8 lanes keeps its own online (m, l, acc),
// and the groups meet in the (m, l, acc) monoid at the end. Scores are in log2
// units.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"
#include "rows_io.h"

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
    const uint8_t* __restrict__ tile_kind, const uint64_t* __restrict__ tile_bits, int64_t n_rows,
    int xcd_remap) {
  constexpr int LPK = D / 8;     // lanes per key
  constexpr int KPW = 64 / LPK;  // keys per load step
  constexpr int KB = KPW * U;    // keys per batch
  static_assert(KB <= 32, "a batch fits the ring with a tile's worth of room");
  __shared__ int s_pend[4][64];  // per wave: the ring of pending visible keys
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPK;  // which key of a load step
  const int ds = lane % LPK;   // this lane's 8-element slice of d
  int* pend = s_pend[wave];
  const int n_cols = (Lk + kRowTile - 1) / kRowTile;
  const int64_t off = int64_t(Lk) - Lq;  // bottom-right causal alignment

  // The hardware deals consecutive workgroups to the 8 XCDs in turn; with
  // xcd_remap, XCD x takes the x-th eighth of the rows instead, so the rows of
  // a head run on one XCD and its L2 serves the keys they share (window and
  // global keys).
  const int64_t n_wg = gridDim.x;
  const int64_t blk = xcd_remap ? (blockIdx.x % 8) * (n_wg / 8) + blockIdx.x / 8 : int64_t(blockIdx.x);
  for (int64_t row = blk * 4 + wave; row < n_rows; row += n_wg * 4) {
    const int64_t bh = row / Lq;
    const int i = int(row % Lq);
    const uint4 qv = *reinterpret_cast<const uint4*>(q + row * D + 8 * ds);
    // K and V of the head as buffer resources: a hidden key's lanes load from
    // an offset past the end, which reads 0 without touching memory, so every
    // group issues the same loads and their count is known to the compiler.
    const uint32_t head_bytes = uint32_t(Lk) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = row_rsrc(k + bh * int64_t(Lk) * D, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = row_rsrc(v + bh * int64_t(Lk) * D, head_bytes);
    // last visible key of the row (causal rule and sequence end)
    int64_t last = causal ? int64_t(i) + off : int64_t(Lk) - 1;
    if (last > Lk - 1) last = Lk - 1;
    const int j_end = last < 0 ? 0 : int(last / kRowTile) + 1;
    const int64_t mrow = int64_t(i / kRowTile) * n_cols;

    float m = kNegInf, l = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    // The row's visible keys, gathered into batches of KB keys (in a fixed
    // order: per chunk of 64 tiles, the sparse tiles' keys, then the dense
    // tiles'). The mask is read 64 tiles at a time: lane j reads tile J0 + j's
    // kind and this row's word of it. A dense tile's word comes back to the
    // whole wave by readlane, and its set bits are appended to this wave's list
    // of pending keys in LDS (a 64-entry ring): lane j writes key k0 + j at its
    // rank among the set bits.
    // Tiles with at most kSparse visible keys (most of a sparse row) are not
    // visited one by one: every lane holding such a tile writes its keys at
    // once, at positions from a wave-wide exclusive scan of the counts (three
    // ballots of the count's bits and mbcnt), as long as the ring has room.
    // Denser tiles go one at a time, all lanes writing one key each.
    constexpr int kSparse = 4;
    int J0 = -kRowTile, k0 = 0, head = 0, n_pend = 0;
    uint64_t wl = 0, todo = 0, word = 0, ws = 0;  // ws: this lane's sparse tile keys still to take
    bool sparse_left = false;
    auto mbcnt64 = [](uint64_t m) {
      return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
    };
    auto fill = [&]() {
      while (n_pend < KB) {
        if (sparse_left) {
          const int cnt = __builtin_popcountll(ws);  // 0 .. kSparse
          const uint64_t b0 = __builtin_amdgcn_ballot_w64((cnt & 1) != 0);
          const uint64_t b1 = __builtin_amdgcn_ballot_w64((cnt & 2) != 0);
          const uint64_t b2 = __builtin_amdgcn_ballot_w64((cnt & 4) != 0);
          const int excl = mbcnt64(b0) + 2 * mbcnt64(b1) + 4 * mbcnt64(b2);
          const int total = __builtin_popcountll(b0) + 2 * __builtin_popcountll(b1) + 4 * __builtin_popcountll(b2);
          const int room = 64 - n_pend;
          uint64_t w = ws;
#pragma unroll
          for (int j = 0; j < kSparse; ++j)
            if (w != 0 && excl + j < room) {
              pend[(head + n_pend + excl + j) & 63] = (J0 + lane) * kRowTile + __builtin_ctzll(w);
              w &= w - 1;
            }
          ws = w;
          n_pend += total < room ? total : room;
          sparse_left = __builtin_amdgcn_ballot_w64(ws != 0) != 0;
          continue;
        }
        if (word == 0) {
          if (todo == 0) {
            J0 += 64;
            if (J0 >= j_end) return;
            const int Jl = J0 + lane;
            wl = 0;
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
            const bool dense = __builtin_popcountll(wl) > kSparse;
            ws = dense ? 0 : wl;
            todo = __builtin_amdgcn_ballot_w64(dense);
            sparse_left = __builtin_amdgcn_ballot_w64(ws != 0) != 0;
            continue;
          }
          const int jl = __builtin_ctzll(todo);
          todo &= todo - 1;
          const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(wl), jl);
          const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(wl >> 32), jl);
          word = (uint64_t(hi) << 32) | lo;
          k0 = (J0 + jl) * kRowTile;
        }
        // Take as many of the dense tile's keys as the ring has room for.
        const int rank = mbcnt64(word);
        const bool take = ((word >> lane) & 1) != 0 && rank < 64 - n_pend;
        if (take) pend[(head + n_pend + rank) & 63] = k0 + lane;
        const uint64_t taken = __builtin_amdgcn_ballot_w64(take);
        n_pend += __builtin_popcountll(taken);
        word &= ~taken;
      }
    };
    // The next batch: lane (u, sub) gets key u KPW + sub of it, or -1 past its
    // end; returns the batch size (0 when the row is done).
    auto take_batch = [&](int (&key)[U]) {
      fill();
      const int nb = n_pend < KB ? n_pend : KB;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sl = u * KPW + sub;
        key[u] = sl < nb ? pend[(head + sl) & 63] : -1;
      }
      head = (head + nb) & 63;
      n_pend -= nb;
      return nb;
    };
    // Loads of one batch: this lane's 16 bytes of its key, or 0 (an offset past
    // the end reads 0 without touching memory).
    auto issue = [&](const int (&key)[U], uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t boff = key[u] >= 0 ? uint32_t(key[u]) * (D * 2) + 16u * uint32_t(ds) : 0x80000000u;
        const buf_u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rk, int(boff), 0, kBufNonTemporal);
        const buf_u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rv, int(boff), 0, kBufNonTemporal);
        kr[u] = make_uint4(a[0], a[1], a[2], a[3]);
        vr[u] = make_uint4(b[0], b[1], b[2], b[3]);
      }
    };
    // The online update with one batch.
    auto consume = [&](const int (&key)[U], const uint4 (&kr)[U], const uint4 (&vr)[U]) {
      float ts[U];
      float bm = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dsum = dot2_bf16r(kr[u].x, qv.x, 0.f);
        dsum = dot2_bf16r(kr[u].y, qv.y, dsum);
        dsum = dot2_bf16r(kr[u].z, qv.z, dsum);
        dsum = dot2_bf16r(kr[u].w, qv.w, dsum);
        dsum = group_sum<LPK>(dsum);
        ts[u] = key[u] >= 0 ? dsum * scale_log2 : kNegInf;
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
    };
    // Two batches in flight: the next batch's loads go out before the current
    // one is consumed (unrolled by two, so no register copies).
    int key_a[U], key_b[U];
    uint4 ka[U], va[U], kb2[U], vb2[U];
    bool have_a = take_batch(key_a) > 0;
    if (have_a) issue(key_a, ka, va);
    while (have_a) {
      const bool have_b = take_batch(key_b) > 0;
      if (have_b) issue(key_b, kb2, vb2);
      consume(key_a, ka, va);
      if (!have_b) break;
      have_a = take_batch(key_a) > 0;
      if (have_a) issue(key_a, ka, va);
      consume(key_b, kb2, vb2);
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
  const int xcd_remap = grid % 8 == 0 ? 1 : 0;
  const float scale_log2 = float(double(scale) * 1.4426950408889634);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(o);
  if (d == 128)
    hipLaunchKernelGGL((attention_rowwise_kernel<128, 4>), dim3(grid), dim3(256), 0, stream, qq, kk, vv, oo, lse, Lq,
                       Lk, scale_log2, causal, tile_kind, tile_bits, n_rows, xcd_remap);
  else
    hipLaunchKernelGGL((attention_rowwise_kernel<64, 4>), dim3(grid), dim3(256), 0, stream, qq, kk, vv, oo, lse, Lq,
                       Lk, scale_log2, causal, tile_kind, tile_bits, n_rows, xcd_remap);
  return hipGetLastError();
}

}  // namespace rf
