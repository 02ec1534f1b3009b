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
//   - Each wave runs its stages one tile apart: the score
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
//   - A split mode cuts each head's key tiles into contiguous ranges and writes
//     normalised fp32 partials with their LSE for a log-sum-exp merge (decode
//     with grouped queries: the query heads sharing a key/value head are the
//     rows of one query tile).
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"

namespace rf {
namespace {

// Launch shape per head dim: waves per workgroup (32 query rows each) and
// waves per SIMD the register allocation must allow.
#ifndef RF_SPLIT_SMALL_TILES
#define RF_SPLIT_SMALL_TILES 1
#endif
#ifndef RF_ATT_NW_D128
#define RF_ATT_NW_D128 4
#endif
#ifndef RF_ATT_WPE_D128
#define RF_ATT_WPE_D128 2
#endif
#ifndef RF_ATT_NW_D64
#define RF_ATT_NW_D64 2
#endif
#ifndef RF_ATT_PRIO
#define RF_ATT_PRIO 1
#endif
#ifndef RF_ATT_SREAD_AHEAD_D128
#define RF_ATT_SREAD_AHEAD_D128 2
#endif
#ifndef RF_ATT_SREAD_AHEAD
#define RF_ATT_SREAD_AHEAD 4
#endif
#ifndef RF_ATT_VREAD_AHEAD
#define RF_ATT_VREAD_AHEAD 2
#endif
#ifndef RF_ATT_SPLIT_NT
#define RF_ATT_SPLIT_NT 1
#endif
#ifndef RF_ATT_HEAD_GROUP
#define RF_ATT_HEAD_GROUP 2
#endif
#ifndef RF_ATT_SP_SCHED
#define RF_ATT_SP_SCHED 1
#endif
#ifndef RF_ATT_WPE_D64
#define RF_ATT_WPE_D64 2
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// Cache-policy bit of a buffer load: non-temporal.
constexpr int kLoadNonTemporal = 2;

// Raw buffer access: loads outside [0, bytes) return zero, so ragged tiles
// need no predication.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte rows supplied by lanes i/4,
// i/4 + 4, i/4 + 8, i/4 + 12 of its group.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

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

// Score modifications of one call. The MOD kernel instance turns each score
// tile into log2-unit scores t = scale log2(e) (q . k) and then applies, in this
// order, a softcap t <- cap2 tanh(t / cap2) (cap2 = softcap log2 e, the natural
// softcap moved to log2 units) and an ALiBi bias t <- t + slope_h log2(e)
// (j - p_i), p_i = i + Lk - Lq; a window keeps keys j > p_i - window.
struct ScoreMod {
  const float* slopes = nullptr;  // ALiBi slope per head (natural units per position), or none
  int H = 1;                      // heads: the slope of item head bh is slopes[bh % H]
  float cap2 = 0.f;               // softcap in log2 units, 0 = none
  float tk = 0.f;                 // 2 log2(e) / cap2: tanh(y) = 1 - 2 / (1 + 2^(t tk)), y = t / cap2
  int window = 0;                 // keys per row window, 0 = none
  int rev = 0;                    // visit the key tiles last to first (no block mask only)
};

// Walks the key tiles a workgroup must visit, in order. Without a block mask it
// is every tile below kt_end. With one, the mask bytes of the next 64 tiles are
// read once per 64 tiles (one byte per lane) and turned into two wave-uniform
// 64-bit words by ballot: tiles active for any of the workgroup's mask rows, and
// tiles active for this wave's own mask row. The scan itself is scalar bit work.
// ONE_ROW: the workgroup's rows are one mask row (64 query rows), so a wave's
// own words are the workgroup's and are not kept twice.
template <bool ONE_ROW, int MR>
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

  // This lane's mask bytes for tile b + lane, one per mask row of the
  // workgroup (MR rows at most): unconditional loads of clamped (valid)
  // addresses, without waiting for them; apply_kinds drops what the clamp
  // stood in for.
  __device__ void load_kinds(int b, uint32_t (&kinds)[MR]) const {
    const int kt = b + int(threadIdx.x & 63);
    const int mc = min(kt * bn / kMaskTile, n_mask_cols - 1);
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int mr = min(mr0 + i, ONE_ROW ? mr0 : mr1);
      kinds[i] = mask[int64_t(mr) * n_mask_cols + mc];
    }
  }
  __device__ void refill(int b) {
    uint32_t kinds[MR];
    load_kinds(b, kinds);
    apply_kinds(b, kinds);
  }
  // The tile words of tiles b .. b + 63 from the lanes' mask bytes.
  __device__ void apply_kinds(int b, const uint32_t (&kinds)[MR]) {
    bool any = false, mine = false, part = false, anypart = false;
    const bool in_range = b + int(threadIdx.x & 63) < kt_end;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const uint32_t kind = (in_range && mr0 + i <= (ONE_ROW ? mr0 : mr1)) ? kinds[i] : 0u;
      const bool a = kind != 0;
      const bool pa = bits && kind != 0 && kind != 1;
      any |= a;
      mine |= (ONE_ROW || mr0 + i == mr_w) && a;
      anypart |= pa;
      part |= (ONE_ROW || mr0 + i == mr_w) && pa;
    }
    wg_bits = __builtin_amdgcn_ballot_w64(any);
    if (!ONE_ROW) wv_bits = __builtin_amdgcn_ballot_w64(mine);
    if (bits) {
      pg_bits = __builtin_amdgcn_ballot_w64(anypart);
      if (!ONE_ROW) pv_bits = __builtin_amdgcn_ballot_w64(part);
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
        *mine = ONE_ROW ? true : ((wv_bits >> (kt - base)) & 1) != 0;
        if (part != nullptr) {
          const int pg = int((pg_bits >> (kt - base)) & 1);
          *part = ONE_ROW ? pg * 3 : (int((pv_bits >> (kt - base)) & 1) | (pg << 1));
        }
        return kt;
      }
      kt = base + 64;
    }
    *mine = false;
    return kt_end;
  }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS tiles. K and V travel global -> LDS with buffer loads that write
// LDS themselves (no staging registers, no LDS store instructions). Such a load
// writes lane i's 16 bytes at (LDS base + 16 i), so a tile lands as unpadded
// rows; bank conflicts are avoided by XOR-swizzling the 16-byte chunks of each
// row instead: K chunk c of row r sits in slot c ^ (r mod KCH), which spreads the
// 16 rows that one 16-lane read touches over 16 slots; V chunk c of row r sits in
// slot c ^ s(r mod 4) (s = 4 for d = 128, 2 for d = 64), which spreads the 4 rows
// x 2 chunks of one transposed 16-lane read over 8 slots.
// ---------------------------------------------------------------------------
template <int D>
struct Swz {
  static constexpr int KCH = D / 8;
  static constexpr int VX = D >= 128 ? 4 : 2;
  __device__ static int k_slot(int row, int c) { return c ^ (row & (KCH - 1)); }
  __device__ static int v_slot(int row, int c) { return c ^ (VX * (row & 3)); }
};

// One wave-wide direct-to-LDS load of 1 KiB of tile row bitmaps into bb
// (lane i writes bytes 16 i .. 16 i + 15); off is this lane's byte offset.
__device__ __forceinline__ void dma_bits(const uint64_t* bits, uint32_t bytes, uint64_t* bb, uint32_t off) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(bits, bytes);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(bb), 16, off, 0, 0, 0);
}

// One tensor's share of a tile: this wave's n direct-to-LDS instructions.
// Each instruction's LDS destination (M0) is formed from one opaque base at
// the point of use: otherwise the compiler keeps every (buffer, instruction)
// destination of the loop in its own scalar register, and under pressure
// spills them to vector lanes and reloads one before each load.
// AUX is the loads' cache policy (kLoadNonTemporal for data read once).
// The tile's first byte (base < head_bytes) becomes the resource's base, by
// scalar arithmetic, so the lanes' offsets go in unchanged: no vector add per
// instruction. The range still ends where the head does, so rows past the
// last key read zero.
template <int AUX = 0>
__device__ __forceinline__ void dma_one(const uint16_t* head, uint32_t head_bytes, uint16_t* dst, uint32_t base,
                                        const uint32_t* lane_off, int ins0, int n) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char*>(head) + base, head_bytes - base);
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  uint32_t lds = uint32_t((uintptr_t)(lds_u8*)dst) + uint32_t(ins0) * 1024u;
  asm volatile("" : "+s"(lds));
#pragma unroll
  for (int j = 0; j < n; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(uintptr_t)(lds + j * 1024u),
                                             16, lane_off[j], 0, 0, AUX);
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
// Software-pipelined attention kernel.
//
// Within one wave the three stages of a key tile (score product, softmax
// update, P.V product) depend on each other, so run back to back they leave
// the matrix core idle during the exponentials and the vector ALU idle during
// the products. Here every wave runs them one tile apart, in three phases per
// step (tile j current, tile j+1 next):
//
//   phase A :  S(j+1) = K(j+1) Q^T          with P = exp of keys 0..31 of tile j
//   phase B1:  O^T += V^T P^T, keys 0..31   with P = exp of keys 32..63 of tile j
//   phase B2:  O^T += V^T P^T, keys 32..63
//
// so each phase pairs a run of MFMAs with independent vector work. Every
// tile's K and V are loaded one step ahead (K of tile j+2 and V of tile j+1
// during step j), double-buffered; one barrier per half-step publishes the
// loads issued in the half-step before it and frees the buffers read there.
//
// P is formed against a lazy reference m: while a lane's sum of its 16 P of a
// half tile stays within 2^kRescaleSlack (so every P is within the bound) the
// P are kept; otherwise the half tile's exact maximum decides, and when it
// exceeds m by more than the slack, m moves, O and the sums are rescaled and
// that half's P is formed again (the sum guard, commit_half).
// ---------------------------------------------------------------------------
//
// SPLIT: split-KV partials. Item = (head, split, query tile); split s visits
// key tiles [s kt_split, (s + 1) kt_split) only, and writes its output,
// normalised, in fp32 with its LSE into ws_o [head rows, n_splits, D] and
// ws_lse [head rows, n_splits] for a log-sum-exp merge. Used for decode with
// grouped queries, where the query heads sharing one key/value head are the
// rows of the query tile.
//
// MOD: score modifications (ScoreMod) applied to each score tile before the mask;
// 1 = bias and window, 2 = also the softcap.
//
// MASK: whether the call has a block mask (or tile kinds); without one the tile
// walk is a plain count and its state takes no registers.
template <int D, int NW, int WPE, bool BITS, bool SPLIT = false, int MOD = 0, bool MASK = true>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attention_bf16_sp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, float c_log2, int q_mode, int causal,
    const uint8_t* __restrict__ block_mask, int n_qt, int64_t n_items, int xcd_remap, int head_group,
    int64_t item_base, const uint64_t* __restrict__ tile_bits, uint32_t bits_bytes, int n_splits = 1,
    int kt_split = 0, float* __restrict__ ws_o = nullptr, float* __restrict__ ws_lse = nullptr,
    ScoreMod mod = ScoreMod{}) {
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
  // K fragments read ahead of the score MFMAs: two at d = 128 measured 0.8%
  // faster on causal prefill than four (with the wave priority below).
  constexpr int kSreadAhead = D >= 128 ? RF_ATT_SREAD_AHEAD_D128 : RF_ATT_SREAD_AHEAD;
  static_assert(kSreadAhead > 0, "read-ahead");

  // Split (decode) items stream their K and V once, with no reuse by other
  // items: their direct-to-LDS loads are non-temporal (1.25 against 1.41 ms
  // on grouped-query decode, 0.184 against 0.210 ms on the shared cache).
  // Prefill-type items re-read K and V through the L2, and lose with it
  // (0.61 against 0.545 ms on causal prefill).
  constexpr int kKVAux = (SPLIT && RF_ATT_SPLIT_NT != 0) ? kLoadNonTemporal : 0;
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
    // Output addresses of this wave's rows. The masked instances form them
    // here and hold them in VGPRs until the epilogue: as scalars they stayed
    // live across the tile walk and took its spill slots. The others form
    // them in the epilogue.
    uint16_t* obase_m = nullptr;
    float* lse_m = nullptr;
    int rows_m = 0;
    if constexpr (MASK && !SPLIT) {
      obase_m = o + (bh * Lq + q0w) * int64_t(D);
      lse_m = lse != nullptr ? lse + bh * Lq + q0w : nullptr;
      rows_m = Lq - q0w;
      asm volatile("" : "+v"(obase_m), "+v"(lse_m), "+v"(rows_m));
    }

    int64_t last_key = int64_t(min(q0 + BM, Lq) - 1) + (causal ? off : int64_t(Lk));
    if (last_key > Lk - 1) last_key = Lk - 1;
    const int kt_all = last_key < 0 ? 0 : int(last_key / BN) + 1;
    // With a window, tiles wholly before the first row's lowest key are skipped.
    const int64_t lo_first = int64_t(q0) + off - mod.window + 1;
    const int kt_begin = SPLIT ? split * kt_split : ((MOD && mod.window > 0 && lo_first > 0) ? int(lo_first / BN) : 0);
    const int kt_end = SPLIT ? min(kt_all, kt_begin + kt_split) : kt_all;
    TileWalker<BM == kMaskTile, (BM + kMaskTile - 1) / kMaskTile> walk{
        MASK ? block_mask : nullptr, n_mask_cols, q0 / kMaskTile, min(q0 + BM - 1, Lq - 1) / kMaskTile,
        min(q0w, Lq - 1) / kMaskTile, kt_end, BN};
    walk.bits = BITS;
    // The item's first memory accesses go out together: the mask bytes of its
    // first 64 key tiles, then its Q rows; only then is the mask read (to pick
    // the first K and V tiles), and one wait before the first score product
    // covers Q and those tiles: two memory latencies instead of three.
    uint32_t kinds0[(BM + kMaskTile - 1) / kMaskTile];
    const bool first_kinds = MASK && block_mask != nullptr && kt_begin < kt_end;
    if (first_kinds) walk.load_kinds(kt_begin & ~63, kinds0);

    uint4 qf[KSTEPS];
    if constexpr (MOD == 0) {
      // The wave's 32 rows through a buffer resource that covers only them:
      // rows past Lq read as zero, with no branch around each load.
      const int n_rows = __builtin_amdgcn_readfirstlane(max(0, min(32, Lq - q0w)));
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh + int64_t(q0w) * D, uint32_t(n_rows) * D * 2);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        qf[ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, (l32 * D + 16 * ks + 8 * h) * 2, 0, 0));
    } else {
      // (the score-modification instances keep plain loads and wait for them
      // here: their register allocation is tight, and this keeps it spill-free)
      const int qi = q0w + l32;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qi < Lq) x = *reinterpret_cast<const uint4*>(qh + int64_t(qi) * D + 16 * ks + 8 * h);
        qf[ks] = x;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (MASK) __builtin_amdgcn_sched_barrier(0);  // the Q loads stay ahead of the wait for the mask bytes
    if (first_kinds) {
      // the bytes stay raw until here, so the first wait for them comes after the Q loads
#pragma unroll
      for (int i = 0; i < (BM + kMaskTile - 1) / kMaskTile; ++i) asm volatile("" : "+v"(kinds0[i]));
      walk.apply_kinds(kt_begin & ~63, kinds0);
    }
    // A negative scale negates Q, a zero scale zeroes it (see score_coef);
    // applied once the loads have landed.
    auto q_modes = [&]() {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        uint4 x = qf[ks];
        if (q_mode == 1) { x.x ^= 0x80008000u; x.y ^= 0x80008000u; x.z ^= 0x80008000u; x.w ^= 0x80008000u; }
        if (q_mode == 2) x = make_uint4(0, 0, 0, 0);
        qf[ks] = x;
      }
    };

    f32x16_t acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_ref = kNegInf, l_run = 0.f, l_rnd = 0.f;
    const int64_t row_last = causal ? int64_t(q0w + l32) + off : int64_t(Lk) - 1;
    const int row_lim = int(row_last < int64_t(Lk) - 1 ? (row_last < -1 ? -1 : row_last) : int64_t(Lk) - 1);
    // Score modifications: scores become log2-unit t before the exponentials,
    // which then take them as they are.
    const float c_exp = MOD ? 1.f : c_log2;
    // This lane's query position (below 2^31: the boundary bounds Lk d 2 by 2^31).
    const int qpos = q0w + l32 + int(off);
    const float sl2 = (MOD && mod.slopes != nullptr) ? mod.slopes[bh % mod.H] * kLog2e : 0.f;
    // Window: this row's lowest visible key, and the largest such bound in the
    // wave (tiles starting below it need the element mask).
    const int64_t lo_row = int64_t(qpos) - mod.window + 1;
    const int row_lo = (MOD && mod.window > 0) ? int(lo_row < 0 ? 0 : (lo_row > Lk ? Lk : lo_row)) : 0;
    const int64_t lo_wave = int64_t(q0w + 31) + off - mod.window + 1;
    // The per-tile edge tests in 32 bits (one scalar each; the 64-bit forms
    // took register pairs the masked walk could not spare): a causal tile
    // needs the element mask when k0 > diag_edge, a window tile when
    // k0 < lo_edge. Clamping keeps both tests exact for any k0 in [0, Lk).
    auto clamp_i32 = [](int64_t x) { return int(x < INT32_MIN ? INT32_MIN : (x > INT32_MAX ? INT32_MAX : x)); };
    const int diag_edge = clamp_i32(int64_t(q0w) + off - (BN - 1));
    const int lo_edge = clamp_i32(lo_wave);

    // Key tile of walk position t: the walk runs first to last; with rev the
    // tiles are visited last to first (the diagonal first under an ALiBi
    // bias, so the reference starts at the row's largest scores).
    const bool rev = MOD && mod.rev != 0;
    auto tile = [&](int t) { return rev ? kt_begin + kt_end - 1 - t : t; };

    // ---- stage pieces (inlined into the phase bodies below) ----
    auto score_mfmas = [&](const uint16_t* ks_, f32x16_t (&sacc)[MB]) {
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[a][r] = 0.f;
      // K fragments in a rolling window of KAHEAD reads ahead of their product.
      constexpr int KAHEAD = kSreadAhead;
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
          const float p0 = fast_exp2(fmaf(st[mb][r], c_exp, -mu));
          const float p1 = fast_exp2(fmaf(st[mb][r + 1], c_exp, -mu));
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
    // Score modifications of a fresh score tile (before its mask): t = c S,
    // then the softcap, then the ALiBi bias. Lane (row l32, half h) holds key
    // k0 + 4 h + 32 mb + 8 (r / 4) + r % 4 in st[mb][r].
    auto mod_base = [&](int kt) { return sl2 * float(kt * BN + 4 * h - qpos); };
    auto mod_elem = [&](f32x16_t (&st)[MB], int mb, int r, float base) {
      const float bias = fmaf(sl2, float(32 * mb + 8 * (r >> 2) + (r & 3)), base);
      if constexpr (MOD == 2) {
        float t = st[mb][r] * c_log2;
        const float e = fast_exp2(t * mod.tk);
        t = fmaf(-2.f * mod.cap2, __builtin_amdgcn_rcpf(1.f + e), mod.cap2);
        st[mb][r] = t + bias;
      } else {
        st[mb][r] = fmaf(st[mb][r], c_log2, bias);
      }
    };
    auto mod_tile = [&](f32x16_t (&st)[MB], int kt) {
      if constexpr (MOD) {
        const float base = mod_base(kt);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mod_elem(st, mb, r, base);
      }
    };
    auto mask_tile = [&](f32x16_t (&st)[MB], int kt, bool mine, int part, uint64_t word) {
      const int k0 = kt * BN;
      const bool bitmap = BITS && (part & 1);
      const bool below_window = MOD && mod.window > 0 && k0 < lo_edge;
      const bool edge = !mine || bitmap || below_window || (causal && k0 > diag_edge) || (k0 + BN > Lk);
      if (edge) {
        const int lim = mine ? row_lim - k0 - 4 * h : -BN;
        const int lo = row_lo - k0 - 4 * h;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int idx = 32 * mb + 8 * (r >> 2) + (r & 3);
            if (idx > lim || (MOD && idx < lo)) st[mb][r] = kNegInf;
          }
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
      const float mt = mx * c_exp;
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
      const float p0 = fast_exp2(fmaf(st[mb][2 * r], c_exp, -mu));
      const float p1 = fast_exp2(fmaf(st[mb][2 * r + 1], c_exp, -mu));
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
    static_assert(MB == 2, "two halves per tile");
    // Wave priority: at d = 128 a wave issuing its score MFMAs (phase A) or
    // the pure MFMA run of phase B2 wins the SIMD's arbitration over the other
    // wave's softmax work, so the matrix core is fed first and that vector work
    // fills the cycles between MFMAs (about 2% on causal prefill). At d = 64,
    // where the vector work per MFMA doubles, it measured no better.
    constexpr bool kIssuePrio = RF_ATT_PRIO != 0 && D >= 128;
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
        constexpr int KAHEAD = kSreadAhead;
        auto kread = [&](int i) {
          const int kstep = i / MB, mb = i % MB;
          const int row = 32 * mb + l32;
          return *reinterpret_cast<const uint4*>(ks_next + row * D + 8 * SW::k_slot(row, 2 * kstep + h));
        };
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        uint4 kfrag[KAHEAD];
        if constexpr (kIssuePrio) __builtin_amdgcn_s_setprio(1);
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
        if constexpr (kIssuePrio) __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[0][i]));
      asm volatile("" ::"v"(lt0), "v"(ltr0));
      commit_half(s_cur, pk, 0, lt0, ltr0);
      // With score modifications, d = 64 runs them (and then the mask) in the
      // shadow of phase B2; d = 128 has no registers for the unmasked scores
      // to live that long and runs them here.
      constexpr bool MOD_IN_B2 = MOD != 0 && D <= 64;
      if constexpr (!MOD_IN_B2) {
        mod_tile(s_next, kt_next);
        mask_tile(s_next, kt_next, mine_next, part_next, D <= 64 ? word_next : row_word(part_next, bb_next));
      }
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
      if constexpr (MOD_IN_B2) {
        // Phase B2 issues only matrix-core work: the next tile's score
        // modifications run in its shadow, then its mask.
        constexpr int NB2 = NPV - NPV / 2;
        const float base = mod_base(kt_next);
        pv_range(vs_cur, pk, NPV / 2, NPV, [&](int j) {
#pragma unroll
          for (int e = j * 16 * MB / NB2; e < (j + 1) * 16 * MB / NB2; ++e) mod_elem(s_next, e / 16, e % 16, base);
#if RF_ATT_SP_SCHED
          __builtin_amdgcn_sched_barrier(0);
#endif
        });
        mask_tile(s_next, kt_next, mine_next, part_next, ~uint64_t(0));
      } else {
        if constexpr (kIssuePrio) __builtin_amdgcn_s_setprio(1);
        pv_range(vs_cur, pk, NPV / 2, NPV, [](int) {});
        if constexpr (kIssuePrio) __builtin_amdgcn_s_setprio(0);
      }
    };
    // The last tile: exponentials and P.V product only.
    auto finish = [&](const uint16_t* vs_cur, const f32x16_t (&s_cur)[MB]) {
      uint32_t pk[MB][8];
      float lt = 0.f, ltr = 0.f;
      exp_tile(s_cur, pk, lt, ltr);
      commit_tile(s_cur, pk, lt, ltr);
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
      dma_one<kKVAux>(khead, head_bytes, kb0, uint32_t(tile(t0)) * BN * D * 2, kv_off, wave * IPW, IPW);
      dma_one<kKVAux>(vhead, head_bytes, vb0, uint32_t(tile(t0)) * BN * D * 2, vv_off, wave * IPW, IPW);
      load_bits(bb0, tile(t0), p0);
      if (t1 < kt_end) {
        dma_one<kKVAux>(khead, head_bytes, kb1, uint32_t(tile(t1)) * BN * D * 2, kv_off, wave * IPW, IPW);
        load_bits(bb1, tile(t1), p1);
      }
      publish_lds_loads();  // Q, K(t0), K(t1), V(t0) resident
      q_modes();
      score_mfmas(kb0, s0);
      mod_tile(s0, tile(t0));
      mask_tile(s0, tile(t0), m0, p0, row_word(p0, bb0));
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
          dma_one<kKVAux>(khead, head_bytes, kb0, uint32_t(tile(t2)) * BN * D * 2, kv_off, wave * IPW, IPW);
          load_bits(bb0, tile(t2), p2);
        }
        dma_one<kKVAux>(vhead, head_bytes, vb1, uint32_t(tile(t1)) * BN * D * 2, vv_off, wave * IPW, IPW);
        step(kb1, vb0, s0, s1, tile(t1), m1, p1, bb1);

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
          dma_one<kKVAux>(khead, head_bytes, kb1, uint32_t(tile(t3)) * BN * D * 2, kv_off, wave * IPW, IPW);
          load_bits(bb1, tile(t3), p3);
        }
        dma_one<kKVAux>(vhead, head_bytes, vb0, uint32_t(tile(t2)) * BN * D * 2, vv_off, wave * IPW, IPW);
        step(kb0, vb1, s1, s0, tile(t2), m2, p2, bb0);
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
    } else {
    // Output: each wave's 32 rows are one contiguous block of O. Lanes l and
    // l + 32 hold alternate 8-byte pieces of a row; one v_permlane32_swap per
    // dword gives each lane a 16-byte run, which goes through this wave's own
    // slice of the (now idle) K buffers so that every store instruction writes
    // 1 KiB of consecutive bytes.
    {
      static_assert(NW >= 2 && NW * 32 <= 2 * BN, "output staging: a wave pair per K buffer");
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
      uint16_t* obase = MASK ? obase_m : o + (bh * Lq + q0w) * int64_t(D);
#pragma unroll
      for (int i = 0; i < 32 * OCH / 64; ++i) {
        const int g = 64 * i + lane, row = g / OCH, c = g % OCH;
        const uint4 x = *reinterpret_cast<const uint4*>(stage + row * D + 8 * (c ^ (row & (OCH - 1))));
        // O is written once: non-temporal stores keep the L2 for K and V
        // (0.3-0.8% on prefill and block-sparse; non-temporal Q loads lost 1%)
        if (MASK ? row < rows_m : q0w + row < Lq) nt_store(x, reinterpret_cast<uint4*>(obase + row * D + 8 * c));
      }
    }
    if constexpr (MASK) {
      if (lse_m != nullptr && h == 0 && l32 < rows_m) lse_m[l32] = live ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
    } else {
      if (lse != nullptr && h == 0 && qi < Lq) lse[bh * Lq + qi] = live ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
    }
  }
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

// One workgroup per item (b, h, query tile); more items than one grid allows go
// in chunks (then without the XCD placement, which assumes the whole item range).
template <int D, int NW, int WPE, bool BITS, int MOD = 0, bool MASK = true>
hipError_t launch_sp_inst(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                     float scale, int causal, const uint8_t* block_mask, const uint64_t* tile_bits,
                     hipStream_t stream, ScoreMod mod = ScoreMod{}) {
  constexpr int BM = 32 * NW;
  const int n_qt = (Lq + BM - 1) / BM;
  const int64_t n_items = int64_t(B) * H * n_qt;
  int q_mode = 0;
  const float c = score_coef(scale, &q_mode);
  const int64_t cap = 1LL << 22;
  const int xcd_remap = (n_items % 8 == 0 && n_items <= cap) ? 1 : 0;
  // Causal items go in head groups (work_item). A masked call takes one head
  // at a time: its items visit few tiles each, and with two heads the pair's
  // K/V outgrows the L2 and is read about 1.3 times; with one, the traffic
  // equals Q, K and V read once, at the same speed.
  const int head_group = (causal && xcd_remap) ? (MASK ? 1 : RF_ATT_HEAD_GROUP) : 1;
  // Bytes of the row-bitmap array (validated below 2^32 at the boundary).
  const uint32_t bits_bytes =
      BITS ? uint32_t(int64_t((Lq + kMaskTile - 1) / kMaskTile) * ((Lk + kMaskTile - 1) / kMaskTile) * 512) : 0u;
  for (int64_t base = 0; base < n_items; base += cap) {
    const int64_t n = n_items - base < cap ? n_items - base : cap;
    hipLaunchKernelGGL((attention_bf16_sp_kernel<D, NW, WPE, BITS, false, MOD, MASK>), dim3(unsigned(n)), dim3(NW * 64),
                       0, stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Lq, Lk, c, q_mode, causal,
                       block_mask, n_qt, n, xcd_remap, head_group, base,
                       tile_bits, bits_bytes, 1, 0, nullptr, nullptr, mod);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The block-mask-free instance for calls without one (the walk state then
// costs no registers); element bitmaps always come with tile kinds.
template <int D, int NW, int WPE, bool BITS, int MOD = 0>
hipError_t launch_sp(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                     float scale, int causal, const uint8_t* block_mask, const uint64_t* tile_bits,
                     hipStream_t stream, ScoreMod mod = ScoreMod{}) {
  if constexpr (!BITS) {
    if (block_mask == nullptr)
      return launch_sp_inst<D, NW, WPE, BITS, MOD, false>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, nullptr,
                                                          tile_bits, stream, mod);
  }
  return launch_sp_inst<D, NW, WPE, BITS, MOD, true>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal, block_mask,
                                                     tile_bits, stream, mod);
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
    hipLaunchKernelGGL((attention_bf16_sp_kernel<D, NW, WPE, false, true, 0, false>), dim3(unsigned(n)), dim3(NW * 64), 0,
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
  // A decode item has as many query rows as query heads share a key/value
  // head. Where they fill only a fraction of the 128-row tile, a 32- or
  // 64-row workgroup does the same K/V streaming with a quarter or a half of
  // the padded matrix and softmax work, which otherwise competes with the
  // stream for issue slots.
  if (d == 128) {
#if RF_SPLIT_SMALL_TILES
    // The 1- and 2-wave workgroups take 64 KiB of LDS each, so at most one
    // wave per SIMD is resident anyway; their register allocation is sized
    // for one (the split epilogue does not fit two waves' 256 registers).
    if (Lq <= 32)
      return launch_split<128, 1, 1>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale, n_splits, stream);
    if (Lq <= 64)
      return launch_split<128, 2, 1>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale, n_splits, stream);
#endif
    return launch_split<128, RF_ATT_NW_D128, RF_ATT_WPE_D128>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale,
                                                               n_splits, stream);
  }
  return launch_split<64, RF_ATT_NW_D64, RF_ATT_WPE_D64>(q, k, v, ws_o, ws_lse, n_heads, Lq, Lk, scale, n_splits,
                                                          stream);
}

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Lq, int Lk, int d, float scale, int causal, const uint8_t* block_mask,
                                 const uint64_t* tile_bits, hipStream_t stream, int window,
                                 const float* alibi_slopes, float softcap) {
  if (window > 0 || alibi_slopes != nullptr || softcap > 0.f) {  // score modifications
    ScoreMod m;
    m.slopes = alibi_slopes;
    m.H = H;
    m.cap2 = softcap > 0.f ? float(double(softcap) * 1.4426950408889634) : 0.f;
    m.tk = softcap > 0.f ? float(2.0 / double(softcap)) : 0.f;
    m.window = window;
    // ALiBi slopes are positive by convention, so a row's scores grow toward its
    // own position: walk from the diagonal back (the visiting order changes no
    // result, only how often the lazy reference moves).
    m.rev = (alibi_slopes != nullptr && block_mask == nullptr) ? 1 : 0;
    if (softcap > 0.f) {
      if (d == 128)
        return launch_sp<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, false, 2>(q, k, v, o, lse, B, H, Lq, Lk, scale,
                                                                        causal, block_mask, nullptr, stream, m);
      return launch_sp<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, false, 2>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                   block_mask, nullptr, stream, m);
    }
    if (d == 128)
      return launch_sp<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, false, 1>(q, k, v, o, lse, B, H, Lq, Lk, scale,
                                                                      causal, block_mask, nullptr, stream, m);
    return launch_sp<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, false, 1>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                 block_mask, nullptr, stream, m);
  }
  if (tile_bits != nullptr) {  // element bitmaps inside partial tiles
    if (d == 128)
      return launch_sp<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, true>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                    block_mask, tile_bits, stream);
    return launch_sp<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, true>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                               block_mask, tile_bits, stream);
  }
  if (d == 128)
    return launch_sp<128, RF_ATT_NW_D128, RF_ATT_WPE_D128, false>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                                   block_mask, nullptr, stream);
  return launch_sp<64, RF_ATT_NW_D64, RF_ATT_WPE_D64, false>(q, k, v, o, lse, B, H, Lq, Lk, scale, causal,
                                                              block_mask, nullptr, stream);
}

}  // namespace rf
