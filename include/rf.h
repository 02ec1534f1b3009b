/*
 * rf.h — C ABI of the fused online-softmax attention library for AMD MI355X (gfx950).
 *
 * What is computed is the cascaded reduction behind safe softmax — a row max,
 * then a sum of exponentials that depends on that max, then a normalisation —
 * optionally followed by the P·V contraction of attention, run as one pass in
 * incremental form: a running max m and running sum l are rescaled by
 * exp(m_old - m_new) as each tile of the reduction axis arrives, so on-chip
 * state stays constant in sequence length.
 *
 * Sources (web summaries of the papers):
 *   - RedFuser page, "Résumé technique": 1. Problématique (cascaded reductions,
 *     safe softmax followed by a GEMM in attention), 2. Méthodologie (the
 *     definition d_i = ⊕ F_i(X[l], D_i), fusion into one reduction tree, the
 *     incremental form with O(1) on-chip state), 3. Contributions clés
 *     (single-segment and multi-segment strategies; FlashDecoding as a
 *     special case of the latter).
 *   - FLASHLIGHT page, Metodologia item 3 (online softmax via e^{x-y} = e^x/e^y).
 *   - STOF page, Résumé technique (block masks; skip masked tiles rather than
 *     compute and reset them; full and partial outer tiles).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer into caller-owned memory. The
 *     library never allocates or frees device memory and never keeps a
 *     pointer after a call returns.
 *   - All tensors are dense, contiguous and row-major.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. Work is enqueued asynchronously and the call returns once it is
 *     enqueued; the caller synchronises.
 *   - Every argument is validated before any HIP API call, so a validation
 *     error is returned synchronously, enqueues nothing and leaves the
 *     library usable. A HIP launch failure returns RF_ERR_HIP. The detail of
 *     the last failing call on the calling thread is in rf_last_error_message().
 *   - Outputs are fully overwritten, never accumulated into. Inputs must not
 *     alias outputs.
 *   - Floating-point arithmetic is fp32 (accumulation, running max and sum);
 *     bf16 inputs are widened exactly, bf16 outputs are rounded to nearest
 *     even. LSE values are natural logarithms.
 *   - No C++ exception crosses this boundary. There is no global mutable
 *     state besides the thread-local error text, so calls on different
 *     streams may run concurrently.
 */
#ifndef RF_H_
#define RF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RF_F32 = 0, RF_BF16 = 1 } rf_dtype;

typedef enum {
  RF_OK = 0,
  RF_ERR_INVALID_ARG = 1,  /* NULL pointer, negative or overflowing size, bad enum */
  RF_ERR_UNSUPPORTED = 2,  /* a valid request this build has no kernel for */
  RF_ERR_WORKSPACE = 3,    /* caller workspace missing or smaller than required */
  RF_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} rf_status;

/* Tile edge, in tokens, of the attention block mask (both axes). */
#define RF_MASK_TILE 64

/*
 * Row-wise safe softmax: y[r, :] = exp(x[r, :] - max_r) / sum_j exp(x[r, j] - max_r).
 * Source: RedFuser page, 1. Problématique / 2. Méthodologie (max → exp-sum →
 * normalise as one fused reduction tree, the input read once).
 *   x, y   : [rows, cols] of `dtype` (RF_F32 or RF_BF16), device pointers.
 *   rows   : >= 0 (0 enqueues nothing); cols >= 1.
 * Each element is read once and written once when the row fits on chip
 * (cols <= 65536); longer rows take a second
 * read. A row whose entries are all -inf yields NaN.
 * Errors: RF_ERR_INVALID_ARG (NULL pointer with rows > 0, rows < 0, cols < 1,
 * rows*cols overflowing int64, unknown dtype).
 */
int rf_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int dtype, void* stream);

/*
 * Mixture-of-experts routing: for each token t, the softmax over its E expert
 * logits and its k most probable experts.
 *   p_te = exp(x_te - m_t) / sum_j exp(x_tj - m_t),  m_t = max_j x_tj;
 *   topk_idx[t, r] = the r-th expert in descending order of x_t (equal logits:
 *                    lower expert index first; the softmax is monotone, so this
 *                    is the order of p_t);
 *   topk_w[t, r]   = p_t,idx, or p_t,idx / sum_r' p_t,idx[r'] when renorm != 0.
 * Source: RedFuser page, 1. Problématique (MoE routing among the cascaded
 * reductions: max, sum of exponentials, normalisation, then the selection) and
 * 4. Résultats Expérimentaux (MoE routing workload).
 *   logits   : [T, E] of `dtype` (RF_F32 or RF_BF16), device pointer.
 *   topk_idx : int32 [T, k], written;  topk_w : fp32 [T, k], written.
 *   1 <= k <= E. Each logit is read once.
 * A token whose logits are all -inf gets NaN weights, as the definition does.
 * Supported: E <= 1024, k <= 32 (else RF_ERR_UNSUPPORTED).
 * Errors: RF_ERR_INVALID_ARG (unknown dtype, T < 0, E < 1, k outside 1..E,
 * overflow, NULL or misaligned pointers with T > 0), RF_ERR_UNSUPPORTED,
 * RF_ERR_HIP.
 */
int rf_moe_route(const void* logits, int32_t* topk_idx, float* topk_w, int64_t T, int E, int k, int renorm,
                 int dtype, void* stream);

/*
 * Row-wise layer normalisation: per row r, with n = cols,
 *   mean_r = (1/n) sum_j x_rj,  var_r = (1/n) sum_j (x_rj - mean_r)^2,
 *   y_rj   = (x_rj - mean_r) / sqrt(var_r + eps) * gamma_j + beta_j.
 * Source: RedFuser page, 1. Problématique (normalisation layers are cascaded
 * reductions: the mean, then the squared deviations from it) and 2.
 * Méthodologie (the chain fused into one reduction tree, input read once);
 * the Korean page reports variance as a workload.
 *   x, y   : [rows, cols] of `dtype` (RF_F32 or RF_BF16), device pointers.
 *   gamma, beta : fp32 [cols] or NULL (1 and 0).
 *   mean, rstd  : fp32 [rows] or NULL; written with mean_r and 1/sqrt(var_r + eps).
 *   eps    : finite, >= 0 (eps = 0 and a constant row give NaN, as the
 *            definition does).
 * Each element is read once and written once when the row fits in registers
 * (cols <= 32768 with 16-byte aligned rows, gamma and beta and cols a
 * multiple of 4 (fp32) or 8 (bf16); cols <= 16384 otherwise); longer rows
 * take a second read.
 * Errors: RF_ERR_INVALID_ARG (NULL x or y with rows > 0, rows < 0, cols < 1,
 * bad eps, overflow, misalignment, unknown dtype).
 */
int rf_layernorm_rows(const void* x, const float* gamma, const float* beta, void* y, float* mean, float* rstd,
                      int64_t rows, int64_t cols, float eps, int dtype, void* stream);

/*
 * Attention forward with the online softmax, single-segment strategy (one
 * workgroup sweeps every visible key tile of its query tile).
 * Source: RedFuser page, 1. Problématique (safe softmax then GEMM) and
 * 3. Contributions clés (single-segment strategy); FLASHLIGHT page,
 * Metodologia 2–4 (max() fused into QK^T, softmax(QK^T)V fused); STOF page,
 * Méthodologie 1 (block mask, full / partial outer tiles, masked tiles skipped).
 *   q          : [B, H, Lq, d] of `dtype`.
 *   k, v       : [B, H, Lk, d] of `dtype`.
 *   o          : [B, H, Lq, d] of `dtype`, written.
 *   lse        : [B, H, Lq] fp32, written; may be NULL (then not written).
 *   scale      : scores are s_ij = scale * (q_i . k_j).
 *   causal     : nonzero masks key j for query i unless j <= i + (Lk - Lq)
 *                (bottom-right aligned; identical to the usual mask when Lq == Lk).
 *   block_mask : NULL (dense), or a device uint8 array [ceil(Lq/64), ceil(Lk/64)];
 *                tile (I, J) is visible iff block_mask[I * ceil(Lk/64) + J] != 0.
 *                One mask is shared by all (b, h). Masked tiles are skipped.
 * Visible(i, j) = causal rule AND block rule AND j < Lk. A query row with no
 * visible key gets O = 0 and LSE = -inf.
 * Supported: RF_BF16 with d in {64, 128} and Lk * d * 2 < 2^31 (bytes of one
 * head's K); RF_F32 with 1 <= d <= 128.
 * B, H, Lq, Lk >= 0 (any of B, H, Lq zero enqueues nothing).
 * Errors: RF_ERR_INVALID_ARG (NULL pointers when work exists, negative sizes,
 * non-finite scale, unknown dtype), RF_ERR_UNSUPPORTED (other d), RF_ERR_HIP.
 */
int rf_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Lq, int Lk, int d, float scale, int causal,
                     const uint8_t* block_mask, int dtype, void* stream);

/*
 * rf_attention_fwd with element-level sparsity inside partial tiles.
 * Source: STOF page, Méthodologie 1, two-level storage format: outer 64 x 64
 * tiles are skipped, "full" (every element valid) or "partial", and the valid
 * elements of a partial tile are held as 64-bit bitmaps.
 *   tile_kind : device uint8 [ceil(Lq/64), ceil(Lk/64)], shared by all (b, h):
 *               0 = empty (never loaded), 1 = full, any other value = partial.
 *   tile_bits : device uint64 [ceil(Lq/64), ceil(Lk/64), 64], 16-byte aligned:
 *               word r of tile (I, J) holds the visibility of query row
 *               64 I + r for keys 64 J .. 64 J + 63 (bit j mod 64). Read only
 *               for partial tiles. (The page groups the same 4096 bits of a
 *               tile by 8 x 8 blocks; here a tile's words are its rows, since
 *               one lane owns one query row.)
 *   Other arguments as rf_attention_fwd.
 * Visible(i, j) = causal rule AND tile rule AND j < Lk, where the tile rule
 * is kind == 1, or kind not in {0, 1} and the bit of (i, j) set.
 * Supported as rf_attention_fwd, and the bitmap array must be below 2^32
 * bytes (RF_ERR_UNSUPPORTED otherwise).
 * Errors: as rf_attention_fwd, plus RF_ERR_INVALID_ARG for NULL tile_kind or
 * tile_bits when work exists, or misaligned tile_bits.
 */
int rf_attention_fwd_bitmap(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int Lq, int Lk, int d, float scale, int causal, const uint8_t* tile_kind,
                            const uint64_t* tile_bits, int dtype, void* stream);

/*
 * Attention with score modifications: rf_attention_fwd with, per head h,
 * query row i at position p_i = i + Lk - Lq (bottom-right, as the causal
 * rule) and key j,
 *   s = scale * (q_i . k_j);
 *   softcap > 0         : s <- softcap * tanh(s / softcap);
 *   alibi_slopes != NULL: s <- s + alibi_slopes[h] * (j - p_i);
 *   window > 0          : key j is visible only if j > p_i - window
 *                         (with causal = 1: the window keys up to the row's own);
 * then the masked softmax of rf_attention_fwd (causal rule and block mask
 * apply as there). A row with no visible key gives O = 0, LSE = -inf.
 * Source: FLASHLIGHT page, Risultati (the FlexAttention variants ALiBi,
 * Softcap, Causal and Sliding Window; Softcap attention in LLaMa-3.2-1B).
 *   window       : >= 0, 0 = no window.
 *   alibi_slopes : fp32 [H] device pointer (natural-log units per position) or
 *                  NULL for no bias; slopes may have any sign.
 *   softcap      : finite, >= 0, 0 = no softcap.
 * Tiles wholly before every row's window are neither loaded nor computed.
 * Supported sizes and errors as rf_attention_fwd, plus RF_ERR_INVALID_ARG for
 * window < 0, a negative or non-finite softcap, or misaligned alibi_slopes.
 */
int rf_attention_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Lq, int Lk, int d, float scale, int causal,
                         const uint8_t* block_mask, int window, const float* alibi_slopes, float softcap,
                         int dtype, void* stream);

/*
 * Row-wise masked attention: exactly what rf_attention_fwd_bitmap computes
 * (causal rule, tile kinds, row bitmaps inside partial tiles), by the row
 * kernel of the dual-kernel strategy: one wavefront per query row walks only
 * the key tiles its mask row keeps and loads and multiplies only their visible
 * keys (in batches of 16 keys at d = 128, 32 at d = 64), with lane-level
 * reductions and no synchronisation across wavefronts. Suited to highly sparse masks on short sequences; the tile
 * kernel (rf_attention_fwd_bitmap) to the rest. rf_attention_plan chooses.
 * Source: STOF page, Méthodologie 1 (dual-kernel strategy: row-wise kernel and
 * block-wise kernel, chosen by an analytic model).
 *   tile_kind : uint8 [ceil(Lq/64), ceil(Lk/64)] device pointer or NULL (every
 *               tile full); tile_bits : uint64 [same tiles, 64] or NULL (every
 *               nonzero kind is a full tile), 8-byte aligned.
 *   q, k, v, o, lse and scale as rf_attention_fwd; q, k, v, o 16-byte aligned.
 * Supported: RF_BF16 with d in {64, 128} and Lk * d * 2 < 2^31 bytes per head.
 * Errors: RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_HIP.
 */
int rf_attention_fwd_rowwise(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Lq, int Lk, int d, float scale, int causal,
                             const uint8_t* tile_kind, const uint64_t* tile_bits, int dtype, void* stream);

/*
 * The analytic kernel choice for a masked call (host only, no GPU work): from
 * HOST copies of the mask (tile_kind / tile_bits as for rf_attention_fwd_rowwise,
 * NULL allowed), counts the work of each kernel exactly:
 *   tile_work  : 64 x 64 tiles of matrix-core work per head, i.e. for every
 *                workgroup of query rows (128 rows at d = 128, 64 at d = 64)
 *                the key tiles any of its rows needs, times rows / 64;
 *   row_batches: batches per head the row kernel processes, each up to
 *                16 visible keys of one row at d = 128 (32 at d = 64), i.e.
 *                the sum over rows of ceil(visible keys / batch size);
 * and prices them with a cost model of both kernels on MI355X, fitted to
 * measured calls: a launch term plus the larger of a throughput term (the work
 * of all B * H heads over the whole chip) and a critical-path term (the work of
 * the busiest workgroup for the tile kernel, of the busiest query row for the
 * row kernel):
 *   kernel = 1 (row kernel) if its estimate is lower, else 0 (tile kernel).
 * Source: STOF page, Méthodologie 1 (kernel selection by an analytic model from
 * mask sparsity and sequence length).
 * Output pointers other than kernel may be NULL.
 * Errors: RF_ERR_INVALID_ARG (NULL kernel, negative sizes, bits without
 * kinds), RF_ERR_UNSUPPORTED (d not 64 or 128).
 */
int rf_attention_plan(const uint8_t* tile_kind, const uint64_t* tile_bits, int B, int H, int Lq, int Lk, int d,
                      int causal, int* kernel, double* est_tile_us, double* est_row_us, int64_t* tile_work,
                      int64_t* row_batches);

/*
 * Bytes of device workspace that rf_attention_decode_splitkv needs:
 * B*H*num_splits*(d + 1) fp32 values (normalised partial outputs and their
 * LSE), rounded up to 256 bytes. Returns 0 for invalid arguments.
 */
size_t rf_attention_decode_splitkv_workspace_size(int B, int H, int d, int num_splits);

/*
 * Split-KV decode: one query token per (b, h) against Lk cached keys, with the
 * multi-segment strategy: the Lk keys are cut into num_splits contiguous
 * chunks of ceil(Lk / num_splits) keys (trailing chunks may be short or
 * empty); each chunk yields a normalised partial (O_s, lse_s) and the
 * partials are merged by log-sum-exp as rf_lse_merge does.
 * Source: RedFuser page, 3. Contributions clés (multi-segment strategy,
 * FlashDecoding as its special case); STOF page, Méthodologie 1 (row-wise kernel).
 *   q          : [B, H, 1, d] of `dtype`;  k, v : [B, H, Lk, d] of `dtype`.
 *   o          : [B, H, 1, d] of `dtype`, written.
 *   lse        : [B, H] fp32, written; may be NULL.
 *   num_splits : 1 .. 1024.
 *   workspace  : device buffer of at least
 *                rf_attention_decode_splitkv_workspace_size(B, H, d, num_splits)
 *                bytes, 256-byte aligned; its contents on entry are ignored.
 *                It must stay untouched until the enqueued work completes.
 * No causal or block mask applies: the query sees every cached key. Lk == 0
 * gives O = 0, LSE = -inf.
 * Supported: RF_BF16 with d in {64, 128}.
 * Errors: RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_WORKSPACE (NULL,
 * misaligned or too small workspace), RF_ERR_HIP.
 */
int rf_attention_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Lk, int d, float scale, int num_splits,
                                void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * rf_attention_decode_splitkv for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (without the workspace),
 * same kernels, same result bit for bit. The partials live in a device array
 * of the library's own, RF_DECODE_SCRATCH_BYTES (32 MiB) per GPU, held from
 * the first call on that GPU until the process ends; it fits the partials of
 * B*H*num_splits*(d + 1) fp32 values laid out as the workspace above (about
 * 65,000 rows B*H*num_splits at d = 128; 2048 heads with 16 splits need 16.1 MiB).
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (concurrent streams, or host threads) race and must be serialised by the
 * caller. Nothing in the array needs clearing between calls: each call writes
 * every partial it reads. The first call on a GPU looks the array's address up
 * on that GPU; every call asks the stream for its device and launches the two
 * kernels. No call allocates or frees memory.
 * Errors: as rf_attention_decode_splitkv, and RF_ERR_WORKSPACE when the
 * partials need more than RF_DECODE_SCRATCH_BYTES (checked before any HIP
 * call).
 */
#define RF_DECODE_SCRATCH_BYTES (32u << 20)
int rf_attention_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                        int B, int H, int Lk, int d, float scale, int num_splits, int dtype,
                                        void* stream);

/*
 * Bytes of device workspace that rf_attention_decode_gqa needs: 0 when
 * num_splits == 1 (no partials), else B*Hq*num_splits*(d + 1) fp32 values laid
 * out and rounded as for rf_attention_decode_splitkv. Returns 0 for invalid
 * arguments too.
 */
size_t rf_attention_decode_gqa_workspace_size(int B, int Hq, int d, int num_splits);

/*
 * Decode with grouped queries: Hq = G * Hkv query heads, one token each, where
 * query head hq attends the cached keys and values of head hq / G (the G
 * consecutive query heads G j .. G j + G - 1 share key/value head j). Hkv = 1
 * is the sharing pattern of MLA decode: every query head reads one cache. The
 * result per query head is exactly rf_attention_decode_splitkv's with H = Hq
 * and each key/value head repeated G times; here each key/value tile is read
 * once for its G query heads, which are the rows of one matrix-core tile.
 * Source: RedFuser page, 4. Résultats Expérimentaux (MHA and MLA workloads)
 * and 3. Contributions clés (multi-segment strategy, merge of partials).
 *   q, o       : [B, Hq, d] of `dtype` (o written);  k, v : [B, Hkv, Lk, d].
 *   lse        : [B, Hq] fp32, written; may be NULL.
 *   num_splits : 1 .. 1024. Keys go in tiles of 64; split s covers tiles
 *                [s T, (s + 1) T), T = ceil(ceil(Lk / 64) / num_splits);
 *                trailing splits may be empty. Each split yields a normalised
 *                fp32 partial and its LSE, merged as rf_lse_merge does. With
 *                num_splits == 1 the result is written directly and no
 *                workspace is used (workspace may be NULL).
 *   workspace  : for num_splits > 1, a device buffer of at least
 *                rf_attention_decode_gqa_workspace_size(B, Hq, d, num_splits)
 *                bytes, 256-byte aligned, untouched until the work completes.
 * No mask applies. Lk == 0 gives O = 0, LSE = -inf. The latent widths of MLA
 * (576-wide keys, 512-wide values) are not supported.
 * Supported: RF_BF16 with d in {64, 128} and Lk * d * 2 < 2^31.
 * Errors: RF_ERR_INVALID_ARG (including Hq not a multiple of Hkv),
 * RF_ERR_UNSUPPORTED, RF_ERR_WORKSPACE, RF_ERR_HIP.
 */
int rf_attention_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int Lk, int d, float scale, int num_splits, void* workspace,
                            size_t workspace_bytes, int dtype, void* stream);

/*
 * Log-sum-exp merge of normalised partial results (the merge step of the
 * multi-segment strategy; order-free because the (O, lse) pairs form a
 * commutative monoid with identity (anything, -inf)).
 * Source: RedFuser page, 2. Méthodologie (fusion conditions: commutative
 * monoid, distributivity) and 3. Contributions clés (merge of partial results).
 * Per row r: M = max_s lse[r, s]; w_s = exp(lse[r, s] - M); W = sum_s w_s;
 *            o[r, :] = sum_s w_s * o_parts[r, s, :] / W;  lse_out[r] = M + ln W.
 * A part with lse = -inf has weight exactly zero and its o_parts row is not
 * read. If every part is -inf: o[r, :] = 0 and lse_out[r] = -inf.
 *   o_parts   : [n_rows, num_splits, d] fp32;  lse_parts : [n_rows, num_splits] fp32.
 *   o         : [n_rows, d] of out_dtype (RF_F32 or RF_BF16), written.
 *   lse       : [n_rows] fp32, written; may be NULL.
 *   n_rows >= 0; 1 <= num_splits <= 1024; d >= 1.
 * Errors: RF_ERR_INVALID_ARG, RF_ERR_HIP.
 */
int rf_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                 int64_t n_rows, int num_splits, int d, int out_dtype, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* rf_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). Valid until
 * the next rf_* call on the same thread. */
const char* rf_last_error_message(void);

/* ABI version of this header: bumped when a signature or semantic changes. */
#define RF_ABI_VERSION 7
int rf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RF_H_ */
