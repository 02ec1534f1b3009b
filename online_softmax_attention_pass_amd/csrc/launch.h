// Host-side launchers of the rf kernels. Each returns hipSuccess or the launch
// error; all argument checks happen in the C-ABI layer before these are
// called. Declarations only: nothing here changes a kernel's code, so the
// source hash that dates a kernel's traffic counters leaves this file out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rf {
hipError_t launch_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int dtype,
                               hipStream_t stream);
// Mixture-of-experts routing: logits [T, E] (fp32 or bf16) -> top-k expert
// indices and weights [T, k]; 1 <= k <= min(E, 32), E <= 1024.
hipError_t launch_moe_route(const void* logits, int32_t* idx, float* w, int64_t T, int E, int k, int renorm,
                            int dtype, hipStream_t stream);
hipError_t launch_layernorm_rows(const void* x, const float* gamma, const float* beta, void* y, float* mean,
                                 float* rstd, int64_t rows, int64_t cols, float eps, int dtype, hipStream_t stream);
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                            int64_t n_rows, int num_splits, int d, int out_dtype, hipStream_t stream);
hipError_t launch_decode_partials(const void* q, const void* k, const void* v, float* o_parts,
                                  float* lse_parts, int B, int H, int Lk, int d, float scale,
                                  int num_splits, hipStream_t stream);
// Split-KV decode with the partials in the library's own device scratch array
// (no allocation, no workspace argument): partials, then the merge into o, lse.
// The partial LSEs start lse_off bytes into the scratch; the caller has checked
// that the layout fits in kDecodeScratchBytes.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_decode_splitkv_scratch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                         int H, int Lk, int d, float scale, int num_splits, size_t lse_off,
                                         hipStream_t stream);
// block_mask: NULL (dense) or tile kinds [ceil(Lq/64), ceil(Lk/64)]. tile_bits:
// NULL (every nonzero kind is a full tile) or uint64 [same tiles, 64] row
// bitmaps, used where the kind is neither 0 nor 1.
hipError_t launch_attention_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                                int B, int H, int Lq, int Lk, int d, float scale, int causal,
                                const uint8_t* block_mask, const uint64_t* tile_bits, hipStream_t stream,
                                int window = 0, const float* alibi_slopes = nullptr, float softcap = 0.f);
// Split-KV partials of the pipelined bf16 kernel (no mask): n_heads heads of
// Lq query rows, fp32 normalised partials into ws_o [n_heads * Lq, n_splits, d]
// and ws_lse [n_heads * Lq, n_splits].
hipError_t launch_attention_bf16_split(const void* q, const void* k, const void* v, float* ws_o, float* ws_lse,
                                       int n_heads, int Lq, int Lk, int d, float scale, int n_splits,
                                       hipStream_t stream);
// Score modifications (window > 0, alibi_slopes [H] device pointer, softcap > 0)
// select the instance that applies them; tile_bits is then ignored (the entry
// point with modifications takes no bitmaps).
hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int Lq, int Lk, int d, float scale, int causal,
                                 const uint8_t* block_mask, const uint64_t* tile_bits, hipStream_t stream,
                                 int window = 0, const float* alibi_slopes = nullptr, float softcap = 0.f);
// Row-wise masked attention (bf16, d in {64, 128}): one wavefront per query row,
// only the row's visible keys, in batches. tile_kind NULL = every tile full; tile_bits
// NULL = every nonzero kind is a full tile.
hipError_t launch_attention_rowwise(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int Lq, int Lk, int d, float scale, int causal, const uint8_t* tile_kind,
                                    const uint64_t* tile_bits, hipStream_t stream);
}  // namespace rf
