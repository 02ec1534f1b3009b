// C-ABI entry points of librf: argument validation, dispatch, error reporting.
//
// Every check runs before the first HIP API call of an entry point, so a
// rejected call is synchronous, enqueues nothing and needs no GPU. Kernels
// are launched asynchronously on the caller's stream. No C++ exception
// crosses the boundary.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <exception>
#include <string>

#include "rf.h"
#include "launch.h"
#include "rf_internal.h"

namespace {

static_assert(rf::kDecodeScratchBytes == RF_DECODE_SCRATCH_BYTES, "one scratch size on both sides of the ABI");

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return RF_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(RF_ERR_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

// a * b * c * ... without int64 overflow; false when the product would overflow.
bool mul_ok(int64_t& acc, int64_t x) {
  if (x < 0) return false;
  if (x != 0 && acc > INT64_MAX / x) return false;
  acc *= x;
  return true;
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct DecodeWs {
  size_t o_bytes, lse_off, total;
};

bool decode_ws_layout(int B, int H, int d, int S, DecodeWs& w) {
  if (B < 0 || H < 0 || d < 1 || S < 1 || S > 1024) return false;
  int64_t n = 1;
  if (!mul_ok(n, B) || !mul_ok(n, H) || !mul_ok(n, S)) return false;
  int64_t nod = n;
  if (!mul_ok(nod, d) || !mul_ok(nod, 4)) return false;
  if (n > INT64_MAX / 8) return false;
  w.o_bytes = size_t(nod);
  w.lse_off = round_up(w.o_bytes, 256);
  w.total = w.lse_off + round_up(size_t(n) * 4, 256);
  return true;
}

}  // namespace

extern "C" {

const char* rf_status_string(int s) {
  switch (s) {
    case RF_OK: return "RF_OK";
    case RF_ERR_INVALID_ARG: return "RF_ERR_INVALID_ARG";
    case RF_ERR_UNSUPPORTED: return "RF_ERR_UNSUPPORTED";
    case RF_ERR_WORKSPACE: return "RF_ERR_WORKSPACE";
    case RF_ERR_HIP: return "RF_ERR_HIP";
    default: return "RF_UNKNOWN_STATUS";
  }
}

const char* rf_last_error_message(void) { return g_last_error.c_str(); }

int rf_abi_version(void) { return RF_ABI_VERSION; }

int rf_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int dtype, void* stream) {
  try {
    if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: unknown dtype %d", dtype);
    if (rows < 0) return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: rows = %lld < 0", (long long)rows);
    if (cols < 1) return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: cols = %lld < 1", (long long)cols);
    int64_t n = rows;
    if (!mul_ok(n, cols) || !mul_ok(n, dtype == RF_F32 ? 4 : 2))
      return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: rows * cols overflows");
    if (rows == 0) return ok();
    if (x == nullptr || y == nullptr) return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: NULL x or y");
    const size_t es = dtype == RF_F32 ? 4 : 2;
    if (!aligned(x, es) || !aligned(y, es))
      return fail(RF_ERR_INVALID_ARG, "rf_softmax_rows: x and y must be aligned to their element size");
    return hip_status(rf::launch_softmax_rows(x, y, rows, cols, dtype, static_cast<hipStream_t>(stream)),
                      "rf_softmax_rows");
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "rf_softmax_rows: %s", e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "rf_softmax_rows: unknown exception");
  }
}

int rf_layernorm_rows(const void* x, const float* gamma, const float* beta, void* y, float* mean, float* rstd,
                      int64_t rows, int64_t cols, float eps, int dtype, void* stream) {
  try {
    if (dtype != RF_F32 && dtype != RF_BF16)
      return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: unknown dtype %d", dtype);
    if (rows < 0) return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: rows < 0");
    if (cols < 1) return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: cols < 1");
    if (!std::isfinite(eps) || eps < 0.f) return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: eps must be finite and >= 0");
    int64_t n = 1;
    if (!mul_ok(n, rows) || !mul_ok(n, cols) || !mul_ok(n, 4))
      return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: rows * cols overflows int64");
    if (rows == 0) return ok();
    if (x == nullptr || y == nullptr) return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: NULL x or y");
    const size_t es = dtype == RF_F32 ? 4 : 2;
    if (!aligned(x, es) || !aligned(y, es) || (gamma != nullptr && !aligned(gamma, 4)) ||
        (beta != nullptr && !aligned(beta, 4)) || (mean != nullptr && !aligned(mean, 4)) ||
        (rstd != nullptr && !aligned(rstd, 4)))
      return fail(RF_ERR_INVALID_ARG, "rf_layernorm_rows: misaligned pointer");
    return hip_status(rf::launch_layernorm_rows(x, gamma, beta, y, mean, rstd, rows, cols, eps, dtype,
                                                static_cast<hipStream_t>(stream)),
                      "rf_layernorm_rows");
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "rf_layernorm_rows: %s", e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "rf_layernorm_rows: unknown exception");
  }
}

int rf_attention_fwd_rowwise(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                             int Lq, int Lk, int d, float scale, int causal, const uint8_t* tile_kind,
                             const uint64_t* tile_bits, int dtype, void* stream) {
  const char* name = "rf_attention_fwd_rowwise";
  try {
    if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0)
      return fail(RF_ERR_INVALID_ARG, "%s: negative size (B=%d H=%d Lq=%d Lk=%d)", name, B, H, Lq, Lk);
    if (d < 1) return fail(RF_ERR_INVALID_ARG, "%s: d = %d < 1", name, d);
    if (!std::isfinite(scale)) return fail(RF_ERR_INVALID_ARG, "%s: scale is not finite", name);
    if (dtype != RF_BF16) return fail(RF_ERR_UNSUPPORTED, "%s: only bf16 is supported", name);
    if (d != 64 && d != 128) return fail(RF_ERR_UNSUPPORTED, "%s: d must be 64 or 128, got %d", name, d);
    int64_t nq = 1, nk = 1;
    if (!mul_ok(nq, B) || !mul_ok(nq, H) || !mul_ok(nq, Lq) || !mul_ok(nq, d) || !mul_ok(nq, 2) ||
        !mul_ok(nk, B) || !mul_ok(nk, H) || !mul_ok(nk, Lk) || !mul_ok(nk, d) || !mul_ok(nk, 2))
      return fail(RF_ERR_INVALID_ARG, "%s: tensor size overflows int64", name);
    if (int64_t(B) * H * Lq == 0) return ok();
    if (q == nullptr || o == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL q or o", name);
    if (Lk > 0 && (k == nullptr || v == nullptr)) return fail(RF_ERR_INVALID_ARG, "%s: NULL k or v", name);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
      return fail(RF_ERR_UNSUPPORTED, "%s: needs 16-byte aligned q, k, v and o", name);
    if (lse != nullptr && !aligned(lse, 4)) return fail(RF_ERR_INVALID_ARG, "%s: lse misaligned", name);
    if (tile_bits != nullptr && !aligned(tile_bits, 8))
      return fail(RF_ERR_INVALID_ARG, "%s: tile_bits must be 8-byte aligned", name);
    if (tile_bits != nullptr && Lk > 0 && tile_kind == nullptr)
      return fail(RF_ERR_INVALID_ARG, "%s: NULL tile_kind", name);
    if (int64_t(Lk) * d * 2 > INT32_MAX)
      return fail(RF_ERR_UNSUPPORTED, "%s: needs Lk * d * 2 < 2^31 bytes per head", name);
    return hip_status(rf::launch_attention_rowwise(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal != 0, tile_kind,
                                                   tile_bits, static_cast<hipStream_t>(stream)),
                      name);
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

namespace {
// Cost of one masked call on MI355X, in microseconds: a launch term plus the
// larger of a throughput term (all the work spread over the chip) and a
// critical-path term (the busiest workgroup of the tile kernel, the busiest
// query row of the row kernel), the latter deciding when there are too few
// workgroups or rows to fill 256 compute units. Row-kernel work is its batches
// of visible keys plus row_per_tile of a batch for every tile the row visits.
// Fitted to bf16 calls of both kernels over causal square masks (1k-8k) and
// non-causal short-query masks (64-256 queries over 4k-16k keys), 1-100% of
// tiles and 1-50% of bits kept.
struct PlanCost {
  double tile_launch, tile_per_tile, tile_per_wg_tile;  // us, us per tile unit, us per tile unit of one workgroup
  double row_launch, row_per_batch, row_per_row_batch;  // us, us per batch, us per batch of one row
  double row_per_tile;                                  // batches per visited tile
};
PlanCost plan_cost(int d) {
  if (d == 128) return {11.0, 3.36e-3, 1.05, 12.0, 7.12e-4, 5e-4, 0.1};
  return {10.0, 2.65e-3, 1.50, 13.0, 7.12e-4, 5e-4, 0.1};
}
}  // namespace

int rf_attention_plan(const uint8_t* tile_kind, const uint64_t* tile_bits, int B, int H, int Lq, int Lk, int d,
                      int causal, int* kernel, double* est_tile_us, double* est_row_us, int64_t* tile_work,
                      int64_t* row_batches) {
  const char* name = "rf_attention_plan";
  try {
    if (kernel == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL kernel", name);
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0)
      return fail(RF_ERR_INVALID_ARG, "%s: negative size (B=%d H=%d Lq=%d Lk=%d)", name, B, H, Lq, Lk);
    if (d != 64 && d != 128) return fail(RF_ERR_UNSUPPORTED, "%s: d must be 64 or 128, got %d", name, d);
    if (tile_bits != nullptr && tile_kind == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL tile_kind", name);
    const int n_ct = (Lk + 63) / 64;
    const int64_t off = int64_t(Lk) - Lq;
    const int bm = d == 128 ? 128 : 64;        // query rows per tile-kernel workgroup
    const int kb = d == 128 ? 16 : 32;         // visible keys per row-kernel batch
    auto kind_at = [&](int I, int J) -> int { return tile_kind == nullptr ? 1 : tile_kind[int64_t(I) * n_ct + J]; };
    // tile kernel: per workgroup, the tiles any of its rows needs, each worth bm / 64 tiles of work
    double tiles = 0.0, wg_max = 0.0;
    for (int q0 = 0; q0 < Lq; q0 += bm) {
      double wg_tiles = 0.0;
      const int q1 = q0 + bm < Lq ? q0 + bm : Lq;
      int64_t last = causal ? int64_t(q1 - 1) + off : int64_t(Lk) - 1;
      if (last > Lk - 1) last = Lk - 1;
      const int j_end = last < 0 ? 0 : int(last / 64) + 1;
      for (int J = 0; J < j_end; ++J) {
        bool any = false;
        for (int I = q0 / 64; I <= (q1 - 1) / 64; ++I) any |= kind_at(I, J) != 0;
        if (any) wg_tiles += bm / 64;
      }
      tiles += wg_tiles;
      wg_max = wg_tiles > wg_max ? wg_tiles : wg_max;
    }
    // row kernel: per row, its batches of kb visible keys and the tiles it visits
    const PlanCost c = plan_cost(d);
    double batches = 0.0, row_work = 0.0, row_max = 0.0;
    for (int i = 0; i < Lq; ++i) {
      int64_t last = causal ? int64_t(i) + off : int64_t(Lk) - 1;
      if (last > Lk - 1) last = Lk - 1;
      const int j_end = last < 0 ? 0 : int(last / 64) + 1;
      int64_t vis = 0, tiles_i = 0;
      for (int J = 0; J < j_end; ++J) {
        const int kind = kind_at(i / 64, J);
        if (kind == 0) continue;
        uint64_t word = (tile_bits != nullptr && kind != 1) ? tile_bits[(int64_t(i / 64) * n_ct + J) * 64 + i % 64]
                                                            : ~uint64_t(0);
        if (int64_t(J) * 64 + 63 > last) word &= (uint64_t(1) << int(last - int64_t(J) * 64 + 1)) - 1;
        if (word == 0) continue;
        vis += __builtin_popcountll(word);
        tiles_i += 1;
      }
      const double b_i = double((vis + kb - 1) / kb);
      const double w_i = b_i + c.row_per_tile * double(tiles_i);
      batches += b_i;
      row_work += w_i;
      row_max = w_i > row_max ? w_i : row_max;
    }
    const double heads = double(B) * H;
    auto mx = [](double a, double b) { return a > b ? a : b; };
    const double t_tile = c.tile_launch + mx(c.tile_per_tile * tiles * heads, c.tile_per_wg_tile * wg_max);
    const double t_row = c.row_launch + mx(c.row_per_batch * row_work * heads, c.row_per_row_batch * row_max);
    *kernel = t_row < t_tile ? 1 : 0;
    if (est_tile_us != nullptr) *est_tile_us = t_tile;
    if (est_row_us != nullptr) *est_row_us = t_row;
    if (tile_work != nullptr) *tile_work = int64_t(tiles);
    if (row_batches != nullptr) *row_batches = int64_t(batches);
    return ok();
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

int rf_moe_route(const void* logits, int32_t* topk_idx, float* topk_w, int64_t T, int E, int k, int renorm,
                 int dtype, void* stream) {
  const char* name = "rf_moe_route";
  try {
    if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
    if (T < 0) return fail(RF_ERR_INVALID_ARG, "%s: T < 0", name);
    if (E < 1) return fail(RF_ERR_INVALID_ARG, "%s: E = %d < 1", name, E);
    if (k < 1 || k > E) return fail(RF_ERR_INVALID_ARG, "%s: k = %d outside 1..E (E = %d)", name, k, E);
    if (E > 1024 || k > 32) return fail(RF_ERR_UNSUPPORTED, "%s: needs E <= 1024 and k <= 32 (E = %d, k = %d)", name, E, k);
    int64_t n = T, nk = T;
    if (!mul_ok(n, E) || !mul_ok(n, 4) || !mul_ok(nk, k) || !mul_ok(nk, 4))
      return fail(RF_ERR_INVALID_ARG, "%s: size overflows int64", name);
    if (T == 0) return ok();
    if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr)
      return fail(RF_ERR_INVALID_ARG, "%s: NULL logits, topk_idx or topk_w", name);
    if (!aligned(logits, dtype == RF_F32 ? 4 : 2) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
      return fail(RF_ERR_INVALID_ARG, "%s: misaligned pointer", name);
    return hip_status(rf::launch_moe_route(logits, topk_idx, topk_w, T, E, k, renorm != 0 ? 1 : 0, dtype,
                                           static_cast<hipStream_t>(stream)),
                      name);
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

namespace {
// Shared body of the two attention entry points; `name` labels the errors.
int attention_common(const char* name, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Lq, int Lk, int d, float scale, int causal, const uint8_t* block_mask,
                     const uint64_t* tile_bits, int dtype, void* stream, int window = 0,
                     const float* alibi_slopes = nullptr, float softcap = 0.f) {
  try {
    if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0)
      return fail(RF_ERR_INVALID_ARG, "%s: negative size (B=%d H=%d Lq=%d Lk=%d)", name, B, H, Lq, Lk);
    if (d < 1) return fail(RF_ERR_INVALID_ARG, "%s: d = %d < 1", name, d);
    if (!std::isfinite(scale)) return fail(RF_ERR_INVALID_ARG, "%s: scale is not finite", name);
    if (dtype == RF_BF16 && d != 64 && d != 128)
      return fail(RF_ERR_UNSUPPORTED, "%s: bf16 supports d in {64, 128}, got %d", name, d);
    if (dtype == RF_F32 && d > 128) return fail(RF_ERR_UNSUPPORTED, "%s: fp32 supports d <= 128, got %d", name, d);
    const int es = dtype == RF_F32 ? 4 : 2;
    int64_t nq = 1, nk = 1;
    if (!mul_ok(nq, B) || !mul_ok(nq, H) || !mul_ok(nq, Lq) || !mul_ok(nq, d) || !mul_ok(nq, es) ||
        !mul_ok(nk, B) || !mul_ok(nk, H) || !mul_ok(nk, Lk) || !mul_ok(nk, d) || !mul_ok(nk, es))
      return fail(RF_ERR_INVALID_ARG, "%s: tensor size overflows int64", name);
    if (tile_bits != nullptr) {
      // 64 words of 8 bytes per 64 x 64 tile; the bf16 kernel addresses the
      // array with 32-bit offsets.
      const int64_t bytes = int64_t((Lq + 63) / 64) * ((Lk + 63) / 64) * 512;
      if (bytes > int64_t(UINT32_MAX))
        return fail(RF_ERR_UNSUPPORTED, "%s: tile bitmaps of %lld bytes exceed 2^32", name, (long long)bytes);
    }
    if (int64_t(B) * H * Lq == 0) return ok();
    if (q == nullptr || o == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL q or o", name);
    if (Lk > 0 && (k == nullptr || v == nullptr)) return fail(RF_ERR_INVALID_ARG, "%s: NULL k or v", name);
    if (tile_bits != nullptr && Lk > 0 && block_mask == nullptr)
      return fail(RF_ERR_INVALID_ARG, "%s: NULL tile_kind", name);
    if (tile_bits != nullptr && !aligned(tile_bits, 16))
      return fail(RF_ERR_INVALID_ARG, "%s: tile_bits must be 16-byte aligned", name);
    if (dtype == RF_BF16) {
      if (int64_t(Lk) * d * 2 > INT32_MAX)
        return fail(RF_ERR_UNSUPPORTED, "%s: bf16 path needs Lk * d * 2 < 2^31 bytes per head", name);
      if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 8))
        return fail(RF_ERR_UNSUPPORTED, "%s: bf16 path needs 16-byte aligned q, k, v and 8-byte aligned o", name);
    } else if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(o, 4)) {
      return fail(RF_ERR_INVALID_ARG, "%s: fp32 tensors must be 4-byte aligned", name);
    }
    if (lse != nullptr && !aligned(lse, 4)) return fail(RF_ERR_INVALID_ARG, "%s: lse misaligned", name);
    if (alibi_slopes != nullptr && !aligned(alibi_slopes, 4))
      return fail(RF_ERR_INVALID_ARG, "%s: alibi_slopes misaligned", name);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e =
        dtype == RF_BF16
            ? rf::launch_attention_bf16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal != 0, block_mask, tile_bits,
                                        s, window, alibi_slopes, softcap)
            : rf::launch_attention_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), static_cast<float*>(o), lse, B, H, Lq, Lk,
                                       d, scale, causal != 0, block_mask, tile_bits, s, window, alibi_slopes,
                                       softcap);
    return hip_status(e, name);
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}
}  // namespace

int rf_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                     int Lk, int d, float scale, int causal, const uint8_t* block_mask, int dtype, void* stream) {
  return attention_common("rf_attention_fwd", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, block_mask,
                          nullptr, dtype, stream);
}

int rf_attention_fwd_bitmap(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int Lq, int Lk, int d, float scale, int causal, const uint8_t* tile_kind,
                            const uint64_t* tile_bits, int dtype, void* stream) {
  if (int64_t(B) * H * Lq > 0 && Lk > 0 && tile_bits == nullptr)
    return fail(RF_ERR_INVALID_ARG, "rf_attention_fwd_bitmap: NULL tile_bits");
  return attention_common("rf_attention_fwd_bitmap", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, tile_kind,
                          tile_bits, dtype, stream);
}

int rf_attention_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                         int Lk, int d, float scale, int causal, const uint8_t* block_mask, int window,
                         const float* alibi_slopes, float softcap, int dtype, void* stream) {
  const char* name = "rf_attention_fwd_mod";
  if (window < 0) return fail(RF_ERR_INVALID_ARG, "%s: window = %d < 0", name, window);
  if (!std::isfinite(softcap) || softcap < 0.f)
    return fail(RF_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0", name);
  return attention_common(name, q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, block_mask, nullptr, dtype, stream,
                          window, alibi_slopes, softcap);
}

size_t rf_attention_decode_splitkv_workspace_size(int B, int H, int d, int num_splits) {
  DecodeWs w;
  if (!decode_ws_layout(B, H, d, num_splits, w)) return 0;
  return w.total;
}

}  // extern "C"

namespace {

// Argument checks shared by the two split-KV decode entry points; on success
// w holds the partials' layout. Returns RF_OK, or the failing status with its
// message set. Makes no HIP call.
int decode_args(const char* name, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Lk, int d, float scale, int num_splits, int dtype, DecodeWs& w) {
  if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
  if (B < 0 || H < 0 || Lk < 0)
    return fail(RF_ERR_INVALID_ARG, "%s: negative size (B=%d H=%d Lk=%d)", name, B, H, Lk);
  if (d < 1) return fail(RF_ERR_INVALID_ARG, "%s: d = %d < 1", name, d);
  if (num_splits < 1 || num_splits > 1024)
    return fail(RF_ERR_INVALID_ARG, "%s: num_splits = %d outside 1..1024", name, num_splits);
  if (!std::isfinite(scale)) return fail(RF_ERR_INVALID_ARG, "%s: scale is not finite", name);
  if (dtype != RF_BF16) return fail(RF_ERR_UNSUPPORTED, "%s: only bf16 is supported", name);
  if (d != 64 && d != 128) return fail(RF_ERR_UNSUPPORTED, "%s: d must be 64 or 128, got %d", name, d);
  int64_t nk = 1;
  if (!mul_ok(nk, B) || !mul_ok(nk, H) || !mul_ok(nk, Lk) || !mul_ok(nk, d) || !mul_ok(nk, 2))
    return fail(RF_ERR_INVALID_ARG, "%s: tensor size overflows int64", name);
  if (!decode_ws_layout(B, H, d, num_splits, w)) return fail(RF_ERR_INVALID_ARG, "%s: workspace size overflows", name);
  if (int64_t(B) * H == 0) return RF_OK;
  if (q == nullptr || o == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL q or o", name);
  if (Lk > 0 && (k == nullptr || v == nullptr)) return fail(RF_ERR_INVALID_ARG, "%s: NULL k or v", name);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 8))
    return fail(RF_ERR_UNSUPPORTED, "%s: needs 16-byte aligned q, k, v and 8-byte aligned o", name);
  if (lse != nullptr && !aligned(lse, 4)) return fail(RF_ERR_INVALID_ARG, "%s: lse misaligned", name);
  return RF_OK;
}

}  // namespace

extern "C" {

int rf_attention_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                int Lk, int d, float scale, int num_splits, void* workspace,
                                size_t workspace_bytes, int dtype, void* stream) {
  const char* name = "rf_attention_decode_splitkv";
  try {
    DecodeWs w;
    const int st = decode_args(name, q, k, v, o, lse, B, H, Lk, d, scale, num_splits, dtype, w);
    if (st != RF_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    if (workspace == nullptr || workspace_bytes < w.total || !aligned(workspace, 256))
      return fail(RF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu at %p)", name,
                  w.total, workspace_bytes, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* o_parts = static_cast<float*>(workspace);
    float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.lse_off);
    hipError_t e = rf::launch_decode_partials(q, k, v, o_parts, lse_parts, B, H, Lk, d, scale, num_splits, s);
    if (e != hipSuccess) return hip_status(e, "rf_attention_decode_splitkv (partials)");
    e = rf::launch_lse_merge(o_parts, lse_parts, o, lse, int64_t(B) * H, num_splits, d, RF_BF16, s);
    return hip_status(e, "rf_attention_decode_splitkv (merge)");
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

int rf_attention_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                        int H, int Lk, int d, float scale, int num_splits, int dtype, void* stream) {
  const char* name = "rf_attention_decode_splitkv_noalloc";
  try {
    DecodeWs w;
    const int st = decode_args(name, q, k, v, o, lse, B, H, Lk, d, scale, num_splits, dtype, w);
    if (st != RF_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    if (w.total > rf::kDecodeScratchBytes)
      return fail(RF_ERR_WORKSPACE,
                  "%s: the partials of B*H*num_splits = %lld rows need %zu bytes, above the library's %zu-byte "
                  "scratch; use rf_attention_decode_splitkv with a caller workspace",
                  name, (long long)(int64_t(B) * H * num_splits), w.total, rf::kDecodeScratchBytes);
    const hipError_t e = rf::launch_decode_splitkv_scratch(q, k, v, o, lse, B, H, Lk, d, scale, num_splits,
                                                           w.lse_off, static_cast<hipStream_t>(stream));
    return hip_status(e, name);
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

size_t rf_attention_decode_gqa_workspace_size(int B, int Hq, int d, int num_splits) {
  DecodeWs w;
  if (!decode_ws_layout(B, Hq, d, num_splits, w)) return 0;
  return num_splits == 1 ? 0 : w.total;
}

int rf_attention_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int Lk, int d, float scale, int num_splits, void* workspace,
                            size_t workspace_bytes, int dtype, void* stream) {
  const char* name = "rf_attention_decode_gqa";
  try {
    if (dtype != RF_F32 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
    if (B < 0 || Hq < 0 || Lk < 0)
      return fail(RF_ERR_INVALID_ARG, "%s: negative size (B=%d Hq=%d Lk=%d)", name, B, Hq, Lk);
    if (Hkv < 1 || Hq % Hkv != 0)
      return fail(RF_ERR_INVALID_ARG, "%s: Hq = %d is not a multiple of Hkv = %d >= 1", name, Hq, Hkv);
    if (d < 1) return fail(RF_ERR_INVALID_ARG, "%s: d = %d < 1", name, d);
    if (num_splits < 1 || num_splits > 1024)
      return fail(RF_ERR_INVALID_ARG, "%s: num_splits = %d outside 1..1024", name, num_splits);
    if (!std::isfinite(scale)) return fail(RF_ERR_INVALID_ARG, "%s: scale is not finite", name);
    if (dtype != RF_BF16) return fail(RF_ERR_UNSUPPORTED, "%s: only bf16 is supported", name);
    if (d != 64 && d != 128) return fail(RF_ERR_UNSUPPORTED, "%s: d must be 64 or 128, got %d", name, d);
    int64_t nq = 1, nk = 1;
    if (!mul_ok(nq, B) || !mul_ok(nq, Hq) || !mul_ok(nq, d) || !mul_ok(nq, 2) || !mul_ok(nk, B) ||
        !mul_ok(nk, Hkv) || !mul_ok(nk, Lk) || !mul_ok(nk, d) || !mul_ok(nk, 2))
      return fail(RF_ERR_INVALID_ARG, "%s: tensor size overflows int64", name);
    if (int64_t(Lk) * d * 2 > INT32_MAX)
      return fail(RF_ERR_UNSUPPORTED, "%s: needs Lk * d * 2 < 2^31 bytes per key/value head", name);
    if (int64_t(B) * Hq > INT32_MAX) return fail(RF_ERR_UNSUPPORTED, "%s: B * Hq must be below 2^31", name);
    DecodeWs w;
    if (!decode_ws_layout(B, Hq, d, num_splits, w)) return fail(RF_ERR_INVALID_ARG, "%s: workspace size overflows", name);
    if (int64_t(B) * Hq == 0) return ok();
    if (q == nullptr || o == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: NULL q or o", name);
    if (Lk > 0 && (k == nullptr || v == nullptr)) return fail(RF_ERR_INVALID_ARG, "%s: NULL k or v", name);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 8))
      return fail(RF_ERR_UNSUPPORTED, "%s: needs 16-byte aligned q, k, v and 8-byte aligned o", name);
    if (lse != nullptr && !aligned(lse, 4)) return fail(RF_ERR_INVALID_ARG, "%s: lse misaligned", name);
    if (num_splits > 1 && (workspace == nullptr || workspace_bytes < w.total || !aligned(workspace, 256)))
      return fail(RF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu at %p)", name,
                  w.total, workspace_bytes, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int G = Hq / Hkv;
    // q [B, Hq, d] is [B, Hkv, G, d]: the G query heads of a key/value head are
    // the rows of its query tile.
    if (num_splits == 1)
      return hip_status(rf::launch_attention_bf16(q, k, v, o, lse, B, Hkv, G, Lk, d, scale, false, nullptr,
                                                  nullptr, s),
                        name);
    float* o_parts = static_cast<float*>(workspace);
    float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.lse_off);
    hipError_t e =
        rf::launch_attention_bf16_split(q, k, v, o_parts, lse_parts, B * Hkv, G, Lk, d, scale, num_splits, s);
    if (e != hipSuccess) return hip_status(e, "rf_attention_decode_gqa (partials)");
    e = rf::launch_lse_merge(o_parts, lse_parts, o, lse, int64_t(B) * Hq, num_splits, d, RF_BF16, s);
    return hip_status(e, "rf_attention_decode_gqa (merge)");
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "%s: %s", name, e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "%s: unknown exception", name);
  }
}

int rf_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int64_t n_rows, int num_splits,
                 int d, int out_dtype, void* stream) {
  try {
    if (out_dtype != RF_F32 && out_dtype != RF_BF16)
      return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: unknown out_dtype %d", out_dtype);
    if (n_rows < 0) return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: n_rows < 0");
    if (num_splits < 1 || num_splits > 1024)
      return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: num_splits = %d outside 1..1024", num_splits);
    if (d < 1) return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: d = %d < 1", d);
    int64_t n = n_rows;
    if (!mul_ok(n, num_splits) || !mul_ok(n, d) || !mul_ok(n, 4))
      return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: size overflows int64");
    if (n_rows == 0) return ok();
    if (o_parts == nullptr || lse_parts == nullptr || o == nullptr)
      return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: NULL o_parts, lse_parts or o");
    if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(o, out_dtype == RF_F32 ? 4 : 2) ||
        (lse != nullptr && !aligned(lse, 4)))
      return fail(RF_ERR_INVALID_ARG, "rf_lse_merge: misaligned pointer");
    return hip_status(rf::launch_lse_merge(o_parts, lse_parts, o, lse, n_rows, num_splits, d, out_dtype,
                                           static_cast<hipStream_t>(stream)),
                      "rf_lse_merge");
  } catch (const std::exception& e) {
    return fail(RF_ERR_HIP, "rf_lse_merge: %s", e.what());
  } catch (...) {
    return fail(RF_ERR_HIP, "rf_lse_merge: unknown exception");
  }
}

}  // extern "C"
