// Row-wise layer normalisation as one fused reduction tree over a single read.
//
// The cascade mean -> sum of squared deviations from the mean -> normalise is
// a cascaded reduction (RedFuser page, 1. Problématique: normalisation
// layers; the Korean page reports variance as a workload): the second
// reduction depends on the first's root. It fuses into ONE tree over triples
// (n, mean, M2), M2 = sum of squared deviations from mean, which form a
// commutative monoid under the pairwise update
//   (n_a, u_a, M_a) (+) (n_b, u_b, M_b) = (n, u_a + d n_b / n, M_a + M_b + d^2 n_a n_b / n),
//   n = n_a + n_b, d = u_b - u_a,  identity (0, 0, 0),
// the numerically stable form of the decomposition sum (x - u)^2 = sum x^2 - n u^2.
// Each lane reduces its own elements exactly (two passes over registers),
// the lanes meet in the tree, and the row, still in registers, is normalised
// and written: one HBM read and one write per element. All statistics are
// taken relative to the row's first element, so rows far from zero keep their
// fp32 precision. Rows too long for registers take a streaming variant (one
// statistics read, then a normalising read and write).
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"
#include "rows_io.h"

namespace rf {
namespace {

__device__ __forceinline__ void nmm_combine(float& n, float& u, float& m2, float n2, float u2, float m22) {
  const float N = n + n2;
  const float d = u2 - u;
  const float f = N > 0.f ? n2 / N : 0.f;  // two empty triples stay empty
  u = fmaf(d, f, u);
  m2 = m2 + m22 + d * d * n * f;
  n = N;
}

// One butterfly level: this lane's triple meets (n2, u2, m22), the triple of
// the lane group it is paired with. The lower group's triple always goes
// first, so both sides compute the same expression and hold identical bits.
__device__ __forceinline__ void nmm_level(float& n, float& u, float& m2, float n2, float u2, float m22, bool upper) {
  float an = upper ? n2 : n, au = upper ? u2 : u, am = upper ? m22 : m2;
  const float bn = upper ? n : n2, bu = upper ? u : u2, bm = upper ? m2 : m22;
  nmm_combine(an, au, am, bn, bu, bm);
  n = an;
  u = au;
  m2 = am;
}

template <int CTRL>
__device__ __forceinline__ void nmm_dpp_level(float& n, float& u, float& m2, bool upper) {
  nmm_level(n, u, m2, dpp_mov<CTRL>(n), dpp_mov<CTRL>(u), dpp_mov<CTRL>(m2), upper);
}

// Wavefront reduction of the triple with no lane-address registers: DPP
// within rows of 16 lanes (xor 1, xor 2, half mirror, mirror), a swizzle
// across the two rows of each half, and v_permlane32_swap across the halves.
// Every lane ends with the same bits.
__device__ __forceinline__ void wave_nmm(float& n, float& u, float& m2) {
  const int lane = threadIdx.x & 63;
  nmm_dpp_level<0xB1>(n, u, m2, lane & 1);
  nmm_dpp_level<0x4E>(n, u, m2, lane & 2);
  nmm_dpp_level<0x141>(n, u, m2, lane & 4);
  nmm_dpp_level<0x140>(n, u, m2, lane & 8);
  nmm_level(n, u, m2, swizzle_xor16(n), swizzle_xor16(u), swizzle_xor16(m2), lane & 16);
  const auto rn = __builtin_amdgcn_permlane32_swap(__float_as_uint(n), __float_as_uint(n), false, false);
  const auto ru = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(u), false, false);
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2), __float_as_uint(m2), false, false);
  n = __uint_as_float(rn[0]);  // low half first
  u = __uint_as_float(ru[0]);
  m2 = __uint_as_float(rm[0]);
  nmm_combine(n, u, m2, __uint_as_float(rn[1]), __uint_as_float(ru[1]), __uint_as_float(rm[1]));
}

template <int BLOCK>
__device__ __forceinline__ void block_nmm(float& n, float& u, float& m2, float* sn, float* su, float* sm2) {
  constexpr int NW = BLOCK / 64;
  wave_nmm(n, u, m2);
  if constexpr (NW > 1) {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      sn[w] = n;
      su[w] = u;
      sm2[w] = m2;
    }
    __syncthreads();
    n = sn[0];
    u = su[0];
    m2 = sm2[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) nmm_combine(n, u, m2, sn[i], su[i], sm2[i]);
  }
}

template <typename T>
__device__ __forceinline__ float first_elem(const T* p);
template <>
__device__ __forceinline__ float first_elem<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float first_elem<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}

// gamma / beta for EPV consecutive columns through a buffer resource: 16-byte
// loads when EPV >= 4 (the host takes the vector path only for 16-byte aligned
// gamma and beta); a zero-length resource (absent gamma or beta) reads 0.
template <int EPV>
__device__ __forceinline__ void load_affine(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[EPV]) {
  if constexpr (EPV % 4 == 0) {
#pragma unroll
    for (int e = 0; e < EPV; e += 4) {
      const buf_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off + 4 * e), 0, 0);
      o[e] = __uint_as_float(v[0]);
      o[e + 1] = __uint_as_float(v[1]);
      o[e + 2] = __uint_as_float(v[2]);
      o[e + 3] = __uint_as_float(v[3]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, int(off + 4 * e), 0, 0));
  }
}

// Register-resident row: thread t owns vectors t, t + BLOCK, ..., t + (NV-1) BLOCK
// of EPV elements. Every access goes through row-sized buffer resources, so
// the vectors past the row's end read 0 and are never written, with no
// branches; only the statistics mask them out.
//
// RAGGED (fp32, and bf16 of even width): cols need not be a multiple of EPV. The row's last vector
// then straddles its end (raw buffer accesses are range-checked per dword: the
// dwords past the end read 0 and are not written); it sits at a slot and lane
// fixed by cols, and its missing elements are set so that they add nothing to
// either sum (to x0 before the shift, to the lane mean before the squares).
template <typename T, int EPV, int BLOCK, int NV, bool RAGGED = false>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(NV * EPV >= 64 ? 4 : 1))) void layernorm_rows_reg(const T* __restrict__ x, const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, T* __restrict__ y,
                                                            float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                            int64_t rows, int64_t cols, float eps) {
  __shared__ float sn[BLOCK / 64], su[BLOCK / 64], sm2[BLOCK / 64];
  constexpr uint32_t VB = EPV * sizeof(T);      // bytes per row vector
  constexpr uint32_t VA = EPV * sizeof(float);  // bytes per gamma / beta vector
  // vectors touching the row (without RAGGED the host guarantees cols % EPV == 0)
  const int64_t nvec = RAGGED ? (cols + EPV - 1) / EPV : cols / EPV;
  const uint32_t row_bytes = uint32_t(cols) * uint32_t(sizeof(T));
  const int64_t owned = (nvec - int64_t(threadIdx.x) + BLOCK - 1) / BLOCK;
  const int nv = int(owned < NV ? owned : NV);  // vectors of this lane inside the row
  // RAGGED: the last vector (index nvec - 1) is vector kp of lane lp, rem valid elements.
  const int kp = RAGGED ? int((nvec - 1) / BLOCK) : 0;
  const int lp = RAGGED ? int((nvec - 1) % BLOCK) : 0;
  const int rem = RAGGED ? int(cols - (nvec - 1) * EPV) : EPV;
  const float n = float(nv * EPV - ((RAGGED && int(threadIdx.x) == lp) ? EPV - rem : 0));
  // Sets the straddling vector's elements past the row's end to val.
  auto fill_past_end = [&](float (&v)[NV][EPV], float val) {
    if constexpr (RAGGED) {
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (k == kp && int(threadIdx.x) == lp) {
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            if (e >= rem) v[k][e] = val;
        }
    }
  };
  const bool has_gamma = gamma != nullptr;
  const __amdgpu_buffer_rsrc_t gs = row_rsrc(gamma, has_gamma ? uint32_t(cols) * 4u : 0u);
  const __amdgpu_buffer_rsrc_t bs = row_rsrc(beta, beta != nullptr ? uint32_t(cols) * 4u : 0u);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T* xr = x + r * cols;
    const __amdgpu_buffer_rsrc_t xs = row_rsrc(xr, row_bytes);
    const __amdgpu_buffer_rsrc_t ys = row_rsrc(y + r * cols, row_bytes);
    const float x0 = first_elem(xr);  // shift: statistics of x - x0
    float v[NV][EPV];
#pragma unroll
    for (int k = 0; k < NV; ++k) BufIo<T, EPV>::load(xs, (threadIdx.x + k * BLOCK) * VB, v[k]);
    // Lane-local triple, exact two-pass over registers. Vectors past the row's
    // end were read as 0; shifting them by 0 (instead of x0, then u) keeps
    // them 0, so they add nothing to either sum.
    fill_past_end(v, x0);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float sh = k < nv ? x0 : 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        v[k][e] -= sh;
        s += v[k][e];
      }
    }
    float u = n > 0.f ? s / n : 0.f;
    fill_past_end(v, u);
    float m2 = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float sh = k < nv ? u : 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float dv = v[k][e] - sh;
        m2 = fmaf(dv, dv, m2);
      }
    }
    float N = n;
    block_nmm<BLOCK>(N, u, m2, sn, su, sm2);
    const float rstd = 1.f / sqrtf(m2 / N + eps);
    // Output offsets are recomputed from an opaque copy of the lane index, so
    // the per-vector load offsets need not stay live across the reduction.
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const uint32_t vi = t + k * BLOCK;
      float g[EPV], b[EPV];
      load_affine<EPV>(gs, vi * VA, g);
      load_affine<EPV>(bs, vi * VA, b);
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[k][e] = fmaf((v[k][e] - u) * rstd, has_gamma ? g[e] : 1.f, b[e]);
      BufIo<T, EPV>::store(ys, vi * VB, v[k]);
    }
    if (threadIdx.x == 0) {
      if (mean_out != nullptr) mean_out[r] = x0 + u;
      if (rstd_out != nullptr) rstd_out[r] = rstd;
    }
    if (BLOCK > 64 && r + gridDim.x < rows) __syncthreads();  // sn/su/sm2 reused by the next row
  }
}

// Rows too long for registers: one statistics pass (lane triples combined
// vector by vector), then a normalising read + write.
template <typename T, int EPV, int BLOCK>
__global__ __launch_bounds__(BLOCK) void layernorm_rows_stream(const T* __restrict__ x, const float* __restrict__ gamma,
                                                               const float* __restrict__ beta, T* __restrict__ y,
                                                               float* __restrict__ mean_out,
                                                               float* __restrict__ rstd_out, int64_t rows,
                                                               int64_t cols, float eps) {
  __shared__ float sn[BLOCK / 64], su[BLOCK / 64], sm2[BLOCK / 64];
  const int64_t nvec = cols / EPV;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T* xr = x + r * cols;
    T* yr = y + r * cols;
    const float x0 = first_elem(xr);
    float n = 0.f, u = 0.f, m2 = 0.f;
    for (int64_t vi = threadIdx.x; vi < nvec; vi += BLOCK) {
      float a[EPV];
      Io<T, EPV>::load(xr + vi * EPV, a);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        a[e] -= x0;
        s += a[e];
      }
      const float ub = s / float(EPV);
      float mb = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) mb = fmaf(a[e] - ub, a[e] - ub, mb);
      nmm_combine(n, u, m2, float(EPV), ub, mb);
    }
    block_nmm<BLOCK>(n, u, m2, sn, su, sm2);
    const float rstd = 1.f / sqrtf(m2 / n + eps);
    for (int64_t vi = threadIdx.x; vi < nvec; vi += BLOCK) {
      float a[EPV];
      Io<T, EPV>::load(xr + vi * EPV, a);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t c = vi * EPV + e;
        float t = (a[e] - x0 - u) * rstd;
        if (gamma != nullptr) t *= gamma[c];
        if (beta != nullptr) t += beta[c];
        a[e] = t;
      }
      Io<T, EPV>::store(yr + vi * EPV, a);
    }
    if (threadIdx.x == 0) {
      if (mean_out != nullptr) mean_out[r] = x0 + u;
      if (rstd_out != nullptr) rstd_out[r] = rstd;
    }
    if (r + gridDim.x < rows) __syncthreads();
  }
}

template <typename T, int EPV, bool RAGGED = false>
hipError_t dispatch(const T* x, const float* gamma, const float* beta, T* y, float* mean, float* rstd, int64_t rows,
                    int64_t cols, float eps, hipStream_t stream) {
  const int64_t nvec = RAGGED ? (cols + EPV - 1) / EPV : cols / EPV;
  const unsigned grid = unsigned(rows < (1 << 30) ? rows : (1 << 30));
  // Register variants: up to 64 row elements per lane (32 with single-element
  // access), each within the VGPRs of its occupancy. (1024 lanes x 32 fits 64
  // VGPRs but measured slower than 512 x 64 here, unlike softmax.) Longer rows
  // stream.
  constexpr int FPL_MAX = EPV == 1 ? 32 : 64;
#define RF_LN_REG(BLOCK, FPL)                                                                           \
  if constexpr ((FPL) <= FPL_MAX) {                                                                     \
    if (nvec <= int64_t(BLOCK) * ((FPL) / EPV)) {                                                       \
      hipLaunchKernelGGL((layernorm_rows_reg<T, EPV, BLOCK, (FPL) / EPV, RAGGED>), dim3(grid), dim3(BLOCK), 0,  \
                         stream, x, gamma, beta, y, mean, rstd, rows, cols, eps);                       \
      return hipGetLastError();                                                                         \
    }                                                                                                   \
  }
  RF_LN_REG(64, 16)
  RF_LN_REG(128, 32)
  RF_LN_REG(256, 32)
  RF_LN_REG(512, 32)
  RF_LN_REG(512, 64)
#undef RF_LN_REG
  if constexpr (RAGGED) return hipErrorInvalidValue;  // the host keeps ragged rows within the table
  hipLaunchKernelGGL((layernorm_rows_stream<T, EPV, 1024>), dim3(grid), dim3(1024), 0, stream, x, gamma, beta, y,
                     mean, rstd, rows, cols, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layernorm_rows(const void* x, const float* gamma, const float* beta, void* y, float* mean,
                                 float* rstd, int64_t rows, int64_t cols, float eps, int dtype, hipStream_t stream) {
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(gamma) % 16 == 0) && (reinterpret_cast<uintptr_t>(beta) % 16 == 0);
  if (dtype == 0) {
    const float* xf = static_cast<const float*>(x);
    float* yf = static_cast<float*>(y);
    if (aligned && cols % 4 == 0) return dispatch<float, 4>(xf, gamma, beta, yf, mean, rstd, rows, cols, eps, stream);
    // Other widths up to the register table's 32768 columns: 16-byte accesses
    // all the same, the last vector of a row straddling its end.
    if (aligned && cols <= 32768)
      return dispatch<float, 4, true>(xf, gamma, beta, yf, mean, rstd, rows, cols, eps, stream);
    return dispatch<float, 1>(xf, gamma, beta, yf, mean, rstd, rows, cols, eps, stream);
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* yb = static_cast<uint16_t*>(y);
  if (aligned && cols % 8 == 0) return dispatch<uint16_t, 8>(xb, gamma, beta, yb, mean, rstd, rows, cols, eps, stream);
  // Even widths: rows start 4-byte aligned and end on a dword boundary.
  if (aligned && cols % 2 == 0 && cols <= 32768)
    return dispatch<uint16_t, 8, true>(xb, gamma, beta, yb, mean, rstd, rows, cols, eps, stream);
  return dispatch<uint16_t, 1>(xb, gamma, beta, yb, mean, rstd, rows, cols, eps, stream);
}

}  // namespace rf
