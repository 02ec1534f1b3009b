// Row-wise safe softmax as one fused reduction tree over a single read of the row.
//
// The cascade max -> sum of exp(x - max) -> normalise (RedFuser page, Résumé
// technique, 1. Problématique; d_i = ⊕ F_i(X[l], D_i) in 2. Méthodologie) is
// fused with the rescale identity e^{x-y} = e^x / e^y (FLASHLIGHT page,
// Metodologia 3): each lane reduces its own elements to a pair (m_t, l_t),
// and the pairs meet in ONE tree under
//   (m_a, l_a) (+) (m_b, l_b) = (M, l_a e^{m_a - M} + l_b e^{m_b - M}).
// The row stays in registers between the reduction and the normalisation, so
// every element is read from HBM once and written once (single-segment
// strategy: one workgroup owns one row, no inter-workgroup synchronisation).
// Rows longer than a workgroup's register capacity take a streaming variant:
// one online (m, l) read, then a normalising read + write.
#include <stdint.h>

#include "launch.h"
#include "rf_internal.h"
#include "rows_io.h"

namespace rf {
namespace {

// One butterfly level of the (m, l) tree: this lane's pair meets (m2, l2), the
// pair of the lane group it is paired with. The lower group's pair always goes
// first, so both sides evaluate the same expression and hold identical bits.
__device__ __forceinline__ void ml_level(float& m, float& l, float m2, float l2, bool upper) {
  float am = upper ? m2 : m, al = upper ? l2 : l;
  const float bm = upper ? m : m2, bl = upper ? l : l2;
  ml_combine_nat(am, al, bm, bl);
  m = am;
  l = al;
}

template <int CTRL>
__device__ __forceinline__ void ml_dpp_level(float& m, float& l, bool upper) {
  ml_level(m, l, dpp_mov<CTRL>(m), dpp_mov<CTRL>(l), upper);
}

// Workgroup-wide (+)-reduction of (m, l) with no lane-address registers: DPP
// within rows of 16 lanes, a swizzle across the two rows of each half,
// v_permlane32_swap across the halves, then LDS across waves. Every lane ends
// with the same bits.
template <int BLOCK>
__device__ __forceinline__ void block_combine(float& m, float& l, float* sm, float* sl) {
  constexpr int NW = BLOCK / 64;
  const int lane = threadIdx.x & 63;
  ml_dpp_level<0xB1>(m, l, lane & 1);
  ml_dpp_level<0x4E>(m, l, lane & 2);
  ml_dpp_level<0x141>(m, l, lane & 4);
  ml_dpp_level<0x140>(m, l, lane & 8);
  ml_level(m, l, swizzle_xor16(m), swizzle_xor16(l), lane & 16);
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  m = __uint_as_float(rm[0]);  // low half first
  l = __uint_as_float(rl[0]);
  ml_combine_nat(m, l, __uint_as_float(rm[1]), __uint_as_float(rl[1]));
  if constexpr (NW > 1) {
    const int w = threadIdx.x >> 6;
    if (lane == 0) {
      sm[w] = m;
      sl[w] = l;
    }
    __syncthreads();
    m = sm[0];
    l = sl[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) ml_combine_nat(m, l, sm[i], sl[i]);
  }
}

// Register-resident row: thread t owns vectors t, t + BLOCK, ..., t + (NV-1) BLOCK
// of EPV elements. Every access goes through row-sized buffer resources: the
// vectors past the row's end read 0 and are never written, with no branches;
// the reduction replaces them by -inf.
// RAGGED (fp32, and bf16 of even width): cols need not be a multiple of EPV.
// The last vector then straddles the row's end: a raw buffer access is
// range-checked per dword, so its dwords past the end read 0 and are not
// written. Rows start only 4-byte aligned, which 16-byte buffer accesses
// allow.
template <typename T, int EPV, int BLOCK, int NV, bool RAGGED = false>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(BLOCK == 1024 && EPV > 1 && NV * EPV == 32 ? 8 : 1))) void softmax_rows_reg(const T* __restrict__ x, T* __restrict__ y,
                                                          int64_t rows, int64_t cols) {
  __shared__ float sm[BLOCK / 64], sl[BLOCK / 64];
  constexpr uint32_t VB = EPV * sizeof(T);  // bytes per vector
  // vectors touching the row (without RAGGED the host guarantees cols % EPV == 0)
  const int64_t nvec = RAGGED ? (cols + EPV - 1) / EPV : cols / EPV;
  const uint32_t row_bytes = uint32_t(cols) * uint32_t(sizeof(T));
  const int64_t owned = (nvec - int64_t(threadIdx.x) + BLOCK - 1) / BLOCK;
  const int nv = int(owned < NV ? owned : NV);  // vectors of this lane inside the row
  // RAGGED: the row's last vector (index nvec - 1) is vector kp of lane lp and
  // holds rem valid elements (the host keeps ragged rows within 65536 columns).
  const int kp = RAGGED ? int((nvec - 1) / BLOCK) : 0;
  const int lp = RAGGED ? int((nvec - 1) % BLOCK) : 0;
  const int rem = RAGGED ? int(cols - (nvec - 1) * EPV) : EPV;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const __amdgpu_buffer_rsrc_t xs = row_rsrc(x + r * cols, row_bytes);
    const __amdgpu_buffer_rsrc_t ys = row_rsrc(y + r * cols, row_bytes);
    float v[NV][EPV];
#pragma unroll
    for (int k = 0; k < NV; ++k) BufIo<T, EPV>::load(xs, (threadIdx.x + k * BLOCK) * VB, v[k]);
    if constexpr (RAGGED) {
      // Only the row's last vector can straddle its end: vector kp of lane lp
      // (both fixed by cols). Its elements past the end (read as 0) become -inf.
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (k == kp && int(threadIdx.x) == lp) {
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            if (e >= rem) v[k][e] = kNegInf;
        }
    }
    // Lane-local pair: m_t = max of its elements, l_t = sum_e e^{x_e - m_t}.
    float m = kNegInf;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        v[k][e] = k < nv ? v[k][e] : kNegInf;
        m = fmaxf(m, v[k][e]);
      }
    const float mu = (m == kNegInf) ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        v[k][e] = fast_exp2((v[k][e] - mu) * kLog2e);
        l += v[k][e];
      }
    float M = m, L = l;
    block_combine<BLOCK>(M, L, sm, sl);
    // y = e^{x - m_t} * e^{m_t - M} / L  (an all -inf row gives NaN, as the definition does)
    const float c = fast_exp2((m - M) * kLog2e) / L;
    // Store offsets are recomputed from an opaque copy of the lane index, so
    // the load offsets need not stay live across the reduction.
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int k = 0; k < NV; ++k) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[k][e] *= c;
      BufIo<T, EPV>::store(ys, (t + k * BLOCK) * VB, v[k]);
    }
    if (BLOCK > 64 && r + gridDim.x < rows) __syncthreads();  // sm/sl reused by the next row
  }
}

// Rows too long for registers: an online (m, l) pass, then a normalising pass.
template <typename T, int EPV, int BLOCK>
__global__ __launch_bounds__(BLOCK) void softmax_rows_stream(const T* __restrict__ x, T* __restrict__ y,
                                                             int64_t rows, int64_t cols) {
  __shared__ float sm[BLOCK / 64], sl[BLOCK / 64];
  const int64_t nvec = cols / EPV;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T* xr = x + r * cols;
    T* yr = y + r * cols;
    float m = kNegInf, l = 0.f;  // running pair, m in natural units
    for (int64_t vi = threadIdx.x; vi < nvec; vi += BLOCK) {
      float a[EPV];
      Io<T, EPV>::load(xr + vi * EPV, a);
      float bm = kNegInf;
#pragma unroll
      for (int e = 0; e < EPV; ++e) bm = fmaxf(bm, a[e]);
      const float mn = fmaxf(m, bm);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) s += fast_exp2((a[e] - mu) * kLog2e);
      l = l * fast_exp2((m - mu) * kLog2e) + s;  // rescale when the running max moves
      m = mn;
    }
    block_combine<BLOCK>(m, l, sm, sl);
    const float inv = 1.f / l;
    for (int64_t vi = threadIdx.x; vi < nvec; vi += BLOCK) {
      float a[EPV];
      Io<T, EPV>::load(xr + vi * EPV, a);
#pragma unroll
      for (int e = 0; e < EPV; ++e) a[e] = fast_exp2((a[e] - m) * kLog2e) * inv;
      Io<T, EPV>::store(yr + vi * EPV, a);
    }
    if (r + gridDim.x < rows) __syncthreads();
  }
}

// Register-resident variants, smallest first: (lanes per workgroup, elements per
// lane). Each stays within the VGPRs of its occupancy without spilling; a row of
// 16k-32k elements goes to 1024 lanes x 32 (64 VGPRs: two workgroups, eight waves
// per SIMD), which streams faster than 512 lanes x 64 (two workgroups, four waves
// per SIMD).
template <typename T, int EPV, bool RAGGED = false>
hipError_t dispatch(const T* x, T* y, int64_t rows, int64_t cols, hipStream_t stream) {
  const int64_t nvec = RAGGED ? (cols + EPV - 1) / EPV : cols / EPV;
  const unsigned grid = unsigned(rows < (1 << 30) ? rows : (1 << 30));
#define RF_SOFTMAX_REG(BLOCK, FPL)                                                                  \
  if (nvec <= int64_t(BLOCK) * ((FPL) / EPV)) {                                                    \
    hipLaunchKernelGGL((softmax_rows_reg<T, EPV, BLOCK, (FPL) / EPV, RAGGED>), dim3(grid), dim3(BLOCK), 0, \
                       stream, x, y, rows, cols);                                                  \
    return hipGetLastError();                                                                      \
  }
  RF_SOFTMAX_REG(64, 16)
  RF_SOFTMAX_REG(128, 32)
  RF_SOFTMAX_REG(256, 32)
  RF_SOFTMAX_REG(512, 32)
  RF_SOFTMAX_REG(1024, 32)
  RF_SOFTMAX_REG(512, 64)
  RF_SOFTMAX_REG(1024, 64)
#undef RF_SOFTMAX_REG
  if constexpr (RAGGED) return hipErrorInvalidValue;  // the host keeps ragged rows within the table
  hipLaunchKernelGGL((softmax_rows_stream<T, EPV, 1024>), dim3(grid), dim3(1024), 0, stream, x, y,
                     rows, cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int dtype,
                               hipStream_t stream) {
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
  if (dtype == 0) {
    const float* xf = static_cast<const float*>(x);
    float* yf = static_cast<float*>(y);
    if (aligned && cols % 4 == 0) return dispatch<float, 4>(xf, yf, rows, cols, stream);
    // Other widths up to the register table's 65536 columns: 16-byte accesses
    // all the same, the last vector of a row straddling its end.
    if (cols <= 65536) return dispatch<float, 4, true>(xf, yf, rows, cols, stream);
    return dispatch<float, 1>(xf, yf, rows, cols, stream);
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* yb = static_cast<uint16_t*>(y);
  if (aligned && cols % 8 == 0) return dispatch<uint16_t, 8>(xb, yb, rows, cols, stream);
  // Even widths: rows start 4-byte aligned and end on a dword boundary, so the
  // straddling last vector works as for fp32.
  if (aligned && cols % 2 == 0 && cols <= 65536) return dispatch<uint16_t, 8, true>(xb, yb, rows, cols, stream);
  return dispatch<uint16_t, 1>(xb, yb, rows, cols, stream);
}

}  // namespace rf
