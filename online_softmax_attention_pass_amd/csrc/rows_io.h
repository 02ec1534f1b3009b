// Row element access (and one lane exchange) shared by the row kernels
// (softmax, layer norm): fp32 or
// bf16 (raw bits), as 16-byte vectors of EPV elements, or single elements
// (EPV = 1) when a row is not 16-byte aligned. Loads and stores are
// non-temporal: every element is touched once.
//
// Io takes global pointers. BufIo goes through a buffer resource (base and
// byte length in scalar registers, a 32-bit byte offset per lane): an access
// whose offset is at or past the length reads 0 and a store there is dropped,
// which is how register-resident row kernels skip their bounds branches.
// Offsets are always passed in the per-lane operand, the one the hardware
// range check covers; the scalar offset is 0.
#pragma once
#include <stdint.h>

#include "rf_internal.h"

namespace rf {

template <typename T, int EPV> struct Io;

template <> struct Io<float, 4> {
  __device__ static void load(const float* p, float (&o)[4]) {
    const float4 v = nt_load(reinterpret_cast<const float4*>(p));
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ static void store(float* p, const float (&o)[4]) {
    float4 v = make_float4(o[0], o[1], o[2], o[3]);
    nt_store(v, reinterpret_cast<float4*>(p));
  }
};
template <> struct Io<float, 1> {
  __device__ static void load(const float* p, float (&o)[1]) { o[0] = *p; }
  __device__ static void store(float* p, const float (&o)[1]) { *p = o[0]; }
};
template <> struct Io<uint16_t, 8> {
  __device__ static void load(const uint16_t* p, float (&o)[8]) {
    const uint4 v = nt_load(reinterpret_cast<const uint4*>(p));
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
  __device__ static void store(uint16_t* p, const float (&o)[8]) {
    uint4 v;
    v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
    nt_store(v, reinterpret_cast<uint4*>(p));
  }
};
template <> struct Io<uint16_t, 1> {
  __device__ static void load(const uint16_t* p, float (&o)[1]) { o[0] = bf16_to_f32(*p); }
  __device__ static void store(uint16_t* p, const float (&o)[1]) { *p = uint16_t(f32_to_bf16_bits(o[0])); }
};

// Lane l exchanges x with lane l ^ 16 (ds_swizzle, bit mode: and 0x1f, xor 16).
__device__ __forceinline__ float swizzle_xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1F));
}

typedef uint32_t buf_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufNonTemporal = 2;  // cache policy bit: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

template <typename T, int EPV> struct BufIo;

template <> struct BufIo<float, 4> {
  __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[4]) {
    const buf_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kBufNonTemporal);
    o[0] = __uint_as_float(v[0]); o[1] = __uint_as_float(v[1]);
    o[2] = __uint_as_float(v[2]); o[3] = __uint_as_float(v[3]);
  }
  __device__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&o)[4]) {
    buf_u32x4 v = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, kBufNonTemporal);
  }
};
template <> struct BufIo<float, 1> {
  __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[1]) {
    o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, kBufNonTemporal));
  }
  __device__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&o)[1]) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[0]), r, int(off), 0, kBufNonTemporal);
  }
};
template <> struct BufIo<uint16_t, 8> {
  __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[8]) {
    const buf_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kBufNonTemporal);
    o[0] = bf16_lo(v[0]); o[1] = bf16_hi(v[0]); o[2] = bf16_lo(v[1]); o[3] = bf16_hi(v[1]);
    o[4] = bf16_lo(v[2]); o[5] = bf16_hi(v[2]); o[6] = bf16_lo(v[3]); o[7] = bf16_hi(v[3]);
  }
  __device__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&o)[8]) {
    buf_u32x4 v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                   pack_bf16x2(o[6], o[7])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, kBufNonTemporal);
  }
};
template <> struct BufIo<uint16_t, 1> {
  __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[1]) {
    o[0] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, kBufNonTemporal));
  }
  __device__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&o)[1]) {
    __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(o[0])), r, int(off), 0, kBufNonTemporal);
  }
};

}  // namespace rf
