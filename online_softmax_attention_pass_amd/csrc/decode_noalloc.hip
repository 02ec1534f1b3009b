// Split-KV decode for callers that cannot allocate: the same partial and merge
// kernels as rf_attention_decode_splitkv (decode_splitkv.hip, lse_merge.hip),
// with the partials (O_s, lse_s) in a device array of the library's own
// instead of a caller workspace.
#include <stdint.h>

#include <mutex>

#include "launch.h"

// The partials of one call, laid out as the caller workspace of
// rf_attention_decode_splitkv. Every GPU the library runs on holds its own copy,
// at its own address, until the process ends; calls on one GPU share it, so
// calls that overlap on one GPU race. Host code never passes this name to a
// kernel (on the host it only stands in for the symbol): the device address
// comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[rf::kDecodeScratchBytes];

namespace rf {
namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current.
hipError_t scratch_on_stream_device(hipStream_t stream, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_splitkv_scratch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                         int H, int Lk, int d, float scale, int num_splits, size_t lse_off,
                                         hipStream_t stream) {
  void* ws = nullptr;
  hipError_t e = scratch_on_stream_device(stream, &ws);
  if (e != hipSuccess) return e;
  float* o_parts = static_cast<float*>(ws);
  float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_off);
  e = launch_decode_partials(q, k, v, o_parts, lse_parts, B, H, Lk, d, scale, num_splits, stream);
  if (e != hipSuccess) return e;
  return launch_lse_merge(o_parts, lse_parts, o, lse, int64_t(B) * H, num_splits, d, 1 /* bf16 */, stream);
}

}  // namespace rf
