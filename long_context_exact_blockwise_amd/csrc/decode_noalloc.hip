// Split-KV decode whose slice states live in a static device buffer of the library, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Same kernels as the workspace form; only
// where the slice states go differs.
//
// The buffer is a file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host that name is only a
// stand-in for the symbol): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress, with that device current, and that address is what the
// kernels receive.  Every call on one GPU shares its copy, so calls that overlap on one GPU
// (two streams, two threads) race on it; the decode kernel writes every slice state it
// later reads, so nothing needs clearing between calls.

#include <mutex>

#include "common.h"

namespace lwm {
namespace {

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on first use.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_bf16_noalloc(const lwm_attn_desc& d, const DecodeLayout& L, const void* q,
                                      const void* k, const void* v, const int32_t* seg_q,
                                      const int32_t* seg_k, const void* table, void* o,
                                      float* lse, hipStream_t stream) {
  if (L.total > kDecodeScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_decode_bf16(d, L, q, k, v, seg_q, seg_k, table, o, lse, ws, stream);
}

}  // namespace lwm
