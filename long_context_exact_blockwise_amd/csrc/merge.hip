// Merge of two partial attention states (m, l, acc) over disjoint key sets, with optional
// finalisation into (O, LSE).
//
// This is the combine step of the LWM pages' ring: each device keeps its query block and
// folds in the contribution of every key/value block that reaches it round the ring (deep
// dive, "RingAttention 为什么必要 / why RingAttention is necessary").  Per row:
//   m' = max(m, mc); l' = l e^(m-m') + lc e^(mc-m'); acc' = acc e^(m-m') + accc e^(mc-m').
// It is pure streaming: 4 floats per thread, bound by HBM bandwidth.

#include <cmath>

#include "common.h"

namespace lwm {
namespace {

// Weight e^(x - m) of a side whose max is x, where m >= x is the merged max; an empty side
// (x = -inf) weighs 0 and a fully empty merge (m = -inf) never subtracts infinities.
__device__ __forceinline__ float side_weight(float x, float m) {
  return x == -INFINITY ? 0.f : expf(x - m);
}

template <bool kHasChunk, bool kFinalize, bool kBf16Out>
__global__ void __launch_bounds__(256) merge_kernel(int64_t rows, int32_t D, float* __restrict__ M,
                                                    float* __restrict__ L, float* __restrict__ ACC,
                                                    const float* __restrict__ Mc,
                                                    const float* __restrict__ Lc,
                                                    const float* __restrict__ ACCc,
                                                    void* __restrict__ O, float* __restrict__ LSE) {
  const int q4 = D / 4;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gid / q4;
  const int part = int(gid % q4);
  if (row >= rows) return;
  const float m1 = M[row], l1 = L[row];
  // an empty state (no key seen) carries m = -inf and l = 0
  LWM_CHECK(q4 * 4 == D && l1 >= 0.f && (m1 != -INFINITY || l1 == 0.f), kChkMerge);
  float4 a = reinterpret_cast<const float4*>(ACC + row * D)[part];
  float m = m1, l = l1;
  if (kHasChunk) {
    const float m2 = Mc[row], l2 = Lc[row];
    const float4 b = reinterpret_cast<const float4*>(ACCc + row * D)[part];
    m = fmaxf(m1, m2);
    const float w1 = side_weight(m1, m), w2 = side_weight(m2, m);
    l = l1 * w1 + l2 * w2;
    a.x = a.x * w1 + b.x * w2;
    a.y = a.y * w1 + b.y * w2;
    a.z = a.z * w1 + b.z * w2;
    a.w = a.w * w1 + b.w * w2;
  }
  if (!kFinalize) {
    reinterpret_cast<float4*>(ACC + row * D)[part] = a;
    if (part == 0) {
      M[row] = m;
      L[row] = l;
    }
    return;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (kBf16Out) {
    __bf16 o4[4] = {(__bf16)(a.x * inv), (__bf16)(a.y * inv), (__bf16)(a.z * inv),
                    (__bf16)(a.w * inv)};
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(O) + row * D)[part] =
        *reinterpret_cast<uint2*>(o4);
  } else {
    reinterpret_cast<float4*>(static_cast<float*>(O) + row * D)[part] =
        make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  }
  if (part == 0) LSE[row] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <bool kHasChunk, bool kFinalize, bool kBf16Out>
hipError_t go(int64_t rows, int32_t D, float* m, float* l, float* acc, const float* mc,
              const float* lc, const float* accc, void* o, float* lse, hipStream_t stream) {
  const int64_t threads = rows * (D / 4);
  merge_kernel<kHasChunk, kFinalize, kBf16Out>
      <<<dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream>>>(rows, D, m, l, acc, mc,
                                                                        lc, accc, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int64_t rows, int32_t D, float* m, float* l, float* acc, const float* mc,
                        const float* lc, const float* accc, int32_t finalize, int32_t out_dtype,
                        void* o, float* lse, hipStream_t stream) {
  const bool chunk = mc != nullptr;
  const bool bf = out_dtype == LWM_BF16;
  if (!finalize) return go<true, false, false>(rows, D, m, l, acc, mc, lc, accc, o, lse, stream);
  if (chunk) {
    return bf ? go<true, true, true>(rows, D, m, l, acc, mc, lc, accc, o, lse, stream)
              : go<true, true, false>(rows, D, m, l, acc, mc, lc, accc, o, lse, stream);
  }
  return bf ? go<false, true, true>(rows, D, m, l, acc, mc, lc, accc, o, lse, stream)
            : go<false, true, false>(rows, D, m, l, acc, mc, lc, accc, o, lse, stream);
}

LWM_DEBUG_READER(merge)

}  // namespace lwm
