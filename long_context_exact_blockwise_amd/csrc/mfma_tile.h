// Device helpers for the bf16 MFMA attention kernels (gfx950 / CDNA4).
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (checked on the hardware), lane l, h = l/32:
//   A (32 x 16):  lane l holds row l%32, k = 8h .. 8h+7      (8 bf16, one 16-byte load)
//   B (16 x 32):  lane l holds column l%32, k = 8h .. 8h+7
//   C (32 x 32):  lane l holds column l%32, rows 8*(i/4) + 4h + (i%4) for slot i = 0..15
//
// Transposed formulation.  Scores are computed as S^T = K Q^T (rows = keys, columns =
// queries), so each lane owns one query column; the row statistics of softmax become
// per-lane scalars (plus one exchange between the two 32-lane halves).  P^T then feeds the
// B operand of O^T = V^T P^T directly, without a trip through LDS, provided the K rows are
// loaded in the order kperm(): swapping bits 2 and 3 of the row index makes C slot
// i = 8a + j (a = 0,1; j = 0..7) of a 32-key block hold key 16a + 8h + j, which is exactly
// the B-operand k index of the a-th 16-key MFMA step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of a 32-row A tile that lane l must load so that C slots come out in B-operand order.
__device__ __forceinline__ int kperm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Key (or query, for the key-major kernels) index within a 32-block held by C slot i of a
// lane in half h, when the A tile was loaded in kperm order.
__device__ __forceinline__ int slot_index(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

// Row index held by C slot i of a lane in half h (plain order).
__device__ __forceinline__ int out_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// max / sum of x over the lane pair (l, l ^ 32): permlane32_swap hands each lane the
// partner value in one of its two results and its own value in the other.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8 bf16 from 8 floats (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

__device__ __forceinline__ bf16x8 lds_load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ uint4 gload16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace lwm
