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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
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

// ---- LDS tiles of 128-wide bf16 rows ------------------------------------------------------
//
// A tile holds rows of 128 bf16 (256 bytes, 16 chunks of 16 bytes).  Chunk c of row r is
// stored at chunk c ^ tile_swz(r), which keeps three access patterns free of bank conflicts:
//   - 16-byte row reads by 16 lanes on 16 distinct rows of an aligned 16-row group (MFMA
//     operands taken along the row),
//   - transposed reads (ds_read_b64_tr_b16) of 4 consecutive rows x 32 columns,
//   - 16-byte writes of one row by 16 lanes while staging from global memory.
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ int tile_off(int row, int col) {
  return row * 128 + ((((col >> 3) ^ tile_swz(row))) << 3) + (col & 7);
}

// MFMA operand read across rows of a tile with ds_read_b64_tr_b16: lane l receives
// T[r0 + 8h + j][c0 + l%32] for j = 0..7 (h = l/32), i.e. the A/B operand of an MFMA whose
// M (or N) index is the tile column and whose k index is the tile row.  Within each group
// of 16 lanes, lane 4j+p supplies the address of row j, columns 4p..4p+3 of its group's
// 4 x 16 block, and the instruction hands lane i column i of rows 0..3.  r0 must be a
// multiple of 8 and c0 a multiple of 32.
__device__ __forceinline__ bf16x8 lds_load_tr8(const uint16_t* tile, int r0, int c0, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int row = r0 + 8 * (g >> 1) + (r >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (r & 3);
  typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tile + tile_off(row, col)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tile + tile_off(row + 4, col)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// exp2 straight from the hardware unit (v_exp_f32, about 1 ulp) without the library's
// denormal range fix-up: results below 2^-126 flush to zero, which softmax weights afford.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 gload16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace lwm
