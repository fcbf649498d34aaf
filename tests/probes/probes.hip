// Microbenchmarks of the gfx950 facts the attention kernels are designed around: the bf16
// MFMA issue rate, the v_exp_f32 issue rate, LDS read bandwidth, streaming HBM read
// bandwidth, and float32 atomic-add throughput to global memory in the pattern an atomic
// dQ accumulation would use.  Test infrastructure: built beside the library, run by
// tests/test_gpu_probes.py and `python bench.py --probes`; the library never uses it.
//
// Every kernel touches only the buffers it is given, within their stated sizes, and ends
// after a fixed number of iterations.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// iters rounds of 4 independent chains of v_mfma_f32_32x32x16_bf16 per wave; one float per
// wave lands in out so nothing is optimised away.  out: gridDim.x * waves floats.
__global__ void __launch_bounds__(256) mfma_probe(int iters, float* out) {
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (threadIdx.x + j));
    b[j] = (__bf16)(0.002f * (threadIdx.x - j));
  }
  f32x16 c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

// iters rounds of 8 independent v_exp_f32 per lane, x -> 2^-x (the negation is a source
// modifier, so the loop is exponentials only and stays in [1/2, 1]).  out: gridDim.x *
// blockDim.x floats.
__global__ void __launch_bounds__(256) exp_probe(int iters, float* out) {
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = 0.001f * (threadIdx.x + j);
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// iters rounds of 16-byte LDS reads over a 64 KiB array (each lane its own chunks, so no
// bank conflicts).  out: gridDim.x * blockDim.x floats.
__global__ void __launch_bounds__(256) lds_probe(int iters, float* out) {
  __shared__ uint4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  // two three-input adds per 16-byte read, so VALU work stays below the LDS rate
  uint32_t acc = 0, acc2 = 0;
  for (int i = 0; i < iters; ++i) {
    const uint4* row = buf + ((threadIdx.x + i) & 255);  // then 16 reads at fixed offsets
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 v = row[256 * j];
      acc = acc + v.x + v.y;
      acc2 = acc2 + v.z + v.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = float(acc ^ acc2);
}

// Streaming read of n uint4 (16 bytes each), grid-stride, four independent loads in flight
// per lane (every index below n); one partial per thread to out (gridDim.x * blockDim.x
// floats).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) read_probe(const u32x4* __restrict__ src, int64_t n, float* out) {
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc += (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) + (c[0] ^ c[1] ^ c[2] ^ c[3]) +
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc += v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = float(acc);
}

// float32 atomic adds of whole 64 x 128 tiles (32 KiB, rows of 512 bytes), the shape of one
// query tile's dQ contribution: workgroup w adds `steps` tiles, tile (w + t) mod ntiles at
// step t, each lane one float per instruction.  dst: ntiles * 8192 floats.
__global__ void __launch_bounds__(256) atomic_probe(float* __restrict__ dst, int64_t ntiles, int steps) {
  for (int t = 0; t < steps; ++t) {
    float* tile = dst + ((int64_t(blockIdx.x) + t) % ntiles) * 8192;
#pragma unroll 4
    for (int i = threadIdx.x; i < 8192; i += 256) unsafeAtomicAdd(tile + i, 1.0f);
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One v_mfma_f32_16x16x32_bf16 with operands loaded in the layout the kernels assume, for a
// check against a host matmul: lane l holds A row l % 16, k = 8 (l / 16) .. + 7; B column
// l % 16, the same k; C column l % 16, rows 4 (l / 16) .. + 3.  A [16][32], B [32][16] and
// C [16][16] are float32 row-major; one wave of 64 lanes.
__global__ void __launch_bounds__(64) mfma16_layout_probe(const float* A, const float* B, float* C) {
  const int l = threadIdx.x, r = l & 15, g = l >> 4;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)A[r * 32 + 8 * g + j];
    b[j] = (__bf16)B[(8 * g + j) * 16 + r];
  }
  const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0, 0, 0, 0}, 0, 0, 0);
  for (int i = 0; i < 4; ++i) C[(4 * g + i) * 16 + r] = c[i];
}

}  // namespace

extern "C" {

int lwm_probe_mfma16_layout(const float* A, const float* B, float* C, void* stream) {
  mfma16_layout_probe<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(A, B, C);
  return int(hipGetLastError());
}

int lwm_probe_mfma(int blocks, int iters, float* out, void* stream) {
  mfma_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return int(hipGetLastError());
}
int lwm_probe_exp(int blocks, int iters, float* out, void* stream) {
  exp_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return int(hipGetLastError());
}
int lwm_probe_lds(int blocks, int iters, float* out, void* stream) {
  lds_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return int(hipGetLastError());
}
int lwm_probe_read(int blocks, const void* src, int64_t n16, float* out, void* stream) {
  read_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src), n16, out);
  return int(hipGetLastError());
}
int lwm_probe_atomic(int blocks, float* dst, int64_t ntiles, int steps, void* stream) {
  atomic_probe<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(dst, ntiles, steps);
  return int(hipGetLastError());
}

}  // extern "C"
