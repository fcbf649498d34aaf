// Rotary position embedding (RoPE) with a large base theta: rotates a [B,H,S,D] tensor of
// queries or keys by global token position, or rotates a gradient back (inverse).
//
// The LWM pages extend the context window by enlarging RoPE's base theta (deep dive, section
// "Stage I：长上下文语言模型" and Tables 11 and 13: theta from 1M at 32K tokens up to 50M at 1M
// tokens).  Pair i = (x[2i], x[2i+1]) of the token at position p turns by the angle
// p * theta^(-2i/D); the inverse turns by the opposite angle.
//
// Precision.  At theta = 5e7 and p near 2^20 the angle of the fastest pair is about 10^6
// radians; a float32 product p * w_i would already be off by several hundredths of a radian.
// So the angle is formed in float64 as revolutions, t = p * w_i / (2 pi), whose fractional
// part t - rint(t) is exact in float64; only that fraction in [-1/2, 1/2] goes to float32
// (rope_math.h, shared with the attention kernels that rotate Q or K at load, so both turn a
// pair by the same angle and round alike).  cos and sin of 2 pi * fraction come from the
// hardware units for bf16 data and from sincospi for float32 data.  The angle error stays
// below 1e-6 radian for every position below 2^32.
//
// Work split.  The kernel streams the tensor once (HBM bound).  A thread owns 8 consecutive
// elements (4 pairs) at one position; a position's D elements take D/8 threads, and the grid
// stride is a multiple of D/8, so a thread meets the same 4 pairs at every position it visits
// and works out their frequencies once.  The angles of a position serve every batch row and
// head, so a thread rotates its 8 elements in a group of four (batch, head) rows of that
// position, one row after the other, after one sin/cos per pair; the grid's y index picks
// the group.  Measured at B1 H32 S131072 D128: four rows per thread taken one at a time reach
// 5.4 TB/s (read + write); two or eight rows, or several rows' loads in flight at once, run
// 10-25 % slower.

#include <cmath>

#include "common.h"
#include "rope_math.h"

namespace lwm {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kRowsPerThread = 4;  // (batch, head) rows per thread and position

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  __bf16 b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)v[i];  // round to nearest even
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(b);
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
rope_kernel(int64_t BH, int64_t rpt, int32_t S, int32_t D, int32_t tpr_shift, int64_t pos0,
            RopeFreq fr, float dir, const T* x, T* y) {  // x and y may be the same buffer
  // D / 8 = 2^tpr_shift threads per position, a divisor of kThreads
  const int64_t total = int64_t(S) << tpr_shift;
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int part = int(g & ((1 << tpr_shift) - 1));
  // revolutions per position of this thread's pairs: theta^(-2i/D) / (2 pi)
  double rev[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) rev[k] = fr.rev[4 * part + k];
  const int64_t rstride = int64_t(S) * D;  // from one (batch, head) row block to the next
  // this workgroup's share of the batch rows and heads: rpt of them
  const int64_t bh0 = int64_t(blockIdx.y) * rpt;
  if (bh0 >= BH) return;
  const int64_t bh1 = bh0 + rpt < BH ? bh0 + rpt : BH;
  x += bh0 * rstride;
  y += bh0 * rstride;
  for (; g < total; g += stride) {
    const int64_t s = g >> tpr_shift;
    float cs[4], sn[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float f = rope_turn(pos0 + s, rev[k]);  // fraction of a turn, |f| <= 1/2
      if constexpr (sizeof(T) == 2)
        rope_cs_turns(f, cs[k], sn[k]);
      else
        sincospif(2.f * f, &sn[k], &cs[k]);
      sn[k] *= dir;
    }
    // every batch row and head shares the position, hence the angles
    const T* xs = x + s * D + 8 * part;
    T* ys = y + s * D + 8 * part;
    auto turn = [&](float* v) {
#pragma unroll
      for (int k = 0; k < 4; ++k) rope_turn_pair(v[2 * k], v[2 * k + 1], cs[k], sn[k]);
    };
    const int64_t n = bh1 - bh0;
    for (int64_t bh = 0; bh < n; ++bh) {
      float v[8];
      load8(xs + bh * rstride, v);
      turn(v);
      store8(ys + bh * rstride, v);
    }
  }
}

}  // namespace

hipError_t launch_rope(int32_t B, int32_t H, int32_t S, int32_t D, int32_t dtype, int64_t pos0,
                       double theta, int32_t inverse, const void* x, void* y, hipStream_t stream) {
  const int64_t threads = int64_t(S) * (D / 8);
  int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;  // grid stride loop beyond that
  const int64_t bh = int64_t(B) * H;
  int64_t rpt = kRowsPerThread;
  if ((bh + rpt - 1) / rpt > 65535) rpt = (bh + 65534) / 65535;  // the grid's y extent
  const int64_t groups = (bh + rpt - 1) / rpt;
  const RopeFreq fr = rope_freqs(D, theta);
  const float dir = inverse ? -1.f : 1.f;
  int shift = 0;
  while ((8 << shift) < D) ++shift;
  if (dtype == LWM_BF16)
    rope_kernel<uint16_t><<<dim3(unsigned(blocks), unsigned(groups)), dim3(kThreads), 0, stream>>>(
        bh, rpt, S, D, shift, pos0, fr, dir, static_cast<const uint16_t*>(x),
        static_cast<uint16_t*>(y));
  else
    rope_kernel<float><<<dim3(unsigned(blocks), unsigned(groups)), dim3(kThreads), 0, stream>>>(
        bh, rpt, S, D, shift, pos0, fr, dir, static_cast<const float*>(x),
        static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace lwm
