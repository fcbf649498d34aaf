// Rotary position embedding arithmetic shared by the standalone RoPE kernel and the
// attention kernels that rotate their register-resident operand at load, so that both give
// the same bits for the same element.
//
// The pages enlarge RoPE's base theta to extend the context (LWM deep dive, section
// "Stage I：长上下文语言模型" and Tables 11 and 13).  Textbook rotary embedding: pair
// i = (x[2i], x[2i+1]) of the token at position p turns by p * theta^(-2i/D).
//
// Precision.  The angle is formed in float64 as revolutions t = p * rev_i with
// rev_i = theta^(-2i/D) / (2 pi); its fractional part t - rint(t), exact in float64, goes to
// float32, so the angle error stays below 1e-6 radian for every position below 2^32.  The
// per-pair factors rev_i are computed once on the host (rope_freqs) and passed to the
// kernels, so every kernel turns a pair by the same angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace lwm {

constexpr int kRopeMaxPairs = 128;  // D <= 256

// rev_i = theta^(-2i/D) / (2 pi) for the D/2 pairs of a row.
struct RopeFreq {
  double rev[kRopeMaxPairs];
};

inline RopeFreq rope_freqs(int D, double theta) {
  RopeFreq f{};
  const double l2t = std::log2(theta);
  for (int i = 0; i < D / 2 && i < kRopeMaxPairs; ++i)
    f.rev[i] = std::exp2(-double(2 * i) / D * l2t) * 0.15915494309189533577;
  return f;
}

// Fraction of a turn, in [-1/2, 1/2], of the angle of a pair with factor rev at position pos.
__device__ __forceinline__ float rope_turn(int64_t pos, double rev) {
  const double t = double(pos) * rev;
  return float(t - rint(t));
}

// cos and sin of 2 pi f from the hardware units, which take their argument in turns
// (|f| <= 1/2 here, well inside their domain); used for bf16 data, whose rounding (2^-9
// relative) dwarfs their error.
__device__ __forceinline__ void rope_cs_turns(float f, float& c, float& s) {
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// (a, b) turned by the angle whose cos and sin are c and s; the roundings are spelled out
// (one product, then one fused multiply-add) so every kernel rounds alike.
__device__ __forceinline__ void rope_turn_pair(float& a, float& b, float c, float s) {
  const float x = fmaf(a, c, -(b * s));
  const float y = fmaf(a, s, b * c);
  a = x;
  b = y;
}

}  // namespace lwm
