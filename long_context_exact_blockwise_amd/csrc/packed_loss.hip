// Packed-sequence loss reweighting: next-token cross-entropy over logits [B,T,V] in which
// every packed sample carries the same total weight, fused with its gradient.
//
// The LWM pages pack many samples into one long sequence and reweight the loss so that it
// matches training the samples unpacked with padding; otherwise samples with many tokens
// (long videos) outweigh samples with few loss tokens (short answers) (deep dive, section
// "Masked sequence packing", second step of the recipe).  With n_s the loss tokens of sample
// s (a segment id within a batch row) and N the samples that have any, a loss token of s has
// weight w = 1 / (N n_s):
//   l_t = logsumexp(x_t) - x_t[y_t],   loss = sum_t w_t l_t,   dx_t = g w_t (softmax(x_t) - e_{y_t}).
//
// Kernels, in stream order:
//   count    one thread per token: integer atomic add into the per-sample counters;
//   samples  one workgroup: N = number of counters above zero;
//   ce       one workgroup per token row, the smallest of 256, 512 or 1024 threads whose
//            registers hold the row: the row's logits are loaded once into registers (8 per
//            chunk, up to 24 chunks per thread for bf16 and 12 for float32; 1024 threads take
//            V up to 131072 or 65536), max and sum of exponentials
//            are reduced across the workgroup, then the gradient row is written; rows that
//            are not loss tokens skip the load and write zeros;
//   sum      one workgroup: the weighted token losses are summed in a fixed order, so the
//            loss is the same on every run.
// The logits are read from HBM once and the gradient written once: the ce kernel is bound
// by HBM bandwidth.

#include <cmath>

#include "common.h"

namespace lwm {
namespace {

constexpr int kMaxWaves = 16;  // largest workgroup: 1024 threads
constexpr float kLog2e = 1.4426950408889634f;

// Packed samples are long runs of one id, so the lanes of a wave almost always count into
// the same counter: the wave groups its lanes by counter (one round per distinct counter)
// and one lane adds the group's size, instead of one atomic per token on a few addresses.
__global__ void __launch_bounds__(256) loss_count_kernel(int64_t tokens, int32_t T, int32_t V,
                                                         int32_t nseg, const int32_t* __restrict__ tg,
                                                         const int32_t* __restrict__ seg,
                                                         int32_t* __restrict__ cnt) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  int64_t key = -1;
  if (i < tokens) {
    const int32_t s = seg[i], y = tg[i];
    if (s >= 0 && s < nseg && y >= 0 && y < V) key = (i / T) * nseg + s;
  }
  bool pending = key >= 0;
  while (__ballot(pending) != 0) {
    // the lowest pending lane's counter; every lane with the same counter joins its group
    const uint64_t pend = __ballot(pending);
    const int leader = __ffsll(static_cast<unsigned long long>(pend)) - 1;
    const int64_t k = __shfl(key, leader);
    const bool mine = pending && key == k;
    const uint64_t group = __ballot(mine);
    if (mine && int(threadIdx.x & 63) == leader) atomicAdd(&cnt[k], __popcll(group));
    pending = pending && !mine;
  }
}

__global__ void __launch_bounds__(256) loss_samples_kernel(int64_t n, const int32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ nsamples) {
  __shared__ int part[256];
  int c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 256) c += cnt[i] > 0;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (int(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) nsamples[0] = part[0];
}

__device__ __forceinline__ void unpack8(const uint4& u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// One chunk = 8 logits: uint4 of bf16, or two float4.
template <typename T> struct Chunk;
template <> struct Chunk<uint16_t> {
  uint4 u;
  __device__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ void get(float* v) const { unpack8(u, v); }
  __device__ static void put(uint16_t* p, const float* v) {
    __bf16 b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)v[i];
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(b);
  }
  __device__ static void zero(uint16_t* p) { *reinterpret_cast<uint4*>(p) = make_uint4(0, 0, 0, 0); }
  __device__ static float at(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
  __device__ static void put1(uint16_t* p, float v) { *reinterpret_cast<__bf16*>(p) = (__bf16)v; }
};
template <> struct Chunk<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void get(float* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static void put(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ static void zero(float* p) {
    reinterpret_cast<float4*>(p)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(p)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ static float at(const float* p) { return *p; }
  __device__ static void put1(float* p, float v) { *p = v; }
};

// 2^x by the hardware instruction alone: results below 2^-126 flush to zero, which moves
// neither a sum of exponentials nor a softmax probability stored in bf16 or float32.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Workgroup-wide reduction through LDS over NW waves; every thread gets the result.
template <bool kMax, int NW>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = kMax ? wave_max(x) : wave_sum(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = lane < NW ? red[lane] : (kMax ? -INFINITY : 0.f);
  r = kMax ? wave_max(r) : wave_sum(r);
  __syncthreads();  // red is reused by the next reduction
  return r;
}

template <typename T, int NT, int R>
__global__ void __launch_bounds__(NT)
loss_ce_kernel(int32_t T_, int32_t V, int32_t nseg, float grad_scale, const T* __restrict__ X,
               const int32_t* __restrict__ tg, const int32_t* __restrict__ seg,
               const int32_t* __restrict__ cnt, const int32_t* __restrict__ nsamples,
               float* __restrict__ wloss, float* __restrict__ token_loss, T* __restrict__ dX) {
  __shared__ float red[kMaxWaves];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = V / 8;
  const int32_t y = tg[row], s = seg[row];
  const bool target_ok = y >= 0 && y < V;
  const bool counted = target_ok && s >= 0 && s < nseg;
  const int32_t n_s = counted ? cnt[(row / T_) * nseg + s] : 0;
  const int32_t N = nsamples[0];
  const float w = counted && n_s > 0 && N > 0 ? 1.f / (float(N) * float(n_s)) : 0.f;
  const T* x = X + row * V;
  T* dx = dX ? dX + row * V : nullptr;
  if (!target_ok) {  // not a loss token: no loss, zero gradient, the row is not read
    if (dx)
      for (int c = tid; c < nch; c += NT) Chunk<T>::zero(dx + 8 * c);
    if (tid == 0) {
      wloss[row] = 0.f;
      if (token_loss) token_loss[row] = 0.f;
    }
    return;
  }
  Chunk<T> ch[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + r * NT;
    if (c < nch) ch[r].load(x + 8 * c);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (tid + r * NT < nch) {
      float v[8];
      ch[r].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, v[e]);
    }
  }
  mx = block_reduce<true, NT / 64>(mx, red);
  const float mx2 = mx * kLog2e;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (tid + r * NT < nch) {
      float v[8];
      ch[r].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += exp2_hw(fmaf(v[e], kLog2e, -mx2));
    }
  }
  sum = block_reduce<false, NT / 64>(sum, red);
  const float lse = mx + logf(sum);
  if (tid == 0) {
    const float l = lse - Chunk<T>::at(x + y);
    wloss[row] = w * l;
    if (token_loss) token_loss[row] = l;
  }
  if (!dx) return;
  // d/dx_j = g w (exp(x_j - lse) - [j == y]); exp(x_j - lse) = exp2(x_j log2e - lse log2e).
  // Every element is written as g w p_j first; the thread that wrote the target's chunk
  // then rewrites the target element with g w (p_y - 1) (same thread, same address: the
  // later store wins).
  const float gw = grad_scale * w;
  const float lse2 = lse * kLog2e;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + r * NT;
    if (c < nch) {
      float v[8];
      ch[r].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gw * exp2_hw(fmaf(v[e], kLog2e, -lse2));
      Chunk<T>::put(dx + 8 * c, v);
    }
  }
  if (tid == (y / 8) % NT) {
    const float p = exp2_hw(fmaf(Chunk<T>::at(x + y), kLog2e, -lse2));
    Chunk<T>::put1(dx + y, gw * (p - 1.f));
  }
}

__global__ void __launch_bounds__(1024) loss_sum_kernel(int64_t n, const float* __restrict__ wloss,
                                                        float* __restrict__ loss) {
  __shared__ float red[kMaxWaves];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) s += wloss[i];
  s = block_reduce<false, 16>(s, red);
  if (threadIdx.x == 0) loss[0] = s;
}

template <typename T, int NT, int R>
void ce(int64_t rows, int32_t T_, int32_t V, int32_t nseg, float g, const void* x, const int32_t* tg,
        const int32_t* seg, const int32_t* cnt, const int32_t* ns, float* wl, float* tl, void* dx,
        hipStream_t stream) {
  loss_ce_kernel<T, NT, R><<<dim3(unsigned(rows)), dim3(NT), 0, stream>>>(
      T_, V, nseg, g, static_cast<const T*>(x), tg, seg, cnt, ns, wl, tl, static_cast<T*>(dx));
}

// Smallest workgroup whose registers hold the row: rows of up to 256 x 8 x 24 bf16 logits
// (12 chunks for float32) fit a 256-thread workgroup, so several rows per CU are in flight.
template <typename T>
void ce_dispatch(int64_t rows, int32_t T_, int32_t V, int32_t nseg, float g, const void* x,
                 const int32_t* tg, const int32_t* seg, const int32_t* cnt, const int32_t* ns,
                 float* wl, float* tl, void* dx, hipStream_t stream) {
  constexpr int kR = sizeof(T) == 2 ? 24 : 12;  // chunks a thread may hold
  const int nch = V / 8;
  const int per = (nch + 255) / 256;  // chunks per thread at 256 threads
  if (per <= 4) {
    ce<T, 256, 4>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
  } else if (per <= 8) {
    ce<T, 256, 8>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
  } else if constexpr (sizeof(T) == 2) {  // bf16: tighter register tiles keep occupancy up
    if (per <= 16)
      ce<T, 256, 16>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
    else if (per <= 20)
      ce<T, 256, 20>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
    else if (per <= kR)
      ce<T, 256, kR>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
    else if ((nch + 511) / 512 <= kR)
      ce<T, 512, kR>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
    else
      ce<T, 1024, 16>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
    return;
  } else if (per <= kR) {
    ce<T, 256, kR>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
  } else if ((nch + 511) / 512 <= kR) {
    ce<T, 512, kR>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
  } else {
    ce<T, 1024, 8>(rows, T_, V, nseg, g, x, tg, seg, cnt, ns, wl, tl, dx, stream);
  }
}

}  // namespace

hipError_t launch_packed_loss(const PackedLossLayout& L, int32_t B, int32_t T_, int32_t V,
                              int32_t nseg, int32_t dtype, const void* logits,
                              const int32_t* targets, const int32_t* seg, float grad_scale,
                              float* loss, float* token_loss, void* dlogits, void* workspace,
                              hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.count_off);
  int32_t* ns = reinterpret_cast<int32_t*>(ws + L.samples_off);
  float* wl = reinterpret_cast<float*>(ws + L.wloss_off);
  const int64_t tokens = int64_t(B) * T_;
  hipError_t e = launch_zero(ws + L.count_off, L.samples_off - L.count_off, stream);
  if (e != hipSuccess) return e;
  if (tokens > 0)
    loss_count_kernel<<<dim3(unsigned((tokens + 255) / 256)), dim3(256), 0, stream>>>(
        tokens, T_, V, nseg, targets, seg, cnt);
  loss_samples_kernel<<<dim3(1), dim3(256), 0, stream>>>(int64_t(B) * nseg, cnt, ns);
  if (tokens > 0) {
    if (dtype == LWM_BF16)
      ce_dispatch<uint16_t>(tokens, T_, V, nseg, grad_scale, logits, targets, seg, cnt, ns, wl,
                            token_loss, dlogits, stream);
    else
      ce_dispatch<float>(tokens, T_, V, nseg, grad_scale, logits, targets, seg, cnt, ns, wl,
                         token_loss, dlogits, stream);
  }
  loss_sum_kernel<<<dim3(1), dim3(1024), 0, stream>>>(tokens, wl, loss);
  return hipGetLastError();
}

}  // namespace lwm
