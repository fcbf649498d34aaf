// float32 attention forward and backward: one thread per query row (forward, dQ) or per
// key row (dK, dV), key/query blocks staged through LDS, float32 throughout.
//
// This path serves fp32 inputs (small workloads and gradient checks); it is written for
// clarity, not speed.  It evaluates the same blockwise online softmax as the bf16 MFMA
// path: key blocks in order, a running max m, denominator l and accumulator acc per row
// (the blockwise evaluation the LWM pages build RingAttention on, deep dive section
// "RingAttention 为什么必要 / why RingAttention is necessary"), with the causal and packing
// masks of sections "核心问题 / core problem" and "Masked sequence packing".

#include <cmath>

#include "common.h"

namespace lwm {
namespace {

constexpr int kBlk = 64;  // rows per workgroup == table block size

__device__ __forceinline__ bool visible(int32_t sq, int32_t sk, int64_t qpos, int64_t kpos,
                                        int causal) {
  return sq >= 0 && sq == sk && (!causal || kpos <= qpos);
}

// Forward: workgroup = 64 query rows of one (b, h); thread = one row.
template <int D>
__global__ void __launch_bounds__(kBlk) fwd_f32_kernel(AttnParams p, TableView t, int mode,
                                                      const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      const int32_t* __restrict__ seg_q,
                                                      const int32_t* __restrict__ seg_k,
                                                      float* __restrict__ O, float* __restrict__ LSE,
                                                      float* __restrict__ Mo, float* __restrict__ Lo,
                                                      float* __restrict__ ACC) {
  __shared__ float ks[kBlk][D + 1];
  __shared__ float vs[kBlk][D + 1];
  __shared__ int32_t sks[kBlk];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int row = qb * kBlk + tid;
  const bool live = row < p.Sq;
  const int64_t bh = int64_t(b) * p.H + h;
  const float* Qh = Q + bh * p.Sq * D;
  const float* Kh = K + bh * p.Sk * D;
  const float* Vh = V + bh * p.Sk * D;

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Qh[int64_t(row) * D + d] : 0.f;
    acc[d] = 0.f;
  }
  const int32_t sq = live ? seg_q[int64_t(b) * p.Sq + row] : -1;
  const int64_t qpos = p.q_offset + row;
  float m = -INFINITY, l = 0.f;

  const int32_t* rng = t.q_range + (int64_t(b) * t.nqb + qb) * 2;
  const int kb_lo = rng[0], kb_hi = rng[1];
  LWM_CHECK(qb < t.nqb && (kb_lo > kb_hi || (kb_lo >= 0 && kb_hi < t.nkb)), kChkF32Range);
  const uint8_t* st_row = t.status + (int64_t(b) * t.nqb + qb) * t.nkb;
  for (int kb = kb_lo; kb <= kb_hi; ++kb) {
    const uint8_t st = st_row[kb];
    LWM_CHECK(st <= LWM_TILE_FULL && kb * kBlk < p.Sk, kChkF32Tile);
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    for (int i = tid; i < kBlk * D; i += kBlk) {
      const int r = i / D, c = i % D;
      const int key = kb * kBlk + r;
      ks[r][c] = key < p.Sk ? Kh[int64_t(key) * D + c] : 0.f;
      vs[r][c] = key < p.Sk ? Vh[int64_t(key) * D + c] : 0.f;
    }
    {
      const int key = kb * kBlk + tid;
      sks[tid] = key < p.Sk ? seg_k[int64_t(b) * p.Sk + key] : -1;
    }
    __syncthreads();
    for (int j = 0; j < kBlk; ++j) {
      const int key = kb * kBlk + j;
      if (st != LWM_TILE_FULL &&
          !(key < p.Sk && live && visible(sq, sks[j], qpos, p.k_offset + key, p.causal)))
        continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[j][d], s);
      s *= p.scale;
      if (s > m) {
        const float alpha = expf(m - s);  // m = -inf gives 0
        l = l * alpha + 1.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], alpha, vs[j][d]);
        m = s;
      } else {
        const float e = expf(s - m);
        l += e;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(e, vs[j][d], acc[d]);
      }
    }
  }
  if (!live) return;
  const int64_t r64 = bh * p.Sq + row;
  if (mode == LWM_OUT_FINAL) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) O[r64 * D + d] = acc[d] * inv;
    LSE[r64] = l > 0.f ? m + logf(l) : -INFINITY;
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) ACC[r64 * D + d] = acc[d];
    Mo[r64] = l > 0.f ? m : -INFINITY;
    Lo[r64] = l;
  }
}

// Delta_i = <dO_i, O_i>, one thread per row.
template <int D>
__global__ void __launch_bounds__(256) delta_f32_kernel(int64_t rows, const float* __restrict__ O,
                                                       const float* __restrict__ dO,
                                                       float* __restrict__ delta) {
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) s = fmaf(O[r * D + d], dO[r * D + d], s);
  delta[r] = s;
}

// dQ: workgroup = 64 query rows; thread = one row; key blocks staged in LDS.
template <int D>
__global__ void __launch_bounds__(kBlk) dq_f32_kernel(AttnParams p, TableView t,
                                                     const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     const float* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     const float* __restrict__ delta,
                                                     const int32_t* __restrict__ seg_q,
                                                     const int32_t* __restrict__ seg_k,
                                                     float* __restrict__ dQ) {
  __shared__ float ks[kBlk][D + 1];
  __shared__ float vs[kBlk][D + 1];
  __shared__ int32_t sks[kBlk];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int row = qb * kBlk + tid;
  const bool live = row < p.Sq;
  const int64_t bh = int64_t(b) * p.H + h;
  const int64_t r64 = bh * p.Sq + row;
  const float* Kh = K + bh * p.Sk * D;
  const float* Vh = V + bh * p.Sk * D;
  float q[D], g[D], dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[r64 * D + d] : 0.f;
    g[d] = live ? dO[r64 * D + d] : 0.f;
    dq[d] = 0.f;
  }
  const float lse = live ? LSE[r64] : 0.f;
  const float dl = live ? delta[r64] : 0.f;
  const int32_t sq = live ? seg_q[int64_t(b) * p.Sq + row] : -1;
  const int64_t qpos = p.q_offset + row;
  const int32_t* rng = t.q_range + (int64_t(b) * t.nqb + qb) * 2;
  LWM_CHECK(qb < t.nqb && (rng[0] > rng[1] || (rng[0] >= 0 && rng[1] < t.nkb)), kChkF32Range);
  const uint8_t* st_row = t.status + (int64_t(b) * t.nqb + qb) * t.nkb;
  for (int kb = rng[0]; kb <= rng[1]; ++kb) {
    const uint8_t st = st_row[kb];
    LWM_CHECK(st <= LWM_TILE_FULL && kb * kBlk < p.Sk, kChkF32Tile);
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    for (int i = tid; i < kBlk * D; i += kBlk) {
      const int r = i / D, c = i % D;
      const int key = kb * kBlk + r;
      ks[r][c] = key < p.Sk ? Kh[int64_t(key) * D + c] : 0.f;
      vs[r][c] = key < p.Sk ? Vh[int64_t(key) * D + c] : 0.f;
    }
    {
      const int key = kb * kBlk + tid;
      sks[tid] = key < p.Sk ? seg_k[int64_t(b) * p.Sk + key] : -1;
    }
    __syncthreads();
    for (int j = 0; j < kBlk; ++j) {
      const int key = kb * kBlk + j;
      if (st != LWM_TILE_FULL &&
          !(key < p.Sk && live && visible(sq, sks[j], qpos, p.k_offset + key, p.causal)))
        continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], ks[j][d], s);
        dp = fmaf(g[d], vs[j][d], dp);
      }
      const float pr = expf(s * p.scale - lse);
      const float ds = pr * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, ks[j][d], dq[d]);
    }
  }
  if (!live) return;
#pragma unroll
  for (int d = 0; d < D; ++d) dQ[r64 * D + d] = dq[d] * p.scale;
}

// dK, dV: workgroup = 64 keys; thread = one key; query blocks staged in LDS.
template <int D>
__global__ void __launch_bounds__(kBlk) dkv_f32_kernel(AttnParams p, TableView t,
                                                      const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      const float* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      const float* __restrict__ delta,
                                                      const int32_t* __restrict__ seg_q,
                                                      const int32_t* __restrict__ seg_k,
                                                      float* __restrict__ dK,
                                                      float* __restrict__ dV) {
  __shared__ float qs[kBlk][D + 1];
  __shared__ float gs[kBlk][D + 1];
  __shared__ float ls[kBlk], dls[kBlk];
  __shared__ int32_t sqs[kBlk];
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int key = kb * kBlk + tid;
  const bool live = key < p.Sk;
  const int64_t bh = int64_t(b) * p.H + h;
  const int64_t k64 = bh * p.Sk + key;
  const float* Qh = Q + bh * p.Sq * D;
  const float* Gh = dO + bh * p.Sq * D;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = live ? K[k64 * D + d] : 0.f;
    v[d] = live ? V[k64 * D + d] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int32_t sk = live ? seg_k[int64_t(b) * p.Sk + key] : -2;
  const int64_t kpos = p.k_offset + key;
  const int32_t* rng = t.k_range + (int64_t(b) * t.nkb + kb) * 2;
  LWM_CHECK(kb < t.nkb && (rng[0] > rng[1] || (rng[0] >= 0 && rng[1] < t.nqb)), kChkF32Range);
  const uint8_t* st_base = t.status + int64_t(b) * t.nqb * t.nkb + kb;
  for (int qb = rng[0]; qb <= rng[1]; ++qb) {
    const uint8_t st = st_base[int64_t(qb) * t.nkb];
    LWM_CHECK(st <= LWM_TILE_FULL && qb * kBlk < p.Sq, kChkF32Tile);
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    for (int i = tid; i < kBlk * D; i += kBlk) {
      const int r = i / D, c = i % D;
      const int row = qb * kBlk + r;
      qs[r][c] = row < p.Sq ? Qh[int64_t(row) * D + c] : 0.f;
      gs[r][c] = row < p.Sq ? Gh[int64_t(row) * D + c] : 0.f;
    }
    {
      const int row = qb * kBlk + tid;
      const bool ok = row < p.Sq;
      ls[tid] = ok ? LSE[bh * p.Sq + row] : 0.f;
      dls[tid] = ok ? delta[bh * p.Sq + row] : 0.f;
      sqs[tid] = ok ? seg_q[int64_t(b) * p.Sq + row] : -1;
    }
    __syncthreads();
    for (int i = 0; i < kBlk; ++i) {
      const int row = qb * kBlk + i;
      if (st != LWM_TILE_FULL &&
          !(row < p.Sq && live && visible(sqs[i], sk, p.q_offset + row, kpos, p.causal)))
        continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qs[i][d], k[d], s);
        dp = fmaf(gs[i][d], v[d], dp);
      }
      const float pr = expf(s * p.scale - ls[i]);
      const float ds = pr * (dp - dls[i]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(pr, gs[i][d], dv[d]);
        dk[d] = fmaf(ds, qs[i][d], dk[d]);
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    dK[k64 * D + d] = dk[d] * p.scale;
    dV[k64 * D + d] = dv[d];
  }
}

template <int D>
hipError_t fwd_f32_launch(const lwm_attn_desc& d, int mode, const float* q, const float* k,
                          const float* v, const int32_t* seg_q, const int32_t* seg_k,
                          const void* table, float* o, float* lse, float* m, float* l, float* acc,
                          hipStream_t stream) {
  const TableView t = table_view(d, table);
  dim3 grid(unsigned(t.nqb), unsigned(d.H), unsigned(d.B));
  fwd_f32_kernel<D><<<grid, dim3(kBlk), 0, stream>>>(attn_params(d), t, mode, q, k, v, seg_q,
                                                       seg_k, o, lse, m, l, acc);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_f32_launch(const lwm_attn_desc& d, int phase, const float* q, const float* k, const float* v,
                          const float* o, const float* dO, const float* lse,
                          const int32_t* seg_q, const int32_t* seg_k, const void* table,
                          float* dq, float* dk, float* dv, float* delta, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const AttnParams p = attn_params(d);
  const int64_t rows = int64_t(d.B) * d.H * d.Sq;
  if (phase < 0 || phase == LWM_BWD_DELTA)
    delta_f32_kernel<D><<<dim3(unsigned((rows + 255) / 256)), dim3(256), 0, stream>>>(rows, o, dO,
                                                                                       delta);
  if (phase < 0 || phase == LWM_BWD_DQ)
    dq_f32_kernel<D><<<dim3(unsigned(t.nqb), unsigned(d.H), unsigned(d.B)), dim3(kBlk), 0, stream>>>(
        p, t, q, k, v, dO, lse, delta, seg_q, seg_k, dq);
  if (phase < 0 || phase == LWM_BWD_DKV)
    dkv_f32_kernel<D><<<dim3(unsigned(t.nkb), unsigned(d.H), unsigned(d.B)), dim3(kBlk), 0, stream>>>(
        p, t, q, k, v, dO, lse, delta, seg_q, seg_k, dk, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const lwm_attn_desc& d, int mode, const float* q, const float* k,
                          const float* v, const int32_t* seg_q, const int32_t* seg_k,
                          const void* table, float* o, float* lse, float* m, float* l,
                          float* acc, hipStream_t stream) {
  switch (d.D) {
    case 32: return fwd_f32_launch<32>(d, mode, q, k, v, seg_q, seg_k, table, o, lse, m, l, acc, stream);
    case 64: return fwd_f32_launch<64>(d, mode, q, k, v, seg_q, seg_k, table, o, lse, m, l, acc, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_f32(const lwm_attn_desc& d, int phase, const float* q, const float* k, const float* v,
                          const float* o, const float* dO, const float* lse,
                          const int32_t* seg_q, const int32_t* seg_k, const void* table,
                          float* dq, float* dk, float* dv, float* delta, hipStream_t stream) {
  switch (d.D) {
    case 32: return bwd_f32_launch<32>(d, phase, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, delta, stream);
    case 64: return bwd_f32_launch<64>(d, phase, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, delta, stream);
    default: return hipErrorInvalidValue;
  }
}

LWM_DEBUG_READER(attn_f32)

}  // namespace lwm
