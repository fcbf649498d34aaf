// bf16 attention on gfx950 MFMA: forward (FINAL or PARTIAL output) and the LSE-recompute
// backward (Delta, dQ, dK/dV), head width 128, float32 accumulation.
//
// The method is the blockwise evaluation behind the LWM pages' RingAttention (deep dive,
// "RingAttention 为什么必要 / why RingAttention is necessary"): a query block stays
// resident while key/value blocks stream past it, and each block updates a running max,
// denominator and accumulator per query row.  The causal mask (sections "核心问题" and
// "模型结构") and the packed-sample mask ("Masked sequence packing") are applied only on
// tiles the block table marks PARTIAL; SKIP tiles are never visited.
//
// Shapes: head width D = 128; a workgroup is 4 waves.  Forward and dQ: 128 query rows per
// workgroup (32 per wave), key tiles of 64 streamed through LDS.  dK/dV: 128 keys per
// workgroup (32 per wave), query tiles of 64 streamed through LDS.  The table is built with
// 64 x 64 blocks; a 128-row tile combines two table rows (or columns).

#include <cmath>

#include "common.h"
#include "mfma_tile.h"

namespace lwm {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;          // query rows per forward / dQ workgroup
constexpr int BK = 64;           // keys per streamed tile
constexpr int TB = 64;           // table block size
constexpr int NT = 256;          // threads per workgroup
constexpr int RSTR = D + 8;      // row stride (bf16) of row-major [row][d] LDS tiles
constexpr int TSTR = BK + 8;     // row stride (bf16) of transposed [d][row] LDS tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint8_t combine_status(uint8_t a, uint8_t b) {
  if (a == LWM_TILE_SKIP && b == LWM_TILE_SKIP) return LWM_TILE_SKIP;
  if (a == LWM_TILE_FULL && b == LWM_TILE_FULL) return LWM_TILE_FULL;
  return LWM_TILE_PARTIAL;
}

// Copy a [64 rows][128 d] bf16 tile (rows row0.., zero past `nrows`) from global into a
// row-major LDS tile, and optionally into a transposed [128 d][64 rows] LDS tile.
template <bool kTranspose, bool kRowMajor>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ src, int row0, int nrows,
                                          uint16_t* rm, uint16_t* tr, int tid) {
#pragma unroll
  for (int it = 0; it < (BK * D / 8) / NT; ++it) {
    const int c = tid + it * NT;
    const int r = c >> 4, c16 = c & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < nrows) v = gload16(src + int64_t(row0 + r) * D + c16 * 8);
    if (kRowMajor) *reinterpret_cast<uint4*>(rm + r * RSTR + c16 * 8) = v;
    if (kTranspose) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tr[(c16 * 8 + 2 * e) * TSTR + r] = uint16_t(w[e] & 0xffff);
        tr[(c16 * 8 + 2 * e + 1) * TSTR + r] = uint16_t(w[e] >> 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------------------

__global__ void __launch_bounds__(NT, 2)
fwd_bf16_kernel(AttnParams p, TableView t, int mode, int nqt, const uint16_t* __restrict__ Q,
                const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_k,
                uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Mo,
                float* __restrict__ Lo, float* __restrict__ ACC) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BK * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * TSTR];
  __shared__ int32_t segk_lds[BK];

  // Longest rows first: rank 0 is the last query tile; heads are interleaved so that
  // consecutive workgroups (spread over the XCDs) share a tile rank.
  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int qt = nqt - 1 - rest % nqt;
  const int b = rest / nqt;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Qh = Q + bh * p.Sq * D;
  const uint16_t* Kh = K + bh * p.Sk * D;
  const uint16_t* Vh = V + bh * p.Sk * D;

  const int qrow = qt * BQ + wave * 32 + col;
  const bool qlive = qrow < p.Sq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qlive) v = gload16(Qh + int64_t(qrow) * D + 16 * s + 8 * hf);
    qreg[s] = *reinterpret_cast<bf16x8*>(&v);
  }
  const int32_t sq = qlive ? seg_q[int64_t(b) * p.Sq + qrow] : -1;
  const int64_t qpos = p.q_offset + qrow;

  const int r0 = 2 * qt, r1 = 2 * qt + 1;
  const bool has_r1 = r1 < t.nqb;
  const int32_t* rg0 = t.q_range + (int64_t(b) * t.nqb + r0) * 2;
  int lo = rg0[0], hi = rg0[1];
  if (has_r1) {
    const int32_t* rg1 = rg0 + 2;
    if (rg1[1] >= rg1[0]) {
      lo = hi >= lo ? min(lo, rg1[0]) : rg1[0];
      hi = max(hi, rg1[1]);
    }
  }
  const uint8_t* st0 = t.status + (int64_t(b) * t.nqb + r0) * t.nkb;
  const uint8_t* st1 = st0 + t.nkb;

  const float c = p.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{0};

  for (int kt = lo; kt <= hi; ++kt) {
    const uint8_t st = combine_status(st0[kt], has_r1 ? st1[kt] : uint8_t(LWM_TILE_SKIP));
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    stage_tile<false, true>(Kh, kt * BK, p.Sk, k_lds, nullptr, tid);
    stage_tile<true, false>(Vh, kt * BK, p.Sk, nullptr, vt_lds, tid);
    if (tid < BK) {
      const int key = kt * BK + tid;
      segk_lds[tid] = key < p.Sk ? seg_k[int64_t(b) * p.Sk + key] : -1;
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sacc[sub] = f32x16{0};
      const uint16_t* krow = k_lds + (32 * sub + kperm(col)) * RSTR + 8 * hf;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) sacc[sub] = mfma32(lds_load8(krow + 16 * s), qreg[s], sacc[sub]);
    }

    if (st == LWM_TILE_PARTIAL) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = 32 * sub + slot_index(i, hf);
          const int key = kt * BK + kl;
          const bool vis = qlive && key < p.Sk && sq >= 0 && sq == segk_lds[kl] &&
                           (!p.causal || p.k_offset + key <= qpos);
          if (!vis) sacc[sub][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[sub][i]);
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = exp2f(fmaf(sacc[sub][8 * a + j], c, -m_use));
          psum += pv[j];
        }
        pb[2 * sub + a] = to_bf16x8(pv);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = mfma32(lds_load8(vt_lds + (32 * db + col) * TSTR + 16 * ks + 8 * hf), pb[ks],
                          oacc[db]);
  }

  const float l_tot = half_sum(l_run);
  if (!qlive) return;
  const int64_t r64 = bh * p.Sq + qrow;
  if (mode == LWM_OUT_FINAL) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = O + r64 * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        __bf16 o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = *reinterpret_cast<uint2*>(o4);
      }
    if (hf == 0) LSE[r64] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  } else {
    float* arow = ACC + r64 * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(arow + d0) =
            make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
      }
    if (hf == 0) {
      Mo[r64] = l_tot > 0.f ? m_run * kLn2 : -INFINITY;
      Lo[r64] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------------------

// Delta_i = <dO_i, O_i> (float32), 16 lanes per row of 128.
__global__ void __launch_bounds__(NT) delta_bf16_kernel(int64_t rows, const uint16_t* __restrict__ O,
                                                        const uint16_t* __restrict__ dO,
                                                        float* __restrict__ delta) {
  const int64_t gid = int64_t(blockIdx.x) * NT + threadIdx.x;
  const int64_t row = gid >> 4;
  const int part = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    const uint4 a = gload16(O + row * D + part * 8);
    const uint4 g = gload16(dO + row * D + part * 8);
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(&a);
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(&g);
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(float(av[j]), float(gv[j]), s);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
  if (row < rows && part == 0) delta[row] = s;
}

// dQ: query-major like the forward.  Per key tile: S^T = K Q^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - Delta), dQ^T += K^T dS^T.
__global__ void __launch_bounds__(NT, 2)
dq_bf16_kernel(AttnParams p, TableView t, int nqt, const uint16_t* __restrict__ Q,
               const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
               const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
               const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
               const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BK * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BK * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[D * TSTR];
  __shared__ int32_t segk_lds[BK];

  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int qt = nqt - 1 - rest % nqt;
  const int b = rest / nqt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Kh = K + bh * p.Sk * D;
  const uint16_t* Vh = V + bh * p.Sk * D;

  const int qrow = qt * BQ + wave * 32 + col;
  const bool qlive = qrow < p.Sq;
  const int64_t r64 = bh * p.Sq + qrow;
  bf16x8 qreg[D / 16], greg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4 a = make_uint4(0, 0, 0, 0), g = make_uint4(0, 0, 0, 0);
    if (qlive) {
      a = gload16(Q + r64 * D + 16 * s + 8 * hf);
      g = gload16(dO + r64 * D + 16 * s + 8 * hf);
    }
    qreg[s] = *reinterpret_cast<bf16x8*>(&a);
    greg[s] = *reinterpret_cast<bf16x8*>(&g);
  }
  const float lse2 = qlive ? LSE[r64] * kLog2e : 0.f;
  const float dl = qlive ? delta[r64] : 0.f;
  const int32_t sq = qlive ? seg_q[int64_t(b) * p.Sq + qrow] : -1;
  const int64_t qpos = p.q_offset + qrow;

  const int r0 = 2 * qt, r1 = 2 * qt + 1;
  const bool has_r1 = r1 < t.nqb;
  const int32_t* rg0 = t.q_range + (int64_t(b) * t.nqb + r0) * 2;
  int lo = rg0[0], hi = rg0[1];
  if (has_r1) {
    const int32_t* rg1 = rg0 + 2;
    if (rg1[1] >= rg1[0]) {
      lo = hi >= lo ? min(lo, rg1[0]) : rg1[0];
      hi = max(hi, rg1[1]);
    }
  }
  const uint8_t* st0 = t.status + (int64_t(b) * t.nqb + r0) * t.nkb;
  const uint8_t* st1 = st0 + t.nkb;
  const float c = p.scale * kLog2e;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{0};

  for (int kt = lo; kt <= hi; ++kt) {
    const uint8_t st = combine_status(st0[kt], has_r1 ? st1[kt] : uint8_t(LWM_TILE_SKIP));
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    stage_tile<true, true>(Kh, kt * BK, p.Sk, k_lds, kt_lds, tid);
    stage_tile<false, true>(Vh, kt * BK, p.Sk, v_lds, nullptr, tid);
    if (tid < BK) {
      const int key = kt * BK + tid;
      segk_lds[tid] = key < p.Sk ? seg_k[int64_t(b) * p.Sk + key] : -1;
    }
    __syncthreads();

    bf16x8 dsb[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc = f32x16{0}, pacc = f32x16{0};
      const int rr = (32 * sub + kperm(col)) * RSTR + 8 * hf;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(lds_load8(k_lds + rr + 16 * s), qreg[s], sacc);
        pacc = mfma32(lds_load8(v_lds + rr + 16 * s), greg[s], pacc);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * a + j;
          float pr = exp2f(fmaf(sacc[i], c, -lse2));
          if (st == LWM_TILE_PARTIAL) {
            const int kl = 32 * sub + slot_index(i, hf);
            const int key = kt * BK + kl;
            const bool vis = qlive && key < p.Sk && sq >= 0 && sq == segk_lds[kl] &&
                             (!p.causal || p.k_offset + key <= qpos);
            if (!vis) pr = 0.f;
          }
          ds[j] = pr * (pacc[i] - dl);
        }
        dsb[2 * sub + a] = to_bf16x8(ds);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dqacc[db] = mfma32(lds_load8(kt_lds + (32 * db + col) * TSTR + 16 * ks + 8 * hf), dsb[ks],
                           dqacc[db]);
  }
  if (!qlive) return;
  uint16_t* out = dQ + r64 * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hf;
      __bf16 o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(dqacc[db][4 * g + e] * p.scale);
      *reinterpret_cast<uint2*>(out + d0) = *reinterpret_cast<uint2*>(o4);
    }
}

// dK, dV: key-major.  Workgroup = 128 keys (32 per wave) held in registers; query tiles of
// 64 stream through LDS in both layouts.  Per 32-query half: S = Q K^T, dP = dO V^T,
// P = exp(S - LSE), dS = P (dP - Delta), dV^T += dO^T P, dK^T += Q^T dS.
__global__ void __launch_bounds__(NT, 1)
dkv_bf16_kernel(AttnParams p, TableView t, int nkt, const uint16_t* __restrict__ Q,
                const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
                const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
                const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dK,
                uint16_t* __restrict__ dV) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[TB * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t g_lds[TB * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t gt_lds[D * TSTR];
  __shared__ __attribute__((aligned(16))) float lse_lds[TB];
  __shared__ __attribute__((aligned(16))) float dl_lds[TB];
  __shared__ int32_t segq_lds[TB];

  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int kt = rest % nkt;  // early keys see the most queries under the causal mask
  const int b = rest / nkt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Qh = Q + bh * p.Sq * D;
  const uint16_t* Gh = dO + bh * p.Sq * D;

  const int key = kt * 128 + wave * 32 + col;
  const bool klive = key < p.Sk;
  const int64_t k64 = bh * p.Sk + key;
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4 a = make_uint4(0, 0, 0, 0), v = make_uint4(0, 0, 0, 0);
    if (klive) {
      a = gload16(K + k64 * D + 16 * s + 8 * hf);
      v = gload16(V + k64 * D + 16 * s + 8 * hf);
    }
    kreg[s] = *reinterpret_cast<bf16x8*>(&a);
    vreg[s] = *reinterpret_cast<bf16x8*>(&v);
  }
  const int32_t sk = klive ? seg_k[int64_t(b) * p.Sk + key] : -2;
  const int64_t kpos = p.k_offset + key;

  const int c0 = 2 * kt, c1 = 2 * kt + 1;
  const bool has_c1 = c1 < t.nkb;
  const int32_t* rg0 = t.k_range + (int64_t(b) * t.nkb + c0) * 2;
  int lo = rg0[0], hi = rg0[1];
  if (has_c1) {
    const int32_t* rg1 = rg0 + 2;
    if (rg1[1] >= rg1[0]) {
      lo = hi >= lo ? min(lo, rg1[0]) : rg1[0];
      hi = max(hi, rg1[1]);
    }
  }
  const uint8_t* stb = t.status + int64_t(b) * t.nqb * t.nkb;
  const float c = p.scale * kLog2e;

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dkacc[i] = f32x16{0};
    dvacc[i] = f32x16{0};
  }

  for (int qb = lo; qb <= hi; ++qb) {
    const uint8_t* row = stb + int64_t(qb) * t.nkb;
    const uint8_t st = combine_status(row[c0], has_c1 ? row[c1] : uint8_t(LWM_TILE_SKIP));
    if (st == LWM_TILE_SKIP) continue;
    __syncthreads();
    stage_tile<true, true>(Qh, qb * TB, p.Sq, q_lds, qt_lds, tid);
    stage_tile<true, true>(Gh, qb * TB, p.Sq, g_lds, gt_lds, tid);
    if (tid < TB) {
      const int r = qb * TB + tid;
      const bool ok = r < p.Sq;
      lse_lds[tid] = ok ? LSE[bh * p.Sq + r] * kLog2e : 0.f;
      dl_lds[tid] = ok ? delta[bh * p.Sq + r] : 0.f;
      segq_lds[tid] = ok ? seg_q[int64_t(b) * p.Sq + r] : -1;
    }
    __syncthreads();

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc = f32x16{0}, pacc = f32x16{0};
      const int rr = (32 * sub + kperm(col)) * RSTR + 8 * hf;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(lds_load8(q_lds + rr + 16 * s), kreg[s], sacc);
        pacc = mfma32(lds_load8(g_lds + rr + 16 * s), vreg[s], pacc);
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int qbase = 32 * sub + 16 * a + 8 * hf;  // 8 consecutive local query rows
        float pv[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * a + j;
          const int ql = qbase + j;
          float pr = exp2f(fmaf(sacc[i], c, -lse_lds[ql]));
          if (st == LWM_TILE_PARTIAL) {
            const int qr = qb * TB + ql;
            const bool vis = klive && qr < p.Sq && segq_lds[ql] >= 0 && segq_lds[ql] == sk &&
                             (!p.causal || kpos <= p.q_offset + qr);
            if (!vis) pr = 0.f;
          }
          pv[j] = pr;
          ds[j] = pr * (pacc[i] - dl_lds[ql]);
        }
        pb[a] = to_bf16x8(pv);
        dsb[a] = to_bf16x8(ds);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int ks = 2 * sub + a;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int tr = (32 * db + col) * TSTR + 16 * ks + 8 * hf;
          dvacc[db] = mfma32(lds_load8(gt_lds + tr), pb[a], dvacc[db]);
          dkacc[db] = mfma32(lds_load8(qt_lds + tr), dsb[a], dkacc[db]);
        }
      }
    }
  }
  if (!klive) return;
  uint16_t* ko = dK + k64 * D;
  uint16_t* vo = dV + k64 * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hf;
      __bf16 k4[4], v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = (__bf16)(dkacc[db][4 * g + e] * p.scale);
        v4[e] = (__bf16)(dvacc[db][4 * g + e]);
      }
      *reinterpret_cast<uint2*>(ko + d0) = *reinterpret_cast<uint2*>(k4);
      *reinterpret_cast<uint2*>(vo + d0) = *reinterpret_cast<uint2*>(v4);
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const lwm_attn_desc& d, int mode, const void* q, const void* k,
                           const void* v, const int32_t* seg_q, const int32_t* seg_k,
                           const void* table, void* o, float* lse, float* m, float* l,
                           float* acc, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  const int64_t grid = int64_t(nqt) * d.H * d.B;
  fwd_bf16_kernel<<<dim3(unsigned(grid)), dim3(NT), 0, stream>>>(
      attn_params(d), t, mode, nqt, static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), seg_q, seg_k,
      static_cast<uint16_t*>(o), lse, m, l, acc);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const lwm_attn_desc& d, int phase, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* seg_q, const int32_t* seg_k, const void* table,
                           void* dq, void* dk, void* dv, float* delta, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const AttnParams p = attn_params(d);
  const int64_t rows = int64_t(d.B) * d.H * d.Sq;
  if (phase < 0 || phase == LWM_BWD_DELTA)
    delta_bf16_kernel<<<dim3(unsigned((rows * 16 + NT - 1) / NT)), dim3(NT), 0, stream>>>(
        rows, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), delta);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  if (phase < 0 || phase == LWM_BWD_DQ)
    dq_bf16_kernel<<<dim3(unsigned(int64_t(nqt) * d.H * d.B)), dim3(NT), 0, stream>>>(
        p, t, nqt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta, seg_q,
        seg_k, static_cast<uint16_t*>(dq));
  const int nkt = (d.Sk + 127) / 128;
  if (phase < 0 || phase == LWM_BWD_DKV)
    dkv_bf16_kernel<<<dim3(unsigned(int64_t(nkt) * d.H * d.B)), dim3(NT), 0, stream>>>(
        p, t, nkt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta, seg_q,
        seg_k, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
  return hipGetLastError();
}

}  // namespace lwm
