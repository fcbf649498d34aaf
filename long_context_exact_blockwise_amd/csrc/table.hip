// Block table: per-block segment statistics -> SKIP / PARTIAL / FULL per tile pair ->
// per-row and per-column ranges of non-SKIP tiles.
//
// The table turns the two masks of the LWM pages into skipped work: the causal order of the
// next-token model (deep dive, "核心问题 / core problem") and the per-sample attention mask
// of masked sequence packing (deep dive, "Masked sequence packing").  All three passes are
// integer work bound by memory latency; they run once per (layout, offsets) and are reused
// by the forward and backward calls.

#include <climits>

#include "common.h"

namespace lwm {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, kWave));
  return x;
}

// One wave per block of `block` (<= 64) tokens: {min id, max id, min non-negative id}.
__global__ void __launch_bounds__(256) block_stats_kernel(const int32_t* __restrict__ seg, int32_t S,
                                                          int32_t block, int32_t nblk, int32_t B,
                                                          int32_t* __restrict__ stats) {
  const int wave = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (wave >= B * nblk) return;
  const int b = wave / nblk, blk = wave % nblk;
  const int pos = blk * block + lane;
  const bool valid = lane < block && pos < S;
  const int id = valid ? seg[int64_t(b) * S + pos] : 0;
  const int mn = wave_min(valid ? id : INT_MAX);
  const int mx = wave_max(valid ? id : INT_MIN);
  const int mnn = wave_min(valid && id >= 0 ? id : INT_MAX);
  if (lane == 0) {
    int32_t* s = stats + int64_t(wave) * 4;
    s[0] = mn;
    s[1] = mx;
    s[2] = mnn;
    s[3] = 0;
  }
}

// One thread per (b, query block, key block).
__global__ void __launch_bounds__(256) classify_kernel(AttnParams p, int32_t block_q, int32_t block_k,
                                                       int32_t nqb, int32_t nkb,
                                                       const int32_t* __restrict__ qstats,
                                                       const int32_t* __restrict__ kstats,
                                                       uint8_t* __restrict__ status) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_b = int64_t(nqb) * nkb;
  if (idx >= per_b * p.B) return;
  const int b = int(idx / per_b);
  const int64_t rem = idx % per_b;
  const int qb = int(rem / nkb), kb = int(rem % nkb);
  const int qf = qb * block_q, ql = min(p.Sq, qf + block_q) - 1;
  const int kf = kb * block_k, kl = min(p.Sk, kf + block_k) - 1;
  const int32_t* qs = qstats + (int64_t(b) * nqb + qb) * 4;
  const int32_t* ks = kstats + (int64_t(b) * nkb + kb) * 4;
  uint8_t st;
  if (qs[1] < 0 || ks[1] < 0) {
    st = LWM_TILE_SKIP;  // one side is all padding
  } else if (qs[2] > ks[1] || ks[2] > qs[1]) {
    st = LWM_TILE_SKIP;  // non-negative segment-id intervals are disjoint
  } else if (p.causal && p.k_offset + kf > p.q_offset + ql) {
    st = LWM_TILE_SKIP;  // every key is later than every query
  } else {
    const bool whole = qf + block_q <= p.Sq && kf + block_k <= p.Sk;
    const bool causal_full = !p.causal || p.k_offset + kl <= p.q_offset + qf;
    const bool one_segment = qs[0] == qs[1] && ks[0] == ks[1] && qs[0] == ks[0] && qs[0] >= 0;
    st = (whole && causal_full && one_segment) ? LWM_TILE_FULL : LWM_TILE_PARTIAL;
  }
  LWM_CHECK(b < p.B && qb < nqb && kb < nkb, kChkTable);
  status[idx] = st;
}

// One wave per query-block row (first B*nqb waves) or key-block column (next B*nkb).
__global__ void __launch_bounds__(256) ranges_kernel(const uint8_t* __restrict__ status, int32_t B,
                                                     int32_t nqb, int32_t nkb,
                                                     int32_t* __restrict__ q_range,
                                                     int32_t* __restrict__ k_range) {
  const int64_t wave = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t nrows = int64_t(B) * nqb, ncols = int64_t(B) * nkb;
  int lo = INT_MAX, hi = -1;
  if (wave < nrows) {
    const uint8_t* row = status + wave * nkb;
    for (int kb = lane; kb < nkb; kb += kWave)
      if (row[kb] != LWM_TILE_SKIP) {
        lo = min(lo, kb);
        hi = max(hi, kb);
      }
  } else if (wave < nrows + ncols) {
    const int64_t c = wave - nrows;
    const int b = int(c / nkb), kb = int(c % nkb);
    const uint8_t* col = status + int64_t(b) * nqb * nkb + kb;
    for (int qb = lane; qb < nqb; qb += kWave)
      if (col[int64_t(qb) * nkb] != LWM_TILE_SKIP) {
        lo = min(lo, qb);
        hi = max(hi, qb);
      }
  } else {
    return;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  LWM_CHECK(hi < (wave < nrows ? nkb : nqb), kChkTable);
  if (lane == 0) {
    int32_t* out = wave < nrows ? q_range + wave * 2 : k_range + (wave - nrows) * 2;
    out[0] = hi < 0 ? 0 : lo;
    out[1] = hi;
  }
}

// Zero fill with 16-byte stores (used instead of a memset so callers may capture it).
__global__ void __launch_bounds__(256) zero_kernel(uint4* __restrict__ dst, int64_t n16) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n16) dst[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = int64_t(bytes / 16);
  if (n16 > 0)
    zero_kernel<<<dim3(unsigned((n16 + 255) / 256)), dim3(256), 0, stream>>>(
        static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_build_table(const lwm_attn_desc& d, const int32_t* seg_q, const int32_t* seg_k,
                              void* table, hipStream_t stream) {
  const TableLayout L = table_layout(d);
  char* base = static_cast<char*>(table);
  int32_t* qstats = reinterpret_cast<int32_t*>(base + L.q_stats_off);
  int32_t* kstats = reinterpret_cast<int32_t*>(base + L.k_stats_off);
  uint8_t* status = reinterpret_cast<uint8_t*>(base + L.status_off);
  int32_t* q_range = reinterpret_cast<int32_t*>(base + L.q_range_off);
  int32_t* k_range = reinterpret_cast<int32_t*>(base + L.k_range_off);
  const AttnParams p = attn_params(d);

  const int64_t qwaves = int64_t(d.B) * L.nqb, kwaves = int64_t(d.B) * L.nkb;
  if (qwaves > 0)
    block_stats_kernel<<<dim3(unsigned((qwaves + 3) / 4)), dim3(256), 0, stream>>>(
        seg_q, d.Sq, d.block_q, L.nqb, d.B, qstats);
  if (kwaves > 0)
    block_stats_kernel<<<dim3(unsigned((kwaves + 3) / 4)), dim3(256), 0, stream>>>(
        seg_k, d.Sk, d.block_k, L.nkb, d.B, kstats);
  const int64_t pairs = int64_t(d.B) * L.nqb * L.nkb;
  if (pairs > 0)
    classify_kernel<<<dim3(unsigned((pairs + 255) / 256)), dim3(256), 0, stream>>>(
        p, d.block_q, d.block_k, L.nqb, L.nkb, qstats, kstats, status);
  // with no keys (or no queries) every range comes out empty: first 0, last -1
  if (qwaves + kwaves > 0)
    ranges_kernel<<<dim3(unsigned((qwaves + kwaves + 3) / 4)), dim3(256), 0, stream>>>(
        status, d.B, L.nqb, L.nkb, q_range, k_range);
  return hipGetLastError();
}

LWM_DEBUG_READER(table)

}  // namespace lwm
