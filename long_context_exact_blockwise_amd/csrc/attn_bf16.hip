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
//
// Streaming: tiles are double-buffered in LDS and filled by the buffer unit directly
// (buffer_load ... lds), so no registers hold tile data in flight; the loads for tile j+1
// go out one instruction at a time between the first score MFMAs of tile j, after the
// barrier that opens it, and one barrier per tile both publishes tile j+1 and retires the
// buffer tile j-1 used.  The loop body is instantiated once per buffer half so every LDS
// address is a register plus a constant offset.  Each tile is stored once, row-major and
// swizzled (mfma_tile.h); operands that run across its rows (V^T, K^T, Q^T, dO^T) are read
// with the gfx950 transposing LDS read.

#include <climits>
#include <cmath>

#include "common.h"
#include "mfma_tile.h"
#include "rope_math.h"

namespace lwm {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;          // query rows per forward / dQ workgroup
constexpr int BK = 64;           // rows per streamed tile
constexpr int TB = 64;           // table block size
constexpr int NT = 256;          // threads per workgroup
constexpr int kTileElems = BK * D;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max moves only when a tile's max exceeds it by more than this (log2 units),
// so weights stay below 2^kTau and the accumulator is rescaled rarely; l and acc always
// refer to the max actually used, so the result is exact up to rounding.
constexpr float kTau = 8.0f;

typedef __attribute__((address_space(3))) void* lds_ptr;

// Values read from the block table are the same on every lane; say so, so that addresses
// and buffer resources built from them stay in scalar registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ uint8_t combine_status(uint8_t a, uint8_t b) {
  if (a == LWM_TILE_SKIP && b == LWM_TILE_SKIP) return LWM_TILE_SKIP;
  if (a == LWM_TILE_FULL && b == LWM_TILE_FULL) return LWM_TILE_FULL;
  return LWM_TILE_PARTIAL;
}

// Union of two inclusive ranges (an empty range has first > last).
__device__ __forceinline__ void range_union(const int32_t* a, const int32_t* b, bool has_b, int& lo,
                                            int& hi) {
  lo = uniform(a[0]);
  hi = uniform(a[1]);
  if (has_b) {
    const int blo = uniform(b[0]), bhi = uniform(b[1]);
    if (bhi >= blo) {
      lo = hi >= lo ? min(lo, blo) : blo;
      hi = max(hi, bhi);
    }
  }
}

// The combined status of the tiles a workgroup visits is staged in LDS, one byte per tile,
// in chunks of kStatChunk tiles: scanning for the next live tile then costs LDS reads
// instead of a dependent global-memory round trip per tile.
constexpr int kStatChunk = 2048;

__device__ __forceinline__ void stage_status_rows(uint8_t* stat, const uint8_t* s0, const uint8_t* s1,
                                                  bool has1, int c0, int c1, int tid) {
  for (int i = tid; i <= c1 - c0; i += NT)
    stat[i] = combine_status(s0[c0 + i], has1 ? s1[c0 + i] : uint8_t(LWM_TILE_SKIP));
}

__device__ __forceinline__ void stage_status_cols(uint8_t* stat, const uint8_t* base, int64_t nkb,
                                                  int col0, bool has1, int c0, int c1, int tid) {
  for (int i = tid; i <= c1 - c0; i += NT) {
    const uint8_t* row = base + int64_t(c0 + i) * nkb;
    stat[i] = combine_status(row[col0], has1 ? row[col0 + 1] : uint8_t(LWM_TILE_SKIP));
  }
}

// First tile k' >= k in [k, c1] whose staged status is not SKIP (c1 + 1 if none).
__device__ __forceinline__ int next_live_lds(const uint8_t* stat, int c0, int k, int c1) {
  while (k <= c1 && stat[k - c0] == LWM_TILE_SKIP) ++k;
  return uniform(k);
}

// Position difference q_offset - k_offset clamped into int32: with it, key j is causally
// visible from query row i iff j - i <= dpos (|j - i| < 2^31 always holds).
__device__ __forceinline__ int clamp_dpos(int64_t q_offset, int64_t k_offset) {
  const int64_t d = q_offset - k_offset;
  return int(d > INT32_MAX ? INT32_MAX : (d < INT32_MIN + 1 ? INT32_MIN + 1 : d));
}

// Visibility inside a PARTIAL tile, segments aside, reduced to one compare per score.
// key_limit: key key0 + o (o in 0..63) is visible from query row qrow iff o <= the result
// (key bound Sk and, when causal, key - qrow <= dpos); -1 when the row sees nothing.
__device__ __forceinline__ int key_limit(int key0, int qrow, int dpos, int Sk, int causal, bool live) {
  int64_t lim = int64_t(Sk) - 1 - key0;
  if (causal) lim = min(lim, int64_t(qrow) + dpos - key0);
  if (!live) lim = -1;
  return int(max<int64_t>(-1, min<int64_t>(64, lim)));
}

// row_window: query row row0 + o (o in 0..63) sees key `key` iff lo <= o <= hi (row bound Sq
// and, when causal, key - row <= dpos); an empty window when the key is dead.
__device__ __forceinline__ void row_window(int row0, int key, int dpos, int Sq, int causal, bool live,
                                           int& lo, int& hi) {
  const int64_t h = int64_t(Sq) - 1 - row0;
  int64_t l = causal ? int64_t(key) - dpos - row0 : -1;
  if (!live) l = 64;
  lo = int(max<int64_t>(-1, min<int64_t>(64, l)));
  hi = int(max<int64_t>(-1, min<int64_t>(64, h)));
}

// Eight consecutive int32 / float from LDS (16-byte aligned).
__device__ __forceinline__ void lds_load_i8(const int32_t* p, int* v) {
  const int4 a = *reinterpret_cast<const int4*>(p);
  const int4 b = *reinterpret_cast<const int4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void lds_load_f8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (V#) over `bytes` bytes at `base`: raw addressing, no stride; loads past
// the end return zero (hardware range check), so tails need no branches.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
               __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff)),
               __builtin_amdgcn_readfirstlane(max(bytes, 0)), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr)(p)));
}

// Asynchronous copy global -> LDS by the buffer unit: every lane fetches `bytes` (16 or 4)
// at rsrc + voff and the unit writes them to LDS at lds_base + lane * bytes.  Issued from
// inline assembly so that the compiler does not serialise later LDS reads of other buffers
// behind it; callers wait (wait_vmem) and synchronise before reading the destination.  It
// has no register results, so nothing the compiler allocates is written after issue.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const i32x4& rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Issue the loads of one 64-row tile (rows row0.. of a [nrows][128] bf16 tensor) straight
// into a swizzled LDS tile.  Each wave moves 4 blocks of 4 rows (1 KiB each); the buffer
// unit writes lane l's 16 bytes to block + 16 l, so lane l fetches the logical chunk that
// belongs at physical chunk l % 16 of its row.  Rows past nrows arrive as zeros.
// Instruction `it` of wave w covers rows 16 it + 4 w + lane / 16.  The swizzle depends on the
// row modulo 16 only, so the four instructions share one lane offset and differ in the
// buffer base (a 16-row step), which keeps the per-lane state to one register; `wave` must
// be wave-uniform so that the LDS bases stay scalar.
__device__ __forceinline__ uint32_t tile_lane_off(int wave, int lane) {
  const int row = 4 * wave + (lane >> 4);
  return row * (D * 2) + (((lane & 15) ^ tile_swz(row)) << 4);
}
__device__ __forceinline__ void tile_async_load(uint16_t* tile, const uint16_t* __restrict__ src,
                                                int row0, int nrows, int wave, int lane) {
  const uint32_t voff = tile_lane_off(wave, lane);
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tile)) + wave * 1024;
  const int nb = min(nrows - row0, BK) * D * 2;
#pragma unroll
  for (int it = 0; it < BK / 16; ++it)
    dma16(make_rsrc(src + int64_t(row0 + 16 * it) * D, nb - it * 16 * D * 2), base + it * 4096, voff);
}

// Issue the load of 64 consecutive 32-bit values (rows row0.. of a per-row vector) into LDS;
// called by one whole wave.  Values past nrows arrive as zeros.
__device__ __forceinline__ void vec_async_load(void* dst, const void* src, int row0, int nrows,
                                               int lane) {
  const i32x4 rs = make_rsrc(static_cast<const char*>(src) + int64_t(row0) * 4, min(nrows - row0, BK) * 4);
  dma4(rs, __builtin_amdgcn_readfirstlane(lds_addr(dst)), lane * 4);
}

// The same loads for a pair of tiles (K and V, or Q and dO), one instruction per call:
// 0-3 fill the first tile, 4-7 the second.  Issued all at once after the barrier, the 32
// instructions of a workgroup's four waves queue in the buffer unit and each wave stalls
// before its first MFMA (in-kernel timestamps of the forward: 450-800 cycles); issued one
// at a time between the score MFMAs, they drain while the matrix pipe works.
struct PairDma {
  const uint16_t* a;
  const uint16_t* b;
  int nb;
  uint32_t ba, bb, voff;
  __device__ __forceinline__ PairDma(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                     int row0, int nrows, uint16_t* da, uint16_t* db, int wave,
                                     int lane)
      : a(A + int64_t(row0) * D), b(B + int64_t(row0) * D), nb(min(nrows - row0, BK) * D * 2),
        ba(__builtin_amdgcn_readfirstlane(lds_addr(da)) + wave * 1024),
        bb(__builtin_amdgcn_readfirstlane(lds_addr(db)) + wave * 1024),
        voff(tile_lane_off(wave, lane)) {}
  __device__ __forceinline__ void operator()(int i) const {
    const int it = i & 3;
    dma16(make_rsrc((i < 4 ? a : b) + it * 16 * D, nb - it * 16 * D * 2), (i < 4 ? ba : bb) + it * 4096,
          voff);
  }
};
struct NoDma {
  __device__ __forceinline__ void operator()(int) const {}
};

// Operand reads after which a chain of 16 MFMAs (reads running four ahead) issues one of the
// eight tile loads: reads 4, 5, 7, 8, 10, 11, 13 and 14, about one load per 1.5 MFMAs.
constexpr unsigned kDmaSlots = 0x6db0;
template <class Dma>
__device__ __forceinline__ void dma_after_read(const Dma& dma, int j) {
  if ((kDmaSlots >> j) & 1) dma(__builtin_popcount(kDmaSlots & ((1u << j) - 1)));
}

// dQ / dK-dV score chains with the next tile's loads spread between them: S = A_tile . ra
// and dP = B_tile . rb over D (16 MFMAs, the A and B operand reads alternating four ahead).
template <class Dma>
__device__ __forceinline__ void sdp_chain(f32x16& sacc, f32x16& pacc, const uint16_t* ab,
                                          const uint16_t* bb, int row, int hf, const bf16x8* ra,
                                          const bf16x8* rb, const Dma& dma) {
  bf16x8 op[2 * D / 16];
#pragma unroll
  for (int j = 0; j < 2 * D / 16; ++j) {
    op[j] = lds_load8(((j & 1) ? bb : ab) + tile_off(row, 16 * (j >> 1) + 8 * hf));
    dma_after_read(dma, j);
  }
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    sacc = mfma32(op[2 * s], ra[s], sacc);
    pacc = mfma32(op[2 * s + 1], rb[s], pacc);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 3);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 3);
}

// RoPE at load (the register-resident operand of a kernel, from unrotated input): the lane's
// 64 elements of its row at global position pos, element 16 s + 8 hf + j in x[s][j], i.e.
// pairs 8 s + 4 hf + k, turned and rounded to bf16 exactly as the standalone RoPE kernel does.
__device__ __forceinline__ void rope_row_bf16(bf16x8* x, int64_t pos, int hf, const RopeFreq& fr) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double rev = hf ? fr.rev[8 * s + 4 + k] : fr.rev[8 * s + k];
      float c, sn;
      rope_cs_turns(rope_turn(pos, rev), c, sn);
      float a = float(x[s][2 * k]), b = float(x[s][2 * k + 1]);
      rope_turn_pair(a, b, c, sn);
      x[s][2 * k] = (__bf16)a;
      x[s][2 * k + 1] = (__bf16)b;
    }
}

// RoPE turned back (the transpose) on a float32 accumulator row in the MFMA output layout:
// slot 4 g + e of block db holds element 32 db + 8 g + 4 hf + e, so slots (4g, 4g+1) and
// (4g+2, 4g+3) are pairs 16 db + 4 g + 2 hf and that + 1.  The row is at position pos.
__device__ __forceinline__ void rope_back_acc(f32x16* acc, int64_t pos, int hf, const RopeFreq& fr) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 16 * db + 4 * g + e;
        const double rev = hf ? fr.rev[i + 2] : fr.rev[i];
        float c, sn;
        rope_cs_turns(rope_turn(pos, rev), c, sn);
        float a = acc[db][4 * g + 2 * e], b = acc[db][4 * g + 2 * e + 1];
        rope_turn_pair(a, b, c, -sn);
        acc[db][4 * g + 2 * e] = a;
        acc[db][4 * g + 2 * e + 1] = b;
      }
}

// Wait until this wave's outstanding vector-memory loads (including loads into LDS) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Race canary.  Built with LWM_RACE_CANARY, every phase of a tile step that reads LDS, or
// issues loads into it, is followed by a wait for this wave's loads and a workgroup barrier,
// so no wave can run ahead of another into a buffer it shares.  A schedule whose single
// barrier per tile leaves a race gives results that differ from this build's; the GPU tests
// compare the two bit for bit.  In the normal build the calls compile to nothing.
__device__ __forceinline__ void canary_sync() {
#ifdef LWM_RACE_CANARY
  wait_vmem();
  __syncthreads();
#endif
}

// ---------------------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------------------

// kSplit (decode): blockIdx.y selects a slice of split_tiles key tiles; the workgroup's
// PARTIAL state for that slice goes to slice blockIdx.y of (Mo, Lo, ACC), each slice holding
// B*H*Sq rows; waves whose 32 query rows all lie past Sq only help load tiles.
// kRope: Q arrives unrotated and is turned by RoPE at its global positions as it is loaded;
// K arrives turned already (the standalone RoPE kernel's output).
template <bool kSplit, bool kRope = false>
__device__ __forceinline__ void fwd_bf16_body(AttnParams p, TableView t, int mode, int nqt,
                                              int split_tiles, const RopeFreq* rf,
                                              const uint16_t* __restrict__ Q,
                                              const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ V,
                                              const int32_t* __restrict__ seg_q,
                                              const int32_t* __restrict__ seg_k,
                                              uint16_t* __restrict__ O, float* __restrict__ LSE,
                                              float* __restrict__ Mo, float* __restrict__ Lo,
                                              float* __restrict__ ACC) {
  // double buffers: half 0 and half 1 of each array
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2 * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2 * kTileElems];
  __shared__ __attribute__((aligned(16))) int32_t segk_lds[2 * BK];
  __shared__ uint8_t stat_lds[kStatChunk];

  // Longest rows first: rank 0 is the last query tile; heads are interleaved so that
  // consecutive workgroups (spread over the XCDs) share a tile rank.
  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int qt = nqt - 1 - rest % nqt;
  const int b = rest / nqt;

  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Qh = Q + bh * p.Sq * D;
  const uint16_t* Kh = K + bh * p.Sk * D;
  const uint16_t* Vh = V + bh * p.Sk * D;
  const int32_t* segk_b = seg_k + int64_t(b) * p.Sk;

  const int qrow = qt * BQ + wave * 32 + col;
  const bool qlive = qrow < p.Sq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qlive) v = gload16(Qh + int64_t(qrow) * D + 16 * s + 8 * hf);
    qreg[s] = *reinterpret_cast<bf16x8*>(&v);
  }
  if constexpr (kRope) rope_row_bf16(qreg, p.q_offset + qrow, hf, *rf);
  const int32_t sq = qlive ? seg_q[int64_t(b) * p.Sq + qrow] : -1;
  const int dpos = clamp_dpos(p.q_offset, p.k_offset);

  const int r0 = 2 * qt;
  const bool has_r1 = r0 + 1 < t.nqb;
  const int32_t* rg0 = t.q_range + (int64_t(b) * t.nqb + r0) * 2;
  int lo, hi;
  range_union(rg0, rg0 + 2, has_r1, lo, hi);
  LWM_CHECK(r0 < t.nqb, kChkFwdRow);
  LWM_CHECK(lo > hi || (lo >= 0 && hi < t.nkb), kChkFwdRange);
  if (kSplit) {
    const int s0 = int(blockIdx.y) * split_tiles;
    lo = max(lo, s0);
    hi = min(hi, s0 + split_tiles - 1);
  }
  const bool wave_live = !kSplit || uniform(qt * BQ + wave * 32) < p.Sq;
  const uint8_t* st0 = t.status + (int64_t(b) * t.nqb + r0) * t.nkb;
  const uint8_t* st1 = st0 + t.nkb;

  const float c = p.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{0};

  auto issue = [&](int kt, uint16_t* kd, uint16_t* vd, int32_t* sd) {
    tile_async_load(kd, Kh, kt * BK, p.Sk, wave, lane);
    tile_async_load(vd, Vh, kt * BK, p.Sk, wave, lane);
    if (wave == 0) vec_async_load(sd, segk_b, kt * BK, p.Sk, lane);
  };

  // S^T = K Q^T for two 32-key blocks (K rows loaded in kperm order).  The operand reads run
  // four MFMAs ahead so LDS latency hides behind the matrix pipe; the next tile's loads
  // (`dma`) go out between them.
  auto scores = [&](f32x16* sacc, const uint16_t* kb_lds, const auto& dma) {
    bf16x8 kop[2 * D / 16];
#pragma unroll
    for (int j = 0; j < 2 * D / 16; ++j) {
      kop[j] = lds_load8(kb_lds + tile_off(32 * (j / (D / 16)) + kperm(col), 16 * (j % (D / 16)) + 8 * hf));
      dma_after_read(dma, j);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sacc[sub] = f32x16{0};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) sacc[sub] = mfma32(kop[sub * (D / 16) + s], qreg[s], sacc[sub]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  };

  // One key tile: wait for its loads, then S^T (starting the next tile's loads into the
  // other buffers), mask, online softmax and O^T += V^T P^T.
  // st_c and kn_c: the status of tile kt and the next live tile after it, read one step
  // ahead, so that no LDS round trip sits between two steps
  int kt = 0, c0 = 0, c1 = -1, st_c = 0, kn_c = 0;
  auto step = [&](const uint16_t* kb_lds, const uint16_t* vb_lds, const int32_t* sb_lds,
                  uint16_t* kn_lds, uint16_t* vn_lds, int32_t* sn_lds) {
    const int st = st_c;
    LWM_CHECK(kt >= c0 && kt <= c1 && kt >= lo && kt <= hi && kt * BK < p.Sk, kChkFwdTile);
    LWM_CHECK(st == LWM_TILE_PARTIAL || st == LWM_TILE_FULL, kChkFwdStatus);
    const int kn = kn_c;
    // the next step's: statuses of tiles kn and kn + 1 (indices kept inside the chunk)
    const int st_n = stat_lds[min(kn, c1) - c0];
    const int s_after = stat_lds[min(kn + 1, c1) - c0];
    auto advance = [&]() {
      st_c = uniform(st_n);
      kn_c = (kn + 1 <= c1 && uniform(s_after) == LWM_TILE_SKIP) ? next_live_lds(stat_lds, c0, kn + 2, c1)
                                                                 : kn + 1;
      kt = kn;
    };
    wait_vmem();
    __syncthreads();
    const bool more = kn <= c1;
    if (!wave_live) {
      if (more) issue(kn, kn_lds, vn_lds, sn_lds);
      // as many canary barriers as the live path below
      canary_sync();
      canary_sync();
      canary_sync();
      advance();
      return;
    }

    f32x16 sacc[2];
    if (more) {
      scores(sacc, kb_lds, PairDma(Kh, Vh, kn * BK, p.Sk, kn_lds, vn_lds, wave, lane));
      if (wave == 0) vec_async_load(sn_lds, segk_b, kn * BK, p.Sk, lane);
    } else {
      scores(sacc, kb_lds, NoDma{});
    }
    canary_sync();

    if (st == LWM_TILE_PARTIAL) {
      // branch-free visibility; rows past Sq carry sq = -1 and see nothing
      const int lim = key_limit(kt * BK + 8 * hf, qrow, dpos, p.Sk, p.causal, sq >= 0);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          int sk8[8];
          lds_load_i8(sb_lds + 32 * sub + 16 * a + 8 * hf, sk8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool vis = (sk8[j] == sq) & (32 * sub + 16 * a + j <= lim);
            sacc[sub][8 * a + j] = vis ? sacc[sub][8 * a + j] : -INFINITY;
          }
        }
    }

    // row max over the lane's 32 scores (four independent chains), then across the halves
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx4[(i & 1) + 2 * sub] = fmaxf(mx4[(i & 1) + 2 * sub], sacc[sub][i]);
    const float mxc = half_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]))) * c;
    const bool upd = mxc > m_run + kTau;  // false while every key so far is masked
    const float alpha = upd ? fast_exp2(m_run - mxc) : 1.f;
    if (upd) m_run = mxc;
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float ps4[4];  // four partial sums, each seeded with its first weight
    bf16x8 pb[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(fmaf(sacc[sub][8 * a + j], c, -m_use));
          ps4[j & 3] = (sub == 0 && a == 0 && j < 4) ? pv[j] : ps4[j & 3] + pv[j];
        }
        pb[2 * sub + a] = to_bf16x8(pv);
      }
    canary_sync();
    l_run = l_run * alpha + ((ps4[0] + ps4[1]) + (ps4[2] + ps4[3]));
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // O^T += V^T P^T over four 16-key steps; V^T read transposed from the row-major tile,
    // operand reads four MFMAs ahead
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = mfma32(lds_load_tr8(vb_lds, 16 * ks, 32 * db, lane), pb[ks], oacc[db]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 2);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);
    canary_sync();
    advance();
  };

  for (c0 = lo; c0 <= hi; c0 += kStatChunk) {
    c1 = min(hi, c0 + kStatChunk - 1);
    __syncthreads();
    stage_status_rows(stat_lds, st0, st1, has_r1, c0, c1, tid);
    __syncthreads();
    kt = next_live_lds(stat_lds, c0, c0, c1);
    if (kt <= c1) {
      st_c = uniform(stat_lds[kt - c0]);
      kn_c = next_live_lds(stat_lds, c0, kt + 1, c1);
    }
    if (kt <= c1) issue(kt, k_lds, v_lds, segk_lds);
    while (kt <= c1) {
      step(k_lds, v_lds, segk_lds, k_lds + kTileElems, v_lds + kTileElems, segk_lds + BK);
      if (kt > c1) break;
      step(k_lds + kTileElems, v_lds + kTileElems, segk_lds + BK, k_lds, v_lds, segk_lds);
    }
  }

  const float l_tot = half_sum(l_run);
  if (!qlive) return;
  LWM_CHECK(b < p.B, kChkFwdOut);
  const int64_t r64 = (kSplit ? int64_t(blockIdx.y) * p.B * p.H * p.Sq : 0) + bh * p.Sq + qrow;
  if (!kSplit && mode == LWM_OUT_FINAL) {
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

__global__ void __launch_bounds__(NT, 2)
fwd_bf16_kernel(AttnParams p, TableView t, int mode, int nqt, const uint16_t* __restrict__ Q,
                const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_k,
                uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Mo,
                float* __restrict__ Lo, float* __restrict__ ACC) {
  fwd_bf16_body<false>(p, t, mode, nqt, 0, nullptr, Q, K, V, seg_q, seg_k, O, LSE, Mo, Lo, ACC);
}

__global__ void __launch_bounds__(NT, 2)
fwd_rope_bf16_kernel(AttnParams p, TableView t, int mode, int nqt, const uint16_t* __restrict__ Q,
                     const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                     const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_k,
                     uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Mo,
                     float* __restrict__ Lo, float* __restrict__ ACC, RopeFreq rf) {
  fwd_bf16_body<false, true>(p, t, mode, nqt, 0, &rf, Q, K, V, seg_q, seg_k, O, LSE, Mo, Lo, ACC);
}

// ---------------------------------------------------------------------------------------
// split-KV decode: the forward per key slice, then the combine of the per-slice states
// ---------------------------------------------------------------------------------------

__global__ void __launch_bounds__(NT, 2)
decode_bf16_kernel(AttnParams p, TableView t, int nqt, int split_tiles,
                   const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const int32_t* __restrict__ seg_q,
                   const int32_t* __restrict__ seg_k, float* __restrict__ Mo,
                   float* __restrict__ Lo, float* __restrict__ ACC) {
  fwd_bf16_body<true>(p, t, LWM_OUT_PARTIAL, nqt, split_tiles, nullptr, Q, K, V, seg_q, seg_k, nullptr,
                      nullptr, Mo, Lo, ACC);
}

// Weight e^(x - m) of a slice whose max is x, where m >= x is the combined max; an empty
// slice (x = -inf) weighs 0, also when every slice is empty (m = -inf).
__device__ __forceinline__ float slice_weight(float x, float m) {
  return x == -INFINITY ? 0.f : expf(x - m);
}

// Exact combine of nsplit partial states per row (the ring's merge applied to all slices
// at once): m = max_s m_s, l = sum_s l_s e^(m_s - m), acc = sum_s acc_s e^(m_s - m), then
// O = acc / l (bf16) and LSE = m + ln l, or O = 0 and LSE = -inf when no slice saw a key.
// A group of 32 lanes owns one row (4 floats per lane); `gpr` groups (1, 2, 4 or 8) share a
// row, each summing every gpr-th slice, and their sums meet in LDS.  Every group first
// finds the row's max itself, its 32 lanes reading 32 slices' m at a time.
__global__ void __launch_bounds__(NT) decode_combine_kernel(int64_t rows, int nsplit, int gpr,
                                                            const float* __restrict__ M,
                                                            const float* __restrict__ L,
                                                            const float* __restrict__ ACC,
                                                            uint16_t* __restrict__ O,
                                                            float* __restrict__ LSE) {
  __shared__ float4 part_acc[NT / 32][32];
  __shared__ float part_l[NT / 32];
  const int tid = threadIdx.x, grp = tid >> 5, lane = tid & 31;
  const int rpb = (NT / 32) / gpr;  // rows per workgroup
  const int sub = grp % gpr;
  const int64_t nrb = (rows + rpb - 1) / rpb;
  LWM_CHECK(gpr >= 1 && (NT / 32) % gpr == 0 && nsplit >= 1, kChkCombine);
  for (int64_t rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
    const int64_t row = rb * rpb + grp / gpr;
    const bool live = row < rows;
    float m = -INFINITY, l = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
      for (int s = lane; s < nsplit; s += 32) m = fmaxf(m, M[int64_t(s) * rows + row]);
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 32));
      for (int s = sub; s < nsplit; s += gpr) {
        const int64_t r = int64_t(s) * rows + row;
        const float w = slice_weight(M[r], m);
        const float4 x = reinterpret_cast<const float4*>(ACC + r * D)[lane];
        l = fmaf(L[r], w, l);
        a.x = fmaf(x.x, w, a.x);
        a.y = fmaf(x.y, w, a.y);
        a.z = fmaf(x.z, w, a.z);
        a.w = fmaf(x.w, w, a.w);
      }
    }
    part_acc[grp][lane] = a;
    if (lane == 0) part_l[grp] = l;
    __syncthreads();
    if (live && sub == 0) {
      for (int g = 1; g < gpr; ++g) {
        const float4 x = part_acc[grp + g][lane];
        a.x += x.x;
        a.y += x.y;
        a.z += x.z;
        a.w += x.w;
        l += part_l[grp + g];
      }
      const float inv = l > 0.f ? 1.f / l : 0.f;
      __bf16 o4[4] = {(__bf16)(a.x * inv), (__bf16)(a.y * inv), (__bf16)(a.z * inv),
                      (__bf16)(a.w * inv)};
      reinterpret_cast<uint2*>(O + row * D)[lane] = *reinterpret_cast<uint2*>(o4);
      if (lane == 0) LSE[row] = l > 0.f ? m + logf(l) : -INFINITY;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------------------

// -Delta_i = -<dO_i, O_i> (stored negated) and LSE_i * log2(e), both float32, 16 lanes per
// row of 128.
__global__ void __launch_bounds__(NT) delta_bf16_kernel(int64_t rows, const uint16_t* __restrict__ O,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        float* __restrict__ delta,
                                                        float* __restrict__ lse2) {
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
  if (row < rows && part == 0) {
    delta[row] = -s;  // stored negated: the dP products start from it (see dq / dkv)
    // a row that sees no key (LSE = -inf) gets +inf, so exp2(s c - lse2) is 0 for every
    // key of it, masked or not, and never inf - inf
    const float l = LSE[row];
    lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// dQ: query-major like the forward.  Per key tile: S^T = K Q^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - Delta), dQ^T += K^T dS^T (K^T read transposed from the K tile).
// kRope: Q arrives unrotated and is turned at load, K arrives turned, and dQ (the gradient
// of the turned Q) is turned back in float32 before it is rounded: the gradient of Q.
template <bool kRope>
__device__ __forceinline__ void dq_bf16_body(AttnParams p, TableView t, int nqt, const RopeFreq* rf,
                                             const uint16_t* __restrict__ Q,
                                             const uint16_t* __restrict__ K,
                                             const uint16_t* __restrict__ V,
                                             const uint16_t* __restrict__ dO,
                                             const float* __restrict__ LSE2,
                                             const float* __restrict__ delta,
                                             const int32_t* __restrict__ seg_q,
                                             const int32_t* __restrict__ seg_k,
                                             uint16_t* __restrict__ dQ) {
  // [K tile | V tile] per buffer half in one array, so V reads reuse the K read addresses
  // with a constant offset
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[4 * kTileElems];
  __shared__ __attribute__((aligned(16))) int32_t segk_lds[2 * BK];
  __shared__ uint8_t stat_lds[kStatChunk];
  uint16_t* const k_lds0 = kv_lds;
  uint16_t* const v_lds0 = kv_lds + kTileElems;
  uint16_t* const k_lds1 = kv_lds + 2 * kTileElems;
  uint16_t* const v_lds1 = kv_lds + 3 * kTileElems;

  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int qt = nqt - 1 - rest % nqt;
  const int b = rest / nqt;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Kh = K + bh * p.Sk * D;
  const uint16_t* Vh = V + bh * p.Sk * D;
  const int32_t* segk_b = seg_k + int64_t(b) * p.Sk;

  const int qrow = qt * BQ + wave * 32 + col;
  const bool qlive = qrow < p.Sq;
  const int64_t r64 = bh * p.Sq + qrow;
  int64_t rbase = bh * p.Sq + qt * BQ + wave * 32;  // row of the wave's lane 0 (uniform)
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
  if constexpr (kRope) rope_row_bf16(qreg, p.q_offset + qrow, hf, *rf);
  const float lse2 = qlive ? LSE2[r64] : 0.f;
  const float ndl = qlive ? delta[r64] : 0.f;  // -Delta of the lane's row
  const int32_t sq = qlive ? seg_q[int64_t(b) * p.Sq + qrow] : -1;
  const int dpos = clamp_dpos(p.q_offset, p.k_offset);

  const int r0 = 2 * qt;
  const bool has_r1 = r0 + 1 < t.nqb;
  const int32_t* rg0 = t.q_range + (int64_t(b) * t.nqb + r0) * 2;
  int lo, hi;
  range_union(rg0, rg0 + 2, has_r1, lo, hi);
  LWM_CHECK(r0 < t.nqb, kChkDqRow);
  LWM_CHECK(lo > hi || (lo >= 0 && hi < t.nkb), kChkDqRange);
  const uint8_t* st0 = t.status + (int64_t(b) * t.nqb + r0) * t.nkb;
  const uint8_t* st1 = st0 + t.nkb;
  const float c = p.scale * kLog2e;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{0};

  auto issue = [&](int kt, uint16_t* kd, uint16_t* vd, int32_t* sd) {
    tile_async_load(kd, Kh, kt * BK, p.Sk, wave, lane);
    tile_async_load(vd, Vh, kt * BK, p.Sk, wave, lane);
    if (wave == 0) vec_async_load(sd, segk_b, kt * BK, p.Sk, lane);
  };

  int kt = 0, c0 = 0, c1 = -1;
  auto step = [&](const uint16_t* kb_lds, const uint16_t* vb_lds, const int32_t* sb_lds,
                  uint16_t* kn_lds, uint16_t* vn_lds, int32_t* sn_lds) {
    const int st = uniform(stat_lds[kt - c0]);
    LWM_CHECK(kt >= c0 && kt <= c1 && kt >= lo && kt <= hi && kt * BK < p.Sk, kChkDqTile);
    LWM_CHECK(st == LWM_TILE_PARTIAL || st == LWM_TILE_FULL, kChkDqStatus);
    const int kn = next_live_lds(stat_lds, c0, kt + 1, c1);
    wait_vmem();
    __syncthreads();
    const bool more = kn <= c1;
    if (more && wave == 0) vec_async_load(sn_lds, segk_b, kn * BK, p.Sk, lane);

    bf16x8 dsb[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc = f32x16{0}, pacc = f32x16{0};
      const int krow = 32 * sub + kperm(col);
      if (sub == 0 && more) {  // the next tile's K and V loads go out between these MFMAs
        sdp_chain(sacc, pacc, kb_lds, vb_lds, krow, hf, qreg, greg,
                  PairDma(Kh, Vh, kn * BK, p.Sk, kn_lds, vn_lds, wave, lane));
      } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int off = tile_off(krow, 16 * s + 8 * hf);
          sacc = mfma32(lds_load8(kb_lds + off), qreg[s], sacc);
          pacc = mfma32(lds_load8(vb_lds + off), greg[s], pacc);
        }
      }
      if (st == LWM_TILE_PARTIAL) {
        // hidden scores become -inf, so their probabilities come out as exactly 0
        const int lim = key_limit(kt * BK + 8 * hf, qrow, dpos, p.Sk, p.causal, sq >= 0);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          int sk8[8];
          lds_load_i8(sb_lds + 32 * sub + 16 * a + 8 * hf, sk8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool vis = (sk8[j] == sq) & (32 * sub + 16 * a + j <= lim);
            sacc[8 * a + j] = vis ? sacc[8 * a + j] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * a + j;
          ds[j] = fast_exp2(fmaf(sacc[i], c, -lse2)) * (pacc[i] + ndl);
        }
        dsb[2 * sub + a] = to_bf16x8(ds);
      }
      if (sub == 1) {
        // dQ of the first 32 keys needs only their dS, so its MFMAs run under the second
        // half's softmax: one MFMA per two operand reads and eight VALU instructions
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            dqacc[db] = mfma32(lds_load_tr8(kb_lds, 16 * ks, 32 * db, lane), dsb[ks], dqacc[db]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 6);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 6);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 6);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 6);
        }
      }
      // keep the two 32-key halves' scores apart: overlapping them would need a second set
      // of score registers, which does not fit beside two waves per SIMD
      __builtin_amdgcn_sched_barrier(0);
      canary_sync();
    }
#pragma unroll
    for (int ks = 2; ks < BK / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dqacc[db] = mfma32(lds_load_tr8(kb_lds, 16 * ks, 32 * db, lane), dsb[ks], dqacc[db]);
    canary_sync();
    kt = kn;
  };

  for (c0 = lo; c0 <= hi; c0 += kStatChunk) {
    c1 = min(hi, c0 + kStatChunk - 1);
    __syncthreads();
    stage_status_rows(stat_lds, st0, st1, has_r1, c0, c1, tid);
    __syncthreads();
    kt = next_live_lds(stat_lds, c0, c0, c1);
    if (kt <= c1) issue(kt, k_lds0, v_lds0, segk_lds);
    while (kt <= c1) {
      step(k_lds0, v_lds0, segk_lds, k_lds1, v_lds1, segk_lds + BK);
      if (kt > c1) break;
      step(k_lds1, v_lds1, segk_lds + BK, k_lds0, v_lds0, segk_lds);
    }
  }
  if (!qlive) return;
  // the output row formed again from scalars, so no 64-bit per-lane offset stays live across
  // the tile loop (it was spilled to scratch at two waves per SIMD)
  asm volatile("" : "+s"(rbase));
  uint16_t* out = dQ + (rbase + col) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] *= p.scale;
  if constexpr (kRope) {
    // the rows' positions from scalars as well (q_offset + rbase - bh Sq is row 0's)
    int64_t pos0 = p.q_offset + qt * BQ + wave * 32;
    asm volatile("" : "+s"(pos0));
    rope_back_acc(dqacc, pos0 + col, hf, *rf);
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hf;
      __bf16 o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)dqacc[db][4 * g + e];
      *reinterpret_cast<uint2*>(out + d0) = *reinterpret_cast<uint2*>(o4);
    }
}

__global__ void __launch_bounds__(NT, 2)
dq_bf16_kernel(AttnParams p, TableView t, int nqt, const uint16_t* __restrict__ Q,
               const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
               const uint16_t* __restrict__ dO, const float* __restrict__ LSE2,
               const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
               const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dQ) {
  dq_bf16_body<false>(p, t, nqt, nullptr, Q, K, V, dO, LSE2, delta, seg_q, seg_k, dQ);
}

__global__ void __launch_bounds__(NT, 2)
dq_rope_bf16_kernel(AttnParams p, TableView t, int nqt, const uint16_t* __restrict__ Q,
                    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                    const uint16_t* __restrict__ dO, const float* __restrict__ LSE2,
                    const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
                    const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dQ, RopeFreq rf) {
  dq_bf16_body<true>(p, t, nqt, &rf, Q, K, V, dO, LSE2, delta, seg_q, seg_k, dQ);
}

// dK/dV accumulation into AGPRs.  The dK/dV kernel needs more than 256 registers; built
// with MFMAs in VGPR form (see build.py), its score and dP accumulators sit in VGPRs that the
// softmax reads directly, while the constraint here keeps the long-lived dK/dV accumulators
// in AGPRs.  The compiler's hazard checks do not see inside asm, so the asm carries them:
// s_nop 1 gives the two wait states an MFMA needs after a VALU write of its A/B operand
// (ds_read results are covered by the compiler's lgkmcnt waits); mfma_agpr_fence covers the
// AGPR writes before the first MFMA and the MFMA results before the first AGPR read.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr_fence(f32x16* x, f32x16* y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(y[0]), "+a"(y[1]), "+a"(y[2]),
                 "+a"(y[3]));
}

// dK, dV: key-major.  Workgroup = 128 keys (32 per wave) held in registers; query tiles of
// 64 stream through LDS.  Per 32-query half: S = Q K^T, dP = dO V^T, P = exp(S - LSE),
// dS = P (dP - Delta), dV^T += dO^T P, dK^T += Q^T dS (dO^T, Q^T read transposed).
// kRope: K arrives unrotated and is turned at load, Q arrives turned, and dK is turned back
// in float32 before it is rounded.
template <bool kRope>
__device__ __forceinline__ void dkv_bf16_body(AttnParams p, TableView t, int nkt, const RopeFreq* rf,
                                              const uint16_t* __restrict__ Q,
                                              const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ V,
                                              const uint16_t* __restrict__ dO,
                                              const float* __restrict__ LSE2,
                                              const float* __restrict__ delta,
                                              const int32_t* __restrict__ seg_q,
                                              const int32_t* __restrict__ seg_k,
                                              uint16_t* __restrict__ dK, uint16_t* __restrict__ dV) {
  // [Q tile | dO tile] per buffer half in one array, so dO reads reuse the Q read addresses
  // with a constant offset
  __shared__ __attribute__((aligned(16))) uint16_t qg_lds[4 * kTileElems];
  uint16_t* const q_lds0 = qg_lds;
  uint16_t* const g_lds0 = qg_lds + kTileElems;

  // per query row of the tile: LSE*log2(e), -Delta and the segment id (as raw 32-bit words)
  __shared__ __attribute__((aligned(16))) float row_lds[2 * 3 * TB];
  __shared__ uint8_t stat_lds[kStatChunk];

  const int idx = blockIdx.x;
  const int h = idx % p.H;
  const int rest = idx / p.H;
  const int kt = rest % nkt;  // early keys see the most queries under the causal mask
  const int b = rest / nkt;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = int64_t(b) * p.H + h;
  const uint16_t* Qh = Q + bh * p.Sq * D;
  const uint16_t* Gh = dO + bh * p.Sq * D;
  const float* lse_h = LSE2 + bh * p.Sq;
  const float* dl_h = delta + bh * p.Sq;
  const int32_t* segq_b = seg_q + int64_t(b) * p.Sq;

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
  if constexpr (kRope) rope_row_bf16(kreg, p.k_offset + key, hf, *rf);
  const int32_t sk = klive ? seg_k[int64_t(b) * p.Sk + key] : -2;
  const int dpos = clamp_dpos(p.q_offset, p.k_offset);

  const int c0 = 2 * kt;
  const bool has_c1 = c0 + 1 < t.nkb;
  const int32_t* rg0 = t.k_range + (int64_t(b) * t.nkb + c0) * 2;
  int lo, hi;
  range_union(rg0, rg0 + 2, has_c1, lo, hi);
  LWM_CHECK(c0 < t.nkb, kChkDkvCol);
  LWM_CHECK(lo > hi || (lo >= 0 && hi < t.nqb), kChkDkvRange);
  const uint8_t* stb = t.status + int64_t(b) * t.nqb * t.nkb;
  const float c = p.scale * kLog2e;

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dkacc[i] = f32x16{0};
    dvacc[i] = f32x16{0};
  }
  static_assert(D / 32 == 4, "mfma_agpr_fence takes four accumulators of each kind");
  mfma_agpr_fence(dkacc, dvacc);

  auto issue_rows = [&](int qb, float* rd) {
    if (wave == 0) vec_async_load(rd, lse_h, qb * TB, p.Sq, lane);
    if (wave == 1) vec_async_load(rd + TB, dl_h, qb * TB, p.Sq, lane);
    if (wave == 2) vec_async_load(rd + 2 * TB, segq_b, qb * TB, p.Sq, lane);
  };
  auto issue = [&](int qb, uint16_t* qd, uint16_t* gd, float* rd) {
    tile_async_load(qd, Qh, qb * TB, p.Sq, wave, lane);
    tile_async_load(gd, Gh, qb * TB, p.Sq, wave, lane);
    issue_rows(qb, rd);
  };

  // st_c and qn_c: the status of tile qb and the next live tile after it, read one step
  // ahead, so that no LDS round trip sits between two steps
  int qb = 0, w0 = 0, w1 = -1, st_c = 0, qn_c = 0;
  auto step = [&](const uint16_t* qb_lds, const uint16_t* gb_lds, const float* rb_lds,
                  uint16_t* qn_lds, uint16_t* gn_lds, float* rn_lds) {
    const int st = st_c;
    LWM_CHECK(qb >= w0 && qb <= w1 && qb >= lo && qb <= hi && qb * TB < p.Sq, kChkDkvTile);
    LWM_CHECK(st == LWM_TILE_PARTIAL || st == LWM_TILE_FULL, kChkDkvStatus);
    const int qn = qn_c;
    // the next step's: statuses of tiles qn and qn + 1 (indices kept inside the chunk)
    const int st_n = stat_lds[min(qn, w1) - w0];
    const int s_after = stat_lds[min(qn + 1, w1) - w0];
    wait_vmem();
    __syncthreads();
    const bool more = qn <= w1;
    if (more) issue_rows(qn, rn_lds);

    // both 32-row halves' S and dP first (the next tile's loads spread between the first
    // half's MFMAs), then the masks, the softmax of both halves and their dV/dK updates
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // dP starts from -Delta of each query row (slot 8a + j holds row 32 sub + 16a + 8hf + j),
      // so the products deliver dP - Delta directly
      sacc[sub] = f32x16{0};
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float ndl[8];
        lds_load_f8(rb_lds + TB + 32 * sub + 16 * a + 8 * hf, ndl);
#pragma unroll
        for (int j = 0; j < 8; ++j) pacc[sub][8 * a + j] = ndl[j];
      }
    }
    if (more)
      sdp_chain(sacc[0], pacc[0], qb_lds, gb_lds, kperm(col), hf, kreg, vreg,
                PairDma(Qh, Gh, qn * TB, p.Sq, qn_lds, gn_lds, wave, lane));
    else
      sdp_chain(sacc[0], pacc[0], qb_lds, gb_lds, kperm(col), hf, kreg, vreg, NoDma{});
    sdp_chain(sacc[1], pacc[1], qb_lds, gb_lds, 32 + kperm(col), hf, kreg, vreg, NoDma{});
    canary_sync();
    if (st == LWM_TILE_PARTIAL) {
      // hidden scores become -inf, so their probabilities come out as exactly 0; keys past Sk
      // carry sk = -2 and see no row
      int rlo, rhi;
      row_window(qb * TB + 8 * hf, key, dpos, p.Sq, p.causal, sk >= 0, rlo, rhi);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          int sq8[8];
          lds_load_i8(reinterpret_cast<const int32_t*>(rb_lds + 2 * TB) + 32 * sub + 16 * a + 8 * hf, sq8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int o = 32 * sub + 16 * a + j;
            const bool vis = (sq8[j] == sk) & (o >= rlo) & (o <= rhi);
            sacc[sub][8 * a + j] = vis ? sacc[sub][8 * a + j] : -INFINITY;
          }
        }
    }
    // dV/dK operand reads (transposed dO and Q tiles) run kAhead MFMAs ahead of their use in a
    // fixed order: at one wave per SIMD the scheduler, which cannot see into the asm MFMAs,
    // placed them too late.  The first ones go out before the softmax.  MFMA m updates dV
    // (even m) or dK (odd m) for key step ks = m / 8 and column block db = (m / 2) % 4.
    constexpr int kAhead = 6;
    bf16x8 op[32];
    auto opread = [&](int m) {
      const int ks = m >> 3, db = (m >> 1) & 3;
      op[m] = lds_load_tr8((m & 1) ? qb_lds : gb_lds, 16 * ks, 32 * db, lane);
    };
#pragma unroll
    for (int m = 0; m < kAhead; ++m) opread(m);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pb[4], dsb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int qbase = 16 * ks + 8 * hf;  // 8 consecutive local query rows
      float lsev[8];
      lds_load_f8(rb_lds + qbase, lsev);
      float pv[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * (ks & 1) + j;
        pv[j] = fast_exp2(fmaf(sacc[ks >> 1][i], c, -lsev[j]));
        ds[j] = pv[j] * pacc[ks >> 1][i];
      }
      pb[ks] = to_bf16x8(pv);
      dsb[ks] = to_bf16x8(ds);
    }
    canary_sync();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int ks = m >> 3, db = (m >> 1) & 3;
      if (m & 1)
        mfma32_agpr(dkacc[db], op[m], dsb[ks]);
      else
        mfma32_agpr(dvacc[db], op[m], pb[ks]);
      if (m + kAhead < 32) opread(m + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    canary_sync();
    st_c = uniform(st_n);
    qn_c = (qn + 1 <= w1 && uniform(s_after) == LWM_TILE_SKIP) ? next_live_lds(stat_lds, w0, qn + 2, w1)
                                                                : qn + 1;
    qb = qn;
  };

  for (w0 = lo; w0 <= hi; w0 += kStatChunk) {
    w1 = min(hi, w0 + kStatChunk - 1);
    __syncthreads();
    stage_status_cols(stat_lds, stb, t.nkb, c0, has_c1, w0, w1, tid);
    __syncthreads();
    qb = next_live_lds(stat_lds, w0, w0, w1);
    if (qb <= w1) {
      st_c = uniform(stat_lds[qb - w0]);
      qn_c = next_live_lds(stat_lds, w0, qb + 1, w1);
    }
    // unrolled by two, so every LDS address is a register plus a constant offset
    if (qb <= w1) issue(qb, q_lds0, g_lds0, row_lds);
    while (qb <= w1) {
      step(q_lds0, g_lds0, row_lds, q_lds0 + 2 * kTileElems, g_lds0 + 2 * kTileElems, row_lds + 3 * TB);
      if (qb > w1) break;
      step(q_lds0 + 2 * kTileElems, g_lds0 + 2 * kTileElems, row_lds + 3 * TB, q_lds0, g_lds0, row_lds);
    }
  }
  mfma_agpr_fence(dkacc, dvacc);
  if (!klive) return;
  uint16_t* ko = dK + k64 * D;
  uint16_t* vo = dV + k64 * D;
  f32x16 dks[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dks[db][i] = dkacc[db][i] * p.scale;
  if constexpr (kRope) rope_back_acc(dks, p.k_offset + key, hf, *rf);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hf;
      __bf16 k4[4], v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = (__bf16)dks[db][4 * g + e];
        v4[e] = (__bf16)(dvacc[db][4 * g + e]);
      }
      *reinterpret_cast<uint2*>(ko + d0) = *reinterpret_cast<uint2*>(k4);
      *reinterpret_cast<uint2*>(vo + d0) = *reinterpret_cast<uint2*>(v4);
    }
}

__global__ void __launch_bounds__(NT, 1)
dkv_bf16_kernel(AttnParams p, TableView t, int nkt, const uint16_t* __restrict__ Q,
                const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                const uint16_t* __restrict__ dO, const float* __restrict__ LSE2,
                const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
                const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dK,
                uint16_t* __restrict__ dV) {
  dkv_bf16_body<false>(p, t, nkt, nullptr, Q, K, V, dO, LSE2, delta, seg_q, seg_k, dK, dV);
}

__global__ void __launch_bounds__(NT, 1)
dkv_rope_bf16_kernel(AttnParams p, TableView t, int nkt, const uint16_t* __restrict__ Q,
                     const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                     const uint16_t* __restrict__ dO, const float* __restrict__ LSE2,
                     const float* __restrict__ delta, const int32_t* __restrict__ seg_q,
                     const int32_t* __restrict__ seg_k, uint16_t* __restrict__ dK,
                     uint16_t* __restrict__ dV, RopeFreq rf) {
  dkv_bf16_body<true>(p, t, nkt, &rf, Q, K, V, dO, LSE2, delta, seg_q, seg_k, dK, dV);
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

// Forward with RoPE at load: q unrotated, k turned already.
hipError_t launch_fwd_rope_bf16(const lwm_attn_desc& d, int mode, double theta, const void* q,
                                const void* k, const void* v, const int32_t* seg_q,
                                const int32_t* seg_k, const void* table, void* o, float* lse,
                                float* m, float* l, float* acc, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  const int64_t grid = int64_t(nqt) * d.H * d.B;
  fwd_rope_bf16_kernel<<<dim3(unsigned(grid)), dim3(NT), 0, stream>>>(
      attn_params(d), t, mode, nqt, static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), seg_q, seg_k,
      static_cast<uint16_t*>(o), lse, m, l, acc, rope_freqs(D, theta));
  return hipGetLastError();
}

// Backward with RoPE at load: the dQ pass takes q unrotated and k turned, the dK/dV pass k
// unrotated and q turned (q_rot); dq and dk are the gradients of the unrotated q and k.
hipError_t launch_bwd_rope_bf16(const lwm_attn_desc& d, double theta, const void* q,
                                const void* q_rot, const void* k, const void* k_rot, const void* v,
                                const void* o, const void* dO, const float* lse,
                                const int32_t* seg_q, const int32_t* seg_k, const void* table,
                                void* dq, void* dk, void* dv, float* workspace, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const AttnParams p = attn_params(d);
  const RopeFreq fr = rope_freqs(D, theta);
  const int64_t rows = int64_t(d.B) * d.H * d.Sq;
  float* delta = workspace;
  float* lse2 = workspace + align256(size_t(rows) * sizeof(float)) / sizeof(float);
  delta_bf16_kernel<<<dim3(unsigned((rows * 16 + NT - 1) / NT)), dim3(NT), 0, stream>>>(
      rows, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), lse, delta, lse2);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  dq_rope_bf16_kernel<<<dim3(unsigned(int64_t(nqt) * d.H * d.B)), dim3(NT), 0, stream>>>(
      p, t, nqt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_rot),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse2, delta, seg_q, seg_k,
      static_cast<uint16_t*>(dq), fr);
  const int nkt = (d.Sk + 127) / 128;
  dkv_rope_bf16_kernel<<<dim3(unsigned(int64_t(nkt) * d.H * d.B)), dim3(NT), 0, stream>>>(
      p, t, nkt, static_cast<const uint16_t*>(q_rot), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse2, delta, seg_q, seg_k,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), fr);
  return hipGetLastError();
}

// Split-KV decode: the forward in PARTIAL form with grid (query tiles x heads x batch,
// slices), then the combine.  Workspace layout: L.
hipError_t launch_decode_bf16(const lwm_attn_desc& d, const DecodeLayout& L, const void* q,
                              const void* k, const void* v, const int32_t* seg_q,
                              const int32_t* seg_k, const void* table, void* o, float* lse,
                              void* workspace, hipStream_t stream) {
  const TableView t = table_view(d, table);
  char* ws = static_cast<char*>(workspace);
  float* m = reinterpret_cast<float*>(ws + L.m_off);
  float* l = reinterpret_cast<float*>(ws + L.l_off);
  float* acc = reinterpret_cast<float*>(ws + L.acc_off);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  const int64_t grid = int64_t(nqt) * d.H * d.B;
  decode_bf16_kernel<<<dim3(unsigned(grid), unsigned(L.nsplit)), dim3(NT), 0, stream>>>(
      attn_params(d), t, nqt, int(L.split_tiles), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), seg_q, seg_k, m, l, acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(d.B) * d.H * d.Sq;
  const int gpr = L.nsplit >= 8 ? 8 : L.nsplit >= 4 ? 4 : L.nsplit >= 2 ? 2 : 1;
  const int64_t nrb = (rows + (NT / 32) / gpr - 1) / ((NT / 32) / gpr);
  const unsigned cgrid = unsigned(nrb < (int64_t(1) << 20) ? nrb : (int64_t(1) << 20));
  decode_combine_kernel<<<dim3(cgrid), dim3(NT), 0, stream>>>(
      rows, int(L.nsplit), gpr, m, l, acc, static_cast<uint16_t*>(o), lse);
  return hipGetLastError();
}

// Workspace: -Delta [rows] then LSE * log2(e) [rows], rows = B*H*Sq, each 256-byte aligned.
hipError_t launch_bwd_bf16(const lwm_attn_desc& d, int phase, const void* q, const void* k,
                           const void* v, const void* o, const void* dO, const float* lse,
                           const int32_t* seg_q, const int32_t* seg_k, const void* table,
                           void* dq, void* dk, void* dv, float* workspace, hipStream_t stream) {
  const TableView t = table_view(d, table);
  const AttnParams p = attn_params(d);
  const int64_t rows = int64_t(d.B) * d.H * d.Sq;
  float* delta = workspace;
  float* lse2 = workspace + align256(size_t(rows) * sizeof(float)) / sizeof(float);
  if (phase < 0 || phase == LWM_BWD_DELTA)
    delta_bf16_kernel<<<dim3(unsigned((rows * 16 + NT - 1) / NT)), dim3(NT), 0, stream>>>(
        rows, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), lse, delta, lse2);
  const int nqt = (d.Sq + BQ - 1) / BQ;
  if (phase < 0 || phase == LWM_BWD_DQ)
    dq_bf16_kernel<<<dim3(unsigned(int64_t(nqt) * d.H * d.B)), dim3(NT), 0, stream>>>(
        p, t, nqt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse2, delta, seg_q,
        seg_k, static_cast<uint16_t*>(dq));
  const int nkt = (d.Sk + 127) / 128;
  if (phase < 0 || phase == LWM_BWD_DKV)
    dkv_bf16_kernel<<<dim3(unsigned(int64_t(nkt) * d.H * d.B)), dim3(NT), 0, stream>>>(
        p, t, nkt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse2, delta, seg_q,
        seg_k, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
  return hipGetLastError();
}

LWM_DEBUG_READER(attn_bf16)

}  // namespace lwm
