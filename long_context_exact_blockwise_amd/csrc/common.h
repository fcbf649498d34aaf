// Internal declarations shared by the HIP kernels and the host-side C-ABI glue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lwm_attn.h"

namespace lwm {

// Block-table buffer layout: q_range, k_range, status, then the per-block segment
// statistics the builder derives them from, each part on a 256-byte boundary.
struct TableLayout {
  int32_t nqb, nkb;
  size_t q_range_off, k_range_off, status_off, q_stats_off, k_stats_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- device checks (debug builds) ------------------------------------------------------
// Built with LWM_DEBUG, the kernels check the indices they derive from the block table (the
// query and key ranges, the tile statuses, the slots of the status chunk staged in LDS) and
// from their launch shape against the extents they index.  A failed check does not trap: it
// sets bit `code` of the first word of a device array private to its source file and, for the
// first failure only, stores code << 24 | workgroup in the second; lwm_attn_debug_status reads
// and clears every file's words.  Without LWM_DEBUG a check compiles to nothing.
enum DebugCheck : unsigned {
  kChkFwdRow = 1,      // forward / decode: the query tile's table rows exist
  kChkFwdRange = 2,    // forward / decode: key range of those rows inside the table
  kChkFwdTile = 3,     // forward / decode: visited key tile inside the range, chunk and keys
  kChkFwdStatus = 4,   // forward / decode: visited tile's status is PARTIAL or FULL
  kChkFwdOut = 5,      // forward / decode: output row inside the outputs
  kChkDqRow = 6,       // dQ: the query tile's table rows exist
  kChkDqRange = 7,     // dQ: key range inside the table
  kChkDqTile = 8,      // dQ: visited key tile inside the range, chunk and keys
  kChkDqStatus = 9,    // dQ: visited tile's status
  kChkDkvCol = 10,     // dK/dV: the key tile's table columns exist
  kChkDkvRange = 11,   // dK/dV: query range inside the table
  kChkDkvTile = 12,    // dK/dV: visited query tile inside the range, chunk and queries
  kChkDkvStatus = 13,  // dK/dV: visited tile's status
  kChkCombine = 14,    // decode combine: row inside the outputs
  kChkF32Range = 15,   // float32 kernels: table range inside the table
  kChkF32Tile = 16,    // float32 kernels: visited tile inside the range and the sequence
  kChkTable = 17,      // table builder: block index and status value in range
  kChkMerge = 18,      // merge: row inside the states
  kChkSelfTest = 31,   // set on request by lwm_attn_debug_status, to test the reporting
};

#ifdef LWM_DEBUG
static __device__ unsigned int g_debug_words[2];
__device__ __forceinline__ void debug_fail(unsigned code) {
  atomicOr(&g_debug_words[0], 1u << code);
  atomicCAS(&g_debug_words[1], 0u, (code << 24) | (blockIdx.x & 0xFFFFFFu));
}
#define LWM_CHECK(cond, code)                  \
  do {                                         \
    if (!(cond)) ::lwm::debug_fail(code);      \
  } while (0)
// Defines debug_read_<name>: copies this file's two words to w and clears them.
#define LWM_DEBUG_READER(name)                                                            \
  hipError_t debug_read_##name(unsigned* w) {                                            \
    hipError_t e = hipMemcpyFromSymbol(w, HIP_SYMBOL(g_debug_words), 2 * sizeof(unsigned)); \
    if (e != hipSuccess) return e;                                                        \
    const unsigned z[2] = {0u, 0u};                                                       \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_debug_words), z, sizeof z);                     \
  }
hipError_t debug_read_attn_bf16(unsigned* w);
hipError_t debug_read_attn_f32(unsigned* w);
hipError_t debug_read_table(unsigned* w);
hipError_t debug_read_merge(unsigned* w);
hipError_t debug_read_api(unsigned* w);
#else
#define LWM_CHECK(cond, code) \
  do {                        \
  } while (0)
#define LWM_DEBUG_READER(name)
#endif

inline TableLayout table_layout(const lwm_attn_desc& d) {
  TableLayout t;
  t.nqb = (d.Sq + d.block_q - 1) / d.block_q;
  t.nkb = (d.Sk + d.block_k - 1) / d.block_k;
  t.q_range_off = 0;
  t.k_range_off = align256(size_t(d.B) * t.nqb * 2 * sizeof(int32_t));
  t.status_off = t.k_range_off + align256(size_t(d.B) * t.nkb * 2 * sizeof(int32_t));
  t.q_stats_off = t.status_off + align256(size_t(d.B) * t.nqb * t.nkb);
  t.k_stats_off = t.q_stats_off + align256(size_t(d.B) * t.nqb * 4 * sizeof(int32_t));
  t.total = t.k_stats_off + align256(size_t(d.B) * t.nkb * 4 * sizeof(int32_t));
  return t;
}

// Device view of a built table.
struct TableView {
  const int32_t* q_range;  // [B][nqb][2]
  const int32_t* k_range;  // [B][nkb][2]
  const uint8_t* status;   // [B][nqb][nkb]
  int32_t nqb, nkb;
};

inline TableView table_view(const lwm_attn_desc& d, const void* table) {
  TableLayout L = table_layout(d);
  const char* base = static_cast<const char*>(table);
  return TableView{reinterpret_cast<const int32_t*>(base + L.q_range_off),
                   reinterpret_cast<const int32_t*>(base + L.k_range_off),
                   reinterpret_cast<const uint8_t*>(base + L.status_off), L.nqb, L.nkb};
}

// Scalars every attention kernel needs, passed by value.
struct AttnParams {
  int32_t B, H, Sq, Sk;
  int64_t q_offset, k_offset;
  float scale;
  int32_t causal;
};

inline AttnParams attn_params(const lwm_attn_desc& d) {
  return AttnParams{d.B, d.H, d.Sq, d.Sk, d.q_offset, d.k_offset, d.scale, d.causal};
}

// Split-KV decode (bf16 path): the key tiles are cut into nsplit slices of split_tiles
// 64-key tiles so that few query rows still fill the chip with about kDecodeGroups
// workgroups; each slice's state (m, l, acc) for every query row lands in the workspace:
// m [nsplit][rows], l [nsplit][rows], acc [nsplit][rows][D] float32, rows = B*H*Sq, each
// part on a 256-byte boundary.  Slices never go below kDecodeMinTiles tiles, and there are
// at most 65535 of them (the grid's y extent).
constexpr int64_t kDecodeGroups = 8192;
constexpr int64_t kDecodeMinTiles = 16;

struct DecodeLayout {
  int64_t split_tiles, nsplit;
  size_t m_off, l_off, acc_off, total;
};

inline DecodeLayout decode_layout_for(const lwm_attn_desc& d, int64_t split_tiles) {
  const int64_t nkt = (int64_t(d.Sk) + 63) / 64;
  DecodeLayout L;
  L.split_tiles = split_tiles;
  L.nsplit = nkt > 0 ? (nkt + split_tiles - 1) / split_tiles : 1;
  const size_t rows = size_t(d.B) * d.H * d.Sq;
  L.m_off = 0;
  L.l_off = align256(size_t(L.nsplit) * rows * sizeof(float));
  L.acc_off = L.l_off + align256(size_t(L.nsplit) * rows * sizeof(float));
  L.total = L.acc_off + align256(size_t(L.nsplit) * rows * d.D * sizeof(float));
  return L;
}

inline DecodeLayout decode_layout(const lwm_attn_desc& d) {
  const int64_t nkt = (int64_t(d.Sk) + 63) / 64;
  const int64_t base = (int64_t(d.Sq) + 127) / 128 * d.H * d.B;
  const int64_t want = base > 0 ? (kDecodeGroups + base - 1) / base : 1;
  int64_t st = (nkt + want - 1) / want;
  if (st < kDecodeMinTiles) st = kDecodeMinTiles;
  if (st < (nkt + 65534) / 65535) st = (nkt + 65534) / 65535;
  return decode_layout_for(d, st);
}

// The same split with at most max_bytes of slice states: fewer, longer slices when the
// default split needs more.  False when even one slice per row does not fit.
inline bool decode_layout_capped(const lwm_attn_desc& d, size_t max_bytes, DecodeLayout* out) {
  DecodeLayout L = decode_layout(d);
  if (L.total > max_bytes) {
    const size_t per_slice = size_t(d.B) * d.H * d.Sq * (size_t(d.D) + 2) * sizeof(float);
    if (per_slice == 0 || max_bytes < 3 * 256 + per_slice) return false;
    const int64_t max_slices = int64_t((max_bytes - 3 * 256) / per_slice);
    const int64_t nkt = (int64_t(d.Sk) + 63) / 64;
    int64_t st = (nkt + max_slices - 1) / max_slices;
    if (st < L.split_tiles) st = L.split_tiles;
    L = decode_layout_for(d, st);
    if (L.total > max_bytes) return false;
  }
  *out = L;
  return true;
}

// Packed-loss workspace: per-sample loss-token counters int32 [B][nseg], the sample count
// (one int32 in a 256-byte slot), then the weighted token losses float32 [B*T], each part on
// a 256-byte boundary.
struct PackedLossLayout {
  size_t count_off, samples_off, wloss_off, total;
};

inline PackedLossLayout packed_loss_layout(int32_t B, int32_t T, int32_t nseg) {
  PackedLossLayout L;
  L.count_off = 0;
  L.samples_off = align256(size_t(B) * nseg * sizeof(int32_t));
  L.wloss_off = L.samples_off + 256;
  L.total = L.wloss_off + align256(size_t(B) * T * sizeof(float));
  return L;
}

// ---- launchers (each returns the launch status) ----------------------------------------

// Zero `bytes` (a multiple of 16) at a 16-byte aligned device address.
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t stream);

hipError_t launch_build_table(const lwm_attn_desc& d, const int32_t* seg_q, const int32_t* seg_k,
                              void* table, hipStream_t stream);

hipError_t launch_fwd_f32(const lwm_attn_desc& d, int mode, const float* q, const float* k,
                          const float* v, const int32_t* seg_q, const int32_t* seg_k,
                          const void* table, float* o, float* lse, float* m, float* l,
                          float* acc, hipStream_t stream);

// Backward launchers run one phase (LWM_BWD_*) or all of them (phase < 0).
hipError_t launch_bwd_f32(const lwm_attn_desc& d, int phase, const float* q, const float* k, const float* v,
                          const float* o, const float* dO, const float* lse,
                          const int32_t* seg_q, const int32_t* seg_k, const void* table,
                          float* dq, float* dk, float* dv, float* delta, hipStream_t stream);

hipError_t launch_fwd_bf16(const lwm_attn_desc& d, int mode, const void* q, const void* k,
                           const void* v, const int32_t* seg_q, const int32_t* seg_k,
                           const void* table, void* o, float* lse, float* m, float* l,
                           float* acc, hipStream_t stream);

// RoPE at load (bf16, D = 128): q unrotated, k turned by the standalone RoPE kernel.
hipError_t launch_fwd_rope_bf16(const lwm_attn_desc& d, int mode, double theta, const void* q,
                                const void* k, const void* v, const int32_t* seg_q,
                                const int32_t* seg_k, const void* table, void* o, float* lse,
                                float* m, float* l, float* acc, hipStream_t stream);

// Backward with RoPE at load; the workspace as for launch_bwd_bf16.
hipError_t launch_bwd_rope_bf16(const lwm_attn_desc& d, double theta, const void* q,
                                const void* q_rot, const void* k, const void* k_rot, const void* v,
                                const void* o, const void* dO, const float* lse,
                                const int32_t* seg_q, const int32_t* seg_k, const void* table,
                                void* dq, void* dk, void* dv, float* workspace, hipStream_t stream);

// Slice states in `workspace` laid out as L (decode_layout or decode_layout_capped).
hipError_t launch_decode_bf16(const lwm_attn_desc& d, const DecodeLayout& L, const void* q,
                              const void* k, const void* v, const int32_t* seg_q,
                              const int32_t* seg_k, const void* table, void* o, float* lse,
                              void* workspace, hipStream_t stream);

// Decode with its slice states in the library's own static device buffer of
// kDecodeScratchBytes per device (decode_noalloc.hip); LWM_ERR_WORKSPACE-worthy sizes are
// rejected by the caller with decode_layout_capped first.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t launch_decode_bf16_noalloc(const lwm_attn_desc& d, const DecodeLayout& L, const void* q,
                                      const void* k, const void* v, const int32_t* seg_q,
                                      const int32_t* seg_k, const void* table, void* o,
                                      float* lse, hipStream_t stream);

hipError_t launch_bwd_bf16(const lwm_attn_desc& d, int phase, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* seg_q, const int32_t* seg_k, const void* table,
                           void* dq, void* dk, void* dv, float* workspace, hipStream_t stream);

// RoPE over rows = B*H*S rows of D elements (D in 8..256, a power of two), in place allowed.
hipError_t launch_rope(int32_t B, int32_t H, int32_t S, int32_t D, int32_t dtype, int64_t pos0,
                       double theta, int32_t inverse, const void* x, void* y, hipStream_t stream);

hipError_t launch_packed_loss(const PackedLossLayout& L, int32_t B, int32_t T, int32_t V,
                              int32_t nseg, int32_t dtype, const void* logits,
                              const int32_t* targets, const int32_t* seg, float grad_scale,
                              float* loss, float* token_loss, void* dlogits, void* workspace,
                              hipStream_t stream);

hipError_t launch_merge(int64_t rows, int32_t D, float* m, float* l, float* acc, const float* mc,
                        const float* lc, const float* accc, int32_t finalize, int32_t out_dtype,
                        void* o, float* lse, hipStream_t stream);

}  // namespace lwm
