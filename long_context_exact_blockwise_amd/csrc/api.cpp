// Host side of the C-ABI declared in include/lwm_attn.h: argument validation, dispatch by
// dtype and head width, launch on the caller's stream, error mapping.  Holds no state.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>

#include "common.h"

namespace {

using lwm::TableLayout;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const lwm_attn_desc* d) {
  if (d == nullptr) return LWM_ERR_INVALID_ARG;
  if (d->dtype != LWM_BF16 && d->dtype != LWM_F32) return LWM_ERR_INVALID_ARG;
  if (d->B <= 0 || d->H <= 0 || d->Sq < 0 || d->Sk < 0 || d->D <= 0) return LWM_ERR_SHAPE;
  if (d->q_offset < 0 || d->k_offset < 0) return LWM_ERR_SHAPE;
  if (d->causal != 0 && d->causal != 1) return LWM_ERR_INVALID_ARG;
  if (!(d->block_q == 16 || d->block_q == 32 || d->block_q == 64)) return LWM_ERR_INVALID_ARG;
  if (!(d->block_k == 16 || d->block_k == 32 || d->block_k == 64)) return LWM_ERR_INVALID_ARG;
  // element counts must fit the 64-bit index math and the 32-bit grid dimensions used
  const int64_t rows_q = int64_t(d->B) * d->H * d->Sq;
  const int64_t rows_k = int64_t(d->B) * d->H * d->Sk;
  if (rows_q > (int64_t(1) << 40) || rows_k > (int64_t(1) << 40)) return LWM_ERR_SHAPE;
  if (d->q_offset > (int64_t(1) << 50) || d->k_offset > (int64_t(1) << 50)) return LWM_ERR_SHAPE;
  return LWM_OK;
}

int check_attention_desc(const lwm_attn_desc* d) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!(d->scale > 0.f) || d->scale == std::numeric_limits<float>::infinity())
    return LWM_ERR_INVALID_ARG;
  if (d->block_q != 64 || d->block_k != 64) return LWM_ERR_UNSUPPORTED;
  if (d->dtype == LWM_BF16 && d->D != 128) return LWM_ERR_UNSUPPORTED;
  if (d->dtype == LWM_F32 && d->D != 32 && d->D != 64) return LWM_ERR_UNSUPPORTED;
  // grid: one workgroup per 128-row tile per (b, h) must fit a 32-bit grid
  const int64_t tiles = int64_t((std::max(d->Sq, d->Sk) + 127) / 128) * d->H * d->B;
  if (tiles >= (int64_t(1) << 31)) return LWM_ERR_SHAPE;
  return LWM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LWM_OK : LWM_ERR_HIP; }

#ifdef LWM_DEBUG
// One failed check on purpose (code kChkSelfTest), so that a test can see the reporting work.
__global__ void debug_self_test_kernel() { LWM_CHECK(threadIdx.x != 0, lwm::kChkSelfTest); }
#endif

}  // namespace

#ifdef LWM_DEBUG
namespace lwm {
LWM_DEBUG_READER(api)
}  // namespace lwm
#endif

extern "C" {

const char* lwm_attn_status_string(int status) {
  switch (status) {
    case LWM_OK: return "LWM_OK";
    case LWM_ERR_INVALID_ARG: return "LWM_ERR_INVALID_ARG: null pointer or invalid argument";
    case LWM_ERR_SHAPE: return "LWM_ERR_SHAPE: inconsistent or out-of-range sizes";
    case LWM_ERR_ALIGNMENT: return "LWM_ERR_ALIGNMENT: device pointer not 16-byte aligned";
    case LWM_ERR_UNSUPPORTED: return "LWM_ERR_UNSUPPORTED: dtype / head width / block size not built";
    case LWM_ERR_WORKSPACE: return "LWM_ERR_WORKSPACE: workspace missing or too small";
    case LWM_ERR_HIP: return "LWM_ERR_HIP: kernel launch failed";
    default: return "LWM_ERR_UNKNOWN";
  }
}

int lwm_attn_version(void) { return 300; }

size_t lwm_attn_block_table_bytes(const lwm_attn_desc* d) {
  if (check_desc(d) != LWM_OK) return 0;
  return lwm::table_layout(*d).total;
}

int lwm_attn_build_block_table(const lwm_attn_desc* d, const int32_t* seg_q, const int32_t* seg_k,
                               void* table, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!table || (d->Sq > 0 && !seg_q) || (d->Sk > 0 && !seg_k)) return LWM_ERR_INVALID_ARG;
  const void* ptrs[] = {seg_q, seg_k, table};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  const TableLayout L = lwm::table_layout(*d);
  if (int64_t(d->B) * L.nqb * L.nkb >= (int64_t(1) << 39)) return LWM_ERR_SHAPE;
  return hip_status(lwm::launch_build_table(*d, seg_q, seg_k, table, static_cast<hipStream_t>(stream)));
}

int lwm_attn_fwd(const lwm_attn_desc* d, int32_t mode, const void* q, const void* k, const void* v,
                 const int32_t* seg_q, const int32_t* seg_k, const void* table, void* o, float* lse,
                 float* m, float* l, float* acc, void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  if (mode != LWM_OUT_FINAL && mode != LWM_OUT_PARTIAL) return LWM_ERR_INVALID_ARG;
  if (d->Sq == 0) return LWM_OK;
  if (!q || !seg_q || !table) return LWM_ERR_INVALID_ARG;
  if (d->Sk > 0 && (!k || !v || !seg_k)) return LWM_ERR_INVALID_ARG;
  if (mode == LWM_OUT_FINAL && (!o || !lse)) return LWM_ERR_INVALID_ARG;
  if (mode == LWM_OUT_PARTIAL && (!m || !l || !acc)) return LWM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, seg_q, seg_k, table, o, lse, m, l, acc};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d->dtype == LWM_BF16)
    e = lwm::launch_fwd_bf16(*d, mode, q, k, v, seg_q, seg_k, table, o, lse, m, l, acc, s);
  else
    e = lwm::launch_fwd_f32(*d, mode, static_cast<const float*>(q), static_cast<const float*>(k),
                            static_cast<const float*>(v), seg_q, seg_k, table,
                            static_cast<float*>(o), lse, m, l, acc, s);
  return hip_status(e);
}

size_t lwm_attn_decode_workspace_bytes(const lwm_attn_desc* d) {
  if (check_attention_desc(d) != LWM_OK || d->dtype != LWM_BF16) return 0;
  return lwm::decode_layout(*d).total;
}

int lwm_attn_decode(const lwm_attn_desc* d, const void* q, const void* k, const void* v,
                    const int32_t* seg_q, const int32_t* seg_k, const void* table, void* o,
                    float* lse, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  if (d->dtype != LWM_BF16) return LWM_ERR_UNSUPPORTED;
  if (d->Sq == 0) return LWM_OK;
  if (!q || !seg_q || !table || !o || !lse) return LWM_ERR_INVALID_ARG;
  if (d->Sk > 0 && (!k || !v || !seg_k)) return LWM_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < lwm_attn_decode_workspace_bytes(d)) return LWM_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, seg_q, seg_k, table, o, lse, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  return hip_status(lwm::launch_decode_bf16(*d, lwm::decode_layout(*d), q, k, v, seg_q, seg_k,
                                            table, o, lse, workspace,
                                            static_cast<hipStream_t>(stream)));
}

int lwm_attn_decode_noalloc(const lwm_attn_desc* d, const void* q, const void* k, const void* v,
                            const int32_t* seg_q, const int32_t* seg_k, const void* table,
                            void* o, float* lse, void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  if (d->dtype != LWM_BF16) return LWM_ERR_UNSUPPORTED;
  if (d->Sq == 0) return LWM_OK;
  if (!q || !seg_q || !table || !o || !lse) return LWM_ERR_INVALID_ARG;
  if (d->Sk > 0 && (!k || !v || !seg_k)) return LWM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, seg_q, seg_k, table, o, lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  lwm::DecodeLayout L;
  if (!lwm::decode_layout_capped(*d, lwm::kDecodeScratchBytes, &L)) return LWM_ERR_WORKSPACE;
  return hip_status(lwm::launch_decode_bf16_noalloc(*d, L, q, k, v, seg_q, seg_k, table, o, lse,
                                                    static_cast<hipStream_t>(stream)));
}

int lwm_attn_merge_chunk(int64_t rows, int32_t D, float* m, float* l, float* acc, const float* mc,
                         const float* lc, const float* accc, int32_t finalize, int32_t out_dtype,
                         void* o, float* lse, void* stream) {
  if (rows < 0 || D <= 0 || D % 4 != 0 || D > 256) return LWM_ERR_SHAPE;
  if (rows > (int64_t(1) << 40) / 64) return LWM_ERR_SHAPE;
  if (finalize != 0 && finalize != 1) return LWM_ERR_INVALID_ARG;
  if (out_dtype != LWM_BF16 && out_dtype != LWM_F32) return LWM_ERR_INVALID_ARG;
  const bool any_chunk = mc || lc || accc;
  const bool all_chunk = mc && lc && accc;
  if (any_chunk && !all_chunk) return LWM_ERR_INVALID_ARG;
  if (!all_chunk && !finalize) return LWM_ERR_INVALID_ARG;
  if (rows == 0) return LWM_OK;
  if (!m || !l || !acc) return LWM_ERR_INVALID_ARG;
  if (finalize && (!o || !lse)) return LWM_ERR_INVALID_ARG;
  const void* ptrs[] = {m, l, acc, mc, lc, accc, o, lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  return hip_status(lwm::launch_merge(rows, D, m, l, acc, mc, lc, accc, finalize, out_dtype, o,
                                      lse, static_cast<hipStream_t>(stream)));
}

int lwm_attn_rope(int32_t B, int32_t H, int32_t S, int32_t D, int32_t dtype, int64_t pos_offset,
                  double theta, int32_t inverse, const void* x, void* out, void* stream) {
  if (dtype != LWM_BF16 && dtype != LWM_F32) return LWM_ERR_INVALID_ARG;
  if (inverse != 0 && inverse != 1) return LWM_ERR_INVALID_ARG;
  if (!(theta > 1.0) || theta == std::numeric_limits<double>::infinity()) return LWM_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || S < 0 || pos_offset < 0) return LWM_ERR_SHAPE;
  if (!(D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256)) return LWM_ERR_UNSUPPORTED;
  if (pos_offset + int64_t(S) > (int64_t(1) << 32)) return LWM_ERR_SHAPE;
  const int64_t rows = int64_t(B) * H * S;
  if (rows > (int64_t(1) << 40) / D) return LWM_ERR_SHAPE;
  if (rows == 0) return LWM_OK;
  if (!x || !out) return LWM_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out)) return LWM_ERR_ALIGNMENT;
  // in place or disjoint; a partial overlap would let threads overwrite rows others read
  const size_t bytes = size_t(rows) * D * (dtype == LWM_BF16 ? 2 : 4);
  const char* xa = static_cast<const char*>(x);
  const char* oa = static_cast<const char*>(out);
  if (xa != oa && xa < oa + bytes && oa < xa + bytes) return LWM_ERR_INVALID_ARG;
  return hip_status(lwm::launch_rope(B, H, S, D, dtype, pos_offset, theta, inverse, x, out,
                                     static_cast<hipStream_t>(stream)));
}

// RoPE at load: bf16 with D = 128 only, theta > 1 and finite, positions below 2^32.
static int check_rope(const lwm_attn_desc* d, double theta) {
  if (!(theta > 1.0) || theta == std::numeric_limits<double>::infinity()) return LWM_ERR_INVALID_ARG;
  if (d->dtype != LWM_BF16 || d->D != 128) return LWM_ERR_UNSUPPORTED;
  if (d->q_offset + int64_t(d->Sq) > (int64_t(1) << 32) || d->k_offset + int64_t(d->Sk) > (int64_t(1) << 32))
    return LWM_ERR_SHAPE;
  return LWM_OK;
}

int lwm_attn_fwd_rope(const lwm_attn_desc* d, int32_t mode, double theta, const void* q,
                      const void* k_rot, const void* v, const int32_t* seg_q, const int32_t* seg_k,
                      const void* table, void* o, float* lse, float* m, float* l, float* acc,
                      void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  rc = check_rope(d, theta);
  if (rc) return rc;
  if (mode != LWM_OUT_FINAL && mode != LWM_OUT_PARTIAL) return LWM_ERR_INVALID_ARG;
  if (d->Sq == 0) return LWM_OK;
  if (!q || !seg_q || !table) return LWM_ERR_INVALID_ARG;
  if (d->Sk > 0 && (!k_rot || !v || !seg_k)) return LWM_ERR_INVALID_ARG;
  if (mode == LWM_OUT_FINAL && (!o || !lse)) return LWM_ERR_INVALID_ARG;
  if (mode == LWM_OUT_PARTIAL && (!m || !l || !acc)) return LWM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k_rot, v, seg_q, seg_k, table, o, lse, m, l, acc};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  return hip_status(lwm::launch_fwd_rope_bf16(*d, mode, theta, q, k_rot, v, seg_q, seg_k, table, o,
                                              lse, m, l, acc, static_cast<hipStream_t>(stream)));
}

static int check_packed_loss(int32_t B, int32_t T, int32_t V, int32_t nseg) {
  if (B < 0 || T < 0 || nseg < 1) return LWM_ERR_SHAPE;
  if (V < 8 || V % 8 != 0 || V > 131072) return LWM_ERR_UNSUPPORTED;
  if (int64_t(B) * T >= (int64_t(1) << 31)) return LWM_ERR_SHAPE;  // one workgroup per token
  if (int64_t(B) * nseg > (int64_t(1) << 31) / 4) return LWM_ERR_SHAPE;
  if (int64_t(B) * T * V > (int64_t(1) << 42)) return LWM_ERR_SHAPE;
  return LWM_OK;
}

size_t lwm_attn_packed_loss_workspace_bytes(int32_t B, int32_t T, int32_t V, int32_t num_segments) {
  if (check_packed_loss(B, T, V, num_segments) != LWM_OK) return 0;
  return lwm::packed_loss_layout(B, T, num_segments).total;
}

int lwm_attn_packed_loss(int32_t B, int32_t T, int32_t V, int32_t num_segments, int32_t dtype,
                         const void* logits, const int32_t* targets, const int32_t* seg,
                         float grad_scale, float* loss, float* token_loss, void* dlogits,
                         void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_packed_loss(B, T, V, num_segments);
  if (rc) return rc;
  if (dtype != LWM_BF16 && dtype != LWM_F32) return LWM_ERR_INVALID_ARG;
  if (dtype == LWM_F32 && V > 65536) return LWM_ERR_UNSUPPORTED;
  if (!std::isfinite(grad_scale)) return LWM_ERR_INVALID_ARG;
  if (!loss) return LWM_ERR_INVALID_ARG;
  const bool any = int64_t(B) * T > 0;
  if (any && (!logits || !targets || !seg)) return LWM_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < lwm_attn_packed_loss_workspace_bytes(B, T, V, num_segments))
    return LWM_ERR_WORKSPACE;
  const void* ptrs[] = {logits, targets, seg, loss, token_loss, dlogits, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  return hip_status(lwm::launch_packed_loss(lwm::packed_loss_layout(B, T, num_segments), B, T, V,
                                            num_segments, dtype, logits, targets, seg, grad_scale,
                                            loss, token_loss, dlogits, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t lwm_attn_bwd_workspace_bytes(const lwm_attn_desc* d) {
  if (check_desc(d) != LWM_OK) return 0;
  // Delta and LSE * log2(e), one float32 per query row each
  return 2 * lwm::align256(size_t(d->B) * d->H * d->Sq * sizeof(float));
}

static int bwd_impl(const lwm_attn_desc* d, int phase, const void* q, const void* k,
                    const void* v, const void* o, const void* dO, const float* lse,
                    const int32_t* seg_q, const int32_t* seg_k, const void* table, void* dq,
                    void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  if (phase < -1 || phase > LWM_BWD_DKV) return LWM_ERR_INVALID_ARG;
  if (d->Sq == 0 && d->Sk == 0) return LWM_OK;
  if (!table) return LWM_ERR_INVALID_ARG;
  if (d->Sq > 0 && (!q || !o || !dO || !lse || !seg_q || !dq)) return LWM_ERR_INVALID_ARG;
  if (d->Sk > 0 && (!k || !v || !seg_k || !dk || !dv)) return LWM_ERR_INVALID_ARG;
  const size_t need = lwm_attn_bwd_workspace_bytes(d);
  if (need > 0 && (!workspace || ws_bytes < need)) return LWM_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LWM_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  if (d->Sq == 0 || d->Sk == 0) {
    // no pairs: every gradient is zero (row bytes D*esz are a multiple of 16 for every
    // supported D)
    const size_t esz = d->dtype == LWM_BF16 ? 2 : 4;
    hipError_t e = hipSuccess;
    if (d->Sq > 0 && (phase < 0 || phase == LWM_BWD_DQ))
      e = lwm::launch_zero(dq, size_t(d->B) * d->H * d->Sq * d->D * esz, s);
    if (e == hipSuccess && d->Sk > 0 && (phase < 0 || phase == LWM_BWD_DKV)) {
      e = lwm::launch_zero(dk, size_t(d->B) * d->H * d->Sk * d->D * esz, s);
      if (e == hipSuccess) e = lwm::launch_zero(dv, size_t(d->B) * d->H * d->Sk * d->D * esz, s);
    }
    return hip_status(e);
  }
  hipError_t e;
  if (d->dtype == LWM_BF16)
    e = lwm::launch_bwd_bf16(*d, phase, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv,
                             delta, s);
  else
    e = lwm::launch_bwd_f32(*d, phase, static_cast<const float*>(q), static_cast<const float*>(k),
                            static_cast<const float*>(v), static_cast<const float*>(o),
                            static_cast<const float*>(dO), lse, seg_q, seg_k, table,
                            static_cast<float*>(dq), static_cast<float*>(dk),
                            static_cast<float*>(dv), delta, s);
  return hip_status(e);
}

int lwm_attn_bwd(const lwm_attn_desc* d, const void* q, const void* k, const void* v,
                 const void* o, const void* dO, const float* lse, const int32_t* seg_q,
                 const int32_t* seg_k, const void* table, void* dq, void* dk, void* dv,
                 void* workspace, size_t ws_bytes, void* stream) {
  return bwd_impl(d, -1, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, workspace,
                  ws_bytes, stream);
}

int lwm_attn_bwd_rope(const lwm_attn_desc* d, double theta, const void* q, const void* q_rot,
                      const void* k, const void* k_rot, const void* v, const void* o,
                      const void* dO, const float* lse, const int32_t* seg_q, const int32_t* seg_k,
                      const void* table, void* dq, void* dk, void* dv, void* workspace,
                      size_t ws_bytes, void* stream) {
  int rc = check_attention_desc(d);
  if (rc) return rc;
  rc = check_rope(d, theta);
  if (rc) return rc;
  if (d->Sq == 0 || d->Sk == 0)  // no pairs: zero gradients, as without RoPE
    return bwd_impl(d, -1, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, workspace,
                    ws_bytes, stream);
  if (!table || !q || !q_rot || !o || !dO || !lse || !seg_q || !dq) return LWM_ERR_INVALID_ARG;
  if (!k || !k_rot || !v || !seg_k || !dk || !dv) return LWM_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < lwm_attn_bwd_workspace_bytes(d)) return LWM_ERR_WORKSPACE;
  const void* ptrs[] = {q, q_rot, k, k_rot, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LWM_ERR_ALIGNMENT;
  return hip_status(lwm::launch_bwd_rope_bf16(*d, theta, q, q_rot, k, k_rot, v, o, dO, lse, seg_q,
                                              seg_k, table, dq, dk, dv,
                                              static_cast<float*>(workspace),
                                              static_cast<hipStream_t>(stream)));
}

int lwm_attn_bwd_phase(const lwm_attn_desc* d, int32_t phase, const void* q, const void* k,
                       const void* v, const void* o, const void* dO, const float* lse,
                       const int32_t* seg_q, const int32_t* seg_k, const void* table, void* dq,
                       void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream) {
  if (phase < 0) return LWM_ERR_INVALID_ARG;
  return bwd_impl(d, phase, q, k, v, o, dO, lse, seg_q, seg_k, table, dq, dk, dv, workspace,
                  ws_bytes, stream);
}

int lwm_attn_debug_status(uint32_t* words, int32_t flags) {
  if (words == nullptr || (flags & ~LWM_DEBUG_SELF_TEST) != 0) return LWM_ERR_INVALID_ARG;
  words[0] = words[1] = 0;
#ifdef LWM_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return LWM_ERR_HIP;
  if (flags & LWM_DEBUG_SELF_TEST) {
    debug_self_test_kernel<<<1, 64>>>();
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return LWM_ERR_HIP;
  }
  hipError_t (*const readers[])(unsigned*) = {lwm::debug_read_attn_bf16, lwm::debug_read_attn_f32,
                                               lwm::debug_read_table, lwm::debug_read_merge,
                                               lwm::debug_read_api};
  for (auto rd : readers) {
    unsigned w[2] = {0u, 0u};
    if (rd(w) != hipSuccess) return LWM_ERR_HIP;
    words[0] |= w[0];
    if (words[1] == 0) words[1] = w[1];
  }
  return LWM_OK;
#else
  return LWM_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
