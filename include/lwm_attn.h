/*
 * lwm_attn.h -- C-ABI of the MI355X (gfx950) exact blockwise causal attention library.
 *
 * What the calls compute.  Exact softmax attention, not windowed and not sparse, over a
 * sequence that may hold several packed samples.  The LWM pages state the three parts:
 *   - exact full attention at million-token length, evaluated block by block with
 *     key/value blocks arriving from a device ring: LWM deep dive, section
 *     "RingAttention 为什么必要" (why RingAttention is necessary);
 *   - a causal next-token model over one unified token sequence: same page, sections
 *     "核心问题" (core problem) and "模型结构" (model structure, "Training objective");
 *   - packed samples that only attend to themselves: same page, section
 *     "Masked sequence packing", first step of the LWM recipe.
 * The pages give no formula; the library uses the textbook reading.  For query row i
 * (global position q_offset + i) and key j (global position k_offset + j):
 *   visible(i,j) = seg_q[i] >= 0 && seg_q[i] == seg_k[j] && (!causal || k_offset+j <= q_offset+i)
 *   s_ij = scale * <q_i, k_j>,   P_i = softmax over visible j,   O_i = sum_j P_ij v_j,
 *   LSE_i = max_j s_ij + ln(sum_j exp(s_ij - max_j s_ij))   (natural log)
 * A row with no visible key has O = 0 and LSE = -inf.
 *
 * Conventions for every call:
 *   - Tensors are dense and contiguous: Q, O, dO, dQ are [B,H,Sq,D]; K, V, dK, dV are
 *     [B,H,Sk,D]; D is innermost.  LSE, m, l are float32 [B,H,Sq]; the partial
 *     accumulator is float32 [B,H,Sq,D].  Segment ids are int32 [B,Sq] / [B,Sk], shared by
 *     all heads.  A negative segment id marks padding: it sees nothing and nothing sees it.
 *   - Every pointer is a device pointer owned by the caller; the library never allocates,
 *     frees or synchronises (lwm_attn_debug_status, a test aid, synchronises).  Its only
 *     mutable global state is the static device buffer of lwm_attn_decode_noalloc (one per
 *     GPU), and in the debug build the device-check records.  `stream` is a hipStream_t
 *     (NULL = the null stream); every other call only enqueues work on it and returns.
 *   - Device pointers must be 16-byte aligned.  All arguments are validated on the host
 *     before anything is enqueued; on error nothing is enqueued.
 *   - Return value: LWM_OK (0) or a negative LWM_ERR_* code; lwm_attn_status_string()
 *     names it.  LWM_ERR_HIP reports a failed kernel launch (hipGetLastError).
 *   - NaN or Inf in the inputs is propagated, not checked.
 */
#ifndef LWM_ATTN_H
#define LWM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LWM_BF16 = 0, LWM_F32 = 1 } lwm_dtype;

/* FINAL writes the normalised output O and LSE.  PARTIAL writes the unnormalised state
 * (m, l, acc) of the keys given, for later merging with lwm_attn_merge_chunk. */
typedef enum { LWM_OUT_FINAL = 0, LWM_OUT_PARTIAL = 1 } lwm_out_mode;

enum {
  LWM_OK = 0,
  LWM_ERR_INVALID_ARG = -1, /* NULL pointer, bad enum, negative size, bad block size   */
  LWM_ERR_SHAPE = -2,       /* inconsistent or overflowing sizes                        */
  LWM_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned                   */
  LWM_ERR_UNSUPPORTED = -4, /* dtype / head width / block size combination not built     */
  LWM_ERR_WORKSPACE = -5,   /* workspace missing or smaller than the size query returns */
  LWM_ERR_HIP = -6          /* a kernel launch failed                                    */
};

/* Tile classes stored in the block table. */
enum { LWM_TILE_SKIP = 0, LWM_TILE_PARTIAL = 1, LWM_TILE_FULL = 2 };

typedef struct {
  int32_t B, H, Sq, Sk, D; /* Q [B,H,Sq,D]; K,V [B,H,Sk,D]                               */
  int64_t q_offset;        /* global position of query row 0 (ring share); else 0       */
  int64_t k_offset;        /* global position of key row 0 (ring share); else 0         */
  float scale;             /* score scale, e.g. 1/sqrt(D)                                */
  int32_t causal;          /* 1: key visible only if its global position <= the query's */
  int32_t block_q;         /* query rows per table block (the query-chunk size knob)   */
  int32_t block_k;         /* keys per table block                                      */
  int32_t dtype;           /* lwm_dtype of Q, K, V, O, dO, dQ, dK, dV                    */
} lwm_attn_desc;

/*
 * Block table.  Classifies each (query block, key block) pair so the kernels can skip
 * pairs with no visible key and drop masking where every pair is visible; it is how the
 * causal and packing masks of the pages become skipped work.  The two masks: a packed
 * sample only attends to itself (LWM deep dive, section "Masked sequence packing", first
 * step of the recipe) and the model predicts the next token of one sequence (sections
 * "核心问题" and "模型结构"); the block sizes are the query-chunk knob of the pages' blockwise
 * attention (0539edu article, section "模型训练关键参数配置": scan_query_chunk_size).
 *   status  uint8 [B][nqb][nkb]: LWM_TILE_SKIP if no pair can be visible (causally empty,
 *           all padding, or disjoint segment-id intervals), LWM_TILE_FULL if the block lies
 *           inside [0,Sq)x[0,Sk) and every pair is visible, else LWM_TILE_PARTIAL.
 *           SKIP is exact when segment ids are non-decreasing along the sequence (what
 *           packing produces) and conservative (never wrong) for any ids.
 *   q_range int32 [B][nqb][2]: first and last non-SKIP key block of each query block
 *           (first > last when there is none).
 *   k_range int32 [B][nkb][2]: first and last non-SKIP query block of each key block.
 * with nqb = ceil(Sq/block_q), nkb = ceil(Sk/block_k).  Buffer layout: q_range, then
 * k_range, then status, then per-block segment statistics the builder uses internally,
 * each part starting on a 256-byte boundary; lwm_attn_block_table_bytes gives the total.
 * block_q and block_k must each be 16, 32 or 64; the attention kernels need 64 x 64.
 * The table depends on desc (B, Sq, Sk, offsets, causal, blocks) and the segment ids only.
 */
size_t lwm_attn_block_table_bytes(const lwm_attn_desc* desc);
int lwm_attn_build_block_table(const lwm_attn_desc* desc, const int32_t* seg_q,
                               const int32_t* seg_k, void* table, void* stream);

/*
 * Forward attention of Q against the keys K, V given (one KV chunk or the whole sequence).
 * This is one query block's pass over streamed key/value blocks of the pages' blockwise
 * (ring) attention, with a running max, denominator and accumulator per query row.
 *   mode FINAL:   o [B,H,Sq,D] (desc dtype) and lse float32 [B,H,Sq]; m, l, acc unused.
 *   mode PARTIAL: m, l float32 [B,H,Sq] and acc float32 [B,H,Sq,D] such that
 *                 l = sum_j exp(s_ij - m), acc = sum_j exp(s_ij - m) v_j over the visible
 *                 keys given; a row with none gets (m, l, acc) = (-inf, 0, 0).
 *                 m is finite whenever l > 0 but need not equal max_j s_ij; o, lse unused.
 * Supported: dtype LWM_BF16 with D = 128 (bf16 MFMA, float32 accumulation) and
 * LWM_F32 with D in {32, 64}; table built with block_q = block_k = 64.
 */
int lwm_attn_fwd(const lwm_attn_desc* desc, int32_t mode, const void* q, const void* k,
                 const void* v, const int32_t* seg_q, const int32_t* seg_k, const void* table,
                 void* o, float* lse, float* m, float* l, float* acc, void* stream);

/*
 * Merge a chunk's partial state into a running state (the ring step's combine; LWM deep
 * dive, section "RingAttention 为什么必要": each device keeps its query block while key/value
 * blocks arrive round the ring, and the result is exact full attention): per row
 *   m' = max(m, mc),  l' = l e^(m-m') + lc e^(mc-m'),  acc' = acc e^(m-m') + accc e^(mc-m').
 * An empty side (l = 0) contributes nothing; two empty sides stay empty (-inf, 0, 0).
 * rows = B*H*Sq; m, l, mc, lc are float32 [rows]; acc, accc float32 [rows, D].
 *   finalize = 0: the merged state is written back to m, l, acc; o and lse are unused.
 *   finalize = 1: o [rows, D] (out_dtype) = acc'/l' and lse [rows] = m' + ln l' are
 *                 written and m, l, acc are left unchanged.  mc, lc, accc may all be NULL
 *                 to finalize the running state alone.
 * D must be a multiple of 4 and at most 256.
 */
int lwm_attn_merge_chunk(int64_t rows, int32_t D, float* m, float* l, float* acc,
                         const float* mc, const float* lc, const float* accc, int32_t finalize,
                         int32_t out_dtype, void* o, float* lse, void* stream);

/*
 * Decode: the FINAL forward for a few query rows (new tokens) against a long key/value
 * cache, the inference side of the pages' million-token model (deep dive, section
 * "RingAttention 为什么必要": 1M-token inference needs a v4-128 slice; section "局限与风险":
 * inference cost).  Same result as lwm_attn_fwd(FINAL) on the same arguments, up to the
 * order of float32 rounding; what differs is how the work is spread: the key tiles are cut
 * into slices, every (query tile, head, slice) is one workgroup writing a partial state
 * (m, l, acc) into the workspace, and one combine pass merges the slices exactly and
 * normalises.  So few rows (Sq = 1 .. 128 per head) still fill the GPU and stream the cache
 * at memory bandwidth; any Sq is accepted.  For new tokens at the end of a cache of Sk keys,
 * pass causal = 1 and q_offset = k_offset + Sk - Sq.
 *   o [B,H,Sq,D] bf16 and lse float32 [B,H,Sq] as for lwm_attn_fwd FINAL.
 *   workspace: device memory of at least lwm_attn_decode_workspace_bytes(desc) bytes, owned
 *   by the caller, contents on entry irrelevant (about nsplit * B*H*Sq * (D+2) * 4 bytes; a
 *   few MiB for one token per head against a 1M-token cache).
 * Supported: dtype LWM_BF16 with D = 128 (LWM_ERR_UNSUPPORTED otherwise), table built with
 * block_q = block_k = 64.  The workspace size query returns 0 for a desc that is invalid or
 * not supported.
 */
size_t lwm_attn_decode_workspace_bytes(const lwm_attn_desc* desc);
int lwm_attn_decode(const lwm_attn_desc* desc, const void* q, const void* k, const void* v,
                    const int32_t* seg_q, const int32_t* seg_k, const void* table, void* o,
                    float* lse, void* workspace, size_t ws_bytes, void* stream);

/*
 * lwm_attn_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The slice states go to a static device buffer of the library instead,
 * LWM_DECODE_SCRATCH_BYTES per GPU, one copy on each GPU the library runs on, held until the
 * process ends; the call itself allocates nothing.  When the default split would need more
 * than the buffer holds, fewer and longer key slices are used (same result up to the order
 * of float32 rounding).  A request whose states do not fit even with one slice per query
 * row, i.e. B*H*Sq*(D+2)*4 bytes beyond the buffer (B*H*Sq above about 129000 rows at
 * D = 128), returns LWM_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU share
 * its buffer: calls that overlap on one GPU (two streams or two threads) race and must be
 * serialised by the caller.  Other arguments, results and errors as lwm_attn_decode.
 */
#define LWM_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
int lwm_attn_decode_noalloc(const lwm_attn_desc* desc, const void* q, const void* k,
                            const void* v, const int32_t* seg_q, const int32_t* seg_k,
                            const void* table, void* o, float* lse, void* stream);

/*
 * Backward of the forward above for an upstream gradient dO, recomputing P from the saved
 * LSE (P_ij = exp(s_ij - LSE_i) on visible pairs).  The pages train the model through this
 * attention at every context stage (LWM deep dive, sections "大模型训练路线图" and "Stage I：长上下文语言模型",
 * Tables 11 and 13) but print no gradient; these are the textbook derivatives of the
 * definition above:
 *   Delta_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - Delta_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
 * sums running over the keys given and the queries given.  o and lse are the forward's
 * outputs for the same rows (for a ring share: the outputs after all chunks were merged,
 * and dq is then this chunk's contribution).  dq, dk, dv are written (not accumulated).
 * workspace: device memory of at least lwm_attn_bwd_workspace_bytes(desc) bytes, owned by
 * the caller; its contents on entry do not matter.
 * Supported combinations are those of lwm_attn_fwd.
 */
size_t lwm_attn_bwd_workspace_bytes(const lwm_attn_desc* desc);
int lwm_attn_bwd(const lwm_attn_desc* desc, const void* q, const void* k, const void* v,
                 const void* o, const void* dO, const float* lse, const int32_t* seg_q,
                 const int32_t* seg_k, const void* table, void* dq, void* dk, void* dv,
                 void* workspace, size_t ws_bytes, void* stream);

/*
 * One phase of lwm_attn_bwd, same arguments and buffers.  The phases in order:
 *   LWM_BWD_DELTA  Delta = rowsum(dO * O) into the workspace (its own layout);
 *   LWM_BWD_DQ     dq from Delta (query-major pass over key tiles);
 *   LWM_BWD_DKV    dk, dv from Delta (key-major pass over query tiles).
 * DQ and DKV read the workspace DELTA wrote and are independent of each other, so a caller
 * may run them on two streams once DELTA has completed.  lwm_attn_bwd runs all three on
 * one stream.  For Sq == 0 or Sk == 0 the DQ / DKV phases zero their outputs.
 */
enum { LWM_BWD_DELTA = 0, LWM_BWD_DQ = 1, LWM_BWD_DKV = 2 };
int lwm_attn_bwd_phase(const lwm_attn_desc* desc, int32_t phase, const void* q, const void* k,
                       const void* v, const void* o, const void* dO, const float* lse,
                       const int32_t* seg_q, const int32_t* seg_k, const void* table, void* dq,
                       void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream);

/*
 * Rotary position embedding (RoPE) with a large base theta, the step before Q K^T in every
 * layer of the LWM model: the pages extend the context by enlarging theta (deep dive, section
 * "Stage I：长上下文语言模型" and Tables 11 and 13: 1M at 32K tokens, 10M at 128K and 256K, 25M at
 * 512K, 50M at 1M).  The pages give no formula; the textbook rotary embedding is used: pair
 * i = (x[2i], x[2i+1]) of the row of the token at position p turns by the angle
 * p * theta^(-2i/D):
 *   out[2i]   = x[2i] cos(a) - x[2i+1] sin(a),   out[2i+1] = x[2i] sin(a) + x[2i+1] cos(a).
 * inverse = 1 turns by -a instead (the transpose: it carries dQ, dK of the rotated vectors
 * back to the unrotated ones).  x and out are [B,H,S,D] (dtype LWM_BF16 or LWM_F32), row s
 * at position pos_offset + s; use the attention desc's q_offset / k_offset so positions are
 * global.  out may be x itself (in place) or a disjoint buffer.
 * Angles are reduced to a fraction of a turn in float64 before float32 sin/cos, so the
 * angle error stays below 1e-6 radian at every position; bf16 results are rounded to
 * nearest even.  Requires D in {8, 16, 32, 64, 128, 256}, theta > 1 and finite,
 * pos_offset >= 0, pos_offset + S <= 2^32.  B*H*S = 0 does nothing.
 */
int lwm_attn_rope(int32_t B, int32_t H, int32_t S, int32_t D, int32_t dtype, int64_t pos_offset,
                  double theta, int32_t inverse, const void* x, void* out, void* stream);

/*
 * Attention with RoPE applied inside the tile loop's register load, for the step before
 * Q K^T of every layer of the LWM model (deep dive, section "Stage I：长上下文语言模型" and
 * Tables 11 and 13: RoPE with a base theta grown from 1M to 50M as the context grows).  The
 * operand a kernel keeps in registers arrives unrotated and is turned at load by global
 * position; the operand it streams arrives turned already, from lwm_attn_rope with the same
 * theta and positions (q_offset / k_offset of desc).  The turn at load computes exactly what
 * lwm_attn_rope computes for the same element, so the result equals lwm_attn_fwd /
 * lwm_attn_bwd on turned inputs.
 *   lwm_attn_fwd_rope: q unrotated, k_rot = lwm_attn_rope(k, k_offset, theta); otherwise as
 *     lwm_attn_fwd (both modes).
 *   lwm_attn_bwd_rope: q and k unrotated, q_rot and k_rot turned; o and lse from the forward.
 *     dq and dk are the gradients of the unrotated q and k (the gradients of the turned ones,
 *     turned back in float32 before rounding), dv as lwm_attn_bwd.  Workspace as lwm_attn_bwd.
 * Supported: dtype LWM_BF16 with D = 128 (else LWM_ERR_UNSUPPORTED); theta > 1 and finite
 * (else LWM_ERR_INVALID_ARG); q_offset + Sq and k_offset + Sk at most 2^32 (else
 * LWM_ERR_SHAPE).  Over a training step this replaces six streaming RoPE passes (Q and K
 * before the forward and again before the backward, dQ and dK after it) by three (K before
 * the forward, Q and K before the backward).
 */
int lwm_attn_fwd_rope(const lwm_attn_desc* desc, int32_t mode, double theta, const void* q,
                      const void* k_rot, const void* v, const int32_t* seg_q,
                      const int32_t* seg_k, const void* table, void* o, float* lse, float* m,
                      float* l, float* acc, void* stream);
int lwm_attn_bwd_rope(const lwm_attn_desc* desc, double theta, const void* q, const void* q_rot,
                      const void* k, const void* k_rot, const void* v, const void* o,
                      const void* dO, const float* lse, const int32_t* seg_q,
                      const int32_t* seg_k, const void* table, void* dq, void* dk, void* dv,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * Packed-sequence loss reweighting, the step after attention in the packed path: the LWM
 * pages reweight the loss of a packed sequence so that it equals training its samples
 * unpacked with padding, so that samples with many tokens (long videos) do not outweigh
 * samples with few loss tokens (short answers) (deep dive, section "Masked sequence
 * packing", second step of the recipe; abstract page, contribution (b)).  The pages give no
 * formula; the reading: unpacked training averages over each sample's loss tokens, then
 * over samples.  So with n_s the loss tokens of sample s and N the samples (over the whole
 * batch) that have any, a loss token t of sample s has weight w_t = 1 / (N n_s), and
 *   l_t = logsumexp(x_t) - x_t[y_t],    loss = sum_t w_t l_t,
 *   dlogits_t = grad_scale * w_t * (softmax(x_t) - onehot(y_t)).
 *   logits   [B,T,V] (dtype LWM_BF16 or LWM_F32), the next-token logits of each position;
 *   targets  int32 [B,T]: the target token, or negative for a position with no loss;
 *   seg      int32 [B,T]: the sample (segment id) of each position within its batch row, the
 *            same ids the attention mask uses; negative for padding.  Ids must be below
 *            num_segments; a sample is (batch row, id), ids need not be contiguous runs.
 *            A loss token has seg in [0, num_segments) and target in [0, V); positions whose
 *            target is outside [0, V) count as positions with no loss.
 *   loss     float32 device scalar (written); 0 when there is no loss token.
 *   token_loss float32 [B,T] or NULL: l_t for every position with a target in [0, V)
 *            (also padding ones, which have weight 0), 0 elsewhere.
 *   dlogits  [B,T,V] in the logits' dtype or NULL (loss only); rows with weight 0 are zero.
 *   workspace  at least lwm_attn_packed_loss_workspace_bytes(B, T, V, num_segments) bytes;
 *            contents on entry irrelevant.
 * The loss is summed in a fixed order: repeated calls give identical bits.  Requires V a
 * multiple of 8 in [8, 131072] (float32 logits: V <= 65536, else LWM_ERR_UNSUPPORTED),
 * num_segments >= 1, B*T < 2^31; grad_scale finite.
 */
size_t lwm_attn_packed_loss_workspace_bytes(int32_t B, int32_t T, int32_t V, int32_t num_segments);
int lwm_attn_packed_loss(int32_t B, int32_t T, int32_t V, int32_t num_segments, int32_t dtype,
                         const void* logits, const int32_t* targets, const int32_t* seg,
                         float grad_scale, float* loss, float* token_loss, void* dlogits,
                         void* workspace, size_t ws_bytes, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* lwm_attn_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int lwm_attn_version(void);

/* Device checks of a debug build (the library compiled with LWM_DEBUG, built beside the
 * normal one as liblwm_attn_debug.so).  No passage of the pages defines it: it is for tests
 * and for callers chasing a wrong table or launch.  In such a build every kernel checks the
 * indices it derives from the block table (query and key ranges, tile statuses, status-chunk
 * slots) and from its launch shape against the extents it indexes, and the merge checks that
 * an empty state carries l = 0; a failed check does not trap, it is recorded on the device.
 *   words  host uint32_t[2], written: words[0] has bit c set for every failed check code c
 *          since the last call (codes 1-18, listed in the library's sources; 31 is the self
 *          test), words[1] = code << 24 | workgroup of the first failure, or 0.
 *   flags  0, or LWM_DEBUG_SELF_TEST to fail check 31 once on purpose before reading.
 * Synchronises the current device, then reads and clears the records.  Returns
 * LWM_ERR_UNSUPPORTED (words zeroed) in a library built without LWM_DEBUG, LWM_ERR_INVALID_ARG
 * for a NULL words or unknown flags, LWM_ERR_HIP if the synchronisation or a copy fails. */
#define LWM_DEBUG_SELF_TEST 1
int lwm_attn_debug_status(uint32_t* words, int32_t flags);

#ifdef __cplusplus
}
#endif

#endif /* LWM_ATTN_H */
