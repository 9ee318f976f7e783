/*
 * tl.h — C ABI of the MI355X (gfx950) looped-transformer runtime.
 *
 * The model is  embed -> pre blocks -> one shared loop block (or a stack of
 * n_loop layers) applied L times -> post blocks -> final RMSNorm -> head
 * ("Benchmark Comparison / vs generic runtimes" page, section "Where Generic
 * Runtimes Lose On Looped Checkpoints").  L is an argument of every call, never
 * a property of the weights ("Dynamic-L Inference" page, "The Core Idea").
 *
 * Conventions shared by every entry point
 *   - Pointers named *_dev are device pointers (HIP device memory); *_host are
 *     host pointers.  The caller owns every pointer it passes; the library never
 *     frees them and keeps none of them after the call returns.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls enqueue device work
 *     on it and return without waiting; device outputs are valid once the stream
 *     has reached that point.  Host outputs are written before the call returns.
 *     Calls of one model may use different streams: a call on a stream other than
 *     the previous call's first makes its stream wait for the work the previous
 *     call enqueued (the model's staging area and workspaces are shared), so the
 *     previous call's stream must not have been destroyed.
 *   - On any status other than TL_OK nothing has been enqueued and the model and
 *     its lanes are unchanged (validation happens before any device work), except
 *     TL_E_HIP, which reports a failed HIP call; tl_last_error() gives the reason.
 *   - A model is used by one host thread at a time.
 *   - There are no silent fallbacks: an unsupported shape or dtype is an error.
 *   - Environment variable TL_LOG_LEVEL (read once; stderr only; the pages' CLI
 *     has a log-level variable of the same range, "CLI Reference" page,
 *     Environment Variables): 0 or unset silent, 1 prints the reason of every
 *     failing call, 2 also one line per load and per forward or decode call;
 *     any other value counts as 1.  It never changes what a call computes.
 */
#ifndef TL_H
#define TL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TL_ABI_VERSION 1

typedef enum {
  TL_OK = 0,
  TL_E_ARG = -1,          /* an argument is out of range or a required pointer is NULL */
  TL_E_OOM = -2,          /* the allocator returned NULL; model state unchanged */
  TL_E_HIP = -3,          /* a HIP runtime call failed */
  TL_E_STATE = -4,        /* lane state does not allow the call (never prefilled, full) */
  TL_E_UNSUPPORTED = -5   /* shape, dtype or device not supported (not gfx950) */
} tl_status;

typedef enum {
  TL_DT_F32 = 0,
  TL_DT_F16 = 1,
  TL_DT_BF16 = 2,
  /* Symmetric INT4, one fp16 scale per 128 consecutive input features of an
   * output row: s = fp16(max|w| / 7) (division in fp32), q = clamp(rint(w / s),
   * -7, 7) with ties to even, w ~ q * s.  Min-max without calibration ("Benchmark
   * Comparison" page, section 7); groups of 128 along K ("Benchmark Comparison"
   * page, section 5: 16 groups at K = 2048).  Only for loop blocks, with
   * F16 operands. */
  TL_DT_W4G128 = 3
} tl_dtype;

/* Device memory provider.  alloc returns device memory of at least `bytes`
 * (256-byte aligned) or NULL; dealloc releases it.  Passing NULL for both makes
 * the library use hipMalloc/hipFree. */
typedef void* (*tl_alloc_fn)(size_t bytes, void* user);
typedef void (*tl_dealloc_fn)(void* ptr, void* user);

typedef struct {
  int32_t vocab, d_model, n_heads, head_dim, ffn;
  int32_t n_pre, n_loop, n_post;   /* n_loop = layers in the shared loop stack (>= 1) */
  float rms_eps;                   /* RMSNorm epsilon */
  float rope_base;                 /* rotary base, e.g. 10000 */
  int32_t act_dtype;               /* GEMM operands, activations and KV cache: F32, F16 or BF16 */
  /* Storage type of the weights the caller passes.  Each must equal act_dtype,
   * except BF16 weights with F16 operands (converted once at load, exact for
   * |w| >= 2^-14; the embedding table is read in its stored type), W4G128 loop
   * blocks with F16 operands, and F16 / BF16 weights (all of them) with F32
   * activations: the weights are kept as fp16 (bf16 converted as above), and each
   * product runs on fp16 matrix cores with every fp32 operand x split into
   * x_hi = fp16(x) and x_lo = fp16(x - x_hi), two passes per weight fragment
   * (about 22 significant bits of x); activations, attention and the KV cache are
   * fp32 (K/V cache mode only). */
  int32_t boundary_dtype;          /* embed, head, pre and post blocks: F32, F16 or BF16 */
  int32_t loop_dtype;              /* loop blocks: F32, F16, BF16 or W4G128 */
  /* W4G128 only: 1 = dequantise the loop block once at load to fp16(q * s) and run
   * it as an F16 block (the "FP16 body" of the "CLI Reference" page, environment
   * variable TINYLOOP_EXPERIMENTAL_FP16_BODY). */
  int32_t loop_fp16_body;
  int32_t max_lanes;               /* lanes that can keep a KV cache between calls */
  int32_t max_L;                   /* largest loop count accepted */
  int32_t max_pos;                 /* positions 0 .. max_pos-1 are valid */
  uint64_t kv_arena_bytes;         /* device bytes reserved for lane KV caches (0 = none) */
  /* What a lane's cache slot keeps per position, one of tl_kv_mode (iteration-axis
   * KV compression: "CLI Reference" page, environment variables TINYLOOP_KV_H_MODE
   * with TINYLOOP_KV_INT8 / TINYLOOP_KV_INT4). */
  int32_t kv_mode;
  /* 1: every row's results are independent of which other rows share its passes
   * (bit for bit): the split of each product's K is chosen from its N and K only,
   * one GEMM kernel family runs at every batch size (no few-row GEMVs), decode
   * attention uses one block size for every context, and every RMSNorm sums its
   * squares in one order.  Then continuous-depth decoding (tl_decode_run) equals
   * step-by-step decoding and a mixed batch equals each lane alone exactly.
   * 0: kernels and splits are picked per pass size (faster at small batches). */
  int32_t batch_invariant;
} tl_config;

/* TL_KV_KV: K and V in the operand type (2 d elements per position and slot).
 * TL_KV_H: the block's pre-QKV norm output x in the operand type (d elements).
 * TL_KV_H8: x as int8 codes, one fp16 scale per (position, head): d + 2 H bytes.
 * TL_KV_H4: x as packed two's-complement int4 codes (element 2i in the low nibble)
 *   with one fp16 scale per (position, head): d / 2 + 2 H bytes.
 * TL_KV_D8: iteration-axis delta-KV ("Benchmark Comparison" page, measured
 *   benchmarks, section 9): a loop layer's slot at iteration 1 keeps x in the
 *   operand type (the anchor); at iteration j >= 2 it keeps int8 codes (one fp16
 *   scale per position and head) of x_j minus the reconstruction of iteration
 *   j - 1, the reconstruction being the anchor plus the decoded differences,
 *   summed in fp32 in iteration order.  Pre and post blocks keep x as TL_KV_H.
 * Codes: s = fp16(max|x| / levels) over the head (division in fp32), q =
 * clamp(rint(x / s), -levels, levels), levels 127 / 7, q = 0 where s = 0.
 * In the store-h modes each attention rebuilds K and V of every cached position
 * of the lanes in the pass with the block's own QKV projection, so the cache shrinks
 * and attention costs a projection over the whole context.  Calls without lanes
 * (scoring) keep no cache and compute K and V directly; tl_decode_run needs
 * TL_KV_KV. */
typedef enum { TL_KV_KV = 0, TL_KV_H = 1, TL_KV_H8 = 2, TL_KV_H4 = 3, TL_KV_D8 = 4 } tl_kv_mode;

/* Host weights of one block, canonical layout: linear weights are [out, in]
 * row-major (y = x W^T).  wqkv rows are q (heads 0..H-1, head_dim rows each), then
 * k, then v.  Norm gains are float32 [d_model].  Element type is the block's dtype;
 * a W4G128 block is given as float32 and quantised at load. */
typedef struct {
  const float* norm1;
  const float* norm2;
  const void* wqkv;   /* [3 d, d] */
  const void* wo;     /* [d, d]   */
  const void* wgate;  /* [F, d]   */
  const void* wup;    /* [F, d]   */
  const void* wdown;  /* [d, F]   */
} tl_block_weights;

typedef struct {
  const void* embed;          /* [V, d] boundary dtype */
  const void* head;           /* [V, d] boundary dtype (may equal embed: tied) */
  const float* final_norm;    /* [d] */
  const tl_block_weights* blocks;  /* n_pre + n_loop + n_post, pipeline order */
} tl_weights;

typedef struct tl_model tl_model;

/* Copy host weights to the device and prepare them for the kernels: INT4
 * quantisation and repacking of W4G128 loop blocks, the optional FP16-body
 * dequantisation, row orders that put each rotary pair and each gate/up pair in
 * one tile, the rotary cos/sin table, the KV arena.  Synchronises `stream` before
 * returning, so the host weights may be freed afterwards.
 * Errors: TL_E_ARG (NULL pointer, inconsistent dims), TL_E_UNSUPPORTED (device is
 * not gfx950, head_dim not even or above 128, 16-bit operands with head_dim not a
 * multiple of 32 or d_model/ffn not a multiple of 32, W4G128 with K not a
 * multiple of 128 or with non-F16 operands), TL_E_OOM, TL_E_HIP. */
tl_status tl_load_weights(const tl_config* cfg, const tl_weights* w, tl_alloc_fn alloc,
                          tl_dealloc_fn dealloc, void* alloc_user, void* stream, tl_model** out);

/* Causal forward of n_seqs packed sequences (scoring or prefill).
 *   cu_seqlens_host [n_seqs+1]: prefix sums of sequence lengths (>= 1 each).
 *   tokens_dev [total] int32 ids in [0, vocab).
 *   L: loop count for every sequence, or per-sequence counts in seq_L_host
 *      (non-NULL overrides L).  1 <= L <= max_L.  Sequences with different L run
 *      in one pass; at iteration j only rows whose L >= j are computed and rows
 *      leave after their last iteration ("Dynamic-L Inference" page, "L-Aware
 *      Batching"; "Continuous Depth Batching" summary).
 *   lanes_host [n_seqs] or NULL.  With lanes, each listed lane is (re)initialised
 *      from its sequence: its KV cache keeps one slot per block application (pre
 *      blocks, loop iteration x layer for j <= L, post blocks), capacity
 *      seq_len + max_new_tokens positions ("CLI Reference" page, "Current
 *      Behavior": max_seq = prompt + max_tokens), depth ceiling L, pending token =
 *      greedy token at the last position.  Without lanes the call only scores.
 *   out_hidden_dev [total, d] float32: residual stream after the last block
 *      (before the final norm), or NULL.
 *   out_logits_dev [n_seqs, V] float32 logits at each sequence's last position,
 *      or NULL.
 *   out_next_dev [n_seqs] int32 greedy token at the last position (lowest index on
 *      ties), or NULL.
 *   out_active_log_dev, or NULL: for j = 1..maxL the original row indices active
 *      at iteration j, concatenated (sum_j n_j entries).
 * Errors: TL_E_ARG, TL_E_STATE (seq_len + max_new_tokens > max_pos, KV arena
 * full), TL_E_OOM, TL_E_HIP. */
tl_status tl_forward(tl_model* m, int32_t n_seqs, const int32_t* cu_seqlens_host,
                     const int32_t* tokens_dev, int32_t L, const int32_t* seq_L_host,
                     const int32_t* lanes_host, int32_t max_new_tokens, float* out_hidden_dev,
                     float* out_logits_dev, int32_t* out_next_dev, int32_t* out_active_log_dev,
                     void* stream);

/* Append tokens to prefilled lanes: a cached causal forward of several new
 * positions per lane (the rest of a prompt after a shared prefix, or any chunk).
 *   cu_seqlens_host [n_seqs+1], tokens_dev [total]: as in tl_forward; sequence i
 *      takes the next positions of lanes_host[i] (len .. len + n_i - 1), which
 *      must fit the lane's capacity.
 *   per_seq_L_host [n_seqs]: requested depth; effective depth min(request, lane
 *      ceiling) becomes the new ceiling, as in tl_decode_step.  Every block
 *      application attends to the lane's earlier positions in its own cache slot
 *      and, causally, to the new rows.
 *   out_hidden_dev [total, d], out_logits_dev [n_seqs, V] (last new position),
 *      out_next_dev [n_seqs] (greedy token of the last position, also the lane's
 *      pending token), out_eff_L_host [n_seqs]: each may be NULL.
 * Errors: TL_E_ARG (NULL, empty sequence, lane out of range or repeated, L < 1),
 * TL_E_STATE (lane never prefilled, capacity exceeded), TL_E_OOM, TL_E_HIP. */
tl_status tl_append(tl_model* m, int32_t n_seqs, const int32_t* cu_seqlens_host,
                    const int32_t* tokens_dev, const int32_t* lanes_host,
                    const int32_t* per_seq_L_host, float* out_hidden_dev, float* out_logits_dev,
                    int32_t* out_next_dev, int32_t* out_eff_L_host, void* stream);

/* Shared-prefix reuse ("Benchmark Comparison" page, measured benchmarks, section 2:
 * a prefix's cache is computed once and reused by many requests, in every loop
 * iteration's slot).  Lane dst (re)starts with the first prefix_len positions of
 * lane src: every cache slot up to src's depth ceiling is copied on the device
 * (one strided copy on `stream`), the ceiling is src's, the capacity
 * prefix_len + max_new_tokens.  When prefix_len equals src's length, dst also
 * takes src's pending token; otherwise dst must be appended to (tl_append) before
 * it is decoded.  src is unchanged; dst's previous cache, if any, is released.
 * Errors: TL_E_ARG (lane out of range, src == dst, prefix_len outside
 * [1, src length], max_new_tokens < 0), TL_E_STATE (src never prefilled,
 * prefix_len + max_new_tokens > max_pos, KV arena full), TL_E_HIP. */
tl_status tl_lane_fork(tl_model* m, int32_t src_lane, int32_t dst_lane, int32_t prefix_len,
                       int32_t max_new_tokens, void* stream);

/* One cached greedy decode step for n_lanes prefilled lanes.
 *   per_lane_L_host [n_lanes]: requested depth; the effective depth is
 *      min(request, lane ceiling) and becomes the new ceiling, so depth never rises
 *      within a generation and every cache slot an iteration reads holds all
 *      earlier positions ("CLI Reference" page, "generate", early-exit options:
 *      monotonic clamping).
 *   in_tokens_dev [n_lanes] int32 or NULL (NULL: each lane's pending token).
 *   out_tokens_dev [n_lanes] int32: greedy next token (also the new pending token).
 *   out_logits_dev [n_lanes, V] float32 or NULL; out_hidden_dev [n_lanes, d] or NULL.
 *   out_eff_L_host [n_lanes] or NULL: effective depth used.
 *   out_active_log_dev: as in tl_forward, over the lanes of this call.
 * Errors: TL_E_ARG (lane out of range, repeated lane, L < 1), TL_E_STATE (lane
 * never prefilled or full, or in_tokens_dev NULL for a lane holding no pending
 * token), TL_E_HIP. */
tl_status tl_decode_step(tl_model* m, int32_t n_lanes, const int32_t* lanes_host,
                         const int32_t* per_lane_L_host, const int32_t* in_tokens_dev,
                         int32_t* out_tokens_dev, float* out_logits_dev, float* out_hidden_dev,
                         int32_t* out_eff_L_host, int32_t* out_active_log_dev, void* stream);

/* tl_decode_step for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation during a request.
 * The call allocates nothing (no hipMalloc / hipFree / pinned host memory / any
 * allocating library routine): its workspace (activations, split-K partials, head
 * partials, row descriptors) lives in one device array the library holds on every
 * device it runs on, 64 MiB (TL_NOALLOC_SCRATCH_BYTES) per device, kept until the
 * process ends; the row descriptors go through the pinned host area the model
 * allocated at load.  Results are those of tl_decode_step on the same lanes
 * (the same kernels and split choices), bit for bit.
 *   The array is shared by every call on a device and keeps the last call's
 *   contents (nothing in it is assumed zero): calls that overlap on one device,
 *   from any model or thread, race; serialise them (one stream, or events).
 * Arguments and lane semantics as tl_decode_step (no active-row log).
 * Errors: as tl_decode_step; TL_E_ARG when n_lanes rows need more scratch than
 * TL_NOALLOC_SCRATCH_BYTES (the message gives the bytes; e.g. a 2048-wide model
 * fits about 450 rows, a 5280-wide one about 200); TL_E_UNSUPPORTED for the store-h
 * cache modes (their K/V rebuild buffers are allocated). */
#define TL_NOALLOC_SCRATCH_BYTES (64ull << 20)
tl_status tl_decode_step_noalloc(tl_model* m, int32_t n_lanes, const int32_t* lanes_host,
                                 const int32_t* per_lane_L_host, const int32_t* in_tokens_dev,
                                 int32_t* out_tokens_dev, float* out_logits_dev, float* out_hidden_dev,
                                 int32_t* out_eff_L_host, void* stream);

/* Early-exit rule of a decode call ("CLI Reference" page, "generate": the
 * --early-exit-patience, --early-exit-min-L, --early-exit-tau,
 * --early-exit-peek-every and --early-exit-logit-margin options).  A token is
 * probed after loop iterations j >= min_L with (j - min_L) divisible by
 * peek_every, never after its last iteration.  A probe is stable when the
 * relative L2 change of the token's residual over iteration j,
 * ||h_j - h_(j-1)|| / ||h_j||, is below tau, or, with logit_margin > 0, when
 * top-1 minus top-2 of the head logits at h_j (final norm, head projection)
 * exceeds logit_margin.  patience consecutive stable probes end the token's loop
 * at j; an unstable probe resets the count; patience 0 disables the rule. */
typedef struct tl_early_exit {
  int32_t patience;
  int32_t min_L;
  int32_t peek_every;
  float tau;
  float logit_margin;
} tl_early_exit;

/* tl_decode_step with the early-exit rule decided on the device.  Each token
 * starts at depth min(request, lane ceiling).  After a probed iteration a kernel
 * marks the tokens whose streak reached patience as finished there: their
 * residual at that point is the step's hidden state (and feeds the head), their
 * later cache slots of this position are not written, and they are carried but
 * ignored until the planned compaction drops them.  Nothing in the loop waits for
 * the host; once every token has finished, the remaining iterations' kernels
 * return at once.  The effective depth becomes the lane's ceiling (monotonic
 * clamping).  The call waits for the stream once, at the end, to return
 * out_eff_L_host.
 *   ee: the rule; patience >= 0, min_L >= 1, peek_every >= 1, tau >= 0,
 *       logit_margin >= 0.  Other arguments as tl_decode_step (no active-row log).
 * Errors: as tl_decode_step; TL_E_ARG for a NULL or invalid rule. */
tl_status tl_decode_step_ee(tl_model* m, int32_t n_lanes, const int32_t* lanes_host,
                            const int32_t* per_lane_L_host, const tl_early_exit* ee,
                            const int32_t* in_tokens_dev, int32_t* out_tokens_dev,
                            float* out_logits_dev, float* out_hidden_dev, int32_t* out_eff_L_host,
                            void* stream);

/* Self-speculative greedy decoding ("Dynamic-L Inference" page, "Self-Speculative
 * Decoding": draft at a low L, verify at a high L with the same weights; "CLI
 * Reference" page, "speculate": --draft-loops, --verify-loops, --draft-ahead at
 * temperature 0).  Produces n_tokens greedy tokens per lane at depth
 * Lv = min(L_verify, lane ceiling), the same tokens a sequence of tl_decode_step
 * calls at Lv would give (up to fp32 summation order), in rounds:
 *   draft: k = min(draft_ahead, tokens still wanted - 1) cached greedy steps at
 *     depth min(L_draft, Lv) on the lane's own cache, starting from its pending
 *     token (the ceiling is not lowered);
 *   verify: [pending, d_1 .. d_k] appended at depth Lv in one cached pass, which
 *     rewrites every slot at those positions;
 *   accept: drafts are kept while each equals the verify pass's greedy token
 *     before it; the round emits those verify tokens plus the one after the last
 *     kept draft, which becomes the pending token; rejected positions are
 *     dropped (the lane's length is cut back).
 * The host waits for the stream once per round to read the accepted counts.
 *   out_tokens_dev [n_lanes, n_tokens] int32: generated tokens.
 *   out_accepted_host [n_lanes, n_tokens] or NULL: drafts accepted in each round,
 *     -1 after the lane's last round.
 * Lanes need n_tokens + draft_ahead free positions.  Lane ceilings become Lv.
 * Errors: TL_E_ARG (NULL, lane out of range or repeated, depth < 1, draft_ahead
 * outside [0, 64], n_tokens < 1), TL_E_STATE (lane never prefilled, no pending
 * token, too little room), TL_E_OOM, TL_E_HIP. */
tl_status tl_speculate(tl_model* m, int32_t n_lanes, const int32_t* lanes_host, int32_t L_draft,
                       int32_t L_verify, int32_t draft_ahead, int32_t n_tokens, int32_t* out_tokens_dev,
                       int32_t* out_accepted_host, void* stream);

/* n_steps greedy tokens for each of n_lanes prefilled lanes, scheduled one loop
 * iteration at a time across lanes (continuous depth batching: "Continuous Depth
 * Batching" summary page).  A pool holds one in-flight token per lane, each at its
 * own iteration; every tick applies the loop stack once to the whole pool and
 * compacts out tokens that ran their last iteration.  Those wait in a boundary
 * queue; the boundary stages (post blocks, head, greedy token, embedding, pre
 * blocks) run on the whole queue once it holds boundary_min lanes, or when the
 * pool has nothing left to iterate, and the lanes re-enter the pool at iteration 1
 * with their next token.  Exits are known one tick ahead from the depth schedule,
 * so the host plans every tick before enqueuing any work.
 *   L_req_host [n_lanes, n_steps]: requested depth of each new token; clamped
 *      exactly as in tl_decode_step.  The results equal n_steps calls of
 *      tl_decode_step with these requests (bit for bit with batch_invariant set;
 *      otherwise up to fp32 summation order, as batches of different sizes may
 *      split K differently); only the order of work differs.
 *   in_tokens_dev [n_lanes, n_steps] int32 or NULL: token fed at each step (NULL:
 *      the lane's pending greedy token, i.e. free-running greedy decoding).
 *   out_tokens_dev [n_lanes, n_steps] int32: greedy token of each step.
 *   out_hidden_dev [n_lanes, n_steps, d] float32 or NULL: residual after the last
 *      block for each step.
 *   out_eff_L_host [n_lanes, n_steps] or NULL.
 *   boundary_min: boundary-queue size that triggers the boundary stages (<= 1:
 *      every tick).
 * Errors: as tl_decode_step. */
tl_status tl_decode_run(tl_model* m, int32_t n_lanes, const int32_t* lanes_host, int32_t n_steps,
                        const int32_t* L_req_host, const int32_t* in_tokens_dev, int32_t* out_tokens_dev,
                        float* out_hidden_dev, int32_t* out_eff_L_host, int32_t boundary_min, void* stream);

/* Copy the device-resident INT4 weights of one W4G128 matrix back to canonical
 * form, unpacked by the same device routine the GEMM uses: q_host [N, K] int8 and
 * scale_bits_host [N, K/128] fp16 bit patterns.  matrix: 0 wqkv, 1 wo, 2 wgate,
 * 3 wup, 4 wdown, in canonical row order.  Synchronous.
 * Errors: TL_E_ARG (block not a W4G128 loop block), TL_E_HIP. */
tl_status tl_export_w4(tl_model* m, int32_t block, int32_t matrix, int8_t* q_host,
                       uint16_t* scale_bits_host);

/* Release a lane's KV cache; the lane must be prefilled again before decoding. */
tl_status tl_lane_release(tl_model* m, int32_t lane);

/* Device bytes the model holds: weights, KV arena, workspaces. */
tl_status tl_memory_info(tl_model* m, uint64_t* weight_bytes, uint64_t* kv_bytes,
                         uint64_t* workspace_bytes);

/* Synchronises stream and reports errors the kernels detected since the last
 * check: a token id outside [0, vocab) (it was read as 0) gives TL_E_ARG. */
tl_status tl_sync_errors(tl_model* m, void* stream);

/* Measurement: with timing on, the library records a pair of HIP events on the
 * call's stream around every launch of the kernel classes below and sums their
 * elapsed times.  tl_timing_read waits for the recorded events, writes the total
 * milliseconds and launch counts of each class (arrays of TL_TIMING_CLASSES) and
 * resets the sums.  Classes: */
#define TL_T_GEMM_QKV_LOOP 0
#define TL_T_GEMM_O_LOOP 1
#define TL_T_GEMM_GU_LOOP 2      /* gate/up with the SwiGLU epilogue */
#define TL_T_GEMM_DOWN_LOOP 3
#define TL_T_GEMM_QKV_BOUNDARY 4 /* pre and post blocks */
#define TL_T_GEMM_O_BOUNDARY 5
#define TL_T_GEMM_GU_BOUNDARY 6
#define TL_T_GEMM_DOWN_BOUNDARY 7
#define TL_T_ATTENTION 8
#define TL_T_RMSNORM 9
#define TL_T_HEAD 10             /* head GEMM and greedy-token reduction */
#define TL_T_COMPACT 11          /* active-row compaction and row moves */
#define TL_T_EMBED 12
#define TL_T_HREBUILD 13         /* store-h modes: cache write, read-back and K/V projection */
#define TL_TIMING_CLASSES 14
tl_status tl_timing_enable(tl_model* m, int32_t on);
tl_status tl_timing_read(tl_model* m, double* total_ms, int64_t* launches);
/* Measurement: the kernels' own durations behind the same classes.  While timing
 * is on, every kernel launched inside a timed class hands the runtime a further
 * event pair that the runtime stamps with that kernel's start and end, so these
 * sums leave out the dispatch and event overhead held in tl_timing_read's
 * figures (which the stamping itself raises).  Writes, per class (arrays of
 * TL_TIMING_CLASSES), the summed kernel milliseconds and the number of kernels,
 * and resets the sums.
 * Errors: TL_E_ARG (NULL pointer), TL_E_HIP (a recorded event failed, or some
 * product launches went untimed because no event could be created; the sums
 * then miss them). */
tl_status tl_timing_read_kernels(tl_model* m, double* kernel_ms, int64_t* kernels);

/* Waits for the model's own device work, frees everything the model holds. */
void tl_free(tl_model* m);

/* Message for the last non-OK status on this thread ("" if none). */
const char* tl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TL_H */
