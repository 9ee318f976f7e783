// Host-callable launchers of the gfx950 kernels and the plain structs they share
// with the engine.  No torch types anywhere below the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum DType : int32_t { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_W4G128 = 3 };
// GEMM dispatch type of fp32 activations with fp16 weights: each product runs on
// fp16 MFMA with the fp32 operand split into two fp16 halves (gemm.hip).  Outputs,
// norms, attention and the KV cache are fp32 (DT_F32) in that mode.
constexpr int32_t DT_F32X16 = 16;

// One activation row of a pass.  orig: index of the row in the caller's order;
// lane: KV lane table entry; pos: absolute position; depth: loop iterations the
// row runs; iter: current loop iteration (1-based) of the row.  done / streak:
// early exit of a decode step (done: the row finished at an earlier probe and is
// only carried until the planned compaction drops it; streak: consecutive
// stable probes so far); both 0 elsewhere.
struct RowInfo {
  int32_t orig, lane, pos, depth, iter, tok_slot, done, streak;
};

// KV cache addressing: slot of a block application for a row = s0 + s1 * row.iter.
struct KVParams {
  void* base;
  const int64_t* lane_off;   // element offset of each lane's slot 0
  const int32_t* lane_cap;   // positions per slot of each lane
  int32_t H, dh, s0, s1;
};

enum EpiKind : int32_t { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3, EPI_STORE = 4 };

struct GemmArgs {
  const void* A;          // [M, K] activations, lda = K
  int32_t M, N, K;
  const void* B;          // dense weights [N, K] (act dtype), or NULL for W4
  const uint32_t* Bw4;    // INT4 kernel layout words, or NULL
  const uint16_t* Bs;     // INT4 fp16 scales [K/128][N]
  // split-K workspace: fp32 partial tiles [splits][M][N]
  float* partial;
  int64_t partial_cap;    // floats
  // device count of rows still running (early exit), or NULL: when it reads 0 the
  // kernels return at once
  const int32_t* live;
  // nonzero: the split of K depends on (N, K) only, never on M (rows are cut into
  // chunks when the partials of one launch would not fit partial_cap), and only
  // the LDS-tiled MFMA kernel runs, so a row's result does not depend on the
  // other rows of the product
  int32_t invariant;
  // GEMV only: with norm_h set, A is the fp32 residual norm_h [M, K] normalised on
  // the fly, x = h / sqrt(mean(h^2) + norm_eps) * norm_g rounded to the operand
  // type (the RMSNorm of the producing block, computed by every workgroup); the
  // x rows are also written to x_out when it is set
  const float* norm_h;
  const float* norm_g;
  float norm_eps;
  void* x_out;
  // host pointer, or NULL: when set, a QKV product that is split over K leaves its
  // partials in `partial` unfinished and stores the split count here (0 when the
  // product was finished); the decode attention then finishes them (QkvParts)
  int32_t* defer_split;
};

struct GemmEpi {
  int32_t kind;
  int32_t pair_g;          // row-permutation granularity of paired epilogues
  // EPI_QKV
  void* q_out;             // [M, d] act dtype
  KVParams kv;
  const RowInfo* rows;
  const float* rope_cos;   // [max_pos, dh/2]
  const float* rope_sin;
  int32_t d, H, dh;
  int32_t skip_done;       // rows marked done (finished by early exit) write nothing
  // EPI_RESID: h[r, c] += acc; then, if norm_g is set, norm_out = RMSNorm(h) * norm_g
  // in the operand type (the next GEMM's input), fused with the split-K reduction
  float* h;
  int32_t ldh;
  const float* norm_g;
  void* norm_out;
  float norm_eps;
  // EPI_SWIGLU: u[r, n] = silu(gate) * up
  void* u_out;
  int32_t F;
  // EPI_HEAD: optional logits store + per-tile (max, argmax) partials
  float* logits;
  int64_t ldl;
  float* part_val;
  int32_t* part_idx;
  float* part_val2;        // optional: runner-up value of each tile (logit margin)
  int32_t n_tiles;
  // EPI_STORE: out[r, c] = acc (fp32)
  float* out;
  int32_t ldo;
};

// Returns the number of N tiles the head GEMM uses for N columns (partials per row).
int gemm_head_tiles(int act_dtype, int M, int N);
hipError_t launch_gemm(int act_dtype, const GemmArgs& g, const GemmEpi& e, hipStream_t s);

// With norm_g, x and x_done set (and d a multiple of 4 up to 8192), the gather also
// writes x = RMSNorm(h) * norm_g in x_dtype and sets *x_done.
hipError_t launch_embed(int dtype, const void* E, const int32_t* tokens, int n, int d, float* h,
                        int32_t* err_flag, int vocab, hipStream_t s, const float* norm_g = nullptr, float eps = 0.f,
                        int x_dtype = 0, void* x = nullptr, bool* x_done = nullptr);
hipError_t launch_rmsnorm(int out_dtype, const float* h, const float* g, const int32_t* gather, int n,
                          int d, float eps, void* out, hipStream_t s);
// The split-K partials of a pass's QKV product left unfinished (GemmArgs::defer_split),
// for the decode attention to finish: each (row, head) workgroup sums its q, k and v
// columns in split order, rotates q and k as the QKV epilogue does, stores k and v
// into the row's cache slot and keeps q.  Only for passes with one row per lane
// (another row's workgroup would read this row's K/V while it is written).
struct QkvParts {
  const float* part;       // [S][M][N] fp32, kernel column order; NULL: q is finished in q
  int32_t S, M, N;         // splits, rows of the pass, columns (3 d)
  int32_t G;               // pair granularity: pair (c, c + G) within each 2G-column chunk
  const float* rope_cos;   // [max_pos, dh/2]
  const float* rope_sin;
};
// live: as GemmArgs::live (NULL: always run).  Rows marked done get a zero output.
// max_ctx: an upper bound on pos + 1 over the rows (0: unknown), which picks
// the block size.  qp: see QkvParts (NULL or qp->part NULL: q from `q`).
// part: kAttnPartFloats floats of scratch for splitting long contexts over several
// workgroups per (row, head) when there are few of them (NULL: never split).
constexpr int kAttnPartFloats = 256 * (128 + 2);
hipError_t launch_attention(int dtype, const void* q, const RowInfo* rows, int n, const KVParams& kv,
                            void* out, const int32_t* live, int max_ctx, hipStream_t s,
                            const QkvParts* qp = nullptr, float* part = nullptr);
// A run of up to attn_tile_rows() consecutive rows of one sequence (positions pos0 .. pos0+nrows-1)
// that attend to positions 0 .. pos0+nrows-1 of their lane's slot.  cap > 0: the lane's slot-0
// offset (koff) and capacity are carried here, so the kernel need not read the lane tables;
// cap == 0: read them from the KVParams tables.
struct AttnTile {
  int32_t row0, nrows, pos0, lane, iter, cap;
  int64_t koff;
};
static_assert(sizeof(AttnTile) == 32, "descriptor layout");
// Tiled causal attention (MFMA) for prefill / scoring passes; 16-bit types and
// head_dim in {64, 96, 128} only (attn_tiled_supported).  A tile holds at most
// attn_tile_rows() consecutive rows.
bool attn_tiled_supported(int dtype, int head_dim);
int attn_tile_rows();
// A tile list of regular shape, given in closed form so that the kernel need not
// load its descriptor: tile b is sequence sq = b / tps, rows p0 = (b mod tps) *
// attn_tile_rows() of it, row0 = sq * T + p0, nrows = min(rows, T - p0), pos0 = p0,
// iteration iter, capacity cap > 0 and slot-0 offset koff0 + sq * kstride.
struct AttnGrid {
  int32_t on, T, tps, iter, cap, pad;
  int64_t koff0, kstride;
};
hipError_t launch_attention_tiled(int dtype, const void* q, const AttnTile* tiles, int n_tiles, const KVParams& kv,
                                  void* out, hipStream_t s, const AttnGrid* grid = nullptr);
// Stable filter of the active rows after iteration it (it = 0: each row's own
// iter): rows with depth > it stay (their iter becomes it + 1), the others leave.
// dest[i] = new index or -1.  count_out[0] = number kept.  If log_out is non-NULL
// the kept rows' orig indices are written there; if running_out is non-NULL it
// receives the number of kept rows not marked done.
hipError_t launch_compact(const RowInfo* rows_in, int n, int it, RowInfo* rows_out, int32_t* dest,
                          int32_t* count_out, int32_t* log_out, int32_t* running_out, hipStream_t s);
// h_next[dest[i]] = h[i] for kept rows; h_exit[rows[i].orig] = h[i] for leaving rows
// (not for rows marked done: their exit state was stored when they finished).
hipError_t launch_move_rows(const float* h, const int32_t* dest, const RowInfo* rows, int n, int d,
                            float* h_next, float* h_exit, hipStream_t s);
hipError_t launch_write_orig(const RowInfo* rows, int n, int32_t* out, hipStream_t s);
// launch_compact followed by launch_move_rows in one kernel, for at most
// kCompactMoveRows rows none of which is marked done: kept rows to rows_out /
// h_next (and, with x set, their rows of xrow_bytes bytes from x to x_next), leaving
// rows to h_exit[orig]; count_out[0] = rows kept.  No dest array.
constexpr int kCompactMoveRows = 1024;
hipError_t launch_compact_move(const RowInfo* rows_in, int n, int it, RowInfo* rows_out, int32_t* count_out,
                               int32_t* log_out, const float* h, int d, float* h_next, float* h_exit, const void* x,
                               void* x_next, int xrow_bytes, hipStream_t s);

// Early-exit probe after loop iteration it on n rows (one workgroup per row): rows not
// done are stable when margin[i] > margin_thr (margin != NULL) or when
// ||h_i - h_prev_i|| / ||h_i|| < tau; streak counts consecutive stable probes and
// resets otherwise; at streak >= patience the row is marked done, its state goes to
// h_exit[orig], eff_depth[orig] = it and *live is decremented.  save_prev (hidden
// rule): the rows not done then copy h_i into h_prev_i for a probe at the next
// iteration on the same row list.
hipError_t launch_ee_probe(RowInfo* rows, int n, int it, const float* h, float* h_prev, bool save_prev,
                           const float* margin, float tau, float margin_thr, int patience, int d,
                           float* h_exit, int32_t* eff_depth, int32_t* live, hipStream_t s);
// Per row i of the head GEMM's tile partials (pv/pi: best value and index of each
// of the tiles, pv2: the tile's runner-up value or NULL): greedy token to out[i]
// and out2[scatter[i]] (either may be NULL; scatter NULL = identity), and, when
// margin != NULL, margin[i] = top-1 minus top-2 logit (a repeated maximum gives 0).
hipError_t launch_argmax_reduce(const float* pv, const int32_t* pi, const float* pv2, int n, int tiles, int32_t* out,
                                int32_t* out2, const int32_t* scatter, float* margin, hipStream_t s);
// Self-speculative round: in[i, 0] = pending[lanes[i]], in[i, c] = draft[c - 1, i]
// (draft step-major [k, n]); n lanes, k drafts.
hipError_t launch_spec_pack(const int32_t* pending, const int32_t* lanes, const int32_t* draft, int n, int k,
                            int32_t* in, hipStream_t s);
// Accept rule per lane i: a = leading drafts with draft[r, i] == g[i, r], capped at
// want[i] - 1; out[slot[i] * n_tokens + emitted[i] + c] = g[i, c] for c <= a,
// pending[lanes[i]] = g[i, a], acc[i] = a.
hipError_t launch_spec_accept(const int32_t* draft, const int32_t* g, const int32_t* lanes, const int32_t* want,
                              const int32_t* emitted, const int32_t* slot, int n, int k, int n_tokens,
                              int32_t* out, int32_t* pending, int32_t* acc, hipStream_t s);
// Store-h cache of one block application.  A lane's slot `slot` keeps one row of
// rb bytes per position at base + lane_off[lane] * unit + (slot * lane_cap[lane] +
// pos) * rb.  mode 1: x in the operand type (d elements); mode 2: d int8 codes then
// H fp16 scales; mode 3: d/2 bytes of two's-complement nibbles (element 2i low,
// 2i+1 high) then H fp16 scales.  Codes: s = fp16(max|x| / levels) over the head's
// dh values (division in fp32), q = clamp(rint(x / s), -levels, levels), levels 127
// or 7, q = 0 where s = 0.  mode 4 (delta along the iterations): the first
// n_bound + n_loop slots (pre/post blocks, then iteration 1 of each loop layer)
// keep operand-type rows of rbA bytes, the later slots (iteration j >= 2 of loop
// layer l is slot n_bound + (j - 1) n_loop + l) int8 codes of x minus the
// previous iteration's reconstruction plus H fp16 scales, rows of rbD bytes.
struct HCacheParams {
  uint8_t* base;
  const int64_t* lane_off;
  const int32_t* lane_cap;
  int32_t unit, rb, slot, mode, H, dh;
  int32_t n_bound, n_loop, rbA, rbD;
};
// Write the operand-type rows x [n, d] of rows (lane, pos) into the cache (rows
// marked done are skipped when skip_done).
hipError_t launch_hcache_write(int dtype, const void* x, const RowInfo* rows, int n, const HCacheParams& hp,
                               bool skip_done, hipStream_t s);
// Read cached rows (lane, pos) back as operand-type x [n, d] (codes times scale).
hipError_t launch_hcache_read(int dtype, const HCacheParams& hp, const RowInfo* rows, int n, void* out,
                              hipStream_t s);
// GEMV for 1..4 rows with fp16 operands (INT4 W4G128 or dense fp16 weights; QKV /
// RESID / SWIGLU epilogues; a RESID norm is not fused): no split of K, no
// partials.  gemv_applies tells whether a product takes this path.
bool gemv_applies(const GemmArgs& g, int kind);
hipError_t launch_gemv(const GemmArgs& g, const GemmEpi& e, hipStream_t s);
hipError_t launch_gather_rows(const float* src, const int32_t* idx, int n, int d, float* dst, hipStream_t s);
hipError_t launch_scatter_rows(const float* src, const int32_t* idx, int n, int d, float* dst, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
hipError_t launch_scatter_i32(const int32_t* src, const int32_t* idx, int n, int32_t* dst, hipStream_t s);
hipError_t launch_gather_i32(const int32_t* src, const int32_t* idx, int n, int32_t* dst, hipStream_t s);

// Load-time kernels.  perm[n] = canonical source row of kernel row n.
hipError_t launch_permute_rows(int elem_bytes, const void* src, const int32_t* perm, int N, int K, void* dst,
                               hipStream_t s);
// Row permutation with bf16 -> fp16 conversion (RNE; exact for |w| >= 2^-14).
hipError_t launch_permute_bf16_to_f16(const uint16_t* src, const int32_t* perm, int N, int K, uint16_t* dst,
                                      hipStream_t s);
hipError_t launch_quant_w4(const float* w, const int32_t* perm, int N, int K, uint32_t* words,
                           uint16_t* scales, hipStream_t s);
hipError_t launch_w4_to_f16(const uint32_t* words, const uint16_t* scales, int N, int K, uint16_t* out,
                            hipStream_t s);
// Canonical export: q[perm[n], k], s[perm[n], g] from kernel row n.
hipError_t launch_w4_export(const uint32_t* words, const uint16_t* scales, const int32_t* perm, int N, int K,
                            int8_t* q, uint16_t* s_out, hipStream_t s);

// Scratch of tl_decode_step_noalloc: a device array of this many bytes per device.
// noalloc_scratch_init (device current) looks up its address once per device;
// noalloc_scratch returns it (NULL before the lookup).
constexpr size_t kNoAllocScratchBytes = 64ull << 20;
hipError_t noalloc_scratch_init(int device);
void* noalloc_scratch(int device);

// Kernel-duration timing (measurement only).  While a timer is installed on the
// calling thread, each launch of the library's kernels takes a fresh (start, stop) event pair from it and has the runtime stamp the
// kernel's own start and end into the pair (hipExtLaunchKernel), so that the
// pair's elapsed time excludes the dispatch and event-packet overhead that a
// pair recorded around the launch holds.  take returns false when it has no
// pair to give; the launch then goes ahead untimed.
struct KernelTimer {
  virtual bool take(hipEvent_t* start, hipEvent_t* stop) = 0;

 protected:
  ~KernelTimer() = default;
};
void set_kernel_timer(KernelTimer* t);   // per thread; nullptr: plain launches
KernelTimer* kernel_timer();
