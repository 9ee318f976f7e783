// Host-side state of a loaded looped model (one GPU, one process).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "../../include/tl.h"
#include "kernels.h"

namespace tl {

// First-fit allocator over element offsets of the KV arena.
class KvArena {
 public:
  void reset(uint64_t total);
  bool alloc(uint64_t n, uint64_t* off);
  void release(uint64_t off, uint64_t n);
  uint64_t total() const { return total_; }

 private:
  uint64_t total_ = 0;
  std::map<uint64_t, uint64_t> free_;   // offset -> length
};

// Store-h rebuild of one pass: the cache rows to read and the scratch K/V they are
// projected into, per group of block applications with the same lanes.
struct HPass {
  HCacheParams hp{};                  // slot set per block application
  KVParams skv{};                     // scratch K/V: one slot per lane of the pass
  std::vector<const RowInfo*> rec;    // index 0: pre/post blocks; j: loop iteration j
  std::vector<int> n_rec;
};

struct Lane {
  bool live = false;
  int32_t len = 0;        // positions written
  int32_t cap = 0;        // positions per slot
  int32_t ceiling = 0;    // depth bound of the next token
  int32_t nslots = 0;
  uint64_t off = 0, elems = 0;
  bool pending = false;   // a greedy next token is held on the device
};

// One matrix in kernel row order: dense [N, K] in the operand dtype, or INT4
// words + scales (and optionally the FP16-body dense copy).
struct MatDev {
  int N = 0, K = 0;
  void* dense = nullptr;
  uint32_t* w4 = nullptr;
  uint16_t* s4 = nullptr;
  int32_t* perm = nullptr;   // device: kernel row -> canonical (stacked) row, or NULL = identity
};

struct BlockDev {
  int kind = 0;              // 0 pre, 1 loop, 2 post
  float* norm1 = nullptr;
  float* norm2 = nullptr;
  MatDev qkv, o, gu, down;   // gu = gate/up interleaved [2F, d]
  bool is_w4 = false;
};

// A captured scoring pass, replayed when tl_forward is called again with the same
// arguments (same pointers, lengths and depths) on the same stream.
struct GraphEntry {
  std::vector<int64_t> key;
  hipGraphExec_t exec = nullptr;
  void* stage = nullptr;     // device copy of the call's descriptors (owned)
  uint64_t last_use = 0;
};

struct Workspace {
  int rows = 0, outs = 0;
  int64_t kv_scratch_elems = 0;
  float *hA = nullptr, *hB = nullptr, *hX = nullptr, *hE = nullptr;
  void *x16 = nullptr, *q16 = nullptr, *o16 = nullptr, *u16 = nullptr, *xh = nullptr;
  void* x16b = nullptr;             // x16's partner: normalised rows moved by a compaction
  RowInfo *rowsA = nullptr, *rowsB = nullptr;
  int32_t *dest = nullptr, *count = nullptr, *tok = nullptr, *tok2 = nullptr;
  float* part_v = nullptr;
  int32_t* part_i = nullptr;
  float* part_v2 = nullptr;         // runner-up value per head tile (logit-margin probe)
  void* kv_scratch = nullptr;
  int part_tiles = 0;
  float* splitk = nullptr;          // split-K partial tiles
  float* attn_part = nullptr;       // kAttnPartFloats: decode attention split over positions
};

}  // namespace tl

// A timed launch group: its class, its (start, stop) pair in ev_pool at ev, and
// the kernel-stamped pairs its product launches took, kev_pool[k0, k1).
struct TimedSpan {
  int cls;
  size_t ev, k0, k1;
};

struct tl_model;
struct ModelKernelTimer final : KernelTimer {
  tl_model* m = nullptr;
  bool take(hipEvent_t* start, hipEvent_t* stop) override;
};

struct tl_model {
  tl_config cfg{};
  int device = 0;            // HIP device the model was loaded on
  int act = DT_F16;
  int gdt = DT_F16;          // GEMM dispatch type: act, or DT_F32X16 (fp32 activations, fp16 weights)
  bool wide = false;         // fp32 activations with 16-bit weights (stored as fp16)
  int32_t invariant = 0;     // tl_config.batch_invariant
  int G = 16;
  int esz = 2;               // bytes of an activation / KV element
  int kv_mode = 0;           // tl_kv_mode
  int hrb = 0;               // store-h: bytes of one position of one slot (delta mode: of a delta slot)
  int hrbA = 0;              // delta mode: of a boundary or anchor slot
  tl_alloc_fn alloc = nullptr;
  tl_dealloc_fn dealloc = nullptr;
  void* user = nullptr;
  std::map<void*, size_t> owned;
  uint64_t weight_bytes = 0, kv_bytes = 0, ws_bytes = 0;

  void* embed = nullptr;
  void* head = nullptr;
  float* final_norm = nullptr;
  std::vector<tl::BlockDev> blocks;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;

  void* kv_base = nullptr;
  tl::KvArena arena;
  std::vector<tl::Lane> lanes;
  std::vector<int64_t> h_lane_off;
  std::vector<int32_t> h_lane_cap;
  int64_t* d_lane_off = nullptr;
  int32_t* d_lane_cap = nullptr;
  int32_t* d_pending = nullptr;
  int32_t* d_err = nullptr;

  tl::Workspace ws;
  // per-call upload: pinned host staging mirrored by a device area
  void* stage_host = nullptr;
  void* stage_dev = nullptr;
  size_t stage_bytes = 0;
  hipEvent_t stage_done = nullptr;
  // stream of the previous call (valid once has_last_stream); a call on another
  // stream first waits for it through `handover`
  hipStream_t last_stream = nullptr;
  bool has_last_stream = false;
  hipEvent_t handover = nullptr;
  // second upload channel (store-h rebuild lists, planned inside a pass)
  void* aux_host = nullptr;
  void* aux_dev = nullptr;
  size_t aux_bytes = 0;
  hipEvent_t aux_done = nullptr;
  // store-h rebuild buffers: operand x and throw-away q [h_rows, d], scratch K/V
  void* h_x = nullptr;
  void* h_q = nullptr;
  void* h_kv = nullptr;
  int64_t h_rows = 0, h_kv_elems = 0;
  const tl::HPass* hpass = nullptr;    // set while a store-h pass runs
  // captured scoring passes; a workspace reallocation invalidates them
  std::vector<tl::GraphEntry> graphs;
  uint64_t graph_clock = 0;
  void* stage_override = nullptr;      // descriptor base while capturing a graph
  // early exit of decode steps (allocated on first use)
  const int32_t* gate_live = nullptr;  // set while the loop of an early-exit step runs
  int32_t ctx_hint = 0;                // while a pass runs: 1 + the largest position of its rows (0: unknown)
  int32_t* ee_live = nullptr;          // rows still running
  int32_t* ee_eff = nullptr;           // [ee_rows] effective depth by caller order
  float* ee_hprev = nullptr;           // [ee_rows, d] residual before a probed iteration
  float* ee_margin = nullptr;          // [ee_rows]
  int32_t* ee_eff_host = nullptr;      // pinned mirror of ee_eff
  int ee_rows = 0;
  // self-speculative decoding (allocated on first use)
  int32_t* sp_draft = nullptr;         // [k, n] drafted tokens, step-major
  int32_t* sp_in = nullptr;            // [n, k + 1] tokens of the verify pass
  int32_t* sp_g = nullptr;             // [n, k + 1] greedy token after each verify row
  int32_t* sp_acc = nullptr;           // [n] accepted drafts of the round
  int32_t* sp_acc_host = nullptr;      // pinned mirror of sp_acc
  int64_t sp_elems = 0;                // capacity of the [n, k + 1] buffers
  // kernel-class timing (measurement only)
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<TimedSpan> ev_spans;     // one per timed launch group, in record order
  std::vector<hipEvent_t> kev_pool;    // (start, stop) pairs the product launches stamp
  size_t kev_used = 0;
  size_t span_ev = 0, span_k = 0;      // where the open span's events start
  bool kev_short = false;              // a product launch went untimed (no pair to give)
  ModelKernelTimer ktimer;
  double t_ms[TL_TIMING_CLASSES] = {};
  int64_t t_n[TL_TIMING_CLASSES] = {};
  double tk_ms[TL_TIMING_CLASSES] = {};
  int64_t tk_n[TL_TIMING_CLASSES] = {};
};
