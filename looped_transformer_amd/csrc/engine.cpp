// Host engine of the looped-transformer runtime: weight preparation, the KV arena,
// forward / decode passes scheduled one loop iteration at a time, and the C ABI.
#include "engine.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>

using tl::BlockDev;
using tl::Lane;
using tl::MatDev;

namespace {

thread_local std::string g_err;

// TL_LOG_LEVEL (read once, stderr only): 0 or unset silent, 1 every failing call's
// reason, 2 also one line per load and per call; any other value counts as 1.
// Logging never changes what a call computes.
int log_level() {
  static const int level = [] {
    const char* s = std::getenv("TL_LOG_LEVEL");
    if (!s || !*s) return 0;
    char* end = nullptr;
    const long v = std::strtol(s, &end, 10);
    return (*end || v < 0 || v > 2) ? 1 : (int)v;
  }();
  return level;
}

void tl_log(int level, const char* fmt, ...) {
  if (log_level() < level) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[tl] %s\n", buf);
}

tl_status fail(tl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  if (log_level() >= 1) std::fprintf(stderr, "[tl] error %d: %s\n", (int)st, buf);
  return st;
}

#define HIPCHK(x)                                                                                  \
  do {                                                                                             \
    hipError_t e_ = (x);                                                                           \
    if (e_ != hipSuccess) return fail(TL_E_HIP, "%s failed: %s (%s:%d)", #x, hipGetErrorString(e_), \
                                      __FILE__, __LINE__);                                         \
  } while (0)

#define TRY(x)                        \
  do {                                \
    tl_status s_ = (x);               \
    if (s_ != TL_OK) return s_;       \
  } while (0)

int dtype_size(int dt) { return dt == DT_F32 ? 4 : 2; }

void* dev_alloc(tl_model* m, size_t bytes) {
  bytes = (bytes + 255) & ~(size_t)255;
  if (bytes == 0) bytes = 256;
  void* p = nullptr;
  if (m->alloc) {
    p = m->alloc(bytes, m->user);
  } else if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    p = nullptr;
  }
  if (p) m->owned[p] = bytes;
  return p;
}

void dev_free(tl_model* m, void* p) {
  if (!p) return;
  auto it = m->owned.find(p);
  if (it == m->owned.end()) return;
  m->owned.erase(it);
  if (m->dealloc) m->dealloc(p, m->user);
  else (void)hipFree(p);
}

// ----------------------------------------------------------------- staging
constexpr size_t kStageInitBytes = 1 << 20;
// Host data of one call is assembled here and copied in one transfer to a device
// area; device pointers are offsets into that area.
struct Stage {
  std::vector<uint8_t> buf;
  size_t add(const void* data, size_t bytes) {
    size_t off = (buf.size() + 255) & ~(size_t)255;
    buf.resize(off + bytes);
    if (bytes) std::memcpy(buf.data() + off, data, bytes);
    return off;
  }
  template <class T> size_t add(const std::vector<T>& v) { return add(v.data(), v.size() * sizeof(T)); }
};

template <class T> T* staged(tl_model* m, size_t off) {
  void* base = m->stage_override ? m->stage_override : m->stage_dev;
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

void drop_graphs(tl_model* m) {
  for (auto& g : m->graphs) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    dev_free(m, g.stage);
  }
  m->graphs.clear();
}

// The staging area, the workspaces and the lane tables are shared by every call.
// Before a call enqueues work on a stream other than the previous call's, that
// stream waits for everything the previous call enqueued (which may still read
// them).  The previous call's stream must still exist.
tl_status stream_handover(tl_model* m, hipStream_t s) {
  if (m->has_last_stream && m->last_stream != s) {
    HIPCHK(hipEventRecord(m->handover, m->last_stream));
    HIPCHK(hipStreamWaitEvent(s, m->handover, 0));
  }
  m->last_stream = s;
  m->has_last_stream = true;
  return TL_OK;
}

tl_status stage_upload(tl_model* m, const Stage& st, hipStream_t s) {
  TRY(stream_handover(m, s));
  const size_t need = std::max<size_t>(st.buf.size(), 256);
  if (need > m->stage_bytes) {
    if (m->stage_host) {
      HIPCHK(hipStreamSynchronize(s));
      HIPCHK(hipHostFree(m->stage_host));
      m->stage_host = nullptr;
      dev_free(m, m->stage_dev);
      m->stage_dev = nullptr;
      m->stage_bytes = 0;
    }
    size_t cap = std::max<size_t>(need * 2, 1 << 20);
    HIPCHK(hipHostMalloc(&m->stage_host, cap, hipHostMallocDefault));
    m->stage_dev = dev_alloc(m, cap);
    if (!m->stage_dev) {
      (void)hipHostFree(m->stage_host);
      m->stage_host = nullptr;
      return fail(TL_E_OOM, "staging area of %zu bytes", cap);
    }
    m->stage_bytes = cap;
  } else {
    HIPCHK(hipEventSynchronize(m->stage_done));
  }
  std::memcpy(m->stage_host, st.buf.data(), st.buf.size());
  HIPCHK(hipMemcpyAsync(m->stage_dev, m->stage_host, st.buf.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipEventRecord(m->stage_done, s));
  return TL_OK;
}

// The same for the second channel (lists a pass plans after the call's upload).
tl_status aux_upload(tl_model* m, const Stage& st, hipStream_t s) {
  const size_t need = std::max<size_t>(st.buf.size(), 256);
  if (need > m->aux_bytes) {
    if (m->aux_host) {
      HIPCHK(hipStreamSynchronize(s));
      HIPCHK(hipHostFree(m->aux_host));
      m->aux_host = nullptr;
      dev_free(m, m->aux_dev);
      m->aux_dev = nullptr;
      m->aux_bytes = 0;
    }
    size_t cap = std::max<size_t>(need * 2, 1 << 20);
    HIPCHK(hipHostMalloc(&m->aux_host, cap, hipHostMallocDefault));
    m->aux_dev = dev_alloc(m, cap);
    if (!m->aux_dev) {
      (void)hipHostFree(m->aux_host);
      m->aux_host = nullptr;
      return fail(TL_E_OOM, "staging area of %zu bytes", cap);
    }
    m->aux_bytes = cap;
  } else {
    HIPCHK(hipEventSynchronize(m->aux_done));
  }
  std::memcpy(m->aux_host, st.buf.data(), st.buf.size());
  HIPCHK(hipMemcpyAsync(m->aux_dev, m->aux_host, st.buf.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipEventRecord(m->aux_done, s));
  return TL_OK;
}

// Keep a captured pass (at most 8, least recently used dropped).
tl_status graph_keep(tl_model* m, tl::GraphEntry& ge, hipStream_t s) {
  ge.last_use = ++m->graph_clock;
  if (m->graphs.size() >= 8) {
    auto old = std::min_element(m->graphs.begin(), m->graphs.end(),
                                [](const tl::GraphEntry& a, const tl::GraphEntry& b) { return a.last_use < b.last_use; });
    HIPCHK(hipStreamSynchronize(s));
    (void)hipGraphExecDestroy(old->exec);
    dev_free(m, old->stage);
    m->graphs.erase(old);
  }
  m->graphs.push_back(ge);
  return TL_OK;
}

// ----------------------------------------------------------------- workspace
constexpr int64_t kSplitFloats = 8ll << 20;   // 32 MB of split-K partials
tl_status ensure_ws(tl_model* m, int rows, int outs, int64_t kv_scratch, hipStream_t s) {
  auto& w = m->ws;
  if (rows <= w.rows && outs <= w.outs && kv_scratch <= w.kv_scratch_elems) return TL_OK;
  const tl_config& c = m->cfg;
  const int R = std::max(w.rows, (rows + 63) / 64 * 64);
  const int O = std::max(w.outs, (outs + 63) / 64 * 64);
  const int64_t KS = std::max(w.kv_scratch_elems, kv_scratch);
  HIPCHK(hipStreamSynchronize(s));
  if (m->has_last_stream && m->last_stream != s) HIPCHK(hipStreamSynchronize(m->last_stream));
  drop_graphs(m);
  void* olds[] = {w.hA, w.hB, w.hX, w.hE, w.x16, w.x16b, w.q16, w.o16, w.u16, w.xh, w.rowsA, w.rowsB,
                  w.dest, w.count, w.tok, w.tok2, w.part_v, w.part_i, w.part_v2, w.kv_scratch, w.splitk, w.attn_part};
  for (void* p : olds) dev_free(m, p);
  w = tl::Workspace{};
  m->ws_bytes = 0;
  const int64_t d = c.d_model, F = c.ffn;
  const int tiles = (c.vocab + 63) / 64;   // upper bound over tile widths (64 or 128)
  struct Req { void** p; size_t bytes; } reqs[] = {
      {(void**)&w.hA, (size_t)R * d * 4},           {(void**)&w.hB, (size_t)R * d * 4},
      {(void**)&w.hX, (size_t)R * d * 4},           {(void**)&w.hE, (size_t)R * d * 4},
      {&w.x16, (size_t)R * d * m->esz},             {&w.x16b, (size_t)R * d * m->esz},
      {&w.q16, (size_t)R * d * m->esz},
      {&w.o16, (size_t)R * d * m->esz},             {&w.u16, (size_t)R * F * m->esz},
      {&w.xh, (size_t)std::max(O, 1) * d * m->esz}, {(void**)&w.rowsA, (size_t)R * sizeof(RowInfo)},
      {(void**)&w.rowsB, (size_t)R * sizeof(RowInfo)}, {(void**)&w.dest, (size_t)R * 4},
      {(void**)&w.count, 256},                      {(void**)&w.tok, (size_t)R * 4},
      {(void**)&w.tok2, (size_t)R * 4},
      {(void**)&w.part_v, (size_t)std::max(O, 1) * tiles * 4},
      {(void**)&w.part_i, (size_t)std::max(O, 1) * tiles * 4},
      {(void**)&w.part_v2, (size_t)std::max(O, 1) * tiles * 4},
      {&w.kv_scratch, (size_t)std::max<int64_t>(KS, 1) * m->esz},
      {(void**)&w.splitk, (size_t)kSplitFloats * 4},
      {(void**)&w.attn_part, (size_t)kAttnPartFloats * 4},
  };
  for (auto& r : reqs) {
    *r.p = dev_alloc(m, r.bytes);
    if (!*r.p) {
      for (auto& q : reqs) { dev_free(m, *q.p); *q.p = nullptr; }
      w = tl::Workspace{};
      return fail(TL_E_OOM, "workspace allocation of %zu bytes failed", r.bytes);
    }
    m->ws_bytes += r.bytes;
  }
  w.rows = R;
  w.outs = O;
  w.kv_scratch_elems = KS;
  w.part_tiles = tiles;
  return TL_OK;
}

// ----------------------------------------------------------------- timing
tl_status flush_timing(tl_model* m) {
  if (m->ev_used == 0) return TL_OK;
  HIPCHK(hipEventSynchronize(m->ev_pool[m->ev_used - 1]));
  for (const TimedSpan& sp : m->ev_spans) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, m->ev_pool[sp.ev], m->ev_pool[sp.ev + 1]));
    m->t_ms[sp.cls] += ms;
    m->t_n[sp.cls] += 1;
    for (size_t k = sp.k0; k < sp.k1; k += 2) {
      HIPCHK(hipEventElapsedTime(&ms, m->kev_pool[k], m->kev_pool[k + 1]));
      m->tk_ms[sp.cls] += ms;
      m->tk_n[sp.cls] += 1;
    }
  }
  m->ev_used = 0;
  m->kev_used = 0;
  m->ev_spans.clear();
  return TL_OK;
}

}  // namespace

bool ModelKernelTimer::take(hipEvent_t* start, hipEvent_t* stop) {
  if (m->kev_used + 2 > m->kev_pool.size()) {
    for (int i = 0; i < 256; ++i) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        m->kev_short = true;
        return false;
      }
      m->kev_pool.push_back(e);
    }
  }
  *start = m->kev_pool[m->kev_used++];
  *stop = m->kev_pool[m->kev_used++];
  return true;
}

namespace {

tl_status tbegin(tl_model* m, hipStream_t s) {
  if (!m->timing) return TL_OK;
  // no span is open here: a full pool is emptied by reading what it holds
  if ((m->ev_used + 2 > m->ev_pool.size() && m->ev_pool.size() >= 16384) || m->kev_used >= 16384)
    TRY(flush_timing(m));
  if (m->ev_used + 2 > m->ev_pool.size()) {
    for (int i = 0; i < 512; ++i) {
      hipEvent_t e;
      HIPCHK(hipEventCreate(&e));
      m->ev_pool.push_back(e);
    }
  }
  m->span_ev = m->ev_used;
  m->span_k = m->kev_used;
  HIPCHK(hipEventRecord(m->ev_pool[m->ev_used++], s));
  return TL_OK;
}

tl_status tend(tl_model* m, int cls, hipStream_t s) {
  if (!m->timing) return TL_OK;
  HIPCHK(hipEventRecord(m->ev_pool[m->ev_used++], s));
  m->ev_spans.push_back(TimedSpan{cls, m->span_ev, m->span_k, m->kev_used});
  return TL_OK;
}

// Installs the model's kernel timer on this thread for the launches of one timed
// group, and takes it down however the group ends.
struct TimerScope {
  explicit TimerScope(tl_model* m) : on(m->timing) {
    if (on) {
      m->ktimer.m = m;
      set_kernel_timer(&m->ktimer);
    }
  }
  ~TimerScope() {
    if (on) set_kernel_timer(nullptr);
  }
  TimerScope(const TimerScope&) = delete;
  TimerScope& operator=(const TimerScope&) = delete;
  bool on;
};

#define TIMED(cls, stmt)            \
  do {                              \
    TRY(tbegin(m, s));              \
    {                               \
      TimerScope tl_ts_(m);         \
      stmt;                         \
    }                               \
    TRY(tend(m, (cls), s));         \
  } while (0)

// ----------------------------------------------------------------- passes
// With norm_h set (only on the few-row GEMV path, see small_gemv) the product's
// input is RMSNorm(norm_h) * norm_g, formed inside the GEMV; x_out receives it.
tl_status gemm(tl_model* m, const void* A, int M, const MatDev& W, GemmEpi& e, hipStream_t s,
               const float* norm_h = nullptr, const float* norm_g = nullptr, void* x_out = nullptr,
               int32_t* defer_split = nullptr) {
  if (defer_split) *defer_split = 0;
  GemmArgs g{};
  g.A = A;
  g.norm_h = norm_h;
  g.norm_g = norm_g;
  g.norm_eps = m->cfg.rms_eps;
  g.x_out = x_out;
  g.M = M;
  g.N = W.N;
  g.K = W.K;
  g.B = W.dense;
  g.Bw4 = W.dense ? nullptr : W.w4;
  g.Bs = W.s4;
  g.partial = m->ws.splitk;
  g.partial_cap = kSplitFloats;
  g.live = m->gate_live;
  g.invariant = m->invariant;
  e.pair_g = m->G;
  if (m->act == DT_F16 && !m->invariant && gemv_applies(g, e.kind)) {   // a few rows: no split-K pass
    HIPCHK(launch_gemv(g, e, s));
    if (e.kind == EPI_RESID && e.norm_g)
      HIPCHK(launch_rmsnorm(m->act, e.h, e.norm_g, nullptr, M, g.N, e.norm_eps, e.norm_out, s));
    return TL_OK;
  }
  if (norm_h) return fail(TL_E_STATE, "normalised input outside the GEMV path");
  g.defer_split = defer_split;
  HIPCHK(launch_gemm(m->gdt, g, e, s));
  return TL_OK;
}

// A block whose four products all take the few-row GEMV (fp16 operands, n <= 4
// rows, INT4 or dense weights): its RMSNorms are formed inside the QKV and
// gate/up GEMVs.
bool small_gemv(const tl_model* m, const tl::BlockDev& B, int n) {
  if (m->act != DT_F16 || m->invariant) return false;
  for (const MatDev* W : {&B.qkv, &B.o, &B.gu, &B.down}) {
    GemmArgs g{};
    g.M = n;
    g.N = W->N;
    g.K = W->K;
    g.B = W->dense;
    g.Bw4 = W->dense ? nullptr : W->w4;
    if (!gemv_applies(g, EPI_RESID)) return false;
  }
  return true;
}

// One pre-norm block on n rows.  x_ready: the caller's previous block already left
// this block's normalised input in ws.x16.  next_norm: gain of the norm that
// follows on the same rows (the next block's first norm), fused into the down
// projection's residual update when possible (then ws.x16 holds its output).
// one_row_per_lane: no lane has two rows in the pass (decode steps), so a split QKV
// product can be finished inside the decode attention (QkvParts).
tl_status run_block(tl_model* m, int b, float* h, const RowInfo* rows, int n, const KVParams& kv, hipStream_t s,
                    const AttnTile* tiles = nullptr, int n_tiles = 0, bool x_ready = false,
                    const float* next_norm = nullptr, int hgroup = -1, bool* x_next = nullptr,
                    bool one_row_per_lane = false, const AttnGrid* grid = nullptr) {
  if (x_next) *x_next = false;
  if (n <= 0) return TL_OK;
  const tl_config& c = m->cfg;
  const BlockDev& B = m->blocks[b];
  auto& w = m->ws;
  const int tb = B.kind == 1 ? TL_T_GEMM_QKV_LOOP : TL_T_GEMM_QKV_BOUNDARY;
  const bool gv = small_gemv(m, B, n);   // norms inside the GEMVs, none fused into the residual products
  const bool norm_in_qkv = gv && !x_ready;
  if (!x_ready && !gv)
    TIMED(TL_T_RMSNORM, HIPCHK(launch_rmsnorm(m->act, h, B.norm1, nullptr, n, c.d_model, c.rms_eps, w.x16, s)));
  GemmEpi e{};
  e.kind = EPI_QKV;
  e.q_out = w.q16;
  e.kv = kv;
  e.rows = rows;
  e.rope_cos = m->rope_cos;
  e.rope_sin = m->rope_sin;
  e.d = c.d_model;
  e.H = c.n_heads;
  e.dh = c.head_dim;
  e.skip_done = m->gate_live != nullptr;
  // store-h: K/V live in a per-pass scratch, rebuilt from the cached x rows of
  // every position of the pass's lanes (the current rows' x is cached first)
  const tl::HPass* hpass = (m->hpass && hgroup >= 0) ? m->hpass : nullptr;
  const KVParams& akv = hpass ? hpass->skv : kv;
  e.kv = akv;
  // a decode pass's split QKV product is finished by the attention
  int32_t qkv_splits = 0;
  int32_t* defer = (one_row_per_lane && !tiles && !hpass) ? &qkv_splits : nullptr;
  if (norm_in_qkv) TIMED(tb + 0, TRY(gemm(m, nullptr, n, B.qkv, e, s, h, B.norm1, w.x16)));
  else TIMED(tb + 0, TRY(gemm(m, w.x16, n, B.qkv, e, s, nullptr, nullptr, nullptr, defer)));
  QkvParts qp{};
  if (qkv_splits > 0) qp = QkvParts{m->ws.splitk, qkv_splits, n, B.qkv.N, m->G, m->rope_cos, m->rope_sin};
  if (hpass) {
    HCacheParams hp = hpass->hp;
    hp.slot = kv.s0;
    const RowInfo* rec = hpass->rec[hgroup];
    const int nrec = hpass->n_rec[hgroup];
    TIMED(TL_T_HREBUILD, HIPCHK(launch_hcache_write(m->act, w.x16, rows, n, hp, m->gate_live != nullptr, s)));
    TIMED(TL_T_HREBUILD, HIPCHK(launch_hcache_read(m->act, hp, rec, nrec, m->h_x, s)));
    GemmEpi r2 = e;
    r2.q_out = m->h_q;
    r2.rows = rec;
    r2.skip_done = false;
    TIMED(TL_T_HREBUILD, TRY(gemm(m, m->h_x, nrec, B.qkv, r2, s)));
  }
  if (tiles) TIMED(TL_T_ATTENTION, HIPCHK(launch_attention_tiled(m->act, w.q16, tiles, n_tiles, akv, w.o16, s, grid)));
  else TIMED(TL_T_ATTENTION, HIPCHK(launch_attention(m->act, w.q16, rows, n, akv, w.o16, m->gate_live,
                                                     m->invariant ? 0 : m->ctx_hint, s, &qp, w.attn_part)));
  GemmEpi r{};
  r.kind = EPI_RESID;
  r.h = h;
  r.ldh = c.d_model;
  r.norm_g = gv ? nullptr : B.norm2;
  r.norm_out = w.x16;
  r.norm_eps = c.rms_eps;
  TIMED(tb + 1, TRY(gemm(m, w.o16, n, B.o, r, s)));
  GemmEpi sw{};
  sw.kind = EPI_SWIGLU;
  sw.u_out = w.u16;
  sw.F = c.ffn;
  if (gv) TIMED(tb + 2, TRY(gemm(m, nullptr, n, B.gu, sw, s, h, B.norm2)));
  else TIMED(tb + 2, TRY(gemm(m, w.x16, n, B.gu, sw, s)));
  r.norm_g = gv ? nullptr : next_norm;
  TIMED(tb + 3, TRY(gemm(m, w.u16, n, B.down, r, s)));
  if (x_next) *x_next = r.norm_g != nullptr;
  return TL_OK;
}

struct Pass {
  int n = 0;
  const int32_t* tokens = nullptr;   // device [n]
  const RowInfo* rows0 = nullptr;    // device, caller order, iter = 1
  std::vector<int> n_active;         // n_j for j = 1..maxL
  KVParams kv{};
  bool scoring = false;              // one reusable slot per sequence
  float* final_h = nullptr;          // [n, d], caller order
  int32_t* log = nullptr;
  // tiled attention (prefill / scoring): tile lists per iteration (index j-1);
  // iteration 1's list covers every row in caller order (pre and post blocks too)
  std::vector<const AttnTile*> tiles;
  std::vector<int> n_tiles;
  std::vector<AttnGrid> grids;       // closed form of each list (on = 0: none)
  // early exit (decode steps): rule, or NULL
  const tl_early_exit* ee = nullptr;
  // host copy of rows0 (store-h modes plan the K/V rebuild from it)
  const std::vector<RowInfo>* rows_host = nullptr;
  // decode steps: every lane has one row
  bool one_row_per_lane = false;
  // gain of the final norm, for a pass whose every row is followed by the head: when
  // all rows leave the loop together and no post block follows, the last residual
  // product forms RMSNorm(h) * head_norm into ws.x16 (the same bits the head's own
  // norm would give) and run_pass sets head_norm_done
  const float* head_norm = nullptr;
  bool head_norm_done = false;
};

// Store-h rebuild plan of a pass: every lane's positions 0 .. (last position in
// the pass), for the pre/post blocks (group 0) and for each loop iteration j (the
// lanes whose rows run iteration j); scratch K/V of one slot per lane.
tl_status plan_hpass(tl_model* m, const Pass& p, tl::HPass& hp, hipStream_t s) {
  const tl_config& c = m->cfg;
  const int ml = std::max(c.max_lanes, 1), d = c.d_model;
  std::vector<int> P(ml, 0), depth(ml, 0);
  for (const RowInfo& r : *p.rows_host) {
    P[r.lane] = std::max(P[r.lane], r.pos + 1);
    depth[r.lane] = std::max(depth[r.lane], r.depth);
  }
  std::vector<int64_t> soff(ml, 0);
  std::vector<int32_t> scap(ml, 0);
  int64_t tot = 0;
  for (int l = 0; l < ml; ++l)
    if (P[l] > 0) {
      soff[l] = tot;
      scap[l] = P[l];
      tot += (int64_t)2 * d * P[l];
    }
  const int Lmax = (int)p.n_active.size();
  Stage st;
  std::vector<size_t> offs;
  std::vector<int> counts;
  std::vector<char> prev;
  int64_t maxR = 1;
  for (int g = 0; g <= Lmax; ++g) {
    std::vector<char> in(ml, 0);
    for (int l = 0; l < ml; ++l) in[l] = P[l] > 0 && (g == 0 || depth[l] >= g);
    if (g > 0 && in == prev) {   // same lanes as the previous group: same list
      offs.push_back(offs.back());
      counts.push_back(counts.back());
      continue;
    }
    std::vector<RowInfo> rec;
    for (int l = 0; l < ml; ++l)
      if (in[l])
        for (int q = 0; q < P[l]; ++q) {
          RowInfo r{};
          r.orig = (int)rec.size();
          r.lane = l;
          r.pos = q;
          r.depth = 1;
          r.iter = 1;
          rec.push_back(r);
        }
    offs.push_back(st.add(rec));
    counts.push_back((int)rec.size());
    maxR = std::max<int64_t>(maxR, (int64_t)rec.size());
    prev = in;
  }
  const size_t o_soff = st.add(soff), o_scap = st.add(scap);
  if (maxR > m->h_rows || tot > m->h_kv_elems) {
    HIPCHK(hipStreamSynchronize(s));
    dev_free(m, m->h_x);
    dev_free(m, m->h_q);
    dev_free(m, m->h_kv);
    m->h_rows = std::max(m->h_rows, (maxR + 63) / 64 * 64);
    m->h_kv_elems = std::max(m->h_kv_elems, tot);
    m->h_x = dev_alloc(m, (size_t)m->h_rows * d * m->esz);
    m->h_q = dev_alloc(m, (size_t)m->h_rows * d * m->esz);
    m->h_kv = dev_alloc(m, (size_t)std::max<int64_t>(m->h_kv_elems, 1) * m->esz);
    if (!m->h_x || !m->h_q || !m->h_kv) {
      m->h_rows = m->h_kv_elems = 0;
      return fail(TL_E_OOM, "store-h rebuild buffers (%lld rows, %lld K/V elements)", (long long)maxR,
                  (long long)tot);
    }
  }
  TRY(aux_upload(m, st, s));
  uint8_t* base = static_cast<uint8_t*>(m->aux_dev);
  hp.hp = HCacheParams{static_cast<uint8_t*>(m->kv_base), m->d_lane_off, m->d_lane_cap, m->esz, m->hrb, 0,
                       m->kv_mode, c.n_heads, c.head_dim, c.n_pre + c.n_post, c.n_loop, m->hrbA, m->hrb};
  hp.skv = KVParams{m->h_kv, reinterpret_cast<const int64_t*>(base + o_soff),
                    reinterpret_cast<const int32_t*>(base + o_scap), c.n_heads, c.head_dim, 0, 0};
  hp.rec.clear();
  hp.n_rec = counts;
  for (size_t o : offs) hp.rec.push_back(reinterpret_cast<const RowInfo*>(base + o));
  return TL_OK;
}

// xnorm: the rows already normalised by the final norm (operand type), or NULL to
// normalise h (gathered) here.
tl_status run_head(tl_model* m, const float* h, const int32_t* gather, int n_out, float* logits, int32_t* out_tok,
                   const int32_t* pend_lanes, hipStream_t s, float* margin = nullptr, const void* xnorm = nullptr);

// Iteration j is probed by the early-exit rule (never the last one: it could not
// shorten the loop).
bool ee_probed(const tl_early_exit* ee, int j, int Lmax) {
  return ee && ee->patience > 0 && j < Lmax && j >= ee->min_L && (j - ee->min_L) % ee->peek_every == 0;
}

// Pre blocks on all rows; loop iteration j on the n_j rows still active, each
// application writing its own cache slot; rows leave (compaction) only after an
// iteration that is the last one of some row; post blocks on all rows.
tl_status run_pass(tl_model* m, Pass& p, hipStream_t s) {
  struct GateReset {
    tl_model* m;
    ~GateReset() {
      m->gate_live = nullptr;
      m->ctx_hint = 0;
    }
  } gate_reset{m};
  m->ctx_hint = 0;
  if (p.rows_host)
    for (const RowInfo& r : *p.rows_host) m->ctx_hint = std::max(m->ctx_hint, r.pos + 1);
  const tl_config& c = m->cfg;
  auto& w = m->ws;
  const int d = c.d_model;
  const bool tiled = !p.tiles.empty();
  tl::HPass hps;
  struct HReset {
    tl_model* m;
    ~HReset() { m->hpass = nullptr; }
  } h_reset{m};
  const bool hmode = m->kv_mode != TL_KV_KV && !p.scoring;
  if (hmode) {
    if (!p.rows_host) return fail(TL_E_STATE, "store-h pass without host rows");
    TRY(plan_hpass(m, p, hps, s));
    m->hpass = &hps;
  }
  const int Lmax = (int)p.n_active.size();
  // every row runs the same number of loop iterations (no early exit): no row moves
  // before the last iteration, where all leave at once, so the pass works in
  // p.final_h from the start and that last compaction (which would only copy every
  // row there, in caller order) is skipped
  bool in_final = !p.ee && p.final_h && Lmax > 0;
  for (int j = 0; j < Lmax && in_final; ++j) in_final = p.n_active[j] == p.n;
  float* const h0 = in_final ? p.final_h : w.hA;
  // the first pre block's norm is formed with the gather (x_ready)
  bool x_ready = false;
  TIMED(TL_T_EMBED, HIPCHK(launch_embed(c.boundary_dtype, m->embed, p.tokens, p.n, d, h0, m->d_err, c.vocab, s,
                                        c.n_pre > 0 ? m->blocks[0].norm1 : nullptr, c.rms_eps, m->act, w.x16,
                                        &x_ready)));
  KVParams kv = p.kv;
  kv.s1 = 0;
  const AttnTile* t0 = tiled ? p.tiles[0] : nullptr;
  const int nt0 = tiled ? p.n_tiles[0] : 0;
  auto grid_of = [&](int k) -> const AttnGrid* {
    return (tiled && k < (int)p.grids.size()) ? &p.grids[k] : nullptr;
  };
  // norm gain of the first block after pre block b / loop layer l on the same rows
  auto loop_first = [&]() { return m->blocks[c.n_pre].norm1; };
  for (int b = 0; b < c.n_pre; ++b) {
    kv.s0 = p.scoring ? 0 : b;
    const float* nn = b + 1 < c.n_pre ? m->blocks[b + 1].norm1 : (Lmax > 0 ? loop_first() : nullptr);
    TRY(run_block(m, b, h0, p.rows0, p.n, kv, s, t0, nt0, x_ready, nn, hmode ? 0 : -1, &x_ready,
                  p.one_row_per_lane, grid_of(0)));
  }
  float* h = h0;
  float* hn = w.hB;
  const RowInfo* rows = p.rows0;
  RowInfo* rbuf[2] = {w.rowsA, w.rowsB};
  int flip = 0;
  int64_t log_off = 0;
  bool moved = true;
  bool hprev_saved = false;   // ee_hprev already holds the rows entering the next iteration
  if (p.ee) {
    m->gate_live = m->ee_live;
    // the probe marks rows in the loop's row list: keep the caller-order list the
    // post blocks use untouched
    HIPCHK(hipMemcpyAsync(rbuf[1], rows, (size_t)p.n * sizeof(RowInfo), hipMemcpyDeviceToDevice, s));
    rows = rbuf[1];
  }
  for (int j = 1; j <= Lmax; ++j) {
    const int nj = p.n_active[j - 1];
    if (p.log && moved) HIPCHK(launch_write_orig(rows, nj, p.log + log_off, s));
    const int next = j < Lmax ? p.n_active[j] : 0;
    const bool leaving = next < nj;
    const bool probe = ee_probed(p.ee, j, Lmax);
    const bool by_margin = probe && p.ee->logit_margin > 0.f;
    // the hidden rule compares with this iteration's input rows: copied here, unless
    // the previous iteration's probe left them (same row list) in ee_hprev
    if (probe && !by_margin && !hprev_saved)
      HIPCHK(hipMemcpyAsync(m->ee_hprev, h, (size_t)nj * d * 4, hipMemcpyDeviceToDevice, s));
    const bool save_prev = probe && !by_margin && !leaving && ee_probed(p.ee, j + 1, Lmax);
    // the compaction after this iteration as one kernel (no early exit, few rows)
    const bool fused_move = !p.ee && nj <= kCompactMoveRows;
    for (int l = 0; l < c.n_loop; ++l) {
      kv.s0 = p.scoring ? 0 : c.n_pre + c.n_post + (j - 1) * c.n_loop + l;
      // (a probe leaves the next iteration's normalised input alone: the logit
      // probe normalises into its own buffer, rows it finishes are only carried)
      // rows that stay after a compaction get their next norm here too when the
      // compaction can move the normalised rows along (fused_move)
      const float* nn = l + 1 < c.n_loop ? m->blocks[c.n_pre + l + 1].norm1
                        : !leaving        ? loop_first()
                        : (in_final && next == 0 && c.n_post == 0) ? p.head_norm
                        : (next > 0 && fused_move) ? loop_first() : nullptr;
      TRY(run_block(m, c.n_pre + l, h, rows, nj, kv, s, tiled ? p.tiles[j - 1] : nullptr,
                    tiled ? p.n_tiles[j - 1] : 0, x_ready, nn, hmode ? j : -1, &x_ready, p.one_row_per_lane,
                    grid_of(j - 1)));
    }
    if (probe) {
      if (by_margin) {
        TRY(run_head(m, h, nullptr, nj, nullptr, nullptr, nullptr, s, m->ee_margin));
      }
      HIPCHK(launch_ee_probe(const_cast<RowInfo*>(rows), nj, j, h, m->ee_hprev, save_prev,
                             by_margin ? m->ee_margin : nullptr,
                             p.ee->tau, p.ee->logit_margin, p.ee->patience, d, p.final_h, m->ee_eff, m->ee_live, s));
    }
    hprev_saved = save_prev;
    moved = leaving;
    if (moved && in_final && next == 0) {
      moved = false;   // every row is in p.final_h already, in caller order
    } else if (moved) {
      RowInfo* rout = rbuf[flip];
      int32_t* logn = p.log ? p.log + log_off + nj : nullptr;
      if (fused_move) {
        // the next iteration's normalised rows (if the last product formed them)
        // move with the rows they belong to
        TIMED(TL_T_COMPACT, HIPCHK(launch_compact_move(rows, nj, j, rout, w.count, logn, h, d, hn, p.final_h,
                                                       x_ready ? w.x16 : nullptr, w.x16b, d * m->esz, s)));
        if (x_ready) std::swap(w.x16, w.x16b);
      } else {
        TIMED(TL_T_COMPACT, HIPCHK(launch_compact(rows, nj, j, rout, w.dest, w.count, logn, p.ee ? m->ee_live : nullptr, s));
                            HIPCHK(launch_move_rows(h, w.dest, rows, nj, d, hn, p.final_h, s)));
        x_ready = false;   // rows moved, their normalised rows did not
      }
      rows = rout;
      flip ^= 1;
      std::swap(h, hn);
      moved = false;   // the compaction already logged iteration j + 1
    } else {
      moved = true;    // rows unchanged: log iteration j + 1 from the same list
    }
    log_off += nj;
  }
  m->gate_live = nullptr;
  p.head_norm_done = in_final && c.n_post == 0 && p.head_norm && x_ready;
  x_ready = false;
  for (int b = 0; b < c.n_post; ++b) {
    kv.s0 = p.scoring ? 0 : c.n_pre + b;
    const float* nn = b + 1 < c.n_post ? m->blocks[c.n_pre + c.n_loop + b + 1].norm1 : nullptr;
    TRY(run_block(m, c.n_pre + c.n_loop + b, p.final_h, p.rows0, p.n, kv, s, t0, nt0, x_ready, nn,
                  hmode ? 0 : -1, &x_ready, p.one_row_per_lane, grid_of(0)));
  }
  return TL_OK;
}

// Attention tiles of one iteration: sequences still active, in caller order, each
// cut into runs of at most attn_tile_rows() consecutive rows.  With lane_off /
// lane_cap (indexed like seq_lane) the tiles carry the lanes' slot offsets, which
// must then be the ones of the KVParams the attention runs with.
void add_tiles(std::vector<AttnTile>& out, const std::vector<int>& seq_len, const std::vector<int>& seq_lane,
               const std::vector<int>& Ls, int j, const std::vector<int>* start = nullptr,
               const std::vector<int64_t>* lane_off = nullptr, const std::vector<int32_t>* lane_cap = nullptr) {
  const int tr = attn_tile_rows();
  int row = 0;
  for (size_t sq = 0; sq < seq_len.size(); ++sq) {
    if (Ls[sq] < j) continue;
    for (int p0 = 0; p0 < seq_len[sq]; p0 += tr) {
      AttnTile t{};
      t.row0 = row + p0;
      t.nrows = std::min(tr, seq_len[sq] - p0);
      t.pos0 = (start ? (*start)[sq] : 0) + p0;
      t.lane = seq_lane[sq];
      t.iter = j;
      if (lane_off && lane_cap) {
        t.cap = (*lane_cap)[t.lane];
        t.koff = (*lane_off)[t.lane];
      }
      out.push_back(t);
    }
    row += seq_len[sq];
  }
}

// The closed form of a tile list (AttnGrid) when it has one: equal-length
// sequences cut into consecutive tiles, capacities carried (cap > 0) and slot
// offsets in arithmetic progression; else on = 0.
AttnGrid tile_grid(const std::vector<AttnTile>& t) {
  AttnGrid g{};
  if (t.empty() || t[0].cap <= 0 || t[0].row0 != 0 || t[0].pos0 != 0) return g;
  const int tr = attn_tile_rows();
  int tps = 0;
  while (tps < (int)t.size() && t[tps].koff == t[0].koff) ++tps;
  const int T = t[tps - 1].pos0 + t[tps - 1].nrows;
  if (tps != (T + tr - 1) / tr || t.size() % tps != 0) return g;
  g.T = T;
  g.tps = tps;
  g.iter = t[0].iter;
  g.cap = t[0].cap;
  g.koff0 = t[0].koff;
  g.kstride = t.size() > (size_t)tps ? t[tps].koff - t[0].koff : 0;
  for (size_t b = 0; b < t.size(); ++b) {
    const int sq = (int)b / tps, p0 = ((int)b % tps) * tr;
    const AttnTile& x = t[b];
    if (x.row0 != sq * T + p0 || x.nrows != std::min(tr, T - p0) || x.pos0 != p0 || x.iter != g.iter ||
        x.cap != g.cap || x.koff != g.koff0 + (int64_t)sq * g.kstride)
      return AttnGrid{};
  }
  g.on = 1;
  return g;
}

// Final norm on the selected rows, head GEMM, greedy token (lowest index on ties)
// and, with margin != NULL, the top-1 minus top-2 logit margin of each row.
tl_status run_head(tl_model* m, const float* h, const int32_t* gather, int n_out, float* logits, int32_t* out_tok,
                   const int32_t* pend_lanes, hipStream_t s, float* margin, const void* xnorm) {
  if (n_out <= 0) return TL_OK;
  const tl_config& c = m->cfg;
  auto& w = m->ws;
  TRY(tbegin(m, s));
  TimerScope ts(m);
  if (!xnorm) HIPCHK(launch_rmsnorm(m->act, h, m->final_norm, gather, n_out, c.d_model, c.rms_eps, w.xh, s));
  const int tiles = gemm_head_tiles(m->gdt, n_out, c.vocab);
  GemmArgs g{};
  g.A = xnorm ? xnorm : w.xh;
  g.M = n_out;
  g.N = c.vocab;
  g.K = c.d_model;
  g.B = m->head;
  g.invariant = m->invariant;
  GemmEpi e{};
  e.kind = EPI_HEAD;
  e.logits = logits;
  e.ldl = c.vocab;
  e.part_val = w.part_v;
  e.part_idx = w.part_i;
  e.n_tiles = tiles;
  e.part_val2 = margin ? w.part_v2 : nullptr;
  HIPCHK(launch_gemm(m->gdt, g, e, s));
  if (out_tok || pend_lanes || margin)
    HIPCHK(launch_argmax_reduce(w.part_v, w.part_i, e.part_val2, n_out, tiles, out_tok,
                                pend_lanes ? m->d_pending : nullptr, pend_lanes, margin, s));
  TRY(tend(m, TL_T_HEAD, s));
  return TL_OK;
}

std::vector<int> active_counts(const std::vector<int>& depth) {
  int mx = 0;
  for (int v : depth) mx = std::max(mx, v);
  std::vector<int> n(mx, 0);
  for (int v : depth)
    for (int j = 1; j <= v; ++j) n[j - 1]++;
  return n;
}

int lane_slots(const tl_config& c, int ceiling) { return c.n_pre + c.n_post + c.n_loop * ceiling; }

uint64_t lane_elems(const tl_model* m, int ceiling, int cap) {
  const tl_config& c = m->cfg;
  uint64_t e = (uint64_t)lane_slots(c, ceiling) * 2ull * c.n_heads * (uint64_t)cap * c.head_dim;
  if (m->kv_mode != TL_KV_KV) {   // store-h: rows of hrb bytes, counted in operand elements
    const uint64_t ns = lane_slots(c, ceiling);
    uint64_t bytes = ns * cap * m->hrb;
    if (m->kv_mode == TL_KV_D8) {   // anchor-format slots first, then the deltas
      const uint64_t A = std::min<uint64_t>(ns, c.n_pre + c.n_post + c.n_loop);
      bytes = A * cap * m->hrbA + (ns - A) * cap * m->hrb;
    }
    e = (bytes + m->esz - 1) / m->esz;
  }
  return (e + 63) / 64 * 64;
}

// Row order used by the paired epilogues: each rotary pair (i, i + dh/2) of q and k
// heads, and each (gate_i, up_i), lands G columns apart inside one 2G-wide chunk.
std::vector<int32_t> perm_qkv(const tl_config& c, int G) {
  const int d = c.d_model, dh = c.head_dim, half = dh / 2;
  std::vector<int32_t> p(3 * d);
  for (int n = 0; n < 3 * d; ++n) {
    const int sect = n / d, within = n % d;
    if (sect == 2) {
      p[n] = n;
      continue;
    }
    const int head = within / dh, cd = within % dh;
    const int ci = cd / G, off = cd % G, pi = ci / 2, which = ci % 2;
    p[n] = sect * d + head * dh + which * half + pi * G + off;
  }
  return p;
}

std::vector<int32_t> perm_gu(const tl_config& c, int G) {
  const int F = c.ffn;
  std::vector<int32_t> p(2 * F);
  for (int n = 0; n < 2 * F; ++n) {
    const int ci = n / G, off = n % G, pi = ci / 2, which = ci % 2;
    p[n] = which * F + pi * G + off;
  }
  return p;
}

tl_status upload_bytes(tl_model* m, void** dst, const void* src, size_t bytes, hipStream_t s) {
  *dst = dev_alloc(m, bytes);
  if (!*dst) return fail(TL_E_OOM, "weights: %zu bytes", bytes);
  m->weight_bytes += bytes;
  HIPCHK(hipMemcpyAsync(*dst, src, bytes, hipMemcpyHostToDevice, s));
  return TL_OK;
}

// Upload one matrix (or a stacked pair) in canonical order and produce the kernel layout.
tl_status prepare_matrix(tl_model* m, MatDev& md, const void* src0, const void* src1, int N, int K, int dtype,
                         bool w4, bool fp16_body, const int32_t* perm_dev, hipStream_t s,
                         std::vector<void*>& temps) {
  // dtype: storage type given by the caller; dense matrices end in the operand type
  // (m->act; fp16 with fp32 activations), converting bf16 -> fp16 on the way when
  // the two differ.
  md.N = N;
  md.K = K;
  md.perm = const_cast<int32_t*>(perm_dev);
  const int in_esz = w4 ? 4 : dtype_size(dtype);
  const size_t half_bytes = (size_t)(src1 ? N / 2 : N) * K * in_esz;
  void* canon = dev_alloc(m, (size_t)N * K * in_esz);
  if (!canon) return fail(TL_E_OOM, "weight staging");
  temps.push_back(canon);
  HIPCHK(hipMemcpyAsync(canon, src0, half_bytes, hipMemcpyHostToDevice, s));
  if (src1)
    HIPCHK(hipMemcpyAsync(static_cast<uint8_t*>(canon) + half_bytes, src1, half_bytes, hipMemcpyHostToDevice, s));
  if (w4) {
    const size_t wbytes = (size_t)N * K / 2, sbytes = (size_t)N * (K / 128) * 2;
    md.w4 = static_cast<uint32_t*>(dev_alloc(m, wbytes));
    md.s4 = static_cast<uint16_t*>(dev_alloc(m, sbytes));
    if (!md.w4 || !md.s4) return fail(TL_E_OOM, "INT4 weights");
    m->weight_bytes += wbytes + sbytes;
    HIPCHK(launch_quant_w4(static_cast<const float*>(canon), perm_dev, N, K, md.w4, md.s4, s));
    if (fp16_body) {
      md.dense = dev_alloc(m, (size_t)N * K * 2);
      if (!md.dense) return fail(TL_E_OOM, "FP16 body");
      m->weight_bytes += (size_t)N * K * 2;
      HIPCHK(launch_w4_to_f16(md.w4, md.s4, N, K, static_cast<uint16_t*>(md.dense), s));
    }
    return TL_OK;
  }
  const size_t bytes = (size_t)N * K * (m->wide ? 2 : m->esz);
  md.dense = dev_alloc(m, bytes);
  if (!md.dense) return fail(TL_E_OOM, "dense weights");
  m->weight_bytes += bytes;
  if (dtype == DT_BF16 && (m->act == DT_F16 || m->wide))
    HIPCHK(launch_permute_bf16_to_f16(static_cast<const uint16_t*>(canon), perm_dev, N, K,
                                      static_cast<uint16_t*>(md.dense), s));
  else if (perm_dev) HIPCHK(launch_permute_rows(in_esz, canon, perm_dev, N, K, md.dense, s));
  else HIPCHK(hipMemcpyAsync(md.dense, canon, bytes, hipMemcpyDeviceToDevice, s));
  return TL_OK;
}

tl_status validate_config(const tl_config* c) {
  if (c->vocab < 1 || c->d_model < 1 || c->n_heads < 1 || c->head_dim < 2 || c->ffn < 1)
    return fail(TL_E_ARG, "dimensions must be positive");
  if (c->d_model != c->n_heads * c->head_dim) return fail(TL_E_ARG, "d_model != n_heads * head_dim");
  if (c->n_pre < 0 || c->n_post < 0 || c->n_loop < 1) return fail(TL_E_ARG, "block counts");
  if (c->max_L < 1 || c->max_pos < 1 || c->max_lanes < 0) return fail(TL_E_ARG, "max_L / max_pos / max_lanes");
  if (c->act_dtype < DT_F32 || c->act_dtype > DT_BF16) return fail(TL_E_UNSUPPORTED, "act_dtype");
  // weights are stored in the operand type, or as bf16 with fp16 operands (converted
  // at load), or (loop blocks) as W4G128 with fp16 operands; with fp32 activations
  // either every weight is fp32 or every weight is 16-bit (fp16 / bf16, run as
  // fp16 with the fp32 operands split into two fp16 halves)
  const bool wide = c->act_dtype == DT_F32 && c->boundary_dtype != DT_F32;
  auto storable = [&](int dt) {
    if (wide) return dt == DT_F16 || dt == DT_BF16;
    return dt == c->act_dtype || (dt == DT_BF16 && c->act_dtype == DT_F16);
  };
  if (!storable(c->boundary_dtype)) return fail(TL_E_UNSUPPORTED, "boundary dtype incompatible with act dtype");
  if (!storable(c->loop_dtype) && !(c->loop_dtype == DT_W4G128 && c->act_dtype == DT_F16))
    return fail(TL_E_UNSUPPORTED, "loop dtype must match act dtype (bf16 storage allowed with F16 operands; "
                                  "F16 / BF16 weights with F32 activations), or W4G128 with F16 operands");
  if (wide && c->kv_mode != TL_KV_KV)
    return fail(TL_E_UNSUPPORTED, "fp32 activations with 16-bit weights keep K/V (kv_mode TL_KV_KV)");
  if (c->loop_fp16_body && c->loop_dtype != DT_W4G128) return fail(TL_E_ARG, "loop_fp16_body needs W4G128");
  if (c->head_dim % 2 || c->head_dim > 128) return fail(TL_E_UNSUPPORTED, "head_dim must be even and <= 128");
  if (c->d_model % 8 || c->ffn % 8) return fail(TL_E_UNSUPPORTED, "d_model and ffn must be multiples of 8");
  if (c->act_dtype == DT_F32 && !wide) {
    if (c->head_dim % 4) return fail(TL_E_UNSUPPORTED, "fp32 head_dim must be a multiple of 4");
  } else {
    if (c->head_dim % 32 || c->ffn % 16) return fail(TL_E_UNSUPPORTED, "16-bit: head_dim % 32, ffn % 16");
  }
  if (c->loop_dtype == DT_W4G128 && (c->d_model % 128 || c->ffn % 128))
    return fail(TL_E_UNSUPPORTED, "W4G128 needs d_model and ffn multiples of 128");
  if (c->kv_mode < TL_KV_KV || c->kv_mode > TL_KV_D8) return fail(TL_E_ARG, "kv_mode %d unknown", c->kv_mode);
  if (c->batch_invariant != 0 && c->batch_invariant != 1) return fail(TL_E_ARG, "batch_invariant must be 0 or 1");
  return TL_OK;
}

}  // namespace

// ----------------------------------------------------------------- KV arena
namespace tl {
void KvArena::reset(uint64_t total) {
  total_ = total;
  free_.clear();
  if (total) free_[0] = total;
}
bool KvArena::alloc(uint64_t n, uint64_t* off) {
  for (auto it = free_.begin(); it != free_.end(); ++it) {
    if (it->second >= n) {
      *off = it->first;
      const uint64_t rest = it->second - n, o = it->first + n;
      free_.erase(it);
      if (rest) free_[o] = rest;
      return true;
    }
  }
  return false;
}
void KvArena::release(uint64_t off, uint64_t n) {
  if (!n) return;
  auto it = free_.emplace(off, n).first;
  auto nx = std::next(it);
  if (nx != free_.end() && it->first + it->second == nx->first) {
    it->second += nx->second;
    free_.erase(nx);
  }
  if (it != free_.begin()) {
    auto pv = std::prev(it);
    if (pv->first + pv->second == it->first) {
      pv->second += it->second;
      free_.erase(it);
    }
  }
}
}  // namespace tl

// ----------------------------------------------------------------- C ABI
extern "C" {

const char* tl_last_error(void) { return g_err.c_str(); }

tl_status tl_load_weights(const tl_config* cfg, const tl_weights* w, tl_alloc_fn alloc, tl_dealloc_fn dealloc,
                          void* alloc_user, void* stream, tl_model** out) {
  g_err.clear();
  if (!cfg || !w || !out) return fail(TL_E_ARG, "NULL argument");
  *out = nullptr;
  if ((alloc == nullptr) != (dealloc == nullptr)) return fail(TL_E_ARG, "alloc and dealloc must both be set or NULL");
  TRY(validate_config(cfg));
  const int nb = cfg->n_pre + cfg->n_loop + cfg->n_post;
  if (!w->embed || !w->head || !w->final_norm || !w->blocks) return fail(TL_E_ARG, "NULL weight pointer");
  for (int b = 0; b < nb; ++b) {
    const tl_block_weights& bw = w->blocks[b];
    if (!bw.norm1 || !bw.norm2 || !bw.wqkv || !bw.wo || !bw.wgate || !bw.wup || !bw.wdown)
      return fail(TL_E_ARG, "NULL pointer in block %d", b);
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(TL_E_UNSUPPORTED, "device %s is not gfx950", prop.gcnArchName);

  hipStream_t s = static_cast<hipStream_t>(stream);
  tl_model* m = new tl_model();
  m->cfg = *cfg;
  m->alloc = alloc;
  m->dealloc = dealloc;
  m->user = alloc_user;
  m->act = cfg->act_dtype;
  m->wide = m->act == DT_F32 && cfg->boundary_dtype != DT_F32;   // validated: all weights 16-bit
  m->gdt = m->wide ? DT_F32X16 : m->act;
  m->invariant = cfg->batch_invariant ? 1 : 0;
  m->G = (m->act == DT_F32 && !m->wide) ? 1 : 16;
  m->esz = dtype_size(m->act);
  m->kv_mode = cfg->kv_mode;
  m->device = dev;
  {
    const int d = cfg->d_model, H = cfg->n_heads;
    m->hrb = m->kv_mode == TL_KV_H ? d * m->esz : m->kv_mode == TL_KV_H4 ? d / 2 + 2 * H : d + 2 * H;
    m->hrbA = d * m->esz;   // delta mode: boundary and anchor slots
  }
  std::vector<void*> temps;
  auto cleanup_fail = [&](tl_status st) {
    std::string msg = g_err;
    (void)hipStreamSynchronize(s);
    tl_free(m);
    g_err = msg;
    return st;
  };
#define LTRY(x)                          \
  do {                                   \
    tl_status s_ = (x);                  \
    if (s_ != TL_OK) return cleanup_fail(s_); \
  } while (0)
#define LHIP(x)                                                                                        \
  do {                                                                                                 \
    hipError_t e_ = (x);                                                                               \
    if (e_ != hipSuccess)                                                                              \
      return cleanup_fail(fail(TL_E_HIP, "%s failed: %s", #x, hipGetErrorString(e_)));                \
  } while (0)

  const tl_config& c = m->cfg;
  const int64_t d = c.d_model, F = c.ffn, V = c.vocab;
  const int besz = dtype_size(c.boundary_dtype);
  LTRY(upload_bytes(m, &m->embed, w->embed, (size_t)V * d * besz, s));
  if (c.boundary_dtype == DT_BF16 && (m->act == DT_F16 || m->wide)) {
    // head in the GEMM's weight type (bf16 storage -> fp16); the embedding gather
    // reads the stored type directly
    void* hs = nullptr;
    LTRY(upload_bytes(m, &hs, w->head, (size_t)V * d * besz, s));
    m->head = dev_alloc(m, (size_t)V * d * 2);
    if (!m->head) return cleanup_fail(fail(TL_E_OOM, "head"));
    m->weight_bytes += (size_t)V * d * 2 - (size_t)V * d * besz;
    LHIP(launch_permute_bf16_to_f16(static_cast<const uint16_t*>(hs), nullptr, (int)V, (int)d,
                                    static_cast<uint16_t*>(m->head), s));
    LHIP(hipStreamSynchronize(s));
    dev_free(m, hs);
  } else if (w->head == w->embed) {
    m->head = m->embed;
  } else {
    LTRY(upload_bytes(m, &m->head, w->head, (size_t)V * d * besz, s));
  }
  void* fn = nullptr;
  LTRY(upload_bytes(m, &fn, w->final_norm, (size_t)d * 4, s));
  m->final_norm = static_cast<float*>(fn);

  // row orders of the paired epilogues
  const std::vector<int32_t> pq = perm_qkv(c, m->G), pg = perm_gu(c, m->G);
  void *pq_dev = nullptr, *pg_dev = nullptr;
  LTRY(upload_bytes(m, &pq_dev, pq.data(), pq.size() * 4, s));
  LTRY(upload_bytes(m, &pg_dev, pg.data(), pg.size() * 4, s));

  m->blocks.resize(nb);
  for (int b = 0; b < nb; ++b) {
    const tl_block_weights& bw = w->blocks[b];
    BlockDev& B = m->blocks[b];
    B.kind = b < c.n_pre ? 0 : (b < c.n_pre + c.n_loop ? 1 : 2);
    const int dt = B.kind == 1 ? c.loop_dtype : c.boundary_dtype;
    const bool w4 = dt == DT_W4G128;
    const bool body = w4 && c.loop_fp16_body;
    B.is_w4 = w4;
    void* n1 = nullptr;
    void* n2 = nullptr;
    LTRY(upload_bytes(m, &n1, bw.norm1, (size_t)d * 4, s));
    LTRY(upload_bytes(m, &n2, bw.norm2, (size_t)d * 4, s));
    B.norm1 = static_cast<float*>(n1);
    B.norm2 = static_cast<float*>(n2);
    LTRY(prepare_matrix(m, B.qkv, bw.wqkv, nullptr, 3 * d, d, dt, w4, body, static_cast<int32_t*>(pq_dev), s, temps));
    LTRY(prepare_matrix(m, B.o, bw.wo, nullptr, d, d, dt, w4, body, nullptr, s, temps));
    LTRY(prepare_matrix(m, B.gu, bw.wgate, bw.wup, 2 * F, d, dt, w4, body, static_cast<int32_t*>(pg_dev), s, temps));
    LTRY(prepare_matrix(m, B.down, bw.wdown, nullptr, d, F, dt, w4, body, nullptr, s, temps));
    // Free the canonical copies as soon as their kernels have consumed them.
    LHIP(hipStreamSynchronize(s));
    for (void* t : temps) dev_free(m, t);
    temps.clear();
  }

  // rotary table: cos/sin of p * base^(-2i/dh) in double, stored fp32
  {
    const int half = c.head_dim / 2;
    std::vector<float> cs((size_t)c.max_pos * half), sn((size_t)c.max_pos * half);
    for (int p = 0; p < c.max_pos; ++p)
      for (int i = 0; i < half; ++i) {
        const double th = std::pow((double)c.rope_base, -2.0 * i / c.head_dim);
        cs[(size_t)p * half + i] = (float)std::cos(p * th);
        sn[(size_t)p * half + i] = (float)std::sin(p * th);
      }
    void *a = nullptr, *b = nullptr;
    LTRY(upload_bytes(m, &a, cs.data(), cs.size() * 4, s));
    LTRY(upload_bytes(m, &b, sn.data(), sn.size() * 4, s));
    m->rope_cos = static_cast<float*>(a);
    m->rope_sin = static_cast<float*>(b);
  }

  // KV arena and lane tables
  const uint64_t kv_elems = c.kv_arena_bytes / m->esz;
  if (kv_elems) {
    m->kv_base = dev_alloc(m, kv_elems * m->esz);
    if (!m->kv_base) return cleanup_fail(fail(TL_E_OOM, "KV arena of %llu bytes", (unsigned long long)c.kv_arena_bytes));
    m->kv_bytes = kv_elems * m->esz;
  }
  m->arena.reset(kv_elems);
  const int ml = std::max(c.max_lanes, 1);
  m->lanes.assign(ml, Lane{});
  m->h_lane_off.assign(ml, 0);
  m->h_lane_cap.assign(ml, 0);
  m->d_lane_off = static_cast<int64_t*>(dev_alloc(m, ml * 8));
  m->d_lane_cap = static_cast<int32_t*>(dev_alloc(m, ml * 4));
  m->d_pending = static_cast<int32_t*>(dev_alloc(m, ml * 4));
  m->d_err = static_cast<int32_t*>(dev_alloc(m, 256));
  if (!m->d_lane_off || !m->d_lane_cap || !m->d_pending || !m->d_err) return cleanup_fail(fail(TL_E_OOM, "lane tables"));
  LHIP(hipMemsetAsync(m->d_lane_off, 0, ml * 8, s));
  LHIP(hipMemsetAsync(m->d_lane_cap, 0, ml * 4, s));
  LHIP(hipMemsetAsync(m->d_pending, 0, ml * 4, s));
  LHIP(hipMemsetAsync(m->d_err, 0, 256, s));
  LHIP(hipEventCreateWithFlags(&m->stage_done, hipEventDisableTiming));
  LHIP(hipEventCreateWithFlags(&m->aux_done, hipEventDisableTiming));
  LHIP(hipEventCreateWithFlags(&m->handover, hipEventDisableTiming));
  // a first staging area (later calls grow it when they need more), so that a
  // decode step of the entry point that allocates nothing finds it
  LHIP(hipHostMalloc(&m->stage_host, kStageInitBytes, hipHostMallocDefault));
  m->stage_dev = dev_alloc(m, kStageInitBytes);
  if (!m->stage_dev) return cleanup_fail(fail(TL_E_OOM, "staging area"));
  m->stage_bytes = kStageInitBytes;
  // device address of the scratch array of tl_decode_step_noalloc on this device
  LHIP(noalloc_scratch_init(dev));
  LHIP(hipStreamSynchronize(s));
  *out = m;
  tl_log(2, "loaded: d_model %d, %d heads x %d, ffn %d, vocab %d, blocks %d pre + %d loop + %d post, act %d, "
            "loop weights %d, kv mode %d, device %d, weights %.1f MB, kv arena %.1f MB",
         m->cfg.d_model, m->cfg.n_heads, m->cfg.head_dim, m->cfg.ffn, m->cfg.vocab, m->cfg.n_pre, m->cfg.n_loop,
         m->cfg.n_post, m->cfg.act_dtype, m->cfg.loop_dtype, m->cfg.kv_mode, m->device, m->weight_bytes / 1e6,
         m->kv_bytes / 1e6);
  return TL_OK;
#undef LTRY
#undef LHIP
}

void tl_free(tl_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  drop_graphs(m);
  std::vector<void*> ps;
  for (auto& kv : m->owned) ps.push_back(kv.first);
  for (void* p : ps) dev_free(m, p);
  if (m->stage_host) (void)hipHostFree(m->stage_host);
  if (m->ee_eff_host) (void)hipHostFree(m->ee_eff_host);
  if (m->sp_acc_host) (void)hipHostFree(m->sp_acc_host);
  if (m->stage_done) (void)hipEventDestroy(m->stage_done);
  if (m->aux_done) (void)hipEventDestroy(m->aux_done);
  if (m->handover) (void)hipEventDestroy(m->handover);
  if (m->aux_host) (void)hipHostFree(m->aux_host);
  for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
  for (hipEvent_t e : m->kev_pool) (void)hipEventDestroy(e);
  delete m;
}

tl_status tl_memory_info(tl_model* m, uint64_t* weight_bytes, uint64_t* kv_bytes, uint64_t* workspace_bytes) {
  if (!m) return fail(TL_E_ARG, "NULL model");
  if (weight_bytes) *weight_bytes = m->weight_bytes;
  if (kv_bytes) *kv_bytes = m->kv_bytes;
  if (workspace_bytes) *workspace_bytes = m->ws_bytes;
  return TL_OK;
}

tl_status tl_lane_release(tl_model* m, int32_t lane) {
  g_err.clear();
  if (!m) return fail(TL_E_ARG, "NULL model");
  if (lane < 0 || lane >= m->cfg.max_lanes) return fail(TL_E_ARG, "lane %d out of range", lane);
  Lane& L = m->lanes[lane];
  if (L.live) m->arena.release(L.off, L.elems);
  L = Lane{};
  return TL_OK;
}

tl_status tl_sync_errors(tl_model* m, void* stream) {
  g_err.clear();
  if (!m) return fail(TL_E_ARG, "NULL model");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t flag = 0;
  TRY(stream_handover(m, s));
  HIPCHK(hipStreamSynchronize(s));
  HIPCHK(hipMemcpy(&flag, m->d_err, 4, hipMemcpyDeviceToHost));
  if (flag) {
    HIPCHK(hipMemset(m->d_err, 0, 4));
    return fail(TL_E_ARG, "a token id was outside [0, vocab) (treated as 0)");
  }
  return TL_OK;
}

tl_status tl_forward(tl_model* m, int32_t n_seqs, const int32_t* cu, const int32_t* tokens, int32_t L,
                     const int32_t* seq_L, const int32_t* lanes, int32_t max_new, float* out_hidden,
                     float* out_logits, int32_t* out_next, int32_t* out_log, void* stream) {
  g_err.clear();
  if (!m || !cu || !tokens) return fail(TL_E_ARG, "NULL argument");
  const tl_config& c = m->cfg;
  if (n_seqs < 1) return fail(TL_E_ARG, "n_seqs must be >= 1");
  tl_log(2, "tl_forward: %d sequences, L %d%s, %s", n_seqs, L, seq_L ? " (per sequence)" : "",
         lanes ? "into lanes" : "scoring");
  if (cu[0] != 0) return fail(TL_E_ARG, "cu_seqlens[0] must be 0");
  std::vector<int> Ls(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int len = cu[i + 1] - cu[i];
    if (len < 1) return fail(TL_E_ARG, "sequence %d is empty", i);
    Ls[i] = seq_L ? seq_L[i] : L;
    if (Ls[i] < 1 || Ls[i] > c.max_L) return fail(TL_E_ARG, "L = %d outside [1, %d]", Ls[i], c.max_L);
    const int need = len + (lanes ? max_new : 0);
    if (need > c.max_pos) return fail(TL_E_STATE, "sequence %d needs %d positions > max_pos %d", i, need, c.max_pos);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = cu[n_seqs];

  // lane plan on a copy of the arena so that a failure leaves the state unchanged
  tl::KvArena arena = m->arena;
  std::vector<Lane> new_lanes;
  if (lanes) {
    if (max_new < 0) return fail(TL_E_ARG, "max_new_tokens < 0");
    std::vector<char> seen(c.max_lanes, 0);
    for (int i = 0; i < n_seqs; ++i) {
      const int l = lanes[i];
      if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
      if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
      seen[l] = 1;
      if (m->lanes[l].live) arena.release(m->lanes[l].off, m->lanes[l].elems);
    }
    for (int i = 0; i < n_seqs; ++i) {
      Lane ln;
      ln.live = true;
      ln.pending = true;
      ln.len = cu[i + 1] - cu[i];
      ln.cap = ln.len + max_new;
      ln.ceiling = Ls[i];
      ln.nslots = lane_slots(c, Ls[i]);
      ln.elems = lane_elems(m, Ls[i], ln.cap);
      if (!arena.alloc(ln.elems, &ln.off))
        return fail(TL_E_STATE, "KV arena full (lane %d needs %llu elements)", lanes[i], (unsigned long long)ln.elems);
      new_lanes.push_back(ln);
    }
  }
  const bool want_head = out_logits || out_next || lanes;
  const int n_out = want_head ? n_seqs : 0;
  TRY(ensure_ws(m, T, n_out, lanes ? 0 : (int64_t)T * 2 * c.d_model, s));

  // scoring passes on a stream are replayed from a captured graph when repeated
  const bool graphable = !lanes && s != nullptr && !m->timing;
  std::vector<int64_t> key;
  if (graphable) {
    TRY(stream_handover(m, s));
    key = {n_seqs, (int64_t)(intptr_t)tokens, (int64_t)(intptr_t)out_hidden, (int64_t)(intptr_t)out_logits,
           (int64_t)(intptr_t)out_next, (int64_t)(intptr_t)out_log, (int64_t)(intptr_t)s};
    for (int i = 0; i <= n_seqs; ++i) key.push_back(cu[i]);
    for (int i = 0; i < n_seqs; ++i) key.push_back(Ls[i]);
    for (auto& g : m->graphs) {
      if (g.key == key) {
        g.last_use = ++m->graph_clock;
        HIPCHK(hipGraphLaunch(g.exec, s));
        return TL_OK;
      }
    }
  }

  std::vector<RowInfo> rows(T);
  std::vector<int> depth(T);
  std::vector<int32_t> last(n_seqs), lane_ids(n_seqs);
  std::vector<int64_t> soff(n_seqs);
  std::vector<int32_t> scap(n_seqs);
  int64_t acc = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int len = cu[i + 1] - cu[i];
    for (int p = 0; p < len; ++p) {
      RowInfo& r = rows[cu[i] + p];
      r = RowInfo{};
      r.orig = cu[i] + p;
      r.lane = lanes ? lanes[i] : i;
      r.pos = p;
      r.depth = Ls[i];
      r.iter = 1;
      depth[cu[i] + p] = Ls[i];
    }
    last[i] = cu[i + 1] - 1;
    lane_ids[i] = lanes ? lanes[i] : -1;
    soff[i] = acc;
    scap[i] = len;
    acc += (int64_t)2 * c.d_model * len;
  }
  std::vector<int64_t> loff = m->h_lane_off;
  std::vector<int32_t> lcap = m->h_lane_cap;
  if (lanes)
    for (int i = 0; i < n_seqs; ++i) {
      loff[lanes[i]] = (int64_t)new_lanes[i].off;
      lcap[lanes[i]] = new_lanes[i].cap;
    }
  // attention tiles for each distinct active set (prefill / scoring passes)
  const bool tiled = attn_tiled_supported(m->act, c.head_dim);
  std::vector<int> slen(n_seqs), slane(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    slen[i] = cu[i + 1] - cu[i];
    slane[i] = lanes ? lanes[i] : i;
  }
  const std::vector<int> n_act = active_counts(depth);
  std::vector<std::vector<AttnTile>> tile_lists;
  if (tiled)
    for (size_t j = 1; j <= n_act.size(); ++j) {
      tile_lists.emplace_back();
      // scoring passes attend in the pass's own scratch (soff / scap by sequence)
      add_tiles(tile_lists.back(), slen, slane, Ls, (int)j, nullptr, lanes ? nullptr : &soff,
                lanes ? nullptr : &scap);
    }
  Stage st;
  std::vector<size_t> o_tiles;
  for (auto& tlst : tile_lists) o_tiles.push_back(st.add(tlst));
  const size_t o_rows = st.add(rows), o_last = st.add(last), o_lanes = st.add(lane_ids);
  const size_t o_soff = st.add(soff), o_scap = st.add(scap);
  const size_t o_loff = st.add(loff), o_lcap = st.add(lcap);
  tl::GraphEntry ge;
  if (graphable) {
    // descriptors in a buffer the graph owns, then capture the pass
    ge.stage = dev_alloc(m, st.buf.size());
    if (!ge.stage) return fail(TL_E_OOM, "graph descriptors");
    hipError_t e1 = hipMemcpy(ge.stage, st.buf.data(), st.buf.size(), hipMemcpyHostToDevice);
    if (e1 != hipSuccess) {
      dev_free(m, ge.stage);
      return fail(TL_E_HIP, "graph descriptors: %s", hipGetErrorString(e1));
    }
    m->stage_override = ge.stage;
    e1 = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e1 != hipSuccess) {
      m->stage_override = nullptr;
      dev_free(m, ge.stage);
      return fail(TL_E_HIP, "stream capture: %s", hipGetErrorString(e1));
    }
  } else {
    TRY(stage_upload(m, st, s));
  }
  if (lanes) {
    HIPCHK(hipMemcpyAsync(m->d_lane_off, staged<int64_t>(m, o_loff), loff.size() * 8, hipMemcpyDeviceToDevice, s));
    HIPCHK(hipMemcpyAsync(m->d_lane_cap, staged<int32_t>(m, o_lcap), lcap.size() * 4, hipMemcpyDeviceToDevice, s));
    m->arena = arena;
    for (int i = 0; i < n_seqs; ++i) m->lanes[lanes[i]] = new_lanes[i];
    m->h_lane_off = loff;
    m->h_lane_cap = lcap;
  }
  Pass p;
  p.n = T;
  p.tokens = tokens;
  p.rows0 = staged<RowInfo>(m, o_rows);
  p.rows_host = &rows;
  p.n_active = n_act;
  for (size_t k = 0; k < tile_lists.size(); ++k) {
    p.tiles.push_back(staged<AttnTile>(m, o_tiles[k]));
    p.n_tiles.push_back((int)tile_lists[k].size());
    p.grids.push_back(tile_grid(tile_lists[k]));
  }
  p.kv.H = c.n_heads;
  p.kv.dh = c.head_dim;
  if (lanes) {
    p.kv.base = m->kv_base;
    p.kv.lane_off = m->d_lane_off;
    p.kv.lane_cap = m->d_lane_cap;
  } else {
    p.kv.base = m->ws.kv_scratch;
    p.kv.lane_off = staged<int64_t>(m, o_soff);
    p.kv.lane_cap = staged<int32_t>(m, o_scap);
    p.scoring = true;
  }
  p.final_h = out_hidden ? out_hidden : m->ws.hX;
  p.log = out_log;
  tl_status stt = run_pass(m, p, s);
  if (stt == TL_OK && want_head)
    stt = run_head(m, p.final_h, staged<int32_t>(m, o_last), n_seqs, out_logits, out_next,
                   lanes ? staged<int32_t>(m, o_lanes) : nullptr, s);
  if (graphable) {
    m->stage_override = nullptr;
    hipGraph_t graph = nullptr;
    const hipError_t e2 = hipStreamEndCapture(s, &graph);
    hipError_t e3 = hipSuccess;
    if (stt == TL_OK && e2 == hipSuccess) e3 = hipGraphInstantiate(&ge.exec, graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    if (stt != TL_OK || e2 != hipSuccess || e3 != hipSuccess) {
      if (ge.exec) (void)hipGraphExecDestroy(ge.exec);
      dev_free(m, ge.stage);
      if (stt != TL_OK) return stt;
      return fail(TL_E_HIP, "graph capture: %s", hipGetErrorString(e2 != hipSuccess ? e2 : e3));
    }
    HIPCHK(hipGraphLaunch(ge.exec, s));
    ge.key = key;
    TRY(graph_keep(m, ge, s));
  }
  return stt;
}

tl_status tl_append(tl_model* m, int32_t n_seqs, const int32_t* cu, const int32_t* tokens, const int32_t* lanes,
                    const int32_t* req_L, float* out_hidden, float* out_logits, int32_t* out_next, int32_t* out_eff_L,
                    void* stream) {
  g_err.clear();
  if (!m || !cu || !tokens || !lanes || !req_L) return fail(TL_E_ARG, "NULL argument");
  const tl_config& c = m->cfg;
  if (n_seqs < 1) return fail(TL_E_ARG, "n_seqs must be >= 1");
  if (cu[0] != 0) return fail(TL_E_ARG, "cu_seqlens[0] must be 0");
  std::vector<char> seen(c.max_lanes, 0);
  std::vector<int> eff(n_seqs), slen(n_seqs), slane(n_seqs), start(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int l = lanes[i];
    if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
    if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
    seen[l] = 1;
    slen[i] = cu[i + 1] - cu[i];
    if (slen[i] < 1) return fail(TL_E_ARG, "sequence %d is empty", i);
    if (req_L[i] < 1) return fail(TL_E_ARG, "requested L %d < 1", req_L[i]);
    const Lane& ln = m->lanes[l];
    if (!ln.live) return fail(TL_E_STATE, "lane %d was never prefilled", l);
    if (ln.len + slen[i] > ln.cap)
      return fail(TL_E_STATE, "lane %d has room for %d more positions, %d appended", l, ln.cap - ln.len, slen[i]);
    eff[i] = std::min(req_L[i], ln.ceiling);
    slane[i] = l;
    start[i] = ln.len;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = cu[n_seqs];
  TRY(ensure_ws(m, T, n_seqs, 0, s));
  std::vector<RowInfo> rows(T);
  std::vector<int> depth(T);
  std::vector<int32_t> last(n_seqs), lane_ids(lanes, lanes + n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    for (int p = 0; p < slen[i]; ++p) {
      RowInfo& r = rows[cu[i] + p];
      r = RowInfo{};
      r.orig = cu[i] + p;
      r.lane = lanes[i];
      r.pos = start[i] + p;
      r.depth = eff[i];
      r.iter = 1;
      depth[cu[i] + p] = eff[i];
    }
    last[i] = cu[i + 1] - 1;
  }
  const bool tiled = attn_tiled_supported(m->act, c.head_dim);
  const std::vector<int> n_act = active_counts(depth);
  std::vector<std::vector<AttnTile>> tile_lists;
  if (tiled)
    for (size_t j = 1; j <= n_act.size(); ++j) {
      tile_lists.emplace_back();
      add_tiles(tile_lists.back(), slen, slane, eff, (int)j, &start);
    }
  Stage st;
  std::vector<size_t> o_tiles;
  for (auto& tlst : tile_lists) o_tiles.push_back(st.add(tlst));
  const size_t o_rows = st.add(rows), o_last = st.add(last), o_lanes = st.add(lane_ids);
  TRY(stage_upload(m, st, s));
  Pass p;
  p.n = T;
  p.tokens = tokens;
  p.rows0 = staged<RowInfo>(m, o_rows);
  p.rows_host = &rows;
  p.n_active = n_act;
  for (size_t k = 0; k < tile_lists.size(); ++k) {
    p.tiles.push_back(staged<AttnTile>(m, o_tiles[k]));
    p.n_tiles.push_back((int)tile_lists[k].size());
    p.grids.push_back(tile_grid(tile_lists[k]));
  }
  p.kv = KVParams{m->kv_base, m->d_lane_off, m->d_lane_cap, c.n_heads, c.head_dim, 0, 0};
  p.final_h = out_hidden ? out_hidden : m->ws.hX;
  TRY(run_pass(m, p, s));
  TRY(run_head(m, p.final_h, staged<int32_t>(m, o_last), n_seqs, out_logits, out_next, staged<int32_t>(m, o_lanes), s));
  for (int i = 0; i < n_seqs; ++i) {
    Lane& ln = m->lanes[lanes[i]];
    ln.len += slen[i];
    ln.ceiling = eff[i];
    ln.pending = true;
    if (out_eff_L) out_eff_L[i] = eff[i];
  }
  return TL_OK;
}

tl_status tl_lane_fork(tl_model* m, int32_t src, int32_t dst, int32_t prefix_len, int32_t max_new, void* stream) {
  g_err.clear();
  if (!m) return fail(TL_E_ARG, "NULL model");
  const tl_config& c = m->cfg;
  if (src < 0 || src >= c.max_lanes || dst < 0 || dst >= c.max_lanes)
    return fail(TL_E_ARG, "lane out of range [0, %d)", c.max_lanes);
  if (src == dst) return fail(TL_E_ARG, "a lane cannot be forked onto itself");
  const Lane sl = m->lanes[src];
  if (!sl.live) return fail(TL_E_STATE, "lane %d was never prefilled", src);
  if (prefix_len < 1 || prefix_len > sl.len)
    return fail(TL_E_ARG, "prefix_len %d outside [1, %d]", prefix_len, sl.len);
  if (max_new < 0) return fail(TL_E_ARG, "max_new_tokens < 0");
  if (prefix_len + max_new > c.max_pos)
    return fail(TL_E_STATE, "fork needs %d positions > max_pos %d", prefix_len + max_new, c.max_pos);
  hipStream_t s = static_cast<hipStream_t>(stream);
  tl::KvArena arena = m->arena;
  if (m->lanes[dst].live) arena.release(m->lanes[dst].off, m->lanes[dst].elems);
  Lane ln;
  ln.live = true;
  ln.len = prefix_len;
  ln.cap = prefix_len + max_new;
  ln.ceiling = sl.ceiling;
  ln.nslots = lane_slots(c, sl.ceiling);   // slots below the ceiling lead the lane's layout
  ln.elems = lane_elems(m, sl.ceiling, ln.cap);
  ln.pending = sl.pending && prefix_len == sl.len;
  if (!arena.alloc(ln.elems, &ln.off))
    return fail(TL_E_STATE, "KV arena full (lane %d needs %llu elements)", dst, (unsigned long long)ln.elems);
  std::vector<int64_t> loff = m->h_lane_off;
  std::vector<int32_t> lcap = m->h_lane_cap;
  loff[dst] = (int64_t)ln.off;
  lcap[dst] = ln.cap;
  Stage st;
  const size_t o_loff = st.add(loff), o_lcap = st.add(lcap);
  TRY(stage_upload(m, st, s));
  // every (slot, K/V, head) block is [cap][head_dim] (store-h: every slot is [cap]
  // rows of hrb bytes; delta mode: the anchor-format slots, then the delta slots):
  // copy its first prefix_len rows
  const bool hm = m->kv_mode != TL_KV_KV;
  uint8_t* kvb = static_cast<uint8_t*>(m->kv_base);
  uint8_t* dstb = kvb + ln.off * m->esz;
  const uint8_t* srcb = kvb + sl.off * m->esz;
  auto copy_rows = [&](uint8_t* dp, const uint8_t* sp, size_t row, size_t blocks) -> tl_status {
    if (blocks)
      HIPCHK(hipMemcpy2DAsync(dp, (size_t)ln.cap * row, sp, (size_t)sl.cap * row, (size_t)prefix_len * row, blocks,
                              hipMemcpyDeviceToDevice, s));
    return TL_OK;
  };
  if (m->kv_mode == TL_KV_D8) {
    const size_t A = std::min<size_t>(ln.nslots, c.n_pre + c.n_post + c.n_loop);
    TRY(copy_rows(dstb, srcb, m->hrbA, A));
    TRY(copy_rows(dstb + A * ln.cap * m->hrbA, srcb + A * sl.cap * m->hrbA, m->hrb, ln.nslots - A));
  } else {
    TRY(copy_rows(dstb, srcb, hm ? (size_t)m->hrb : (size_t)c.head_dim * m->esz,
                  hm ? (size_t)ln.nslots : (size_t)ln.nslots * 2 * c.n_heads));
  }
  if (ln.pending) HIPCHK(hipMemcpyAsync(m->d_pending + dst, m->d_pending + src, 4, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(m->d_lane_off, staged<int64_t>(m, o_loff), loff.size() * 8, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(m->d_lane_cap, staged<int32_t>(m, o_lcap), lcap.size() * 4, hipMemcpyDeviceToDevice, s));
  m->arena = arena;
  m->lanes[dst] = ln;
  m->h_lane_off = loff;
  m->h_lane_cap = lcap;
  return TL_OK;
}

// Buffers of self-speculative rounds for n lanes and k drafts.
tl_status ensure_spec(tl_model* m, int n, int k, hipStream_t s) {
  const int64_t need = (int64_t)n * (k + 1);
  if (need <= m->sp_elems && m->sp_acc_host) return TL_OK;
  HIPCHK(hipStreamSynchronize(s));
  dev_free(m, m->sp_draft);
  dev_free(m, m->sp_in);
  dev_free(m, m->sp_g);
  dev_free(m, m->sp_acc);
  if (m->sp_acc_host) HIPCHK(hipHostFree(m->sp_acc_host));
  m->sp_acc_host = nullptr;
  m->sp_elems = 0;
  const int64_t E = (need + 63) / 64 * 64;
  m->sp_draft = static_cast<int32_t*>(dev_alloc(m, (size_t)E * 4));
  m->sp_in = static_cast<int32_t*>(dev_alloc(m, (size_t)E * 4));
  m->sp_g = static_cast<int32_t*>(dev_alloc(m, (size_t)E * 4));
  m->sp_acc = static_cast<int32_t*>(dev_alloc(m, (size_t)E * 4));
  HIPCHK(hipHostMalloc((void**)&m->sp_acc_host, (size_t)E * 4, hipHostMallocDefault));
  if (!m->sp_draft || !m->sp_in || !m->sp_g || !m->sp_acc) return fail(TL_E_OOM, "speculative buffers");
  m->sp_elems = E;
  return TL_OK;
}

tl_status tl_speculate(tl_model* m, int32_t n, const int32_t* lanes, int32_t L_draft, int32_t L_verify,
                       int32_t draft_ahead, int32_t n_tokens, int32_t* out_tokens, int32_t* out_accepted,
                       void* stream) {
  g_err.clear();
  if (!m || !lanes || !out_tokens) return fail(TL_E_ARG, "NULL argument");
  const tl_config& c = m->cfg;
  if (n < 1) return fail(TL_E_ARG, "n_lanes must be >= 1");
  if (L_draft < 1 || L_verify < 1) return fail(TL_E_ARG, "depths must be >= 1");
  if (draft_ahead < 0 || draft_ahead > 64) return fail(TL_E_ARG, "draft_ahead %d outside [0, 64]", draft_ahead);
  if (n_tokens < 1) return fail(TL_E_ARG, "n_tokens must be >= 1");
  std::vector<char> seen(c.max_lanes, 0);
  std::vector<int> Lv(n), Ld(n);
  for (int i = 0; i < n; ++i) {
    const int l = lanes[i];
    if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
    if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
    seen[l] = 1;
    const Lane& ln = m->lanes[l];
    if (!ln.live) return fail(TL_E_STATE, "lane %d was never prefilled", l);
    if (!ln.pending) return fail(TL_E_STATE, "lane %d holds no pending token (append first)", l);
    if (ln.len + n_tokens + draft_ahead > ln.cap)
      return fail(TL_E_STATE, "lane %d needs %d free positions, has %d", l, n_tokens + draft_ahead, ln.cap - ln.len);
    Lv[i] = std::min(L_verify, ln.ceiling);
    Ld[i] = std::min(L_draft, Lv[i]);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int K = draft_ahead;
  TRY(ensure_ws(m, n * (K + 1), n * (K + 1), 0, s));
  TRY(ensure_spec(m, n, K, s));
  if (out_accepted)
    for (int64_t x = 0; x < (int64_t)n * n_tokens; ++x) out_accepted[x] = -1;
  const KVParams kvp{m->kv_base, m->d_lane_off, m->d_lane_cap, c.n_heads, c.head_dim, 0, 0};
  const bool tiled = attn_tiled_supported(m->act, c.head_dim);
  std::vector<int> emitted(n, 0), rounds(n, 0);
  for (;;) {
    // lanes still generating, and this round's draft count
    std::vector<int> act;
    int max_want = 0;
    for (int i = 0; i < n; ++i)
      if (emitted[i] < n_tokens) {
        act.push_back(i);
        max_want = std::max(max_want, n_tokens - emitted[i]);
      }
    if (act.empty()) break;
    const int na = (int)act.size();
    const int k = std::min(K, max_want - 1);
    std::vector<int32_t> alanes(na), want(na), emit(na), slot(na);
    std::vector<int> pos0(na), lv(na), ld(na);
    for (int a = 0; a < na; ++a) {
      const int i = act[a];
      alanes[a] = lanes[i];
      want[a] = n_tokens - emitted[i];
      emit[a] = emitted[i];
      slot[a] = i;
      pos0[a] = m->lanes[lanes[i]].len;
      lv[a] = Lv[i];
      ld[a] = Ld[i];
    }
    // descriptors: k draft steps (one row per lane), then the verify pass
    Stage st;
    std::vector<size_t> o_drows(k);
    std::vector<std::vector<RowInfo>> drows_host(k);
    for (int r = 0; r < k; ++r) {
      std::vector<RowInfo>& rows = drows_host[r];
      rows.resize(na);
      for (int a = 0; a < na; ++a) {
        rows[a] = RowInfo{};
        rows[a].orig = a;
        rows[a].lane = alanes[a];
        rows[a].pos = pos0[a] + r;
        rows[a].depth = ld[a];
        rows[a].iter = 1;
      }
      o_drows[r] = st.add(rows);
    }
    const int T = na * (k + 1);
    std::vector<RowInfo> vrows(T);
    std::vector<int> vdepth(T), slen(na, k + 1);
    for (int a = 0; a < na; ++a)
      for (int q = 0; q <= k; ++q) {
        RowInfo& r = vrows[a * (k + 1) + q];
        r = RowInfo{};
        r.orig = a * (k + 1) + q;
        r.lane = alanes[a];
        r.pos = pos0[a] + q;
        r.depth = lv[a];
        r.iter = 1;
        vdepth[a * (k + 1) + q] = lv[a];
      }
    const std::vector<int> v_act = active_counts(vdepth);
    std::vector<std::vector<AttnTile>> tile_lists;
    if (tiled)
      for (size_t j = 1; j <= v_act.size(); ++j) {
        tile_lists.emplace_back();
        add_tiles(tile_lists.back(), slen, std::vector<int>(alanes.begin(), alanes.end()), lv, (int)j, &pos0);
      }
    std::vector<size_t> o_tiles;
    for (auto& tlst : tile_lists) o_tiles.push_back(st.add(tlst));
    const size_t o_vrows = st.add(vrows), o_lanes = st.add(alanes), o_want = st.add(want), o_emit = st.add(emit),
                 o_slot = st.add(slot);
    TRY(stage_upload(m, st, s));
    const int32_t* lanes_dev = staged<int32_t>(m, o_lanes);
    // draft: k cached greedy steps at the draft depth, the ceiling left alone
    for (int r = 0; r < k; ++r) {
      const int32_t* toks;
      if (r == 0) {
        HIPCHK(launch_gather_i32(m->d_pending, lanes_dev, na, m->ws.tok, s));
        toks = m->ws.tok;
      } else {
        toks = m->sp_draft + (int64_t)(r - 1) * na;
      }
      std::vector<int> dd(ld.begin(), ld.end());
      Pass p;
      p.n = na;
      p.tokens = toks;
      p.rows0 = staged<RowInfo>(m, o_drows[r]);
      p.rows_host = &drows_host[r];
      p.one_row_per_lane = true;
      p.n_active = active_counts(dd);
      p.kv = kvp;
      p.final_h = m->ws.hX;
      TRY(run_pass(m, p, s));
      TRY(run_head(m, p.final_h, nullptr, na, nullptr, m->sp_draft + (int64_t)r * na, nullptr, s));
    }
    // verify: [pending, d_1 .. d_k] of every lane in one cached pass at the verify depth
    HIPCHK(launch_spec_pack(m->d_pending, lanes_dev, m->sp_draft, na, k, m->sp_in, s));
    {
      Pass p;
      p.n = T;
      p.tokens = m->sp_in;
      p.rows0 = staged<RowInfo>(m, o_vrows);
      p.rows_host = &vrows;
      p.n_active = v_act;
      for (size_t q = 0; q < tile_lists.size(); ++q) {
        p.tiles.push_back(staged<AttnTile>(m, o_tiles[q]));
        p.n_tiles.push_back((int)tile_lists[q].size());
        p.grids.push_back(tile_grid(tile_lists[q]));
      }
      p.kv = kvp;
      p.final_h = m->ws.hX;
      TRY(run_pass(m, p, s));
      TRY(run_head(m, p.final_h, nullptr, T, nullptr, m->sp_g, nullptr, s));
    }
    HIPCHK(launch_spec_accept(m->sp_draft, m->sp_g, lanes_dev, staged<int32_t>(m, o_want), staged<int32_t>(m, o_emit),
                              staged<int32_t>(m, o_slot), na, k, n_tokens, out_tokens, m->d_pending, m->sp_acc, s));
    HIPCHK(hipMemcpyAsync(m->sp_acc_host, m->sp_acc, (size_t)na * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    for (int a = 0; a < na; ++a) {
      const int i = act[a], acc = m->sp_acc_host[a];
      if (acc < 0 || acc > k || acc >= want[a]) return fail(TL_E_HIP, "accept count %d out of range", acc);
      Lane& ln = m->lanes[lanes[i]];
      ln.len = pos0[a] + acc + 1;
      ln.ceiling = lv[a];
      ln.pending = true;
      if (out_accepted) out_accepted[(int64_t)i * n_tokens + rounds[i]] = acc;
      emitted[i] += acc + 1;
      rounds[i] += 1;
    }
  }
  return TL_OK;
}

// Validation shared by the decode-step entry points: lanes in range, distinct,
// prefilled, not full, holding a pending token unless one is fed; eff receives
// the clamped depths.
tl_status decode_check(tl_model* m, int32_t n, const int32_t* lanes, const int32_t* req_L, const int32_t* in_tokens,
                       std::vector<int>& eff) {
  const tl_config& c = m->cfg;
  std::vector<char> seen(c.max_lanes, 0);
  eff.assign(n, 0);
  for (int i = 0; i < n; ++i) {
    const int l = lanes[i];
    if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
    if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
    seen[l] = 1;
    if (req_L[i] < 1) return fail(TL_E_ARG, "requested L %d < 1", req_L[i]);
    const Lane& ln = m->lanes[l];
    if (!ln.live) return fail(TL_E_STATE, "lane %d was never prefilled", l);
    if (ln.len >= ln.cap) return fail(TL_E_STATE, "lane %d is full (%d positions)", l, ln.cap);
    if (!in_tokens && !ln.pending) return fail(TL_E_STATE, "lane %d holds no pending token (append first)", l);
    eff[i] = std::min(req_L[i], ln.ceiling);
  }
  return TL_OK;
}

// Row descriptors of a decode step (staged as [rows, lane ids]).
void decode_stage(const tl_model* m, int n, const int32_t* lanes, const std::vector<int>& eff,
                  std::vector<RowInfo>& rows, Stage& st, size_t* o_rows, size_t* o_lanes) {
  rows.assign(n, RowInfo{});
  std::vector<int32_t> lane_ids(lanes, lanes + n);
  for (int i = 0; i < n; ++i) {
    rows[i].orig = i;
    rows[i].lane = lanes[i];
    rows[i].pos = m->lanes[lanes[i]].len;
    rows[i].depth = eff[i];
    rows[i].iter = 1;
  }
  *o_rows = st.add(rows);
  *o_lanes = st.add(lane_ids);
}

// The pass and head of a decode step whose descriptors are staged and whose
// workspace is m->ws; then the lanes advance.
tl_status decode_run_step(tl_model* m, int n, const int32_t* lanes, const std::vector<int>& eff,
                          const std::vector<RowInfo>& rows, size_t o_rows, size_t o_lanes, const int32_t* in_tokens,
                          int32_t* out_tokens, float* out_logits, float* out_hidden, int32_t* out_eff_L,
                          int32_t* out_log, hipStream_t s) {
  const tl_config& c = m->cfg;
  const int32_t* lanes_dev = staged<int32_t>(m, o_lanes);
  const int32_t* toks = in_tokens;
  if (!toks) {
    HIPCHK(launch_gather_i32(m->d_pending, lanes_dev, n, m->ws.tok, s));
    toks = m->ws.tok;
  }
  Pass p;
  p.n = n;
  p.tokens = toks;
  p.rows0 = staged<RowInfo>(m, o_rows);
  p.rows_host = &rows;
  p.n_active = active_counts(eff);
  p.kv = KVParams{m->kv_base, m->d_lane_off, m->d_lane_cap, c.n_heads, c.head_dim, 0, 0};
  p.final_h = out_hidden ? out_hidden : m->ws.hX;
  p.log = out_log;
  p.one_row_per_lane = true;
  p.head_norm = m->final_norm;
  TRY(run_pass(m, p, s));
  TRY(run_head(m, p.final_h, nullptr, n, out_logits, out_tokens, lanes_dev, s, nullptr,
               p.head_norm_done ? m->ws.x16 : nullptr));
  for (int i = 0; i < n; ++i) {
    Lane& ln = m->lanes[lanes[i]];
    ln.len += 1;
    ln.pending = true;
    ln.ceiling = eff[i];
    if (out_eff_L) out_eff_L[i] = eff[i];
  }
  return TL_OK;
}

tl_status tl_decode_step(tl_model* m, int32_t n, const int32_t* lanes, const int32_t* req_L,
                         const int32_t* in_tokens, int32_t* out_tokens, float* out_logits, float* out_hidden,
                         int32_t* out_eff_L, int32_t* out_log, void* stream) {
  g_err.clear();
  if (!m || !lanes || !req_L || !out_tokens) return fail(TL_E_ARG, "NULL argument");
  if (n < 1) return fail(TL_E_ARG, "n_lanes must be >= 1");
  tl_log(2, "tl_decode_step: %d lanes", n);
  std::vector<int> eff;
  TRY(decode_check(m, n, lanes, req_L, in_tokens, eff));
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(ensure_ws(m, n, n, 0, s));
  std::vector<RowInfo> rows;
  Stage st;
  size_t o_rows = 0, o_lanes = 0;
  decode_stage(m, n, lanes, eff, rows, st, &o_rows, &o_lanes);
  TRY(stage_upload(m, st, s));
  return decode_run_step(m, n, lanes, eff, rows, o_rows, o_lanes, in_tokens, out_tokens, out_logits, out_hidden,
                         out_eff_L, out_log, s);
}

// Layout of tl_decode_step_noalloc's scratch for n rows: the workspace of a decode
// step (as ensure_ws lays it out for n rows, with room for the split-K partials
// the products of at most n rows can take: at most 16 splits, never more than the
// kSplitFloats every path is capped at) followed by the staged descriptors.
// Returns the bytes used; with base set, points w's buffers into it and the
// staging area *stage to its place.
size_t noalloc_layout(const tl_model* m, int n, size_t stage_bytes, uint8_t* base, tl::Workspace* w, void** stage) {
  const tl_config& c = m->cfg;
  const size_t R = (size_t)(n + 63) / 64 * 64;
  const size_t d = c.d_model, F = c.ffn;
  const int tiles = (c.vocab + 63) / 64;
  const size_t nmax = std::max({3 * d, 2 * F, d});
  const size_t split_floats = std::min<size_t>((size_t)kSplitFloats, 16 * (size_t)n * nmax);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  tl::Workspace x{};
  x.hA = static_cast<float*>(take(R * d * 4));
  x.hB = static_cast<float*>(take(R * d * 4));
  x.hX = static_cast<float*>(take(R * d * 4));
  x.hE = static_cast<float*>(take(R * d * 4));
  x.x16 = take(R * d * m->esz);
  x.x16b = take(R * d * m->esz);
  x.q16 = take(R * d * m->esz);
  x.o16 = take(R * d * m->esz);
  x.u16 = take(R * F * m->esz);
  x.xh = take(R * d * m->esz);
  x.rowsA = static_cast<RowInfo*>(take(R * sizeof(RowInfo)));
  x.rowsB = static_cast<RowInfo*>(take(R * sizeof(RowInfo)));
  x.dest = static_cast<int32_t*>(take(R * 4));
  x.count = static_cast<int32_t*>(take(256));
  x.tok = static_cast<int32_t*>(take(R * 4));
  x.tok2 = static_cast<int32_t*>(take(R * 4));
  x.part_v = static_cast<float*>(take(R * tiles * 4));
  x.part_i = static_cast<int32_t*>(take(R * tiles * 4));
  x.part_v2 = static_cast<float*>(take(R * tiles * 4));
  x.splitk = static_cast<float*>(take(split_floats * 4));
  x.attn_part = static_cast<float*>(take((size_t)kAttnPartFloats * 4));
  x.kv_scratch = nullptr;
  x.kv_scratch_elems = 0;
  x.rows = (int)R;
  x.outs = (int)R;
  x.part_tiles = tiles;
  void* st = take(stage_bytes);
  if (w) *w = x;
  if (stage) *stage = st;
  return off;
}

tl_status tl_decode_step_noalloc(tl_model* m, int32_t n, const int32_t* lanes, const int32_t* req_L,
                                 const int32_t* in_tokens, int32_t* out_tokens, float* out_logits,
                                 float* out_hidden, int32_t* out_eff_L, void* stream) {
  g_err.clear();
  if (!m || !lanes || !req_L || !out_tokens) return fail(TL_E_ARG, "NULL argument");
  if (n < 1) return fail(TL_E_ARG, "n_lanes must be >= 1");
  if (m->kv_mode != TL_KV_KV)
    return fail(TL_E_UNSUPPORTED, "the store-h cache modes allocate rebuild buffers; use tl_decode_step");
  const size_t stage_need = ((size_t)n * sizeof(RowInfo) + 255) / 256 * 256 + (size_t)n * 4 + 256;
  const size_t need = noalloc_layout(m, n, stage_need, nullptr, nullptr, nullptr);
  if (need > kNoAllocScratchBytes)
    return fail(TL_E_ARG, "%d lanes need %zu bytes of scratch, more than the %zu the library holds per device", n,
                need, (size_t)kNoAllocScratchBytes);
  std::vector<int> eff;
  TRY(decode_check(m, n, lanes, req_L, in_tokens, eff));
  uint8_t* base = static_cast<uint8_t*>(noalloc_scratch(m->device));
  if (!base) return fail(TL_E_STATE, "no scratch on device %d", m->device);
  tl::Workspace w{};
  void* stage_area = nullptr;
  noalloc_layout(m, n, stage_need, base, &w, &stage_area);
  std::vector<RowInfo> rows;
  Stage st;
  size_t o_rows = 0, o_lanes = 0;
  decode_stage(m, n, lanes, eff, rows, st, &o_rows, &o_lanes);
  if (st.buf.size() > stage_need || st.buf.size() > m->stage_bytes || !m->stage_host)
    return fail(TL_E_STATE, "descriptors of %zu bytes do not fit the staging area", st.buf.size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(stream_handover(m, s));
  // descriptors: the model's pinned host area (allocated at load) -> the scratch
  HIPCHK(hipEventSynchronize(m->stage_done));
  std::memcpy(m->stage_host, st.buf.data(), st.buf.size());
  HIPCHK(hipMemcpyAsync(stage_area, m->stage_host, st.buf.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipEventRecord(m->stage_done, s));
  // run on the scratch: the model's own workspace, staging pointer and timing are
  // put back on every return
  struct Restore {
    tl_model* m;
    tl::Workspace ws;
    void* ov;
    bool timing;
    ~Restore() {
      m->ws = ws;
      m->stage_override = ov;
      m->timing = timing;
    }
  } restore{m, m->ws, m->stage_override, m->timing};
  m->ws = w;
  m->stage_override = stage_area;
  m->timing = false;   // timing records events it may first have to create
  return decode_run_step(m, n, lanes, eff, rows, o_rows, o_lanes, in_tokens, out_tokens, out_logits, out_hidden,
                         out_eff_L, nullptr, s);
}

// Early-exit buffers for n rows.
tl_status ensure_ee(tl_model* m, int n, hipStream_t s) {
  const tl_config& c = m->cfg;
  if (n > m->ee_rows) {
    HIPCHK(hipStreamSynchronize(s));
    dev_free(m, m->ee_eff);
    dev_free(m, m->ee_hprev);
    dev_free(m, m->ee_margin);
    if (!m->ee_live) m->ee_live = static_cast<int32_t*>(dev_alloc(m, 256));
    const int R = (n + 63) / 64 * 64;
    m->ee_eff = static_cast<int32_t*>(dev_alloc(m, (size_t)R * 4));
    m->ee_hprev = static_cast<float*>(dev_alloc(m, (size_t)R * c.d_model * 4));
    m->ee_margin = static_cast<float*>(dev_alloc(m, (size_t)R * 4));
    if (m->ee_eff_host) HIPCHK(hipHostFree(m->ee_eff_host));
    m->ee_eff_host = nullptr;
    HIPCHK(hipHostMalloc((void**)&m->ee_eff_host, (size_t)R * 4, hipHostMallocDefault));
    m->ee_rows = (m->ee_live && m->ee_eff && m->ee_hprev && m->ee_margin) ? R : 0;
    if (!m->ee_rows) return fail(TL_E_OOM, "early-exit buffers for %d rows", n);
  }
  return TL_OK;
}

tl_status tl_decode_step_ee(tl_model* m, int32_t n, const int32_t* lanes, const int32_t* req_L,
                            const tl_early_exit* ee, const int32_t* in_tokens, int32_t* out_tokens,
                            float* out_logits, float* out_hidden, int32_t* out_eff_L, void* stream) {
  g_err.clear();
  if (!m || !lanes || !req_L || !out_tokens || !ee) return fail(TL_E_ARG, "NULL argument");
  if (ee->patience < 0 || ee->min_L < 1 || ee->peek_every < 1 || !(ee->tau >= 0.f) || !(ee->logit_margin >= 0.f))
    return fail(TL_E_ARG, "early-exit rule: patience >= 0, min_L >= 1, peek_every >= 1, tau >= 0, logit_margin >= 0");
  const tl_config& c = m->cfg;
  if (n < 1) return fail(TL_E_ARG, "n_lanes must be >= 1");
  std::vector<char> seen(c.max_lanes, 0);
  std::vector<int> eff(n);
  for (int i = 0; i < n; ++i) {
    const int l = lanes[i];
    if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
    if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
    seen[l] = 1;
    if (req_L[i] < 1) return fail(TL_E_ARG, "requested L %d < 1", req_L[i]);
    const Lane& ln = m->lanes[l];
    if (!ln.live) return fail(TL_E_STATE, "lane %d was never prefilled", l);
    if (ln.len >= ln.cap) return fail(TL_E_STATE, "lane %d is full (%d positions)", l, ln.cap);
    if (!in_tokens && !ln.pending) return fail(TL_E_STATE, "lane %d holds no pending token (append first)", l);
    eff[i] = std::min(req_L[i], ln.ceiling);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(ensure_ws(m, n, n, 0, s));
  TRY(ensure_ee(m, n, s));
  std::vector<RowInfo> rows(n);
  std::vector<int32_t> lane_ids(lanes, lanes + n), eff32(eff.begin(), eff.end()), live0(1, n);
  for (int i = 0; i < n; ++i) {
    rows[i] = RowInfo{};
    rows[i].orig = i;
    rows[i].lane = lanes[i];
    rows[i].pos = m->lanes[lanes[i]].len;
    rows[i].depth = eff[i];
    rows[i].iter = 1;
  }
  Stage st;
  const size_t o_rows = st.add(rows), o_lanes = st.add(lane_ids), o_eff = st.add(eff32), o_live = st.add(live0);
  TRY(stage_upload(m, st, s));
  HIPCHK(hipMemcpyAsync(m->ee_eff, staged<int32_t>(m, o_eff), (size_t)n * 4, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(m->ee_live, staged<int32_t>(m, o_live), 4, hipMemcpyDeviceToDevice, s));
  const int32_t* lanes_dev = staged<int32_t>(m, o_lanes);
  const int32_t* toks = in_tokens;
  if (!toks) {
    HIPCHK(launch_gather_i32(m->d_pending, lanes_dev, n, m->ws.tok, s));
    toks = m->ws.tok;
  }
  Pass p;
  p.n = n;
  p.tokens = toks;
  p.rows0 = staged<RowInfo>(m, o_rows);
  p.rows_host = &rows;
  p.n_active = active_counts(eff);
  p.kv = KVParams{m->kv_base, m->d_lane_off, m->d_lane_cap, c.n_heads, c.head_dim, 0, 0};
  p.final_h = out_hidden ? out_hidden : m->ws.hX;
  p.ee = ee;
  p.one_row_per_lane = true;
  TRY(run_pass(m, p, s));
  TRY(run_head(m, p.final_h, nullptr, n, out_logits, out_tokens, lanes_dev, s));
  HIPCHK(hipMemcpyAsync(m->ee_eff_host, m->ee_eff, (size_t)n * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  for (int i = 0; i < n; ++i) {
    Lane& ln = m->lanes[lanes[i]];
    const int e = m->ee_eff_host[i];
    ln.len += 1;
    ln.pending = true;
    ln.ceiling = e;
    if (out_eff_L) out_eff_L[i] = e;
  }
  return TL_OK;
}

tl_status tl_export_w4(tl_model* m, int32_t block, int32_t matrix, int8_t* q_host, uint16_t* s_host) {
  g_err.clear();
  if (!m || !q_host || !s_host) return fail(TL_E_ARG, "NULL argument");
  const tl_config& c = m->cfg;
  if (block < 0 || block >= (int)m->blocks.size() || !m->blocks[block].is_w4)
    return fail(TL_E_ARG, "block %d is not a W4G128 block", block);
  if (matrix < 0 || matrix > 4) return fail(TL_E_ARG, "matrix %d out of range", matrix);
  const BlockDev& B = m->blocks[block];
  const MatDev& md = matrix == 0 ? B.qkv : matrix == 1 ? B.o : matrix == 4 ? B.down : B.gu;
  const int N = md.N, K = md.K;
  int8_t* dq = static_cast<int8_t*>(dev_alloc(m, (size_t)N * K));
  uint16_t* ds = static_cast<uint16_t*>(dev_alloc(m, (size_t)N * (K / 128) * 2));
  if (!dq || !ds) {
    dev_free(m, dq);
    dev_free(m, ds);
    return fail(TL_E_OOM, "export buffers");
  }
  tl_status st = TL_OK;
  hipError_t e = launch_w4_export(md.w4, md.s4, md.perm, N, K, dq, ds, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    // gate/up live stacked [gate; up] in canonical order after export
    const size_t rows = (matrix == 2 || matrix == 3) ? (size_t)c.ffn : (size_t)N;
    const size_t row0 = matrix == 3 ? (size_t)c.ffn : 0;
    e = hipMemcpy(q_host, dq + row0 * K, rows * K, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(s_host, ds + row0 * (K / 128), rows * (K / 128) * 2, hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) st = fail(TL_E_HIP, "export: %s", hipGetErrorString(e));
  dev_free(m, dq);
  dev_free(m, ds);
  return st;
}

tl_status tl_timing_enable(tl_model* m, int32_t on) {
  g_err.clear();
  if (!m) return fail(TL_E_ARG, "NULL model");
  TRY(flush_timing(m));
  m->timing = on != 0;
  return TL_OK;
}

tl_status tl_timing_read(tl_model* m, double* total_ms, int64_t* launches) {
  g_err.clear();
  if (!m || !total_ms || !launches) return fail(TL_E_ARG, "NULL argument");
  TRY(flush_timing(m));
  for (int i = 0; i < TL_TIMING_CLASSES; ++i) {
    total_ms[i] = m->t_ms[i];
    launches[i] = m->t_n[i];
    m->t_ms[i] = 0.0;
    m->t_n[i] = 0;
  }
  return TL_OK;
}

tl_status tl_timing_read_kernels(tl_model* m, double* kernel_ms, int64_t* kernels) {
  g_err.clear();
  if (!m || !kernel_ms || !kernels) return fail(TL_E_ARG, "NULL argument");
  TRY(flush_timing(m));
  for (int i = 0; i < TL_TIMING_CLASSES; ++i) {
    kernel_ms[i] = m->tk_ms[i];
    kernels[i] = m->tk_n[i];
    m->tk_ms[i] = 0.0;
    m->tk_n[i] = 0;
  }
  const bool short_ = m->kev_short;
  m->kev_short = false;
  if (short_) return fail(TL_E_HIP, "some product launches went untimed: no event could be created");
  return TL_OK;
}

// Continuous depth batching ("Continuous Depth Batching" summary page): work is
// scheduled one loop iteration at a time.  A pool holds one in-flight token per
// lane, each at its own iteration; every tick applies the loop stack once to the
// whole pool and compacts out the tokens that just ran their last iteration.
// Those wait in the boundary queue; the boundary stages (post blocks, final norm,
// head, greedy token; then embedding and pre blocks of the lane's next token) run
// on the whole queue once it holds boundary_min lanes or the pool is empty, and
// the lanes re-enter the pool at iteration 1.  The depth of every token is known
// when it enters (clamped request), so the whole schedule, including every exit,
// is computed on the host first, uploaded in one transfer and enqueued without
// waiting on the device.
tl_status tl_decode_run(tl_model* m, int32_t n, const int32_t* lanes, int32_t n_steps, const int32_t* L_req,
                        const int32_t* in_tokens, int32_t* out_tokens, float* out_hidden, int32_t* out_eff_L,
                        int32_t boundary_min, void* stream) {
  g_err.clear();
  if (!m || !lanes || !L_req || !out_tokens) return fail(TL_E_ARG, "NULL argument");
  const tl_config& c = m->cfg;
  if (n < 1 || n_steps < 1) return fail(TL_E_ARG, "n_lanes and n_steps must be >= 1");
  tl_log(2, "tl_decode_run: %d lanes x %d steps, boundary queue %d", n, n_steps, boundary_min);
  if (m->kv_mode != TL_KV_KV) return fail(TL_E_UNSUPPORTED, "continuous depth decoding needs kv_mode TL_KV_KV");
  std::vector<char> seen(c.max_lanes, 0);
  for (int i = 0; i < n; ++i) {
    const int l = lanes[i];
    if (l < 0 || l >= c.max_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", l, c.max_lanes);
    if (seen[l]) return fail(TL_E_ARG, "lane %d listed twice", l);
    seen[l] = 1;
    const Lane& ln = m->lanes[l];
    if (!ln.live) return fail(TL_E_STATE, "lane %d was never prefilled", l);
    if (ln.len + n_steps > ln.cap) return fail(TL_E_STATE, "lane %d has room for %d more positions", l, ln.cap - ln.len);
    if (!ln.pending) return fail(TL_E_STATE, "lane %d holds no pending token (append first)", l);
    for (int t = 0; t < n_steps; ++t)
      if (L_req[(int64_t)i * n_steps + t] < 1) return fail(TL_E_ARG, "requested L < 1 (lane %d step %d)", l, t);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(ensure_ws(m, n, n, 0, s));

  // ---- host simulation of the schedule
  struct Item { int i, j, L, pos; };
  struct Tick {
    int n_exit = 0, n_enter = 0, n_pool = 0, n_keep = 0;
    size_t o_xrows = 0, o_xidx = 0, o_xlanes = 0, o_xout = 0, o_erows = 0, o_elanes = 0, o_etok = 0;
  };
  std::vector<int> t(n, 0), ceil_(n), len(n);
  std::vector<int32_t> eff((size_t)n * n_steps, 0);
  for (int i = 0; i < n; ++i) {
    ceil_[i] = m->lanes[lanes[i]].ceiling;
    len[i] = m->lanes[lanes[i]].len;
  }
  std::vector<Item> pool, waiting;
  std::vector<int> enter(n);
  std::iota(enter.begin(), enter.end(), 0);
  std::vector<Tick> ticks;
  Stage st;
  const int bmin = std::max(1, boundary_min);
  bool first = true;
  while (first || !pool.empty() || !waiting.empty()) {
    Tick tk;
    if (!first && !waiting.empty() && ((int)waiting.size() >= bmin || pool.empty())) {
      // boundary stages for every waiting lane; lanes with steps left re-enter
      std::vector<RowInfo> xr;
      std::vector<int32_t> xi, xl, xo;
      for (const Item& it : waiting) {
        RowInfo r{};
        r.orig = it.i;
        r.lane = lanes[it.i];
        r.pos = it.pos;
        r.depth = it.L;
        r.iter = it.j;
        xr.push_back(r);
        xi.push_back(it.i);
        xl.push_back(lanes[it.i]);
        xo.push_back(it.i * n_steps + t[it.i]);
        t[it.i] += 1;
        if (t[it.i] < n_steps) enter.push_back(it.i);
      }
      tk.n_exit = (int)xr.size();
      tk.o_xrows = st.add(xr);
      tk.o_xidx = st.add(xi);
      tk.o_xlanes = st.add(xl);
      tk.o_xout = st.add(xo);
      waiting.clear();
    }
    first = false;
    if (!enter.empty()) {
      std::vector<RowInfo> er;
      std::vector<int32_t> el, etok;
      for (int i : enter) {
        const int L = std::min(L_req[(int64_t)i * n_steps + t[i]], ceil_[i]);
        ceil_[i] = L;
        eff[(size_t)i * n_steps + t[i]] = L;
        RowInfo r{};
        r.orig = i;
        r.lane = lanes[i];
        r.pos = len[i] + t[i];
        r.depth = L;
        r.iter = 1;
        er.push_back(r);
        el.push_back(lanes[i]);
        etok.push_back(i * n_steps + t[i]);
        pool.push_back(Item{i, 1, L, r.pos});
      }
      tk.n_enter = (int)er.size();
      tk.o_erows = st.add(er);
      tk.o_elanes = st.add(el);
      tk.o_etok = st.add(etok);
      enter.clear();
    }
    tk.n_pool = (int)pool.size();
    std::vector<Item> keep;
    for (Item it : pool) {
      if (it.L > it.j) {
        it.j += 1;
        keep.push_back(it);
      } else {
        waiting.push_back(it);
      }
    }
    tk.n_keep = (int)keep.size();
    pool.swap(keep);
    ticks.push_back(tk);
  }
  TRY(stage_upload(m, st, s));

  // ---- enqueue every tick: boundary batch, entering lanes, one loop-stack pass
  auto& w = m->ws;
  const int d = c.d_model;
  KVParams kv{m->kv_base, m->d_lane_off, m->d_lane_cap, c.n_heads, c.head_dim, 0, 0};
  float* hcur = w.hA;
  float* hnxt = w.hB;
  RowInfo* rcur = w.rowsA;
  RowInfo* rnxt = w.rowsB;
  int npool = 0;
  for (const Tick& tk : ticks) {
    if (tk.n_exit) {
      const RowInfo* xr = staged<RowInfo>(m, tk.o_xrows);
      HIPCHK(launch_gather_rows(w.hX, staged<int32_t>(m, tk.o_xidx), tk.n_exit, d, w.hE, s));
      kv.s1 = 0;
      for (int b = 0; b < c.n_post; ++b) {
        kv.s0 = c.n_pre + b;
        TRY(run_block(m, c.n_pre + c.n_loop + b, w.hE, xr, tk.n_exit, kv, s, nullptr, 0, false, nullptr, -1,
                      nullptr, true));
      }
      TRY(run_head(m, w.hE, nullptr, tk.n_exit, nullptr, w.tok2, staged<int32_t>(m, tk.o_xlanes), s));
      HIPCHK(launch_scatter_i32(w.tok2, staged<int32_t>(m, tk.o_xout), tk.n_exit, out_tokens, s));
      if (out_hidden) HIPCHK(launch_scatter_rows(w.hE, staged<int32_t>(m, tk.o_xout), tk.n_exit, d, out_hidden, s));
    }
    if (tk.n_enter) {
      const RowInfo* er = staged<RowInfo>(m, tk.o_erows);
      float* hin = hcur + (int64_t)npool * d;
      if (in_tokens) HIPCHK(launch_gather_i32(in_tokens, staged<int32_t>(m, tk.o_etok), tk.n_enter, w.tok, s));
      else HIPCHK(launch_gather_i32(m->d_pending, staged<int32_t>(m, tk.o_elanes), tk.n_enter, w.tok, s));
      TIMED(TL_T_EMBED, HIPCHK(launch_embed(c.boundary_dtype, m->embed, w.tok, tk.n_enter, d, hin, m->d_err, c.vocab, s)));
      kv.s1 = 0;
      for (int b = 0; b < c.n_pre; ++b) {
        kv.s0 = b;
        TRY(run_block(m, b, hin, er, tk.n_enter, kv, s, nullptr, 0, false, nullptr, -1, nullptr, true));
      }
      HIPCHK(hipMemcpyAsync(rcur + npool, er, sizeof(RowInfo) * tk.n_enter, hipMemcpyDeviceToDevice, s));
      npool += tk.n_enter;
    }
    if (tk.n_pool) {
      for (int l = 0; l < c.n_loop; ++l) {
        kv.s0 = c.n_pre + c.n_post + l - c.n_loop;
        kv.s1 = c.n_loop;
        TRY(run_block(m, c.n_pre + l, hcur, rcur, npool, kv, s, nullptr, 0, false, nullptr, -1, nullptr, true));
      }
      TIMED(TL_T_COMPACT, HIPCHK(launch_compact(rcur, npool, 0, rnxt, w.dest, w.count, nullptr, nullptr, s));
                          HIPCHK(launch_move_rows(hcur, w.dest, rcur, npool, d, hnxt, w.hX, s)));
      std::swap(hcur, hnxt);
      std::swap(rcur, rnxt);
      npool = tk.n_keep;
    }
  }
  for (int i = 0; i < n; ++i) {
    Lane& ln = m->lanes[lanes[i]];
    ln.len += n_steps;
    ln.ceiling = ceil_[i];
  }
  if (out_eff_L) std::memcpy(out_eff_L, eff.data(), eff.size() * 4);
  return TL_OK;
}

}  // extern "C"
