// Causal softmax attention of each row over its own lane's K/V in the cache slot
// of the current block application (one slot per block application: the K/V a
// loop iteration attends to are the ones that same iteration wrote at earlier
// positions).  Row r at position p attends to positions 0..p of its slot; scale
// 1/sqrt(head_dim); one K/V head per query head.
//
// Rows (decode, or prefill where the tiled kernel does not apply): one workgroup
// per (row, head), its four waves taking every fourth block of positions
// (split over the keys, merged through LDS at the end).  Inside a wave a group of
// lanes holds one key row, 16 bytes per lane, so each load instruction reads
// several whole K (and V) rows; the K and V of a block are requested together.
// The lanes that form a key's score also hold that key's V slice, so P V needs no
// data exchange until the final merge.  Online softmax in fp32.  The tiled kernel
// below serves prefill runs of consecutive rows.
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

#include <algorithm>

namespace {

template <class T> struct Row16;   // 16 bytes of a K/V row
template <> struct Row16<f16> { typedef half8 type; };
template <> struct Row16<bf16> { typedef bf16x8 type; };
template <> struct Row16<float> { typedef floatx4 type; };

// LPK lanes per key (a power of two >= head_dim / elements-per-16-bytes; lanes
// past the row hold zeros), 64 / LPK keys per load instruction, U loads per lane
// per block of P = (64 / LPK) * U positions.  UD = 4 (2) cuts blocks to a quarter
// (half), for contexts one (two) full blocks would hold: all four waves then take
// part.
//
// With qp.part set the workgroup first finishes its row's q, k and v from the QKV
// product's split-K partials (QkvParts): the arithmetic of the split-K QKV epilogue
// (sums in split order, the same rotation and roundings), k and v stored into the
// cache at the row's position, q kept in LDS; one kernel fewer per block on a
// decode pass.
//
// Position split (nsplit > 1, grid y): workgroup (row, head, y) attends to the
// y-th run of a row's position blocks and leaves its unnormalised (max, sum,
// output) in part[((row H + head) nsplit + y)][dh + 2]; attn_merge_kernel then
// combines the runs in order.  Every split forms q; only the split holding the
// row's own position stores its k and v.
template <class T, int LPK, int UD>
__global__ __launch_bounds__(256) void attn_rows_kernel(const T* __restrict__ q, const RowInfo* __restrict__ rows,
                                                       KVParams kv, T* __restrict__ out, int d, float scale,
                                                       const int32_t* live, QkvParts qp, int nsplit,
                                                       float* __restrict__ part) {
  typedef typename Row16<T>::type R16;
  constexpr int EPL = 16 / (int)sizeof(T);   // elements per lane of a key row
  constexpr int KPI = 64 / LPK;              // keys per load instruction
  constexpr int U = (LPK < 16 ? LPK : 16) / UD;
  static_assert(U >= 1, "block");
  constexpr int P = KPI * U;                 // positions per block
  const int H = kv.H, dh = kv.dh;
  const int r = blockIdx.x / H, h = blockIdx.x - r * H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane / LPK, k = lane % LPK;   // key in the instruction, 16-byte chunk of the row
  const bool kin = k * EPL < dh;
  // fused QKV finish: thread t < 3 dh/2 takes section t / (dh/2) (q, k, v) and pair
  // p of the head, kernel columns cd = (p / G) 2G + p mod G and cd + G; the first
  // eight splits' partials are requested before the row descriptor arrives
  const int half = dh >> 1;
  const bool fz = qp.part != nullptr && tid < 3 * half;
  const int sec = tid / half, pq = tid - sec * half;
  const int cd = qp.G > 0 ? (pq / qp.G) * 2 * qp.G + pq % qp.G : 0;
  const int64_t pc = (int64_t)sec * d + h * dh + cd;
  float a0[8], a1[8];
  if (fz) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* pr = qp.part + ((int64_t)min(u, qp.S - 1) * qp.M + r) * qp.N + pc;
      a0[u] = pr[0];
      a1[u] = pr[qp.G];
    }
  }
  // a finished q is likewise requested with the descriptor
  R16 qx{};
  if (!qp.part && kin) qx = *reinterpret_cast<const R16*>(q + (int64_t)r * d + h * dh + k * EPL);
  const RowInfo ri = rows[r];
  if (gate_closed(live)) return;
  T* op = out + (int64_t)r * d + h * dh;
  if (ri.done) {   // finished by early exit: carried only, its state no longer matters
    if (blockIdx.y == 0 && tid < 64 && kin) {
      R16 z;
#pragma unroll
      for (int e = 0; e < EPL; ++e) z[e] = from_f32<T>(0.f);
      if (g == 0) *reinterpret_cast<R16*>(op + k * EPL) = z;
    }
    return;
  }
  const T* Kp = kv_ptr<T>(kv, ri, 0, h, 0);
  const T* Vp = kv_ptr<T>(kv, ri, 1, h, 0);
  const int npos = ri.pos + 1;
  const int nblk = (npos + P - 1) / P;
  // this split's run of position blocks [b0, b1)
  const int bs = (nblk + nsplit - 1) / nsplit;
  const int b0 = min(nblk, (int)blockIdx.y * bs), b1 = min(nblk, b0 + bs);
  const bool own_pos = b0 < b1 && b1 == nblk;   // the run holding the row's own position
  float qv[EPL];
  if (qp.part) {
    // after the rotation the pair's values go to p and p + dh/2 (q, k); V keeps
    // kernel order
    __shared__ float qs[128];
    const int G = qp.G, p = pq;
    if (fz) {
      float v0 = 0.f, v1 = 0.f;   // split order, as the split-K QKV epilogue adds them
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < qp.S) {
          v0 += a0[u];
          v1 += a1[u];
        }
      for (int z = 8; z < qp.S; ++z) {
        const float* pr = qp.part + ((int64_t)z * qp.M + r) * qp.N + pc;
        v0 += pr[0];
        v1 += pr[G];
      }
      if (sec == 2) {
        if (own_pos) {
          T* vp = kv_ptr<T>(kv, ri, 1, h, ri.pos);
          vp[cd] = from_f32<T>(v0);
          vp[cd + G] = from_f32<T>(v1);
        }
      } else {
        const float cs = qp.rope_cos[(int64_t)ri.pos * half + p];
        const float sn = qp.rope_sin[(int64_t)ri.pos * half + p];
        const T x1 = from_f32<T>(rot_x1(v0, v1, cs, sn));
        const T x2 = from_f32<T>(rot_x2(v0, v1, cs, sn));
        if (sec == 0) {
          qs[p] = (float)x1;
          qs[p + half] = (float)x2;
        } else if (own_pos) {
          T* kp = kv_ptr<T>(kv, ri, 0, h, ri.pos);
          kp[p] = x1;
          kp[p + half] = x2;
        }
      }
    }
    // this position's K/V stored (workgroup-visible) and q in LDS
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = kin ? qs[k * EPL + e] * scale : 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = (float)qx[e] * scale;
  }
  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int b = b0 + wv; b < b1; b += 4) {
    const int t0 = b * P;
    R16 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tc = min(t0 + u * KPI + g, npos - 1);   // clamped: masked below, V weighted by 0
      kr[u] = R16{};
      vr[u] = R16{};
      if (kin) {
        kr[u] = *reinterpret_cast<const R16*>(Kp + (int64_t)tc * dh + k * EPL);
        vr[u] = *reinterpret_cast<const R16*>(Vp + (int64_t)tc * dh + k * EPL);
      }
    }
    float sc[U], cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(qv[e], (float)kr[u][e], a);
#pragma unroll
      for (int x = 1; x < LPK; x <<= 1) a += __shfl_xor(a, x, 64);
      sc[u] = (t0 + u * KPI + g < npos) ? a : -INFINITY;
      cm = fmaxf(cm, sc[u]);
    }
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) cm = fmaxf(cm, __shfl_xor(cm, x, 64));
    const float mn = fmaxf(m, cm);
    const float corr = expf(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = expf(sc[u] - mn);
      ls += pu;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pu, (float)vr[u][e], o[e]);
    }
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) ls += __shfl_xor(ls, x, 64);
    l = l * corr + ls;
    m = mn;
  }
  // this wave's output: add the key groups' partial sums
#pragma unroll
  for (int e = 0; e < EPL; ++e)
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) o[e] += __shfl_xor(o[e], x, 64);
  __shared__ float wm[4], wl[4];
  __shared__ float wo[4][128];
  if (lane == 0) {
    wm[wv] = m;
    wl[wv] = l;
  }
  if (g == 0 && kin) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) wo[wv][k * EPL + e] = o[e];
  }
  __syncthreads();
  if (wv == 0 && g == 0 && kin) {
    // wave 0 saw the run's first block: M = -inf only for an empty run of a split
    const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    if (nsplit > 1) {
      float* pp = part + ((int64_t)blockIdx.x * nsplit + blockIdx.y) * (dh + 2);
      float f[4], L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = M == -INFINITY ? 0.f : expf(wm[w] - M);
        L += wl[w] * f[w];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += wo[w][k * EPL + e] * f[w];
        pp[2 + k * EPL + e] = acc;
      }
      if (k == 0) {
        pp[0] = M;
        pp[1] = L;
      }
      return;
    }
    float f[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[w] = expf(wm[w] - M);   // 0 for a wave without positions (m = -inf)
      L += wl[w] * f[w];
    }
    const float inv = 1.0f / L;
    R16 res;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += wo[w][k * EPL + e] * f[w];
      res[e] = from_f32<T>(acc * inv);
    }
    *reinterpret_cast<R16*>(op + k * EPL) = res;
  }
}

// The position-split runs of attn_rows_kernel combined, one workgroup per (row,
// head), thread t < dh taking output dimension t: with M the largest run maximum,
// out = sum_y O_y e^(m_y - M) / sum_y l_y e^(m_y - M), runs added in order (empty
// runs, m = -inf, skipped).  Rows marked done keep the zero output already written.
template <class T>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part, int nsplit, int H, int dh,
                                                        const RowInfo* __restrict__ rows, T* __restrict__ out, int d,
                                                        const int32_t* live) {
  const int rh = blockIdx.x, r = rh / H, h = rh - r * H, t = threadIdx.x;
  const RowInfo ri = rows[r];
  if (gate_closed(live) || ri.done) return;
  const float* pp = part + (int64_t)rh * nsplit * (dh + 2);
  float M = -INFINITY;
  for (int y = 0; y < nsplit; ++y) M = fmaxf(M, pp[y * (dh + 2)]);
  float L = 0.f, acc = 0.f;
  for (int y = 0; y < nsplit; ++y) {
    const float my = pp[y * (dh + 2)];
    if (my == -INFINITY) continue;
    const float f = expf(my - M);
    L += pp[y * (dh + 2) + 1] * f;
    if (t < dh) acc += pp[y * (dh + 2) + 2 + t] * f;
  }
  if (t < dh) out[(int64_t)r * d + h * dh + t] = from_f32<T>(acc * (1.0f / L));
}

// ----------------------------------------------------------------------------
// Tiled causal attention for runs of consecutive query rows of one sequence.
// Workgroup = (tile of kAttnTileRows rows, head); wave w owns query rows
// 16w .. 16w+15.  Keys and values stream through LDS in blocks of 64 positions;
// the next block's K/V are loaded into registers while the current block
// computes (LDS-only barriers, so the loads stay in flight).  S = Q K^T and
// O += P V run on 16x16x32 MFMA (QK^T in the cache type, PV in fp16 with V
// converted on its way into LDS), with a running row max / sum in fp32 (online
// softmax).  The score tile leaves the MFMA in column-per-lane layout, so P goes
// through LDS to become the row-per-lane A operand of PV.
template <class T> struct QkMfma;
template <> struct QkMfma<f16> {
  typedef half8 frag;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct QkMfma<bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int kAttnTileRows = 32;
constexpr int kAttnWaves = kAttnTileRows / 16;

// The tile of this workgroup: from the closed form when the list has one, else
// loaded from the list.
__device__ __forceinline__ AttnTile attn_tile(const AttnTile* __restrict__ tiles, const AttnGrid& ug) {
  if (ug.on) {
    const int b = blockIdx.x, sq = b / ug.tps, p0 = (b - sq * ug.tps) * kAttnTileRows;
    AttnTile t;
    t.row0 = sq * ug.T + p0;
    t.nrows = min(kAttnTileRows, ug.T - p0);
    t.pos0 = p0;
    t.lane = 0;
    t.iter = ug.iter;
    t.cap = ug.cap;
    t.koff = ug.koff0 + (int64_t)sq * ug.kstride;
    return t;
  }
  return tiles[blockIdx.x];
}

template <class T, int DH>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_tiled_kernel(const T* __restrict__ q,
                                                                     const AttnTile* __restrict__ tiles, KVParams kv,
                                                                     T* __restrict__ out, int d, float scale,
                                                                     AttnGrid ug) {
  constexpr int NW = kAttnWaves, NT = 64 * NW;
  constexpr int KB = 64;
  constexpr int LDK = DH + 8;
  constexpr int LDV = KB + 8;
  constexpr int KS = DH / 32;
  constexpr int OT = DH / 16;
  constexpr int CH = KB * DH / 8;   // 16-byte chunks of one K (or V) block
  constexpr int CPT = CH / NT;      // per thread
  static_assert(CH % NT == 0, "block split");
  // V goes to LDS transposed (Vt[dim][key]): thread t < VP loads 8 consecutive keys
  // of one 8-wide dim chunk and writes each dim as one 16-byte row piece; the
  // 8-key slot of row r is XOR-ed with (r / 16) mod 8, so that the 16 lanes of a
  // write phase (dim chunks 0..15) hit distinct banks, and PV's reads undo it.
  constexpr int VP = (KB / 8) * (DH / 8);
  static_assert(VP <= NT && KB / 8 == 8, "V staging");
  typedef typename QkMfma<T>::frag qfrag;
  __shared__ __attribute__((aligned(16))) T Ks[KB * LDK];
  __shared__ __attribute__((aligned(16))) f16 Vt[DH * LDV];
  __shared__ __attribute__((aligned(16))) f16 Ps[NW][16 * LDV];

  const AttnTile tile = attn_tile(tiles, ug);
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int slot = kv.s0 + kv.s1 * tile.iter;
  int64_t cap, koff;
  if (tile.cap > 0) {   // carried by the descriptor: one round of dependent loads less
    cap = tile.cap;
    koff = tile.koff;
  } else {
    cap = kv.lane_cap[tile.lane];
    koff = kv.lane_off[tile.lane];
  }
  const T* Kg = reinterpret_cast<const T*>(kv.base) + koff + ((int64_t)(slot * 2) * kv.H + h) * cap * DH;
  const T* Vg = Kg + (int64_t)kv.H * cap * DH;
  const int kend = tile.pos0 + tile.nrows;

  // K/V block k0 -> registers; positions past the end are clamped to the last
  // valid one (their scores are masked, so P = 0 multiplies finite values)
  u32x4 rk[CPT], rv[8];
  const int vkg = tid / (DH / 8), vdc = tid % (DH / 8);   // V: 8-key group, 8-dim chunk
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i, key = c / (DH / 8), dc = (c % (DH / 8)) * 8;
      const int kp = min(k0 + key, kend - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)kp * DH + dc);
    }
    if (tid < VP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kp = min(k0 + 8 * vkg + i, kend - 1);
        rv[i] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)kp * DH + 8 * vdc);
      }
    }
  };
  load(0);

  const int qr = 16 * w + l16;
  qfrag qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int qrc = min(qr, tile.nrows - 1);
    qa[ks] = *reinterpret_cast<const qfrag*>(q + (int64_t)(tile.row0 + qrc) * d + h * DH + ks * 32 + 8 * g4);
  }
  floatx4 o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
  }
  const int qpos0 = tile.pos0 + 16 * w + 4 * g4;

  for (int k0 = 0; k0 < kend; k0 += KB) {
    lds_barrier();   // every wave is done reading the previous block
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i, key = c / (DH / 8), dc = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[key * LDK + dc]) = rk[i];
    }
    if (tid < VP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        half8 hv;
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = (f16)(float)reinterpret_cast<const T*>(&rv[i])[e];
        const int r = 8 * vdc + e;
        *reinterpret_cast<half8*>(&Vt[r * LDV + 8 * (vkg ^ ((r >> 4) & 7))]) = hv;
      }
    }
    lds_barrier();
    if (k0 + KB < kend) load(k0 + KB);
    asm volatile("" ::: "memory");   // keep the prefetch ahead of this block's math

    floatx4 sacc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      sacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const qfrag b = *reinterpret_cast<const qfrag*>(&Ks[(16 * n + l16) * LDK + ks * 32 + 8 * g4]);
        sacc[n] = QkMfma<T>::run(qa[ks], b, sacc[n]);
      }
    }
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[r] = -INFINITY;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = k0 + 16 * n + l16;
        float v = sacc[n][r] * scale;
        if (kp > qpos0 + r || kp >= kend) v = -INFINITY;
        sacc[n][r] = v;
        mx[r] = fmaxf(mx[r], v);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], off, 64));
    }
    float corr[4], rs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // a row with no key yet in this block keeps m = -inf; exp(-inf - -inf)
      // would be NaN, so its correction is 1 and its probabilities 0
      const float mn = fmaxf(mrow[r], mx[r]);
      corr[r] = mn == -INFINITY ? 1.f : expf(mrow[r] - mn);
      mrow[r] = mn;
      rs[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = sacc[n][r] == -INFINITY ? 0.f : expf(sacc[n][r] - mrow[r]);
        rs[r] += p;
        Ps[w][(4 * g4 + r) * LDV + 16 * n + l16] = (f16)p;
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) rs[r] += __shfl_xor(rs[r], off, 64);
      lrow[r] = lrow[r] * corr[r] + rs[r];
    }
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] *= corr[r];
    // P tile of this wave written by this wave only: a wave-level LDS barrier
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int kk = 0; kk < KB; kk += 32) {
      const half8 a = *reinterpret_cast<const half8*>(&Ps[w][l16 * LDV + kk + 8 * g4]);
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        const half8 b = *reinterpret_cast<const half8*>(&Vt[(16 * t + l16) * LDV + 8 * ((kk / 8 + g4) ^ (t & 7))]);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, o[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rl = 16 * w + 4 * g4 + r;
    if (rl >= tile.nrows) continue;
    const float inv = 1.0f / lrow[r];
    T* op = out + (int64_t)(tile.row0 + rl) * d + h * DH + l16;
#pragma unroll
    for (int t = 0; t < OT; ++t) op[16 * t] = from_f32<T>(o[t][r] * inv);
  }
}

// The same tiling for fp32 Q / K / V on fp16 MFMA: every fp32 operand x is split
// into x_hi = fp16(x) and x_lo = fp16(x - x_hi) on its way into registers or LDS
// (about 22 significant bits), and each product takes the three terms that carry
// them: S = Qh Kh^T + Qh Kl^T + Ql Kh^T, O += Ph Vh + Ph Vl + Pl Vh (the lo * lo
// term is below fp32 rounding).  Softmax statistics stay fp32.
template <int DH>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_tiled_split_kernel(const float* __restrict__ q,
                                                                           const AttnTile* __restrict__ tiles,
                                                                           KVParams kv, float* __restrict__ out, int d,
                                                                           float scale, AttnGrid ug) {
  constexpr int NW = kAttnWaves, NT = 64 * NW;
  constexpr int KB = 64;
  constexpr int LDK = DH + 8;
  constexpr int LDV = KB + 8;
  constexpr int KS = DH / 32;
  constexpr int OT = DH / 16;
  constexpr int CH = KB * DH / 4;   // 16-byte chunks (4 floats) of one K block
  constexpr int CPT = CH / NT;      // per thread
  static_assert(CH % NT == 0, "block split");
  // V: thread t < VP holds 8 consecutive keys of one 8-wide dim chunk (16 words)
  // and writes each dim as one 16-byte piece of the transposed row (hi and lo),
  // the 8-key slot XOR-ed with (row / 16) mod 8 as in attn_tiled_kernel
  constexpr int VP = (KB / 8) * (DH / 8);
  static_assert(VP <= NT && KB / 8 == 8, "V staging");
  __shared__ __attribute__((aligned(16))) f16 Kh[KB * LDK];
  __shared__ __attribute__((aligned(16))) f16 Kl[KB * LDK];
  __shared__ __attribute__((aligned(16))) f16 Vth[DH * LDV];
  __shared__ __attribute__((aligned(16))) f16 Vtl[DH * LDV];
  __shared__ __attribute__((aligned(16))) f16 Ph[NW][16 * LDV];
  __shared__ __attribute__((aligned(16))) f16 Pl[NW][16 * LDV];

  const AttnTile tile = attn_tile(tiles, ug);
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int slot = kv.s0 + kv.s1 * tile.iter;
  int64_t cap, koff;
  if (tile.cap > 0) {
    cap = tile.cap;
    koff = tile.koff;
  } else {
    cap = kv.lane_cap[tile.lane];
    koff = kv.lane_off[tile.lane];
  }
  const float* Kg = reinterpret_cast<const float*>(kv.base) + koff + ((int64_t)(slot * 2) * kv.H + h) * cap * DH;
  const float* Vg = Kg + (int64_t)kv.H * cap * DH;
  const int kend = tile.pos0 + tile.nrows;

  auto split8 = [](const float* x, half8& hi, half8& lo) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f16 xh = (f16)x[e];
      hi[e] = xh;
      lo[e] = (f16)(x[e] - (float)xh);
    }
  };

  u32x4 rk[CPT], rv[8][2];
  const int vkg = tid / (DH / 8), vdc = tid % (DH / 8);
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i, key = c / (DH / 4), dc = (c % (DH / 4)) * 4;
      const int kp = min(k0 + key, kend - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)kp * DH + dc);
    }
    if (tid < VP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kp = min(k0 + 8 * vkg + i, kend - 1);
        rv[i][0] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)kp * DH + 8 * vdc);
        rv[i][1] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)kp * DH + 8 * vdc + 4);
      }
    }
  };
  load(0);

  const int qr = 16 * w + l16;
  half8 qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int qrc = min(qr, tile.nrows - 1);
    const float* qp = q + (int64_t)(tile.row0 + qrc) * d + h * DH + ks * 32 + 8 * g4;
    float x[8];
    const floatx4 a = *reinterpret_cast<const floatx4*>(qp), b = *reinterpret_cast<const floatx4*>(qp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
    split8(x, qh[ks], ql[ks]);
  }
  floatx4 o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
  }
  const int qpos0 = tile.pos0 + 16 * w + 4 * g4;

  for (int k0 = 0; k0 < kend; k0 += KB) {
    lds_barrier();
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i, key = c / (DH / 4), dc = (c % (DH / 4)) * 4;
      const floatx4 v = __builtin_bit_cast(floatx4, rk[i]);
      half2v hi0, hi1, lo0, lo1;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f16 a = (f16)v[e], b = (f16)v[2 + e];
        hi0[e] = a;
        hi1[e] = b;
        lo0[e] = (f16)(v[e] - (float)a);
        lo1[e] = (f16)(v[2 + e] - (float)b);
      }
      *reinterpret_cast<half2v*>(&Kh[key * LDK + dc]) = hi0;
      *reinterpret_cast<half2v*>(&Kh[key * LDK + dc + 2]) = hi1;
      *reinterpret_cast<half2v*>(&Kl[key * LDK + dc]) = lo0;
      *reinterpret_cast<half2v*>(&Kl[key * LDK + dc + 2]) = lo1;
    }
    if (tid < VP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_bit_cast(floatx4, rv[i][e >> 2])[e & 3];
        half8 hv, lv;
        split8(x, hv, lv);
        const int r = 8 * vdc + e;
        const int at = r * LDV + 8 * (vkg ^ ((r >> 4) & 7));
        *reinterpret_cast<half8*>(&Vth[at]) = hv;
        *reinterpret_cast<half8*>(&Vtl[at]) = lv;
      }
    }
    lds_barrier();
    if (k0 + KB < kend) load(k0 + KB);
    asm volatile("" ::: "memory");

    floatx4 sacc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      sacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int at = (16 * n + l16) * LDK + ks * 32 + 8 * g4;
        const half8 bh = *reinterpret_cast<const half8*>(&Kh[at]);
        const half8 bl = *reinterpret_cast<const half8*>(&Kl[at]);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[ks], bh, sacc[n], 0, 0, 0);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[ks], bl, sacc[n], 0, 0, 0);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[ks], bh, sacc[n], 0, 0, 0);
      }
    }
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[r] = -INFINITY;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = k0 + 16 * n + l16;
        float v = sacc[n][r] * scale;
        if (kp > qpos0 + r || kp >= kend) v = -INFINITY;
        sacc[n][r] = v;
        mx[r] = fmaxf(mx[r], v);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], off, 64));
    }
    float corr[4], rs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mn = fmaxf(mrow[r], mx[r]);
      corr[r] = mn == -INFINITY ? 1.f : expf(mrow[r] - mn);
      mrow[r] = mn;
      rs[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = sacc[n][r] == -INFINITY ? 0.f : expf(sacc[n][r] - mrow[r]);
        rs[r] += p;
        const f16 ph = (f16)p;
        Ph[w][(4 * g4 + r) * LDV + 16 * n + l16] = ph;
        Pl[w][(4 * g4 + r) * LDV + 16 * n + l16] = (f16)(p - (float)ph);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) rs[r] += __shfl_xor(rs[r], off, 64);
      lrow[r] = lrow[r] * corr[r] + rs[r];
    }
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] *= corr[r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int kk = 0; kk < KB; kk += 32) {
      const half8 ah = *reinterpret_cast<const half8*>(&Ph[w][l16 * LDV + kk + 8 * g4]);
      const half8 al = *reinterpret_cast<const half8*>(&Pl[w][l16 * LDV + kk + 8 * g4]);
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        const int at = (16 * t + l16) * LDV + 8 * ((kk / 8 + g4) ^ (t & 7));
        const half8 bh = *reinterpret_cast<const half8*>(&Vth[at]);
        const half8 bl = *reinterpret_cast<const half8*>(&Vtl[at]);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, o[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rl = 16 * w + 4 * g4 + r;
    if (rl >= tile.nrows) continue;
    const float inv = 1.0f / lrow[r];
    float* op = out + (int64_t)(tile.row0 + rl) * d + h * DH + l16;
#pragma unroll
    for (int t = 0; t < OT; ++t) op[16 * t] = o[t][r] * inv;
  }
}

}  // namespace

int attn_tile_rows() { return kAttnTileRows; }

bool attn_tiled_supported(int dtype, int head_dim) {
  return (dtype == DT_F16 || dtype == DT_BF16 || dtype == DT_F32) &&
         (head_dim == 64 || head_dim == 96 || head_dim == 128);
}

hipError_t launch_attention_tiled(int dtype, const void* q, const AttnTile* tiles, int n_tiles, const KVParams& kv,
                                  void* out, hipStream_t s, const AttnGrid* grid) {
  if (n_tiles <= 0) return hipSuccess;
  AttnGrid ug{};
  if (grid && grid->on) {
    if (grid->T < 1 || grid->cap < grid->T || grid->tps != (grid->T + kAttnTileRows - 1) / kAttnTileRows ||
        n_tiles % grid->tps != 0)
      return hipErrorInvalidValue;
    ug = *grid;
  }
  const int d = kv.H * kv.dh;
  const float scale = 1.0f / sqrtf((float)kv.dh);
  dim3 grd(n_tiles, kv.H);
#define TL_ATTN_CASE(T, DHV)                                                                                   \
  if (kv.dh == DHV) {                                                                                          \
    TL_LAUNCH((attn_tiled_kernel<T, DHV>), grd, dim3(kAttnWaves * 64), 0, s, (const T*)q, tiles, kv, (T*)out, d, \
                       scale, ug);                                                                             \
    return hipGetLastError();                                                                                  \
  }
  if (dtype == DT_F16) {
    TL_ATTN_CASE(f16, 64)
    TL_ATTN_CASE(f16, 96)
    TL_ATTN_CASE(f16, 128)
  } else if (dtype == DT_BF16) {
    TL_ATTN_CASE(bf16, 64)
    TL_ATTN_CASE(bf16, 96)
    TL_ATTN_CASE(bf16, 128)
  } else if (dtype == DT_F32) {
#define TL_ATTN_SPLIT(DHV)                                                                                     \
  if (kv.dh == DHV) {                                                                                          \
    TL_LAUNCH((attn_tiled_split_kernel<DHV>), grd, dim3(kAttnWaves * 64), 0, s, (const float*)q, tiles, kv, \
                       (float*)out, d, scale, ug);                                                             \
    return hipGetLastError();                                                                                  \
  }
    TL_ATTN_SPLIT(64)
    TL_ATTN_SPLIT(96)
    TL_ATTN_SPLIT(128)
#undef TL_ATTN_SPLIT
  }
#undef TL_ATTN_CASE
  return hipErrorInvalidValue;
}

// Few (row, head) workgroups and long contexts: the positions are split over up to
// kAttnMaxSplit workgroups per (row, head), as many as keep the launch within
// kAttnSplitWGs workgroups, and merged by attn_merge_kernel.  max_ctx = 0 (unknown,
// or batch-invariant passes) never splits.
constexpr int kAttnSplitWGs = 256;
constexpr int kAttnMaxSplit = 16;

template <class T, int LPK>
void attn_rows_launch(const void* q, const RowInfo* rows, int n, const KVParams& kv, void* out, const int32_t* live,
                      int max_ctx, hipStream_t s, const QkvParts& qp, float* part) {
  const int d = kv.H * kv.dh;
  const float scale = 1.0f / sqrtf((float)kv.dh);
  constexpr int P = (64 / LPK) * (LPK < 16 ? LPK : 16);   // positions of a full block
  const int wgs = n * kv.H;
  int ns = 1;
  if (part && max_ctx > 4 * P && wgs < kAttnSplitWGs)
    ns = std::min(std::min(kAttnSplitWGs / wgs, (max_ctx + P - 1) / P), kAttnMaxSplit);
  const int ctx = (max_ctx + ns - 1) / ns;   // positions per run, at most
  const dim3 grid(wgs, ns);
  if (max_ctx > 0 && ctx <= P)
    TL_LAUNCH((attn_rows_kernel<T, LPK, 4>), grid, dim3(256), 0, s, (const T*)q, rows, kv, (T*)out,
                       d, scale, live, qp, ns, part);
  else if (max_ctx > 0 && ctx <= 2 * P)
    TL_LAUNCH((attn_rows_kernel<T, LPK, 2>), grid, dim3(256), 0, s, (const T*)q, rows, kv, (T*)out,
                       d, scale, live, qp, ns, part);
  else
    TL_LAUNCH((attn_rows_kernel<T, LPK, 1>), grid, dim3(256), 0, s, (const T*)q, rows, kv, (T*)out,
                       d, scale, live, qp, ns, part);
  if (ns > 1)
    TL_LAUNCH((attn_merge_kernel<T>), dim3(wgs), dim3(128), 0, s, (const float*)part, ns, kv.H, kv.dh, rows,
                       (T*)out, d, live);
}

template <class T>
hipError_t attn_rows_dispatch(const void* q, const RowInfo* rows, int n, const KVParams& kv, void* out,
                              const int32_t* live, int max_ctx, hipStream_t s, const QkvParts& qp, float* part) {
  const int chunks = kv.dh * (int)sizeof(T) / 16;   // 16-byte chunks of a row (head_dim is checked at load)
  if (chunks <= 4) attn_rows_launch<T, 4>(q, rows, n, kv, out, live, max_ctx, s, qp, part);
  else if (chunks <= 8) attn_rows_launch<T, 8>(q, rows, n, kv, out, live, max_ctx, s, qp, part);
  else if (chunks <= 16) attn_rows_launch<T, 16>(q, rows, n, kv, out, live, max_ctx, s, qp, part);
  else if (chunks <= 32) attn_rows_launch<T, 32>(q, rows, n, kv, out, live, max_ctx, s, qp, part);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const void* q, const RowInfo* rows, int n, const KVParams& kv, void* out,
                            const int32_t* live, int max_ctx, hipStream_t s, const QkvParts* qp, float* part) {
  if (n <= 0) return hipSuccess;
  if (kv.dh > 128 || (kv.dh * 4) % 16 != 0) return hipErrorInvalidValue;
  QkvParts p{};
  if (qp && qp->part) {
    // the prologue's threads cover 3 dh/2 pairs, pairs stay inside a head, and the
    // partials hold n rows of the 3 d columns
    if (3 * (kv.dh / 2) > 256 || qp->G <= 0 || kv.dh % (2 * qp->G) != 0 || qp->S < 1 || qp->M != n ||
        qp->N != 3 * kv.H * kv.dh || !qp->rope_cos || !qp->rope_sin)
      return hipErrorInvalidValue;
    p = *qp;
  }
  switch (dtype) {
    case DT_F32: return attn_rows_dispatch<float>(q, rows, n, kv, out, live, max_ctx, s, p, part);
    case DT_F16: return attn_rows_dispatch<f16>(q, rows, n, kv, out, live, max_ctx, s, p, part);
    case DT_BF16: return attn_rows_dispatch<bf16>(q, rows, n, kv, out, live, max_ctx, s, p, part);
    default: return hipErrorInvalidValue;
  }
}
