// GEMMs of the looped transformer: y = x W^T with fused epilogues.
//
// 16-bit operands (f16 / bf16) run on gfx950 MFMA (v_mfma_f32_16x16x32_*) with
// fp32 accumulation; tiles of A (activations) and B (weights) are staged through
// LDS by all four waves of a workgroup.  INT4 weights (symmetric, 128-wide groups
// along K) are unpacked in registers to exact fp16 integers on their way into LDS;
// each group's MFMA sum is multiplied by its fp32 scale afterwards, so
// sum_k x_k q_k s_g is formed without rounding q * s to fp16.
//
// Epilogues (columns are in the kernel's row order of W, see the engine):
//   QKV    : rotary embedding on q and k pairs, q to its buffer, k and v into the
//            row's KV cache slot (one slot per block application);
//   RESID  : h += acc (fp32 residual stream);
//   SWIGLU : u = silu(gate) * up on interleaved gate/up pairs;
//   HEAD   : optional fp32 logits and a per-tile (max, lowest argmax) partial;
//   STORE  : fp32 store.
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The loads of k step J of a stage's eight: pieces PPS J .. PPS (J + 1) - 1 of NP,
// and every piece left at the last step.
template <int PPS, int NP, int J, class P>
__device__ __forceinline__ void issue_pieces(P&& piece) {
  constexpr int b = PPS * J < NP ? PPS * J : NP;
  constexpr int e = J == 7 ? NP : (PPS * (J + 1) < NP ? PPS * (J + 1) : NP);
  static_for<b, e>(piece);
}

template <class AT> struct Mfma;
template <> struct Mfma<f16> {
  typedef half8 frag;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};


// Workgroup of 4 waves (2 x 2) computes a BM x BN tile over the K range of its
// split (blockIdx.z).  Per BK-wide K stage: global -> registers, issued D-1 stages
// ahead into a ring of D register sets (so D-1 stages of loads are in flight while
// a stage computes), registers -> LDS, then each wave runs (BM/32) x (BN/32)
// 16x16x32 MFMAs per 32-wide k step.  INT4 stages cover whole 128-wide groups; each group's MFMA sum
// is scaled when the group ends.  With several splits each workgroup stores an
// fp32 partial tile and splitk_epilogue_kernel finishes the tile.
//
// XT is the activation type (A in memory, epilogue outputs).  XT = AT: A goes to
// the MFMA as it is.  XT = float with AT = f16 (fp32 activations, fp16 weights):
// each fp32 operand x is split on its way into LDS into x_hi = fp16(x) and
// x_lo = fp16(x - x_hi) (x_hi + x_lo carries about 22 significant bits), and every
// k step runs both halves against the same weight fragment, acc += x_hi w then
// acc += x_lo w, so the product has close to fp32 accuracy on fp16 MFMA.
template <class AT, class XT, bool W4, int BM, int BN, int BK, int D, int KIND>
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmArgs g, GemmEpi e, int kchunk) {
  constexpr bool SPLIT = std::is_same<XT, float>::value;
  static_assert(!SPLIT || (std::is_same<AT, f16>::value && !W4), "split operands: fp16 MFMA, dense weights");
  constexpr int AW = SPLIT ? 2 : 1;   // 16-byte words of one 8-element A chunk
  constexpr int LDK = BK + 8;   // padded LDS row, elements
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int AC = BM * (BK / 8) / 256;                             // 16-byte A chunks per thread
  constexpr int BCH = W4 ? BN * (BK / 32) : BN * (BK / 8);            // 16-byte B chunks per stage
  constexpr int BC = (BCH + 255) / 256;                               // per thread
  constexpr int GPS = BK / 128;                                       // INT4 groups per stage
  static_assert(TM >= 1 && TN >= 2 && (TN % 2) == 0 && AC >= 1, "tile");
  static_assert(!W4 || (BK % 128) == 0, "INT4 stages hold whole groups");
  static_assert(D >= 2, "the ring holds the stage being stored plus D-1 prefetched ones");
  typedef typename Mfma<AT>::frag frag;

  __shared__ __attribute__((aligned(16))) AT As[BM * LDK];
  __shared__ __attribute__((aligned(16))) AT As2[SPLIT ? BM * LDK : 8];   // x_lo of split operands
  __shared__ __attribute__((aligned(16))) AT Bs[BN * LDK];
  __shared__ float Ss[W4 ? GPS : 1][W4 ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K;
  const int S = gridDim.z, z = blockIdx.z;
  const int kb = z * kchunk, ke = min(K, kb + kchunk);
  const XT* A = reinterpret_cast<const XT*>(g.A);
  const int groups = K >> 7;

  floatx4 acc[TM][TN];
  floatx4 tmp[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      tmp[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  // Register ring.  Every load is issued unconditionally from an address clamped
  // into the operand (branch-free code lets the compiler wait for exactly the
  // oldest stage); chunks outside the tile are zeroed when they go to LDS.
  uint4 ra_[D][AC * AW], rb_[D][BC];
  uint16_t rs_[D][W4 ? GPS : 1];
  uint32_t okA_[D], okB_[D];
  // The loads of one stage in pieces: piece p < AC is A chunk p, then the B chunks,
  // then (INT4) the group scales.  Piece 0 clears the stage's in-tile masks.
  constexpr int NPIECE = AC + BC + (W4 ? 1 : 0);
  auto gpiece = [&](auto pc, uint4 (&ra)[AC * AW], uint4 (&rb)[BC], uint16_t (&rs)[W4 ? GPS : 1], uint32_t& okA,
                    uint32_t& okB, int k0) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    if constexpr (p == 0) {
      okA = 0;
      okB = 0;
    }
    if constexpr (p < AC) {
      constexpr int i = p;
      const int c = tid + 256 * i, r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int gr = m0 + r, gk = k0 + kc;
      if constexpr (!W4) okA |= (gr < M && gk < ke) ? (1u << i) : 0u;   // (INT4: scale 0 instead)
      const int grc = min(gr, M - 1), gkc = min(gk, K - 8);
      const XT* src = A + (int64_t)grc * K + gkc;
#pragma unroll
      for (int w = 0; w < AW; ++w) ra[i * AW + w] = *reinterpret_cast<const uint4*>(src + w * (16 / sizeof(XT)));
    } else if constexpr (p < AC + BC) {
      constexpr int i = p - AC;
      if constexpr (W4) {
        // chunk c: group go of the stage, 32-row block of the tile, half hb of the
        // 2 KB fragment block, lane (row mod 32, k half h): 64 consecutive chunks are
        // one contiguous 1 KB half (four words: k steps 4 hb .. 4 hb + 3)
        const int c = min(tid + 256 * i, BCH - 1);
        const int go = c / (BN * 4), rem = c % (BN * 4);
        const int row = (rem >> 7) * 32 + (rem & 31), hb = (rem >> 6) & 1, h = (rem >> 5) & 1;
        const int gn = n0 + row;
        const int gnc = min(gn, N - 1), gic = min((k0 >> 7) + go, groups - 1);
        rb[i] = *reinterpret_cast<const uint4*>(g.Bw4 + w4_word_offset(gnc, gic * 16 + 8 * hb + h, groups));
      } else {
        const AT* B = reinterpret_cast<const AT*>(g.B);
        const int c = min(tid + 256 * i, BCH - 1), r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        const int gn = n0 + r, gk = k0 + kc;
        okB |= (tid + 256 * i < BCH && gn < N && gk < ke) ? (1u << i) : 0u;
        const int gnc = min(gn, N - 1), gkc = min(gk, K - 8);
        rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)gnc * K + gkc);
      }
    } else if constexpr (W4 && p == AC + BC) {
#pragma unroll
      for (int go = 0; go < GPS; ++go) {
        const int gn = n0 + (tid < BN ? tid : 0);
        const bool ok = tid < BN && gn < N && k0 + go * 128 < ke;
        const int gnc = min(gn, N - 1), gic = min((k0 >> 7) + go, groups - 1);
        rs[go] = g.Bs[(int64_t)gic * N + gnc];
        okB |= ok ? (1u << (16 + go)) : 0u;
      }
    }
  };
  auto gload = [&](uint4 (&ra)[AC * AW], uint4 (&rb)[BC], uint16_t (&rs)[W4 ? GPS : 1], uint32_t& okA, uint32_t& okB,
                   int k0) __attribute__((always_inline)) {
    static_for<0, NPIECE>([&](auto pc) __attribute__((always_inline)) { gpiece(pc, ra, rb, rs, okA, okB, k0); });
  };
  auto lstore = [&](const uint4 (&ra)[AC * AW], const uint4 (&rb)[BC], const uint16_t (&rs)[W4 ? GPS : 1],
                    uint32_t okA, uint32_t okB) {
    // keep the masking here: without this the compiler may move it next to the
    // loads and wait for the data as soon as it is requested
    asm volatile("" : "+v"(okA), "+v"(okB));
    // INT4: no operand is masked.  A group outside the tile or the split (columns
    // past N, K past the split's end, padded stages) gets scale 0 below, so its
    // clamped, finite operands add nothing; rows past M are never stored.
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const uint32_t mk = W4 ? ~0u : 0u - ((okA >> i) & 1u);
      if constexpr (SPLIT) {
        half8 hi, lo;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint4 q = ra[i * 2 + w];
          const uint32_t u[4] = {q.x & mk, q.y & mk, q.z & mk, q.w & mk};
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float x = __builtin_bit_cast(float, u[e2]);
            const f16 xh = (f16)x;
            hi[4 * w + e2] = xh;
            lo[4 * w + e2] = (f16)(x - (float)xh);
          }
        }
        *reinterpret_cast<half8*>(&As[r * LDK + kc]) = hi;
        *reinterpret_cast<half8*>(&As2[r * LDK + kc]) = lo;
      } else {
        *reinterpret_cast<uint4*>(&As[r * LDK + kc]) = uint4{ra[i].x & mk, ra[i].y & mk, ra[i].z & mk, ra[i].w & mk};
      }
    }
    if constexpr (W4) {
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const int c = tid + 256 * i;
        if (c < BCH) {
          const int go = c / (BN * 4), rem = c % (BN * 4);
          const int row = (rem >> 7) * 32 + (rem & 31), hb = (rem >> 6) & 1, hk = (rem >> 5) & 1;
          const uint32_t ws[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
          // word wi: k = 16 (4 hb + wi) + 8 hk + (0..7) of the group
          f16* dst = reinterpret_cast<f16*>(&Bs[row * LDK + go * 128 + 64 * hb + 8 * hk]);
#pragma unroll
          for (int wi = 0; wi < 4; ++wi) {
            half8 h;
            half2v t[4];
            w4_pairs(ws[wi], t);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              h[2 * p] = t[p][0];
              h[2 * p + 1] = t[p][1];
            }
            *reinterpret_cast<half8*>(dst + wi * 16) = h;
          }
        }
      }
      if (tid < BN) {
#pragma unroll
        for (int go = 0; go < GPS; ++go)
          Ss[go][tid] = ((okB >> (16 + go)) & 1u) ? (float)__builtin_bit_cast(f16, rs[go]) : 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const int c = tid + 256 * i, r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        const uint32_t mk = 0u - ((okB >> i) & 1u);
        if (c < BCH)
          *reinterpret_cast<uint4*>(&Bs[r * LDK + kc]) = uint4{rb[i].x & mk, rb[i].y & mk, rb[i].z & mk, rb[i].w & mk};
      }
    }
  };

  // One stage's MFMAs; after k step ks the callback may issue a share of the next
  // stage's load pieces, so that they leave between the MFMAs (issued together ahead
  // of them, the wave's in-order issue holds its MFMAs until the memory pipeline has
  // taken every load).
  auto compute = [&](auto&& issue) __attribute__((always_inline)) {
    static_for<0, BK / 32>([&](auto kc) __attribute__((always_inline)) {
      constexpr int kk = decltype(kc)::value * 32;
      frag a[TM], b[TN], a2[SPLIT ? TM : 1];
      const int lrow = lane & 15, lk = kk + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const frag*>(&As[(wm * WTM + i * 16 + lrow) * LDK + lk]);
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          a2[i] = *reinterpret_cast<const frag*>(&As2[(wm * WTM + i * 16 + lrow) * LDK + lk]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const frag*>(&Bs[(wn * WTN + j * 16 + lrow) * LDK + lk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (W4) {
            tmp[i][j] = Mfma<AT>::run(a[i], b[j], tmp[i][j]);
          } else {
            acc[i][j] = Mfma<AT>::run(a[i], b[j], acc[i][j]);
            if constexpr (SPLIT) acc[i][j] = Mfma<AT>::run(a2[i], b[j], acc[i][j]);
          }
        }
      if constexpr (W4) {
        if ((kk & 127) == 96) {   // end of a 128-wide group: apply its scale
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const float sc = Ss[kk >> 7][wn * WTN + j * 16 + (lane & 15)];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              acc[i][j] += sc * tmp[i][j];
              tmp[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
      issue(kc);
    });
  };

  // Stage count padded to a multiple of D so that the loop body is straight-line
  // (every prefetch issued unconditionally; padded stages load clamped addresses
  // and are masked to zero), which lets the compiler wait for just the oldest stage.
  const int nst = ((ke - kb + BK - 1) / BK + D - 1) / D * D;
  // QKV epilogue operands besides the accumulators: thread t < BM takes the cache
  // coordinates of row m0 + t (lane, position, iteration, done, then the lane's
  // slot offset and capacity), every lane the rotary factors of its own rows and
  // columns.  Small tiles (BM <= 64, BN 64: eight rows and one column pair per
  // lane) request them around the first stages, so that their latency overlaps
  // the main loop; larger tiles would hold too many of them in registers across
  // the loop and gather them after it, in two rounds of loads.
  constexpr bool QPRE = KIND == EPI_QKV && BM <= 64 && BN == 64;
  constexpr int QJ = (KIND == EPI_QKV) ? TN / 2 : 1;
  constexpr int QM = (KIND == EPI_QKV) ? TM : 1;
  int qri[4] = {0, 0, 0, 0};
  int qpos[QPRE ? TM : 1][4] = {};
  int64_t qcap = 0, qoff = 0;
  int qsect[QJ] = {}, qhead[QJ] = {}, qcd[QJ] = {}, qrn[QJ] = {};
  float rcos[QM][4][QJ] = {}, rsin[QM][4][QJ] = {};
  auto q_row = [&]() {
    const RowInfo* ri = e.rows + min(m0 + tid, M - 1);
    qri[0] = ri->lane;
    qri[1] = ri->pos;
    qri[2] = ri->iter;
    qri[3] = ri->done;
  };
  // column arithmetic (section, head, rotary index: integer divisions) once per
  // column of this lane
  auto q_cols = [&]() {
#pragma unroll
    for (int jp = 0; jp < QJ; ++jp) {
      const int c = min(n0 + wn * WTN + 2 * jp * 16 + (lane & 15), N - 1);
      qsect[jp] = c / e.d;
      const int cc = c - qsect[jp] * e.d;
      qhead[jp] = cc / e.dh;
      qcd[jp] = cc - qhead[jp] * e.dh;
      const int ci = qcd[jp] / e.pair_g;
      qrn[jp] = (ci >> 1) * e.pair_g + (qcd[jp] - ci * e.pair_g);
    }
  };
  auto q_rope = [&](int i, int r, int pos) {
#pragma unroll
    for (int jp = 0; jp < QJ; ++jp) {
      const int64_t at = (int64_t)max(pos, 0) * (e.dh >> 1) + qrn[jp];
      rcos[i][r][jp] = e.rope_cos[at];
      rsin[i][r][jp] = e.rope_sin[at];
    }
  };
  if constexpr (QPRE) {
    if (S == 1) {
      if (tid < BM) q_row();
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          qpos[i][r] = e.rows[min(m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + r, M - 1)].pos;
    }
  }
#pragma unroll
  for (int u = 0; u < D - 1; ++u) gload(ra_[u], rb_[u], rs_[u], okA_[u], okB_[u], kb + u * BK);
  if (gate_closed(g.live)) return;
  if constexpr (QPRE) {
    if (S == 1) {
      if (tid < BM) {
        qcap = e.kv.lane_cap[qri[0]];
        qoff = e.kv.lane_off[qri[0]];
      }
      q_cols();
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) q_rope(i, r, qpos[i][r]);
    }
  }
  for (int s0 = 0; s0 < nst; s0 += D) {
    static_for<0, D>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int nx = (u + D - 1) % D;
      lstore(ra_[u], rb_[u], rs_[u], okA_[u], okB_[u]);
      lds_barrier();
      const int k0n = kb + (s0 + u + D - 1) * BK;
      if constexpr (BM >= 128) {
        // large tiles: the next stage's loads between this stage's MFMAs (FP16-body
        // forward of 32 x 128 tokens at L = 8: 5.61 -> 5.47 ms); the 32- and 64-row
        // tiles measured no better or slightly worse this way
        compute([&](auto kc) __attribute__((always_inline)) {
          constexpr int KS = BK / 32, PPS = (NPIECE + KS - 1) / KS, ks = decltype(kc)::value;
          static_for<ks * PPS, (ks + 1) * PPS < NPIECE ? (ks + 1) * PPS : NPIECE>(
              [&](auto pc) __attribute__((always_inline)) {
                gpiece(pc, ra_[nx], rb_[nx], rs_[nx], okA_[nx], okB_[nx], k0n);
              });
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
        gload(ra_[nx], rb_[nx], rs_[nx], okA_[nx], okB_[nx], k0n);
        compute([](auto) {});
      }
      lds_barrier();
    });
  }

  const int lc = lane & 15, lr = 4 * (lane >> 4);
  if (S > 1) {
    // split-K: store this split's fp32 partial tile; splitk_epilogue_kernel adds
    // the splits in order and runs the epilogue (the kernel boundary makes the
    // partials visible across XCDs without any cache maintenance here)
    float* part = g.partial + (int64_t)z * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WTM + i * 16 + lr + r;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + lc;
          if (col < N) part[(int64_t)row * N + col] = acc[i][j][r];
        }
      }
    return;
  }

  // ---- epilogue: lane holds column (lane & 15), rows 4*(lane >> 4) + r of each 16x16 tile
  if constexpr (KIND == EPI_HEAD) {
    __shared__ float red_v[BM][2], red_v2[BM][2];
    __shared__ int red_i[BM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow_t = wm * WTM + i * 16 + lr + r;
        const int row = m0 + lrow_t;
        float bv = -INFINITY, b2 = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + lc;
          if (col < N) {
            const float v = acc[i][j][r];
            if (row < M) epi_one<KIND>(e, row, col, v);
            best2_push(bv, bi, b2, v, col);
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float ov = __shfl_xor(bv, o, 64), ov2 = __shfl_xor(b2, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          best2_merge(bv, bi, b2, ov, oi, ov2);
        }
        if (lc == 0) {
          red_v[lrow_t][wn] = bv;
          red_v2[lrow_t][wn] = b2;
          red_i[lrow_t][wn] = bi;
        }
      }
    __syncthreads();
    for (int t = tid; t < BM; t += 256) {
      const int row = m0 + t;
      if (row < M) {
        float bv = red_v[t][0], b2 = red_v2[t][0];
        int bi = red_i[t][0];
        best2_merge(bv, bi, b2, red_v[t][1], red_i[t][1], red_v2[t][1]);
        e.part_val[(int64_t)row * e.n_tiles + blockIdx.x] = bv;
        e.part_idx[(int64_t)row * e.n_tiles + blockIdx.x] = bi;
        if (e.part_val2) e.part_val2[(int64_t)row * e.n_tiles + blockIdx.x] = b2;
      }
    }
  } else if constexpr (KIND == EPI_QKV) {
    // epi_pair's QKV epilogue with its operands gathered as described above;
    // thread t < BM finishes the cache addressing of row m0 + t in LDS.
    __shared__ int64_t q_kb[BM], q_hs[BM];
    __shared__ int q_pos[BM];   // -1: row not written (past M, or finished by early exit)
    if constexpr (!QPRE) {
      if (tid < BM) {
        q_row();
        qcap = e.kv.lane_cap[qri[0]];
        qoff = e.kv.lane_off[qri[0]];
      }
      q_cols();
    }
    if (tid < BM) {
      const int64_t hs = qcap * e.kv.dh;   // one head of one slot
      const int slot = e.kv.s0 + e.kv.s1 * qri[2];
      q_kb[tid] = qoff + (int64_t)(slot * 2) * e.kv.H * hs + (int64_t)qri[1] * e.kv.dh;
      q_hs[tid] = hs;
      q_pos[tid] = (m0 + tid < M && !(e.skip_done && qri[3])) ? qri[1] : -1;
    }
    __syncthreads();
    if constexpr (!QPRE) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) q_rope(i, r, q_pos[wm * WTM + i * 16 + lr + r]);
    }
    const int d = e.d, dh = e.dh, G = e.pair_g, half = dh >> 1;
    XT* const kv = reinterpret_cast<XT*>(e.kv.base);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = wm * WTM + i * 16 + lr + r, row = m0 + lrow;
        if (q_pos[lrow] < 0) continue;
        const int64_t hs = q_hs[lrow], kbase = q_kb[lrow], vbase = kbase + e.kv.H * hs;
#pragma unroll
        for (int jp = 0; jp < QJ; ++jp) {
          const int col = n0 + wn * WTN + 2 * jp * 16 + lc;
          if (col >= N) continue;
          const float v0 = acc[i][2 * jp][r], v1 = acc[i][2 * jp + 1][r];
          if (qsect[jp] == 2) {
            XT* vp = kv + vbase + qhead[jp] * hs;
            vp[qcd[jp]] = from_f32<XT>(v0);
            vp[qcd[jp] + G] = from_f32<XT>(v1);
            continue;
          }
          const float cs = rcos[i][r][jp], sn = rsin[i][r][jp];
          const float x1 = rot_x1(v0, v1, cs, sn);
          const float x2 = rot_x2(v0, v1, cs, sn);
          XT* dst = (qsect[jp] == 0) ? reinterpret_cast<XT*>(e.q_out) + (int64_t)row * d + qhead[jp] * dh
                                     : kv + kbase + qhead[jp] * hs;
          dst[qrn[jp]] = from_f32<XT>(x1);
          dst[qrn[jp] + half] = from_f32<XT>(x2);
        }
      }
  } else if constexpr (KIND == EPI_SWIGLU) {
    // epi_pair's SwiGLU with the output column (a division) worked out once per
    // column of this lane
    constexpr int EJ = TN / 2;
    const int G = e.pair_g;
    int un[EJ];
#pragma unroll
    for (int jp = 0; jp < EJ; ++jp) {
      const int c = min(n0 + wn * WTN + 2 * jp * 16 + lc, N - 1);
      const int ci = c / G;
      un[jp] = (ci >> 1) * G + (c - ci * G);
    }
    XT* const u = reinterpret_cast<XT*>(e.u_out);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WTM + i * 16 + lr + r;
        if (row >= M) continue;
#pragma unroll
        for (int jp = 0; jp < EJ; ++jp) {
          if (n0 + wn * WTN + 2 * jp * 16 + lc >= N) continue;
          const float v0 = acc[i][2 * jp][r], v1 = acc[i][2 * jp + 1][r];
          const float sg = v0 / (1.0f + expf(-v0));
          u[(int64_t)row * e.F + un[jp]] = from_f32<XT>(sg * v1);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WTM + i * 16 + lr + r;
        if (row >= M) continue;
        if constexpr (paired(KIND)) {
#pragma unroll
          for (int j = 0; j < TN; j += 2) {
            const int col = n0 + wn * WTN + j * 16 + lc;
            if (col < N) epi_pair<XT, KIND>(e, row, col, acc[i][j][r], acc[i][j + 1][r]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + lc;
            if (col < N) epi_one<KIND>(e, row, col, acc[i][j][r]);
          }
        }
      }
  }
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Small-M GEMM with INT4 weights (M <= BM <= 64 rows per workgroup).
//
// At decode sizes the product is bound by fixed costs and by how often each CU
// re-reads the activations, so one workgroup takes every row of the pass and a
// BN = 128 * WNB column tile, and K is split across workgroups (blockIdx.z) to
// fill the CUs.  Per 128-wide K stage:
//  * A (BM x 128 fp16) goes global -> registers -> LDS once per workgroup, rows of
//    16 chunks of 16 bytes with the chunk slot XOR-ed by (row mod 16), so both the
//    row-wise stores and the 32-row fragment reads hit 16 distinct slots;
//  * each of the four waves owns all BM rows and WNB 32-column blocks; its INT4
//    fragments come straight from global memory in MFMA order (two coalesced
//    1 KB loads per 32 columns) and are expanded to exact fp16 integers in
//    registers, so every weight is expanded once per workgroup;
//  * 32x32x16 MFMAs form the group's sum in a fresh accumulator, which is then
//    multiplied by the column's fp32 scale and added: sum_k x_k q_k s exactly as
//    in the per-group definition.  A fragments of the next k step are read from
//    LDS while the current step's MFMAs run.
// Global loads run D-1 stages ahead in a register ring (straight-line loop,
// clamped addresses; stages past the split's end are given scale 0).  LDS is
// double-buffered, one barrier per stage.
template <int BM, int WNB, int D, int KIND>
__global__ __launch_bounds__(256) void gemm_skinny_w4_kernel(GemmArgs g, GemmEpi e, int kchunk) {
  constexpr int RBW = BM / 32;           // 32-row blocks (every wave covers all rows)
  constexpr int WN = 32 * WNB;
  constexpr int BN = 4 * WN;
  constexpr int AC = BM / 16;            // 16-byte A chunks per thread per stage
  static_assert(RBW >= 1 && D >= 2, "tile");
  __shared__ u32x4 As[2][BM * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN, wn0 = n0 + wave * WN, wr0 = 0;
  const int M = g.M, N = g.N, K = g.K, groups = K >> 7;
  const int S = gridDim.z, z = blockIdx.z;
  const int kb = z * kchunk, ke = min(K, kb + kchunk);
  const int nreal = (ke - kb) >> 7;
  const int nst = (nreal + D - 1) / D * D;
  const f16* A = reinterpret_cast<const f16*>(g.A);

  floatx16 acc[RBW][WNB];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[D][AC];
  u32x4 rw[D][WNB][2];
  uint16_t rs[D][WNB];

  auto gload = [&](auto uc, int st) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    const int gi = (kb >> 7) + min(st, nreal - 1);
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c >> 4, ch = c & 15;
      const int gr = min(m0 + r, M - 1);
      ra[u][i] = *reinterpret_cast<const u32x4*>(A + (int64_t)gr * K + gi * 128 + ch * 8);
    }
#pragma unroll
    for (int cb = 0; cb < WNB; ++cb) {
      const int nb = min((wn0 >> 5) + cb, (N >> 5) - 1);
      const uint32_t* wp = g.Bw4 + ((int64_t)nb * groups + gi) * 512 + lane * 4;
      rw[u][cb][0] = *reinterpret_cast<const u32x4*>(wp);
      rw[u][cb][1] = *reinterpret_cast<const u32x4*>(wp + 256);
      rs[u][cb] = g.Bs[(int64_t)gi * N + min(wn0 + cb * 32 + (lane & 31), N - 1)];
    }
  };
  auto lstore = [&](auto uc, int buf) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c >> 4, ch = c & 15;
      As[buf][r * 16 + (ch ^ (r & 15))] = ra[u][i];
    }
  };
  auto read_a = [&](half8 (&a)[RBW], int buf, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int r = wr0 + 32 * i + (lane & 31), ch = 2 * j + (lane >> 5);
      a[i] = __builtin_bit_cast(half8, As[buf][r * 16 + (ch ^ (r & 15))]);
    }
  };
  auto compute = [&](auto uc, int buf, bool valid) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    floatx16 tmp[RBW][WNB];
    half8 a[2][RBW];
    read_a(a[0], buf, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < 7) read_a(a[(j + 1) & 1], buf, j + 1);
      half8 b[WNB];
#pragma unroll
      for (int cb = 0; cb < WNB; ++cb) {
        const u32x4 q4 = rw[u][cb][j >> 2];
        const uint32_t w = q4[j & 3];
        half2v t[4];
        w4_pairs(w, t);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          b[cb][2 * p] = t[p][0];
          b[cb][2 * p + 1] = t[p][1];
        }
      }
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int cb = 0; cb < WNB; ++cb) {
          if (j == 0) {
            floatx16 zero;
#pragma unroll
            for (int r = 0; r < 16; ++r) zero[r] = 0.f;
            tmp[i][cb] = mfma32(a[0][i], b[cb], zero);
          } else {
            tmp[i][cb] = mfma32(a[j & 1][i], b[cb], tmp[i][cb]);
          }
        }
    }
#pragma unroll
    for (int cb = 0; cb < WNB; ++cb) {
      const float sc = valid ? (float)__builtin_bit_cast(f16, rs[u][cb]) : 0.f;
#pragma unroll
      for (int i = 0; i < RBW; ++i) acc[i][cb] += sc * tmp[i][cb];
    }
  };

  static_for<0, D - 1>([&](auto uc) __attribute__((always_inline)) { gload(uc, decltype(uc)::value); });
  if (gate_closed(g.live)) return;
  for (int s0 = 0; s0 < nst; s0 += D) {
    static_for<0, D>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      const int st = s0 + u;
      lstore(uc, st & 1);
      lds_barrier();
      gload(std::integral_constant<int, (u + D - 1) % D>{}, st + D - 1);
      // keep the prefetch here: otherwise it is sunk past this stage's MFMAs to
      // where its registers are next used, and nothing overlaps the load latency
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      compute(uc, st & 1, st < nreal);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // C layout of a 32x32 tile: lane holds column (lane & 31), rows
  // 8 (r / 4) + 4 (lane / 32) + (r mod 4) for r = 0 .. 15
  const int lc = lane & 31, lh = lane >> 5;
  if (S > 1) {
    float* part = g.partial + (int64_t)z * M * N;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int cb = 0; cb < WNB; ++cb) {
        const int col = wn0 + 32 * cb + lc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wr0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (row < M && col < N) part[(int64_t)row * N + col] = acc[i][cb][r];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int cb = 0; cb < WNB; ++cb) {
      const int col = wn0 + 32 * cb + lc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wr0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const float v = acc[i][cb][r];
        if constexpr (paired(KIND)) {
          // pair (c, c + 16) of a 32-column chunk: the partner sits 16 lanes away
          const float v1 = __shfl_xor(v, 16, 64);
          if (lc < 16 && row < M && col < N) epi_pair<f16, KIND>(e, row, col, v, v1);
        } else {
          if (row < M && col < N) epi_one<KIND>(e, row, col, v);
        }
      }
    }
}

// Output of a wave that holds RB 32 x 32 tiles (rows r0 + 32 i, columns c0 ..
// c0 + 31) of a row-tiled INT4 product: split partials, or the epilogue.  C layout
// of a 32x32 tile: lane holds column (lane & 31), rows 8 (r / 4) + 4 (lane / 32) +
// (r mod 4) for r = 0 .. 15.
template <int RB, int KIND>
__device__ __forceinline__ void rows_store(const GemmArgs& g, const GemmEpi& e, const floatx16 (&acc)[RB], int r0,
                                           int c0, int lane) {
  const int M = g.M, N = g.N, S = gridDim.z;
  const int lc = lane & 31, lh = lane >> 5;
  const int col = c0 + lc;
  if (S > 1) {
    float* part = g.partial + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < M && col < N) part[(int64_t)row * N + col] = acc[i][r];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
      const float v = acc[i][r];
      if constexpr (paired(KIND)) {
        // pair (c, c + 16) of a 32-column block: the partner sits 16 lanes away
        const float v1 = __shfl_xor(v, 16, 64);
        if (lc < 16 && row < M && col < N) epi_pair<f16, KIND>(e, row, col, v, v1);
      } else {
        if (row < M && col < N) epi_one<KIND>(e, row, col, v);
      }
    }
}

// One 128-wide group of a row-tiled INT4 product on a wave: RB A fragments per k
// step from the LDS stage (16-byte chunks XOR-swizzled by row within the group's 16),
// the wave's 32-column INT4 fragments (two 16-byte words per lane, in MFMA order)
// expanded in registers, 32x32x16 MFMAs into a fresh group sum that is scaled by the
// column's fp32 group scale and added.  The next k step's fragments are read and
// expanded before this step's MFMAs, so the MFMAs do not wait on their own LDS
// reads (gate/up at 128 rows: 20.4 -> 20.0 us per launch in the forward).  After k step j the callback issues piece j of
// the next stage's loads, so that they leave one at a time between the MFMAs: issued
// together ahead of the MFMAs, the wave's in-order issue held its MFMAs until the
// memory pipeline had taken every load (gate/up at 128 rows: 18.9 -> 17.9 us per
// launch with four waves).
template <int RB, int KC, class Issue>
__device__ __forceinline__ void rows_group(floatx16 (&acc)[RB], const u32x4* As, int r0, int ch0, int lane,
                                           const u32x4 (&w)[2], float sc, Issue&& issue) {
  floatx16 tmp[RB];
  auto rd = [&](int j, half8 (&a)[RB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = r0 + 32 * i + (lane & 31), ch = ch0 + 2 * j + (lane >> 5);
      a[i] = __builtin_bit_cast(half8, As[r * KC + ((ch & ~15) | ((ch & 15) ^ (r & 15)))]);
    }
  };
  auto ex = [&](int j, half8& b) __attribute__((always_inline)) {
    half2v t[4];
    w4_pairs(w[j >> 2][j & 3], t);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      b[2 * p] = t[p][0];
      b[2 * p + 1] = t[p][1];
    }
  };
  half8 a[2][RB], b[2];
  rd(0, a[0]);
  ex(0, b[0]);
  static_for<0, 8>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value, c = j & 1;
    if constexpr (j < 7) {
      rd(j + 1, a[1 - c]);
      ex(j + 1, b[1 - c]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if constexpr (j == 0) {
        floatx16 zero;
#pragma unroll
        for (int r = 0; r < 16; ++r) zero[r] = 0.f;
        tmp[i] = mfma32(a[c][i], b[c], zero);
      } else {
        tmp[i] = mfma32(a[c][i], b[c], tmp[i]);
      }
    }
    issue(jc);
  });
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i] += sc * tmp[i];
}

// INT4 GEMM for passes of 65..128 rows (a 128-token forward, prefill chunks): the
// small-M kernel's structure with the rows cut into BM = 64 tiles.
//  * A (64 x 128 fp16 per stage) goes global -> registers -> LDS once per workgroup;
//  * the four waves are arranged WM x (4 / WM): a wave owns 64 / WM rows and one
//    32-column block, whose INT4 fragments it loads straight from global memory
//    (two coalesced 1 KB loads per group) and expands in registers (rows_group);
//  * a two-stage register ring, the next stage's loads issued between this stage's
//    MFMAs.
// At 128 rows of the 2048-wide model (per-launch event timing, a dependent kernel
// before each launch) the down projection (K = 5632, WM = 2, K split 4 ways,
// reduction included) took 17.1 us against 20.7 us on the LDS-tiled kernel.
template <int WM, int KIND>
__global__ __launch_bounds__(256, 2) void gemm_w4_rows_kernel(GemmArgs g, GemmEpi e, int kchunk) {
  constexpr int BM = 64, KC = 16, AC = BM * KC / 256;
  constexpr int WN = 4 / WM;
  constexpr int RB = BM / WM / 32;
  static_assert(WM * WN == 4 && RB >= 1, "tile");
  __shared__ u32x4 As[2][BM * KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, wn0 = blockIdx.x * (WN * 32) + wn * 32, wr0 = wm * (BM / WM);
  const int M = g.M, N = g.N, K = g.K, groups = K >> 7;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  const int g0 = kb >> 7, nreal = (ke >> 7) - g0;
  const int nst = (nreal + 3) & ~3;
  const int nb = min(wn0 >> 5, (N >> 5) - 1);
  const f16* A = reinterpret_cast<const f16*>(g.A);

  floatx16 acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // two-stage register ring; every address is clamped into its operand (stages past
  // the split's end are given scale 0)
  u32x4 ra[2][AC];
  u32x4 rw[2][2];
  uint16_t rs[2];
  // piece p of stage st's loads into ring slot u: the A chunks, then the two INT4
  // words, then the scale
  auto piece = [&](auto uc, auto pc, int st) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value, p = decltype(pc)::value;
    const int gi = min(g0 + min(st, nreal - 1), groups - 1);
    if constexpr (p < AC) {
      const int c = tid + 256 * p, r = c / KC, ch = c % KC;
      ra[u][p] = *reinterpret_cast<const u32x4*>(A + (int64_t)min(m0 + r, M - 1) * K + gi * 128 + ch * 8);
    } else if constexpr (p == AC) {
      rw[u][0] = *reinterpret_cast<const u32x4*>(g.Bw4 + ((int64_t)nb * groups + gi) * 512 + lane * 4);
    } else if constexpr (p == AC + 1) {
      rw[u][1] = *reinterpret_cast<const u32x4*>(g.Bw4 + ((int64_t)nb * groups + gi) * 512 + 256 + lane * 4);
    } else if constexpr (p == AC + 2) {
      rs[u] = g.Bs[(int64_t)gi * N + min(wn0 + (lane & 31), N - 1)];
    }
  };
  auto lstore = [&](auto uc, int buf) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c / KC, ch = c % KC;
      As[buf][r * KC + (ch ^ (r & 15))] = ra[u][i];
    }
  };

  static_for<0, AC + 3>([&](auto pc) __attribute__((always_inline)) { piece(std::integral_constant<int, 0>{}, pc, 0); });
  if (gate_closed(g.live)) return;
  for (int s0 = 0; s0 < nst; s0 += 4) {
    static_for<0, 4>([&](auto sc4) __attribute__((always_inline)) {
      constexpr int u = decltype(sc4)::value & 1;
      const int st = s0 + decltype(sc4)::value;
      lstore(std::integral_constant<int, u>{}, st & 1);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const float sc = st < nreal ? (float)__builtin_bit_cast(f16, rs[u]) : 0.f;
      rows_group<RB, KC>(acc, As[st & 1], wr0, 0, lane, rw[u], sc, [&](auto jc) __attribute__((always_inline)) {
        issue_pieces<2, AC + 3, decltype(jc)::value>([&](auto pc) __attribute__((always_inline)) {
          piece(std::integral_constant<int, 1 - u>{}, pc, st + 1);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }
  rows_store<RB, KIND>(g, e, acc, m0 + wr0, wn0, lane);
}

// Gate/up-shaped products at 65..128 rows: eight waves on one 64 x 128 tile (two
// per SIMD, so that one wave's expansion and LDS reads overlap the other's MFMAs).
// Each stage covers two 128-wide groups: waves 0-3 take the first, waves 4-7 the
// second, each wave all 64 rows of its 32-column block, with the next stage's loads
// issued between its MFMAs; the two halves' sums meet in LDS at the end (the A
// stages' memory) and waves 0-3 apply the epilogue.  Gate/up at 128 rows: 16.4 us
// per launch against 18.9 us for the four-wave row-tiled kernel.
template <int KIND>
__global__ __launch_bounds__(512, 1) void gemm_w4_pair_kernel(GemmArgs g, GemmEpi e, int kchunk) {
  constexpr int BM = 64, KC = 32, RB = 2, AC = BM * KC / 512;
  __shared__ u32x4 As[2][BM * KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 3, kh = wave >> 2;
  const int m0 = blockIdx.y * BM, wn0 = blockIdx.x * 128 + wn * 32;
  const int M = g.M, N = g.N, K = g.K, groups = K >> 7;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  const int g0 = kb >> 7, gend = ke >> 7;
  const int nreal = (gend - g0 + 1) >> 1;   // two-group stages
  const int nst = (nreal + 3) & ~3;
  const int nb = min(wn0 >> 5, (N >> 5) - 1);
  const f16* A = reinterpret_cast<const f16*>(g.A);

  floatx16 acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  u32x4 ra[2][AC];
  u32x4 rw[2][2];
  uint16_t rs[2];
  auto piece = [&](auto uc, auto pc, int st) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value, p = decltype(pc)::value;
    const int s2 = g0 + 2 * min(st, nreal - 1);
    if constexpr (p < AC) {
      const int c = tid + 512 * p, r = c / KC, ch = c % KC;
      const int gk = min(s2 * 128 + ch * 8, K - 8);
      ra[u][p] = *reinterpret_cast<const u32x4*>(A + (int64_t)min(m0 + r, M - 1) * K + gk);
    } else {
      const int gi = min(s2 + kh, groups - 1);
      if constexpr (p == AC) {
        rw[u][0] = *reinterpret_cast<const u32x4*>(g.Bw4 + ((int64_t)nb * groups + gi) * 512 + lane * 4);
      } else if constexpr (p == AC + 1) {
        rw[u][1] = *reinterpret_cast<const u32x4*>(g.Bw4 + ((int64_t)nb * groups + gi) * 512 + 256 + lane * 4);
      } else if constexpr (p == AC + 2) {
        rs[u] = g.Bs[(int64_t)gi * N + min(wn0 + (lane & 31), N - 1)];
      }
    }
  };
  auto lstore = [&](auto uc, int buf) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 512 * i, r = c / KC, ch = c % KC;
      As[buf][r * KC + ((ch & ~15) | ((ch & 15) ^ (r & 15)))] = ra[u][i];
    }
  };

  static_for<0, AC + 3>([&](auto pc) __attribute__((always_inline)) { piece(std::integral_constant<int, 0>{}, pc, 0); });
  if (gate_closed(g.live)) return;
  for (int s0 = 0; s0 < nst; s0 += 4) {
    static_for<0, 4>([&](auto sc4) __attribute__((always_inline)) {
      constexpr int u = decltype(sc4)::value & 1;
      const int st = s0 + decltype(sc4)::value;
      lstore(std::integral_constant<int, u>{}, st & 1);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // an odd group count leaves the last stage's second half empty
      const bool valid = st < nreal && g0 + 2 * st + kh < gend;
      const float sc = valid ? (float)__builtin_bit_cast(f16, rs[u]) : 0.f;
      rows_group<RB, KC>(acc, As[st & 1], 0, 16 * kh, lane, rw[u], sc, [&](auto jc) __attribute__((always_inline)) {
        issue_pieces<2, AC + 3, decltype(jc)::value>([&](auto pc) __attribute__((always_inline)) {
          piece(std::integral_constant<int, 1 - u>{}, pc, st + 1);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }
  // waves 4-7 hand their sums to waves 0-3 through the A stages' LDS (32 KB of 64)
  float* red = reinterpret_cast<float*>(&As[0][0]);
  lds_barrier();
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wn * RB + i) * 16 + r) * 64 + lane] = acc[i][r];
  }
  lds_barrier();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] += red[((wn * RB + i) * 16 + r) * 64 + lane];
  rows_store<RB, KIND>(g, e, acc, m0, wn0, lane);
}

// fp32 operands: a plain LDS-tiled SIMT kernel (64 x 64 tile, 4 x 4 per thread).
// Paired epilogues use adjacent column pairs (row-permutation granularity 1).
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, GemmEpi e) {
  if (g.live && *g.live <= 0) return;
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K;
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* B = reinterpret_cast<const float*>(g.B);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + 256 * it, r = c / BK, k = c % BK;
      const int gk = k0 + k;
      As[k][r] = (m0 + r < M && gk < K) ? A[(int64_t)(m0 + r) * K + gk] : 0.f;
      Bs[k][r] = (n0 + r < N && gk < K) ? B[(int64_t)(n0 + r) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  if constexpr (KIND == EPI_HEAD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      float bv = -INFINITY, b2 = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) {
          if (row < M) epi_one<KIND>(e, row, col, acc[i][j]);
          best2_push(bv, bi, b2, acc[i][j], col);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64), ov2 = __shfl_xor(b2, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        best2_merge(bv, bi, b2, ov, oi, ov2);
      }
      if (tx == 0 && row < M) {
        e.part_val[(int64_t)row * e.n_tiles + blockIdx.x] = bv;
        e.part_idx[(int64_t)row * e.n_tiles + blockIdx.x] = bi;
        if (e.part_val2) e.part_val2[(int64_t)row * e.n_tiles + blockIdx.x] = b2;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
    if constexpr (paired(KIND)) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int col = n0 + tx * 4 + j;
        if (col < N) epi_pair<float, KIND>(e, row, col, acc[i][j], acc[i][j + 1]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) epi_one<KIND>(e, row, col, acc[i][j]);
      }
    }
  }
}

// Split-K reductions with a run-time split count request the partials of
// kSplitBatch splits at a time (indices clamped, the extra ones not added), so that
// their loads overlap instead of following one another; the sum is still taken in
// split order.
constexpr int kSplitBatch = 4;

// Sum of the split-K partials in split order, then the epilogue.  Paired
// epilogues get one thread per (row, pair): columns c and c + G with c in an even
// G-chunk; the others one thread per (row, column).
template <class AT, int KIND>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(GemmArgs g, GemmEpi e, int S) {
  const int M = g.M, N = g.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if constexpr (paired(KIND)) {
    const int G = e.pair_g;
    const int64_t per_row = N / 2;
    if (idx >= (int64_t)M * per_row) return;
    const int row = (int)(idx / per_row);
    const int p = (int)(idx - (int64_t)row * per_row);
    const int c = (p / G) * 2 * G + (p % G);
    QkvRow qr{};
    if constexpr (KIND == EPI_QKV) qr = qkv_row(e, row);   // read with the partials
    float v0 = 0.f, v1 = 0.f;
    for (int z0 = 0; z0 < S; z0 += kSplitBatch) {
      float a0[kSplitBatch], a1[kSplitBatch];
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q) {
        const float* pr = g.partial + ((int64_t)min(z0 + q, S - 1) * M + row) * N;
        a0[q] = pr[c];
        a1[q] = pr[c + G];
      }
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q)
        if (z0 + q < S) {
          v0 += a0[q];
          v1 += a1[q];
        }
    }
    if (gate_closed(g.live)) return;
    if constexpr (KIND == EPI_QKV) qkv_put<AT>(e, qkv_prep(e, qr, row, c), v0, v1);
    else epi_pair<AT, KIND>(e, row, c, v0, v1);
  } else {
    if (idx >= (int64_t)M * N) return;
    const int row = (int)(idx / N);
    const int c = (int)(idx - (int64_t)row * N);
    float v = 0.f;
    for (int z0 = 0; z0 < S; z0 += kSplitBatch) {
      float a[kSplitBatch];
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q) a[q] = g.partial[((int64_t)min(z0 + q, S - 1) * M + row) * N + c];
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q)
        if (z0 + q < S) v += a[q];
    }
    if (gate_closed(g.live)) return;
    epi_one<KIND>(e, row, c, v);
  }
}

// Split-K residual reduction fused with the next RMSNorm: one workgroup per row
// adds the splits in order onto the fp32 residual, then normalises the new row
// (fp32 statistics) into the next GEMM's operand type.  Each thread owns VPT
// groups of 4 consecutive columns (16-byte loads); with SN > 0 the SN splits are
// all requested before any is used, with SN == 0 a loop adds any number,
// kSplitBatch at a time.
template <class AT, int VPT, int SN>
__global__ __launch_bounds__(256) void splitk_resid_norm_kernel(GemmArgs g, GemmEpi e, int S) {
  const int row = blockIdx.x, N = g.N, M = g.M;
  float* hr = e.h + (int64_t)row * e.ldh;
  const floatx4* P = reinterpret_cast<const floatx4*>(g.partial);
  const int64_t zs = (int64_t)M * N / 4, rs = (int64_t)row * N / 4;
  floatx4 acc[VPT], hv0[VPT], gv[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the residual row and the norm gain are requested with the partials: one round
  // of loads before the sums instead of three
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int c4 = min((int)threadIdx.x + 256 * u, N / 4 - 1);
    hv0[u] = *reinterpret_cast<const floatx4*>(hr + 4 * c4);
    gv[u] = *reinterpret_cast<const floatx4*>(e.norm_g + 4 * c4);
  }
  if constexpr (SN > 0) {
    floatx4 p[SN][VPT];
#pragma unroll
    for (int z = 0; z < SN; ++z)
#pragma unroll
      for (int u = 0; u < VPT; ++u) p[z][u] = P[z * zs + rs + min((int)threadIdx.x + 256 * u, N / 4 - 1)];
    if (gate_closed(g.live)) return;
#pragma unroll
    for (int z = 0; z < SN; ++z)
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        acc[u] += p[z][u];
      }
  } else {
    if (gate_closed(g.live)) return;
    for (int z0 = 0; z0 < S; z0 += kSplitBatch) {
      floatx4 p[kSplitBatch][VPT];
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q)
#pragma unroll
        for (int u = 0; u < VPT; ++u) p[q][u] = P[min(z0 + q, S - 1) * zs + rs + min((int)threadIdx.x + 256 * u, N / 4 - 1)];
#pragma unroll
      for (int q = 0; q < kSplitBatch; ++q)
        if (z0 + q < S) {
#pragma unroll
          for (int u = 0; u < VPT; ++u) acc[u] += p[q][u];
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int c4 = (int)threadIdx.x + 256 * u;
    if (c4 * 4 < N) {
      const floatx4 hv = hv0[u] + acc[u];
      *reinterpret_cast<floatx4*>(hr + 4 * c4) = hv;
      acc[u] = hv;
      ss = sumsq4(hv[0], hv[1], hv[2], hv[3], ss);
    }
  }
  const float inv = rms_inv(row_sum256(ss), N, e.norm_eps);
  AT* o = reinterpret_cast<AT*>(e.norm_out) + (int64_t)row * N;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int c4 = (int)threadIdx.x + 256 * u;
    if (c4 * 4 < N) {
      const floatx4 gg = gv[u];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[4 * c4 + q] = from_f32<AT>(acc[u][q] * inv * gg[q]);
    }
  }
}

struct TileCfg {
  int bm, bn, splits, kchunk, bk, depth;
};

constexpr int kCUs = 256;
// rows the split of K is sized for when it must not depend on M (a decode-sized
// product)
constexpr int kInvariantRows = 64;

// Tile and split choice, from sweeps of the 2048-wide model's shapes on MI355X:
// for M <= 128 the kernels are bound by per-workgroup latency, so small tiles
// (BM 32/64 x BN 64, BK 128, two-stage ring, refined by the rules at the end) and
// a split of K that brings the workgroup count to roughly 320 work best; larger
// M uses 128 x 128 tiles and splits K only when the tiles cannot cover the 256
// CUs.  Dense weights at <= 32 rows that get no split (gate/up: 176 tiles of 16
// stages) keep three stages in flight instead of one: 17.5 -> 12.3 us with the
// weights in HBM.  Every tile accumulates k in the same order (32-wide steps, in
// order, within a split), so only the split changes the arithmetic; with
// g.invariant the split is the one kInvariantRows rows would get.
TileCfg pick_tile(int act_dtype, const GemmArgs& g, int kind) {
  if (act_dtype == DT_F32) return {64, 64, 1, g.K, 16, 2};
  TileCfg t{};
  t.depth = 2;
  t.splits = 1;
  t.kchunk = g.K;
  auto shape = [&](int M, int* bm, int* bn, int* bk) {
    if (M <= 128 && kind != EPI_HEAD) {
      *bm = M <= 32 ? 32 : 64;
      *bn = 64;
      *bk = 128;
    } else {
      *bm = M <= 32 ? 32 : ((M <= 64 || g.Bw4) ? 64 : 128);   // INT4 128 x 128 would spill
      *bn = 128;
      *bk = g.Bw4 ? 128 : 64;
    }
  };
  shape(g.M, &t.bm, &t.bn, &t.bk);
  const int Ms = g.invariant ? kInvariantRows : g.M;
  int sbm = t.bm, sbn = t.bn, sbk = t.bk;
  shape(Ms, &sbm, &sbn, &sbk);
  const int64_t tiles = (int64_t)((g.M + t.bm - 1) / t.bm) * ((g.N + t.bn - 1) / t.bn);
  const int64_t stiles = (int64_t)((Ms + sbm - 1) / sbm) * ((g.N + sbn - 1) / sbn);
  const int64_t units = g.K / 128;   // splits cut K at 128-wide group boundaries
  const int64_t target = Ms <= 128 ? 320 : 2 * kCUs;
  if (kind != EPI_HEAD && g.partial && (g.N % 32) == 0 && (g.K % 128) == 0 && stiles < target && units >= 4) {
    int64_t want = std::min<int64_t>(std::min<int64_t>(target / stiles, units / 2), 8);
    if (!g.invariant)
      while (want > 1 && want * g.M * g.N > g.partial_cap) --want;
    if (want > 1) {
      const int64_t per = (units + want - 1) / want;
      t.kchunk = (int)(per * 128);
      t.splits = (int)((units + per - 1) / per);
    }
  }
  if (!g.Bw4 && t.bm == 32 && t.bn == 64 && t.splits == 1) t.depth = 4;
  // one unsplit INT4 64 x 64 tile per CU at most (QKV at 128 rows): nothing else on
  // the CU hides a stage's loads, so keep three stages in flight (171 -> 162 us of
  // QKV per forward; with two tiles on a CU, or a split that pads the stage count,
  // two stages measured faster).  The 16-bit tile of the same shape is faster with
  // two stages (QKV 6144 x 2048 at 96 / 128 rows: 17.9 / 17.5 us with three stages
  // in flight, 16.4 / 16.0 us with one).
  if (g.Bw4 && t.bm == 64 && t.bn == 64 && t.splits == 1 && tiles <= kCUs) t.depth = 4;
  // INT4 64 x 64 tiles whose K range (split) is whole 256-wide stages: two groups
  // per stage, half the stages (with the two-stage ring: four stages of this size
  // spill).  Per forward at 128 rows: QKV 162 -> 152 us, gate/up 180 -> 170 us,
  // O 106 -> 102 us; a split of an odd number of groups would pad a stage.
  if (g.Bw4 && t.bm == 64 && t.bn == 64 && (t.kchunk % 256) == 0) {
    t.bk = 256;
    t.depth = 2;
  }
  return t;
}

// Finish a split-K product: the residual GEMM with a following RMSNorm sums the
// splits in one kernel per row and normalises (fused, *norm_done = true); the
// others sum per element and run their epilogue.  XT: the activation type of the
// outputs.
template <class XT>
hipError_t finish_splits(const GemmArgs& g, const GemmEpi& e, int splits, hipStream_t s, bool* norm_done) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (e.kind == EPI_QKV && g.defer_split) {   // the decode attention finishes the partials
    *g.defer_split = splits;
    return hipSuccess;
  }
  const int vpt = (g.N / 4 + 255) / 256;
  if (e.kind == EPI_RESID && e.norm_g && (g.N % 4) == 0 && (e.ldh % 4) == 0 && vpt <= 6) {
#define TL_RN(VPT_)                                                                                                \
  switch (splits) {                                                                                               \
    case 2: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 2>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    case 3: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 3>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    case 4: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 4>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    case 5: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 5>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    case 6: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 6>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    case 8: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 8>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
    default: TL_LAUNCH((splitk_resid_norm_kernel<XT, VPT_, 0>), dim3(g.M), dim3(256), 0, s, g, e, splits); break; \
  }
    if (vpt <= 2) { TL_RN(2) }
    else { TL_RN(6) }
#undef TL_RN
    *norm_done = true;
    return hipGetLastError();
  }
  const bool pr = paired(e.kind);
  const int64_t items = (int64_t)g.M * (pr ? g.N / 2 : g.N);
  dim3 rg((unsigned)((items + 255) / 256));
  switch (e.kind) {
    case EPI_QKV: TL_LAUNCH((splitk_epilogue_kernel<XT, EPI_QKV>), rg, dim3(256), 0, s, g, e, splits); break;
    case EPI_RESID: TL_LAUNCH((splitk_epilogue_kernel<XT, EPI_RESID>), rg, dim3(256), 0, s, g, e, splits); break;
    case EPI_SWIGLU: TL_LAUNCH((splitk_epilogue_kernel<XT, EPI_SWIGLU>), rg, dim3(256), 0, s, g, e, splits); break;
    case EPI_STORE: TL_LAUNCH((splitk_epilogue_kernel<XT, EPI_STORE>), rg, dim3(256), 0, s, g, e, splits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class AT, class XT, bool W4, int BM, int BN, int BK, int D>
hipError_t launch_mfma_t(const GemmArgs& g, const GemmEpi& e, const TileCfg& t, hipStream_t s, bool* norm_done) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, t.splits);
  switch (e.kind) {
    case EPI_QKV: TL_LAUNCH((gemm_mfma_kernel<AT, XT, W4, BM, BN, BK, D, EPI_QKV>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_RESID: TL_LAUNCH((gemm_mfma_kernel<AT, XT, W4, BM, BN, BK, D, EPI_RESID>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_SWIGLU: TL_LAUNCH((gemm_mfma_kernel<AT, XT, W4, BM, BN, BK, D, EPI_SWIGLU>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_HEAD: TL_LAUNCH((gemm_mfma_kernel<AT, XT, W4, BM, BN, BK, D, EPI_HEAD>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_STORE: TL_LAUNCH((gemm_mfma_kernel<AT, XT, W4, BM, BN, BK, D, EPI_STORE>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    default: return hipErrorInvalidValue;
  }
  if (t.splits > 1) return finish_splits<XT>(g, e, t.splits, s, norm_done);
  return hipGetLastError();
}

template <class AT, class XT, bool W4>
hipError_t launch_mfma(const GemmArgs& g, const GemmEpi& e, const TileCfg& t, hipStream_t s, bool* norm_done) {
  if (t.bn == 64) {
    if constexpr (!W4) {
      if (t.bm == 32 && t.depth == 4) return launch_mfma_t<AT, XT, W4, 32, 64, 128, 4>(g, e, t, s, norm_done);
    }
    if (t.bm == 32) return launch_mfma_t<AT, XT, W4, 32, 64, 128, 2>(g, e, t, s, norm_done);
    if constexpr (W4) {
      if (t.bk == 256) return launch_mfma_t<AT, XT, W4, 64, 64, 256, 2>(g, e, t, s, norm_done);
    }
    if constexpr (!std::is_same<XT, float>::value) {   // (split operands: four stages would spill)
      if (t.depth == 4) return launch_mfma_t<AT, XT, W4, 64, 64, 128, 4>(g, e, t, s, norm_done);
    }
    return launch_mfma_t<AT, XT, W4, 64, 64, 128, 2>(g, e, t, s, norm_done);
  }
  if (t.bm == 32) return launch_mfma_t<AT, XT, W4, 32, 128, 128, 2>(g, e, t, s, norm_done);
  if (t.bm == 64) return launch_mfma_t<AT, XT, W4, 64, 128, 128, 2>(g, e, t, s, norm_done);
  if constexpr (W4) return hipErrorInvalidValue;
  else return launch_mfma_t<AT, XT, W4, 128, 128, 64, 2>(g, e, t, s, norm_done);
}

// ---- small-M INT4 path
struct SkinnyCfg {
  int bm, wnb, splits, kchunk, depth;   // bm == 0: not applicable
};

// Tile and split choice for the small-M INT4 kernel, fitted to a sweep of the
// 2048-wide model's decode shapes at 13..64 rows on MI355X (per-launch event
// timing, the split reduction and the norm included): 32-row tiles at every row
// count (64-row tiles re-read less of A but ran 0.5-4.5 us slower per product),
// two 32-column blocks per wave when one-block tiles would number 32..63 (else
// one), K split so that about 192 workgroups run but at most 8 ways (the down
// projection at 11 splits with a third ring stage: 13.5-17.7 us; at 8 splits and
// two stages: 11.4-13.3 us).  Gate/up at 33..64 rows: 12.7-13.3 us unsplit here
// against 15.0-15.3 us on the LDS-tiled kernel.
SkinnyCfg pick_skinny(const GemmArgs& g, int kind) {
  SkinnyCfg t{0, 1, 1, 0, 2};
  if (!g.Bw4 || g.invariant || g.M > 64 || kind == EPI_HEAD || (g.K % 128) != 0 || (g.N % 32) != 0) return t;
  const int bm = 32;
  const int units = g.K / 128;
  const int64_t rows = (g.M + bm - 1) / bm;
  const int64_t tiles1 = (int64_t)((g.N + 127) / 128) * rows;
  const int wnb = (tiles1 >= 32 && tiles1 < 64) ? 2 : 1;
  const int64_t tiles = (int64_t)((g.N + 128 * wnb - 1) / (128 * wnb)) * rows;
  int sp = (int)std::min<int64_t>(8, std::max<int64_t>(1, (192 + tiles / 2) / tiles));
  sp = std::min(sp, units);
  int per = (units + sp - 1) / sp;
  sp = (units + per - 1) / per;
  while (sp > 1 && (!g.partial || (int64_t)sp * g.M * g.N > g.partial_cap)) {
    ++per;
    sp = (units + per - 1) / per;
  }
  t.bm = bm;
  t.wnb = wnb;
  t.splits = sp;
  t.kchunk = per * 128;
  t.depth = 2;
  return t;
}

template <int BM, int WNB, int D>
hipError_t launch_skinny_t(const GemmArgs& g, const GemmEpi& e, const SkinnyCfg& t, hipStream_t s, bool* norm_done) {
  constexpr int BN = 4 * 32 * WNB;
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, t.splits);
  switch (e.kind) {
    case EPI_QKV: TL_LAUNCH((gemm_skinny_w4_kernel<BM, WNB, D, EPI_QKV>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_RESID: TL_LAUNCH((gemm_skinny_w4_kernel<BM, WNB, D, EPI_RESID>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_SWIGLU: TL_LAUNCH((gemm_skinny_w4_kernel<BM, WNB, D, EPI_SWIGLU>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_STORE: TL_LAUNCH((gemm_skinny_w4_kernel<BM, WNB, D, EPI_STORE>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    default: return hipErrorInvalidValue;
  }
  if (t.splits > 1) return finish_splits<f16>(g, e, t.splits, s, norm_done);
  return hipGetLastError();
}

template <int D>
hipError_t launch_skinny_d(const GemmArgs& g, const GemmEpi& e, const SkinnyCfg& t, hipStream_t s, bool* norm_done) {
  if (t.bm == 32) return t.wnb == 1 ? launch_skinny_t<32, 1, D>(g, e, t, s, norm_done) : launch_skinny_t<32, 2, D>(g, e, t, s, norm_done);
  return hipErrorInvalidValue;
}

hipError_t launch_skinny(const GemmArgs& g, const GemmEpi& e, const SkinnyCfg& t, hipStream_t s, bool* norm_done) {
  if (t.depth == 2) return launch_skinny_d<2>(g, e, t, s, norm_done);
  return hipErrorInvalidValue;
}

// The row-tiled INT4 kernels for 65..128 rows where they measured ahead (see their
// comments): gate/up-shaped products (N >= 8192) unsplit on the eight-wave pair
// kernel; products with K >= 4096 (the down projection) and residual products with
// N <= 4096 (the O projection at 128 rows: 12.4 -> 11.6 us per launch with its
// reduction, forward 0.598 -> 0.587 ms) split 4 ways on the row-tiled kernel with
// WM = 2.  The QKV product stays on the LDS-tiled kernel, whose epilogue gathers
// its operands during the K loop (on the row-tiled kernel: 16.5 -> 23 us per
// launch).  Returns false to keep the LDS-tiled kernel.
bool w4_rows_launch(const GemmArgs& g, const GemmEpi& e, hipStream_t s, bool* norm_done, hipError_t* err) {
  if (!g.Bw4 || g.invariant || g.M <= 64 || g.M > 128 || e.pair_g != 16 || (g.K % 128) || (g.N % 32)) return false;
  if (e.kind != EPI_SWIGLU && e.kind != EPI_RESID && e.kind != EPI_STORE) return false;
  const int units = g.K / 128;
  if (g.N >= 8192) {
    dim3 grid((g.N + 127) / 128, (g.M + 63) / 64, 1);
    switch (e.kind) {
      case EPI_SWIGLU: TL_LAUNCH((gemm_w4_pair_kernel<EPI_SWIGLU>), grid, dim3(512), 0, s, g, e, g.K); break;
      case EPI_RESID: TL_LAUNCH((gemm_w4_pair_kernel<EPI_RESID>), grid, dim3(512), 0, s, g, e, g.K); break;
      default: TL_LAUNCH((gemm_w4_pair_kernel<EPI_STORE>), grid, dim3(512), 0, s, g, e, g.K); break;
    }
    *err = hipGetLastError();
    return true;
  }
  if ((g.K < 4096 && !(e.kind == EPI_RESID && g.N <= 4096)) || !g.partial || (int64_t)4 * g.M * g.N > g.partial_cap)
    return false;
  const int per = (units + 3) / 4;
  const int sp = (units + per - 1) / per;
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, sp);
  switch (e.kind) {
    case EPI_SWIGLU: TL_LAUNCH((gemm_w4_rows_kernel<2, EPI_SWIGLU>), grid, dim3(256), 0, s, g, e, per * 128); break;
    case EPI_RESID: TL_LAUNCH((gemm_w4_rows_kernel<2, EPI_RESID>), grid, dim3(256), 0, s, g, e, per * 128); break;
    default: TL_LAUNCH((gemm_w4_rows_kernel<2, EPI_STORE>), grid, dim3(256), 0, s, g, e, per * 128); break;
  }
  *err = sp > 1 ? finish_splits<f16>(g, e, sp, s, norm_done) : hipGetLastError();
  return true;
}

}  // namespace

namespace {
thread_local KernelTimer* t_kernel_timer = nullptr;
}  // namespace

void set_kernel_timer(KernelTimer* t) { t_kernel_timer = t; }
KernelTimer* kernel_timer() { return t_kernel_timer; }

int gemm_head_tiles(int act_dtype, int M, int N) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = 128;
  const TileCfg t = pick_tile(act_dtype, g, EPI_HEAD);
  return (N + t.bn - 1) / t.bn;
}

static hipError_t launch_gemm_core(int act_dtype, const GemmArgs& g, const GemmEpi& e, hipStream_t s,
                                   bool* norm_done);

namespace {
int act_bytes(int act_dtype) { return (act_dtype == DT_F32 || act_dtype == DT_F32X16) ? 4 : 2; }

// Rows [r0, r0 + M) of a product: A, the epilogue's row-indexed outputs and row
// descriptors offset to that range.
void row_range(int act_dtype, const GemmArgs& g, const GemmEpi& e, int r0, int M, GemmArgs* gc, GemmEpi* ec) {
  const int64_t esz = act_bytes(act_dtype);
  *gc = g;
  *ec = e;
  gc->M = M;
  gc->A = static_cast<const uint8_t*>(g.A) + (int64_t)r0 * g.K * esz;
  if (e.rows) ec->rows = e.rows + r0;
  if (e.q_out) ec->q_out = static_cast<uint8_t*>(e.q_out) + (int64_t)r0 * e.d * esz;
  if (e.h) ec->h = e.h + (int64_t)r0 * e.ldh;
  if (e.norm_out) ec->norm_out = static_cast<uint8_t*>(e.norm_out) + (int64_t)r0 * g.N * esz;
  if (e.u_out) ec->u_out = static_cast<uint8_t*>(e.u_out) + (int64_t)r0 * e.F * esz;
  if (e.out) ec->out = e.out + (int64_t)r0 * e.ldo;
  if (e.logits) ec->logits = e.logits + (int64_t)r0 * e.ldl;
  if (e.part_val) ec->part_val = e.part_val + (int64_t)r0 * e.n_tiles;
  if (e.part_idx) ec->part_idx = e.part_idx + (int64_t)r0 * e.n_tiles;
  if (e.part_val2) ec->part_val2 = e.part_val2 + (int64_t)r0 * e.n_tiles;
}
}  // namespace

// Residual GEMM with a following RMSNorm: fused into the split-K reduction when K
// is split, else the epilogue adds into h and a separate RMSNorm kernel runs.
// With g.invariant a product whose split partials would exceed g.partial_cap runs
// as several launches over consecutive row ranges (same split, same arithmetic).
hipError_t launch_gemm(int act_dtype, const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  if (g.defer_split) *g.defer_split = 0;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.invariant && act_dtype != DT_F32) {
    const TileCfg t = pick_tile(act_dtype, g, e.kind);
    const int64_t per_row = (int64_t)t.splits * g.N;
    if (t.splits > 1 && per_row * g.M > g.partial_cap) {
      const int rows = (int)std::max<int64_t>(1, g.partial_cap / per_row);
      if (rows < 1 || per_row > g.partial_cap) return hipErrorInvalidValue;
      for (int r0 = 0; r0 < g.M; r0 += rows) {
        GemmArgs gc;
        GemmEpi ec;
        row_range(act_dtype, g, e, r0, std::min(rows, g.M - r0), &gc, &ec);
        gc.defer_split = nullptr;   // each row range's partials reuse the buffer: finished here
        const hipError_t err = launch_gemm(act_dtype, gc, ec, s);
        if (err != hipSuccess) return err;
      }
      return hipSuccess;
    }
  }
  bool norm_done = false;
  hipError_t err = launch_gemm_core(act_dtype, g, e, s, &norm_done);
  if (err != hipSuccess || e.kind != EPI_RESID || !e.norm_g || norm_done) return err;
  const int xdt = act_dtype == DT_F32X16 ? DT_F32 : act_dtype;
  return launch_rmsnorm(xdt, e.h, e.norm_g, nullptr, g.M, g.N, e.norm_eps, e.norm_out, s);
}

static hipError_t launch_gemm_core(int act_dtype, const GemmArgs& g, const GemmEpi& e, hipStream_t s,
                                   bool* norm_done) {
  if (act_dtype == DT_F32) {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
    switch (e.kind) {
      case EPI_QKV: TL_LAUNCH(gemm_f32_kernel<EPI_QKV>, grid, dim3(256), 0, s, g, e); break;
      case EPI_RESID: TL_LAUNCH(gemm_f32_kernel<EPI_RESID>, grid, dim3(256), 0, s, g, e); break;
      case EPI_SWIGLU: TL_LAUNCH(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, g, e); break;
      case EPI_HEAD: TL_LAUNCH(gemm_f32_kernel<EPI_HEAD>, grid, dim3(256), 0, s, g, e); break;
      case EPI_STORE: TL_LAUNCH(gemm_f32_kernel<EPI_STORE>, grid, dim3(256), 0, s, g, e); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const TileCfg t = pick_tile(act_dtype, g, e.kind);
  if (act_dtype == DT_F16) {
    if (g.Bw4) {
      if (e.pair_g == 16) {
        const SkinnyCfg k = pick_skinny(g, e.kind);
        if (k.bm) return launch_skinny(g, e, k, s, norm_done);
        hipError_t err = hipSuccess;
        if (w4_rows_launch(g, e, s, norm_done, &err)) return err;
      }
      return launch_mfma<f16, f16, true>(g, e, t, s, norm_done);
    }
    return launch_mfma<f16, f16, false>(g, e, t, s, norm_done);
  }
  if (act_dtype == DT_BF16) {
    if (g.Bw4) return hipErrorInvalidValue;
    return launch_mfma<bf16, bf16, false>(g, e, t, s, norm_done);
  }
  if (act_dtype == DT_F32X16) {
    if (g.Bw4) return hipErrorInvalidValue;
    return launch_mfma<f16, float, false>(g, e, t, s, norm_done);
  }
  return hipErrorInvalidValue;
}
