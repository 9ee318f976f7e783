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

#include <algorithm>

namespace {

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

template <class AT, int KIND>
__device__ __forceinline__ void epi_pair(const GemmEpi& e, int r, int c, float v0, float v1) {
  if constexpr (KIND == EPI_QKV) {
    const int d = e.d, dh = e.dh, G = e.pair_g;
    const int sect = c / d;
    const int cc = c - sect * d;
    const int head = cc / dh;
    const int cd = cc - head * dh;
    const RowInfo ri = e.rows[r];
    if (sect == 2) {
      AT* vp = kv_ptr<AT>(e.kv, ri, 1, head, ri.pos);
      vp[cd] = from_f32<AT>(v0);
      vp[cd + G] = from_f32<AT>(v1);
      return;
    }
    const int half = dh >> 1;
    const int ci = cd / G;
    const int n0 = (ci >> 1) * G + (cd - ci * G);
    const float cs = e.rope_cos[(int64_t)ri.pos * half + n0];
    const float sn = e.rope_sin[(int64_t)ri.pos * half + n0];
    const float x1 = v0 * cs - v1 * sn;
    const float x2 = v1 * cs + v0 * sn;
    AT* dst = (sect == 0) ? reinterpret_cast<AT*>(e.q_out) + (int64_t)r * d + head * dh
                          : kv_ptr<AT>(e.kv, ri, 0, head, ri.pos);
    dst[n0] = from_f32<AT>(x1);
    dst[n0 + half] = from_f32<AT>(x2);
  } else if constexpr (KIND == EPI_SWIGLU) {
    const int G = e.pair_g;
    const int ci = c / G;
    const int n = (ci >> 1) * G + (c - ci * G);
    const float s = v0 / (1.0f + expf(-v0));
    reinterpret_cast<AT*>(e.u_out)[(int64_t)r * e.F + n] = from_f32<AT>(s * v1);
  }
}

template <int KIND>
__device__ __forceinline__ void epi_one(const GemmEpi& e, int r, int c, float v) {
  if constexpr (KIND == EPI_RESID) {
    e.h[(int64_t)r * e.ldh + c] += v;
  } else if constexpr (KIND == EPI_HEAD) {
    if (e.logits) e.logits[(int64_t)r * e.ldl + c] = v;
  } else if constexpr (KIND == EPI_STORE) {
    e.out[(int64_t)r * e.ldo + c] = v;
  }
}

constexpr bool paired(int kind) { return kind == EPI_QKV || kind == EPI_SWIGLU; }

// (value, index) ordering for the greedy token: larger value wins, ties -> lower index.
__device__ __forceinline__ void best_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Workgroup of 4 waves (2 x 2) computes a BM x BN tile over the K range of its
// split (blockIdx.z).  Per 64-wide K stage: global -> registers (issued one stage
// ahead, so the loads of stage s+1 are in flight during the MFMAs of stage s),
// registers -> LDS, then each wave runs (BM/32) x (BN/32) 16x16x32 MFMAs per
// 32-wide k step.  With several splits, every workgroup stores its fp32 partial
// tile; the last one to arrive (per-tile counter) adds the partials in split
// order, so the result does not depend on arrival order, and runs the epilogue.
template <class AT, bool W4, int BM, int BN, int KIND>
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmArgs g, GemmEpi e, int kchunk) {
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;   // padded LDS row, elements
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int AC = BM * (BK / 8) / 256;                 // 16-byte A chunks per thread
  constexpr int BC = W4 ? 1 : BN * (BK / 8) / 256;        // 16-byte B chunks per thread
  static_assert(TM >= 1 && TN >= 2 && (TN % 2) == 0 && AC >= 1 && BC >= 1, "tile");
  typedef typename Mfma<AT>::frag frag;

  __shared__ __attribute__((aligned(16))) AT As[BM * LDK];
  __shared__ __attribute__((aligned(16))) AT Bs[BN * LDK];
  __shared__ float Ss[W4 ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K;
  const int S = gridDim.z, z = blockIdx.z;
  const int kb = z * kchunk, ke = min(K, kb + kchunk);
  const AT* A = reinterpret_cast<const AT*>(g.A);
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

  uint4 ra[AC], rb[BC];
  uint16_t rs = 0;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
      const int gr = m0 + r, gk = k0 + kc;
      ra[i] = uint4{0u, 0u, 0u, 0u};
      if (gr < M && gk < ke) ra[i] = *reinterpret_cast<const uint4*>(A + (int64_t)gr * K + gk);
    }
    if constexpr (W4) {
      const int gidx = k0 >> 7, hsel = (k0 >> 6) & 1;
      const int c = tid;
      rb[0] = uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};   // q = 0
      if (c < BN * 2) {
        const int nb = c >> 5, within = c & 31, row = within >> 1, qq = within & 1;
        const int gn = n0 + nb * 16 + row;
        if (gn < N) {
          const int64_t blk = (int64_t)((n0 >> 4) + nb) * groups + gidx;
          rb[0] = *reinterpret_cast<const uint4*>(g.Bw4 + blk * 256 + row * 16 + hsel * 8 + qq * 4);
        }
      }
      if (hsel == 0 && tid < BN) {
        const int gn = n0 + tid;
        rs = gn < N ? g.Bs[(int64_t)gidx * N + gn] : (uint16_t)0;
      }
    } else {
      const AT* B = reinterpret_cast<const AT*>(g.B);
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
        const int gn = n0 + r, gk = k0 + kc;
        rb[i] = uint4{0u, 0u, 0u, 0u};
        if (gn < N && gk < ke) rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)gn * K + gk);
      }
    }
  };
  auto lstore = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[r * LDK + kc]) = ra[i];
    }
    if constexpr (W4) {
      const int c = tid;
      if (c < BN * 2) {
        const int nb = c >> 5, within = c & 31, row = within >> 1, qq = within & 1;
        const uint32_t ws[4] = {rb[0].x, rb[0].y, rb[0].z, rb[0].w};
        f16* dst = reinterpret_cast<f16*>(&Bs[(nb * 16 + row) * LDK + qq * 32]);
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          half8 h;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const half2v t = w4_pair(ws[wi], p);
            h[2 * p] = t[0];
            h[2 * p + 1] = t[1];
          }
          *reinterpret_cast<half8*>(dst + wi * 8) = h;
        }
      }
      if (((k0 >> 6) & 1) == 0 && tid < BN) Ss[tid] = (float)__builtin_bit_cast(f16, rs);
    } else {
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
        *reinterpret_cast<uint4*>(&Bs[r * LDK + kc]) = rb[i];
      }
    }
  };

  if (kb < ke) gload(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    lstore(k0);
    __syncthreads();
    if (k0 + BK < ke) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      frag a[TM], b[TN];
      const int lrow = lane & 15, lk = kk + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const frag*>(&As[(wm * WTM + i * 16 + lrow) * LDK + lk]);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const frag*>(&Bs[(wn * WTN + j * 16 + lrow) * LDK + lk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (W4) tmp[i][j] = Mfma<AT>::run(a[i], b[j], tmp[i][j]);
          else acc[i][j] = Mfma<AT>::run(a[i], b[j], acc[i][j]);
        }
    }
    if constexpr (W4) {
      if (((k0 >> 6) & 1) == 1) {   // end of a 128-wide group: apply its scale
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float sc = Ss[wn * WTN + j * 16 + (lane & 15)];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            acc[i][j] += sc * tmp[i][j];
            tmp[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    __syncthreads();
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
    __shared__ float red_v[BM][2];
    __shared__ int red_i[BM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow_t = wm * WTM + i * 16 + lr + r;
        const int row = m0 + lrow_t;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + lc;
          if (col < N) {
            const float v = acc[i][j][r];
            if (row < M) epi_one<KIND>(e, row, col, v);
            best_merge(bv, bi, v, col);
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          best_merge(bv, bi, ov, oi);
        }
        if (lc == 0) {
          red_v[lrow_t][wn] = bv;
          red_i[lrow_t][wn] = bi;
        }
      }
    __syncthreads();
    for (int t = tid; t < BM; t += 256) {
      const int row = m0 + t;
      if (row < M) {
        float bv = red_v[t][0];
        int bi = red_i[t][0];
        best_merge(bv, bi, red_v[t][1], red_i[t][1]);
        e.part_val[(int64_t)row * e.n_tiles + blockIdx.x] = bv;
        e.part_idx[(int64_t)row * e.n_tiles + blockIdx.x] = bi;
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
            if (col < N) epi_pair<AT, KIND>(e, row, col, acc[i][j][r], acc[i][j + 1][r]);
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

// fp32 operands: a plain LDS-tiled SIMT kernel (64 x 64 tile, 4 x 4 per thread).
// Paired epilogues use adjacent column pairs (row-permutation granularity 1).
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, GemmEpi e) {
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
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) {
          if (row < M) epi_one<KIND>(e, row, col, acc[i][j]);
          best_merge(bv, bi, acc[i][j], col);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        best_merge(bv, bi, ov, oi);
      }
      if (tx == 0 && row < M) {
        e.part_val[(int64_t)row * e.n_tiles + blockIdx.x] = bv;
        e.part_idx[(int64_t)row * e.n_tiles + blockIdx.x] = bi;
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
    float v0 = 0.f, v1 = 0.f;
    for (int z = 0; z < S; ++z) {
      const float* pr = g.partial + ((int64_t)z * M + row) * N;
      v0 += pr[c];
      v1 += pr[c + G];
    }
    epi_pair<AT, KIND>(e, row, c, v0, v1);
  } else {
    if (idx >= (int64_t)M * N) return;
    const int row = (int)(idx / N);
    const int c = (int)(idx - (int64_t)row * N);
    float v = 0.f;
    for (int z = 0; z < S; ++z) v += g.partial[((int64_t)z * M + row) * N + c];
    epi_one<KIND>(e, row, c, v);
  }
}

struct TileCfg {
  int bm, bn, splits, kchunk;
};

constexpr int kCUs = 256;

// Tile and split choice: enough workgroups to cover the 256 CUs about twice,
// splitting K (in whole 128-wide groups) only when the tiles alone cannot.
TileCfg pick_tile(int act_dtype, const GemmArgs& g, int kind) {
  if (act_dtype == DT_F32) return {64, 64, 1, g.K};
  TileCfg t{g.M <= 32 ? 32 : (g.M <= 64 ? 64 : 128), 128, 1, g.K};
  const int64_t mt = (g.M + t.bm - 1) / t.bm;
  if (mt * ((g.N + 127) / 128) < kCUs) t.bn = 64;
  if (kind == EPI_HEAD) t.bn = 128;
  const int64_t tiles = mt * ((g.N + t.bn - 1) / t.bn);
  const int unit = 128;
  const int64_t units = (g.K + unit - 1) / unit;
  if (kind != EPI_HEAD && tiles < 2 * kCUs && g.partial && units > 1 && (g.N % 32) == 0) {
    int64_t want = (2 * kCUs + tiles - 1) / tiles;
    want = std::min<int64_t>(want, 16);
    want = std::min<int64_t>(want, units);
    while (want > 1 && want * g.M * g.N > g.partial_cap) --want;
    if (want > 1) {
      const int64_t per = (units + want - 1) / want;     // units per split
      t.kchunk = (int)(per * unit);
      t.splits = (int)((units + per - 1) / per);
    }
  }
  return t;
}

template <class AT, bool W4, int BM, int BN>
hipError_t launch_mfma_t(const GemmArgs& g, const GemmEpi& e, const TileCfg& t, hipStream_t s) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, t.splits);
  switch (e.kind) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_mfma_kernel<AT, W4, BM, BN, EPI_QKV>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_mfma_kernel<AT, W4, BM, BN, EPI_RESID>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_mfma_kernel<AT, W4, BM, BN, EPI_SWIGLU>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_HEAD: hipLaunchKernelGGL((gemm_mfma_kernel<AT, W4, BM, BN, EPI_HEAD>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    case EPI_STORE: hipLaunchKernelGGL((gemm_mfma_kernel<AT, W4, BM, BN, EPI_STORE>), grid, dim3(256), 0, s, g, e, t.kchunk); break;
    default: return hipErrorInvalidValue;
  }
  if (t.splits > 1) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool pr = e.kind == EPI_QKV || e.kind == EPI_SWIGLU;
    const int64_t items = (int64_t)g.M * (pr ? g.N / 2 : g.N);
    dim3 rg((unsigned)((items + 255) / 256));
    switch (e.kind) {
      case EPI_QKV: hipLaunchKernelGGL((splitk_epilogue_kernel<AT, EPI_QKV>), rg, dim3(256), 0, s, g, e, t.splits); break;
      case EPI_RESID: hipLaunchKernelGGL((splitk_epilogue_kernel<AT, EPI_RESID>), rg, dim3(256), 0, s, g, e, t.splits); break;
      case EPI_SWIGLU: hipLaunchKernelGGL((splitk_epilogue_kernel<AT, EPI_SWIGLU>), rg, dim3(256), 0, s, g, e, t.splits); break;
      case EPI_STORE: hipLaunchKernelGGL((splitk_epilogue_kernel<AT, EPI_STORE>), rg, dim3(256), 0, s, g, e, t.splits); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <class AT, bool W4>
hipError_t launch_mfma(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  const TileCfg t = pick_tile(DT_F16, g, e.kind);
  if (t.bn == 64) {
    if (t.bm == 32) return launch_mfma_t<AT, W4, 32, 64>(g, e, t, s);
    if (t.bm == 64) return launch_mfma_t<AT, W4, 64, 64>(g, e, t, s);
    return launch_mfma_t<AT, W4, 128, 64>(g, e, t, s);
  }
  if (t.bm == 32) return launch_mfma_t<AT, W4, 32, 128>(g, e, t, s);
  if (t.bm == 64) return launch_mfma_t<AT, W4, 64, 128>(g, e, t, s);
  return launch_mfma_t<AT, W4, 128, 128>(g, e, t, s);
}

}  // namespace

int gemm_head_tiles(int act_dtype, int M, int N) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = 128;
  const TileCfg t = pick_tile(act_dtype, g, EPI_HEAD);
  return (N + t.bn - 1) / t.bn;
}

hipError_t launch_gemm(int act_dtype, const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (act_dtype == DT_F32) {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
    switch (e.kind) {
      case EPI_QKV: hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, grid, dim3(256), 0, s, g, e); break;
      case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, dim3(256), 0, s, g, e); break;
      case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, g, e); break;
      case EPI_HEAD: hipLaunchKernelGGL(gemm_f32_kernel<EPI_HEAD>, grid, dim3(256), 0, s, g, e); break;
      case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, dim3(256), 0, s, g, e); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (act_dtype == DT_F16) {
    if (g.Bw4) return launch_mfma<f16, true>(g, e, s);
    return launch_mfma<f16, false>(g, e, s);
  }
  if (act_dtype == DT_BF16) {
    if (g.Bw4) return hipErrorInvalidValue;
    return launch_mfma<bf16, false>(g, e, s);
  }
  return hipErrorInvalidValue;
}
