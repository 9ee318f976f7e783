// GEMV for decode at batch 1..4: y = x W^T with the GEMM epilogues, for INT4
// weights in the W4G128 fragment layout and for dense fp16 weights.
//
// At a few rows the product is a stream over the weights (each weight used M
// times), so it runs on the vector units, not on MFMA tiles that would be 1/32
// full.  INT4: a workgroup owns one 32-row block of W; its waves take every NW-th
// 128-wide group of K.  In a group's 2 KB fragment block, lane l = r + 32 h of a
// wave reads two coalesced 16-byte words: 64 of row r's 128 codes (k steps
// 0..3 and 4..7, k half h).  The codes become exact fp16 integers (one and/or
// and one packed subtract per pair), dot2 instructions accumulate x * q in fp32,
// and the group's sum is multiplied by its scale, as on the MFMA path.  The two k
// halves meet with one shuffle, the waves through LDS in a fixed order (no split-K
// pass, no atomics), and wave 0 applies the epilogue: a rotary or gate/up pair
// lies 16 columns apart inside the same 32-row block.  Dense fp16: the same
// 32-row blocks, 8 lanes per row streaming 16-byte words of it.  The input is
// either the operand-type x or the fp32 residual, normalised by every workgroup
// as it is staged (the RMSNorm then needs no kernel of its own at these sizes).
#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace {

constexpr int kGemvMaxRows = 4;

// The rows of x in LDS (xs [M][K]): copied from the operand-type A, or formed
// from the fp32 residual as RMSNorm(h) * gain (mean of squares per row, summed in
// a fixed order over the workgroup); workgroup 0 also writes them to x_out.
// Ends with a workgroup barrier.
template <int M, int NW>
__device__ __forceinline__ void gemv_stage_x(const GemmArgs& g, f16* xs) {
  __shared__ float ssw[NW][M];
  const int K = g.K, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int CH = 4;   // residual chunks per thread and row kept in registers
  if (g.norm_h && K <= CH * NW * 256) {
    // x = RMSNorm(h) * gain from the fp32 residual: the rows and gains are read
    // once into registers, the mean of squares is summed per row (per thread in
    // k order, then a fixed-order workgroup sum), then the rows are normalised
    floatx4 hv[M][CH], gv[CH];
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int c = tid * 4 + ch * NW * 256;
      if (c < K) {
        gv[ch] = *reinterpret_cast<const floatx4*>(g.norm_g + c);
#pragma unroll
        for (int m = 0; m < M; ++m)
          hv[m][ch] = *reinterpret_cast<const floatx4*>(g.norm_h + (int64_t)min(m, g.M - 1) * K + c);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        if (tid * 4 + ch * NW * 256 < K) {
          const floatx4 v = hv[m][ch];
          a = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], a))));
        }
      }
      const float sm = wave_sum(a);
      if (lane == 0) ssw[wave][m] = sm;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += ssw[w][m];
      const float inv = 1.0f / sqrtf(t / (float)K + g.norm_eps);
      f16* xo = (g.x_out && blockIdx.x == 0 && m < g.M) ? reinterpret_cast<f16*>(g.x_out) + (int64_t)m * K : nullptr;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int c = tid * 4 + ch * NW * 256;
        if (c < K) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f16 x = (f16)(hv[m][ch][q] * inv * gv[ch][q]);
            xs[m * K + c + q] = x;
            if (xo) xo[c + q] = x;
          }
        }
      }
    }
  } else if (g.norm_h) {
    // x = RMSNorm(h) * gain, formed here from the fp32 residual: mean of squares
    // per row (fixed-order workgroup sum), then the rows in the operand type
    float ss[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float* hr = g.norm_h + (int64_t)min(m, g.M - 1) * K;
      float a = 0.f;
      for (int c = tid * 4; c < K; c += NW * 256) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(hr + c);
        a = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], a))));
      }
      ss[m] = wave_sum(a);
      if (lane == 0) ssw[wave][m] = ss[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += ssw[w][m];
      const float inv = 1.0f / sqrtf(t / (float)K + g.norm_eps);
      const float* hr = g.norm_h + (int64_t)min(m, g.M - 1) * K;
      f16* xo = (g.x_out && blockIdx.x == 0 && m < g.M) ? reinterpret_cast<f16*>(g.x_out) + (int64_t)m * K : nullptr;
      for (int c = tid * 4; c < K; c += NW * 256) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(hr + c);
        const floatx4 gg = *reinterpret_cast<const floatx4*>(g.norm_g + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16 x = (f16)(v[q] * inv * gg[q]);
          xs[m * K + c + q] = x;
          if (xo) xo[c + q] = x;
        }
      }
    }
  } else {
    // x rows to LDS (16-byte chunks)
    const f16* A = reinterpret_cast<const f16*>(g.A);
    for (int c = tid; c < M * K / 8; c += NW * 64) {
      const int m = c / (K / 8), kc = c - m * (K / 8);
      const int mr = min(m, g.M - 1);
      *reinterpret_cast<u32x4*>(&xs[m * K + kc * 8]) = *reinterpret_cast<const u32x4*>(A + (int64_t)mr * K + kc * 8);
    }
  }
  __syncthreads();
}

// The epilogue for row m, called by threads holding one output column each; for
// the paired kinds these are lanes 0..31 of wave 0 (a pair lies 16 columns apart).
// (QKV calls qkv_put instead, with its operands gathered ahead of the product.)
template <int KIND>
__device__ __forceinline__ void gemv_epilogue(const GemmEpi& e, int m, int col, float v) {
  if constexpr (paired(KIND)) {
    const float v1 = __shfl_down(v, 16, 32);   // column col + 16 of the pair
    if ((threadIdx.x & 31) < 16) epi_pair<f16, KIND>(e, m, col, v, v1);
  } else {
    epi_one<KIND>(e, m, col, v);
  }
}

// Weight words requested per lane before the first is used: a wave's whole share
// of a product up to these depths, so a launch costs about one memory round trip
// instead of one per group or chunk.
constexpr int kW4Ring = 8;     // INT4 groups (2 x 16 bytes + a scale each)
constexpr int kF16Ring = 16;   // dense 16-byte words

template <int M, int NW, int KIND>
__global__ __launch_bounds__(NW * 64) void gemv_w4_kernel(GemmArgs g, GemmEpi e) {
  constexpr int D = kW4Ring;
  extern __shared__ __attribute__((aligned(16))) f16 xs[];   // [M][K]
  __shared__ float red[NW][M][32];
  const int nb = blockIdx.x, K = g.K, N = g.N, groups = K >> 7;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hk = lane >> 5;
  const int col = nb * 32 + r;
  const uint32_t* wb = g.Bw4 + (int64_t)nb * groups * 512 + lane * 4;
  const uint16_t* sb = g.Bs + col;
  // ring slot j holds the wave's group wave + (j0 + j) NW; the first D are
  // requested before anything waits
  u32x4 w[D][2];
  uint16_t sc[D];
  // QKV: the epilogue lanes (wave 0, lanes 0..15: the first columns of the
  // pairs) read their rows' cache coordinates before the weights are requested
  constexpr int QR = KIND == EPI_QKV ? M : 1;
  QkvRow qrow[QR];
  QkvPrep qp[QR];
  if constexpr (KIND == EPI_QKV) {
    if (wave == 0 && lane < 16) {
#pragma unroll
      for (int m = 0; m < M; ++m) qrow[m] = qkv_row(e, min(m, g.M - 1));
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int gi = wave + j * NW;
    if (gi < groups) {
      w[j][0] = *reinterpret_cast<const u32x4*>(wb + (int64_t)gi * 512);
      w[j][1] = *reinterpret_cast<const u32x4*>(wb + (int64_t)gi * 512 + 256);
      sc[j] = sb[(int64_t)gi * N];
    } else {
      w[j][0] = w[j][1] = u32x4{0, 0, 0, 0};
      sc[j] = 0;
    }
  }
  if (gate_closed(g.live)) return;   // whole workgroup: no barrier passed yet
  gemv_stage_x<M, NW>(g, xs);
  if constexpr (KIND == EPI_QKV) {   // slot tables and rotary factors: in flight during the product
    if (wave == 0 && lane < 16) {
#pragma unroll
      for (int m = 0; m < M; ++m) qp[m] = qkv_prep(e, qrow[m], m, col);
    }
  }
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (int j0 = 0; wave + j0 * NW < groups; j0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int gi = wave + (j0 + j) * NW;
      if (gi >= groups) break;
      float ga[M];
#pragma unroll
      for (int m = 0; m < M; ++m) ga[m] = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint32_t wd = jj < 4 ? w[j][0][jj] : w[j][1][jj - 4];
        // word jj holds k = 16 jj + 8 hk + 0..7 of the group
        const int k0 = gi * 128 + 16 * jj + 8 * hk;
        half2v q[4];
        w4_pairs(wd, q);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const half8 xv = *reinterpret_cast<const half8*>(&xs[m * K + k0]);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const half2v xp = {xv[2 * p], xv[2 * p + 1]};
            ga[m] = __builtin_amdgcn_fdot2(q[p], xp, ga[m], false);
          }
        }
      }
      const float scale = (float)__builtin_bit_cast(f16, sc[j]);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = fmaf(ga[m], scale, acc[m]);
      const int gn = gi + D * NW;   // refill the slot D groups ahead
      if (gn < groups) {
        w[j][0] = *reinterpret_cast<const u32x4*>(wb + (int64_t)gn * 512);
        w[j][1] = *reinterpret_cast<const u32x4*>(wb + (int64_t)gn * 512 + 256);
        sc[j] = sb[(int64_t)gn * N];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] += __shfl_xor(acc[m], 32, 64);
  if (hk == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][m][r] = acc[m];
  }
  __syncthreads();
  if (wave != 0 || hk != 0) return;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) v += red[w2][m][r];
    if (m >= g.M) continue;
    if constexpr (KIND == EPI_QKV) {
      const float v1 = __shfl_down(v, 16, 32);   // column col + 16 of the pair
      if (r < 16) qkv_put<f16>(e, qp[m], v, v1);
    } else {
      gemv_epilogue<KIND>(e, m, col, v);
    }
  }
}

// Dense fp16 weights [N, K]: a workgroup of NW waves owns R = 8 NW / KS rows; a
// wave takes 8 of them and every KS-th 64-wide chunk of K (KS waves share a row
// group), 8 lanes per row: lane kl reads 16 bytes at k = 64 c + 8 kl of chunk c,
// so a row's 8 lanes cover 128 contiguous bytes.  dot2 into fp32; the 8 lanes of
// a row meet by shuffles, the KS waves through LDS in a fixed order.  Paired
// epilogues need R = 32 (a pair lies 16 columns apart).
template <int M, int NW, int KS, int KIND>
__global__ __launch_bounds__(NW * 64) void gemv_f16_kernel(GemmArgs g, GemmEpi e) {
  constexpr int U = kF16Ring, R = 8 * NW / KS;
  extern __shared__ __attribute__((aligned(16))) f16 xs[];   // [M][K]
  __shared__ float red[KS][R][M];
  const int nb = blockIdx.x, K = g.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane >> 3, kl = lane & 7, rg = wave / KS, kp = wave % KS;
  const int row = nb * R + rg * 8 + rr;
  const f16* wr = reinterpret_cast<const f16*>(g.B) + (int64_t)row * K + 8 * kl;
  const int nc = K / 64;   // chunks per row
  u32x4 w[U];   // slot j: chunk kp + (j0 + j) KS
  // QKV (R = 32): the epilogue threads 0..15 handle the column pairs; their rows'
  // cache coordinates are read first, the rest once the weights are requested
  constexpr int QR = KIND == EPI_QKV ? M : 1;
  QkvRow qrow[QR];
  QkvPrep qp[QR];
  if constexpr (KIND == EPI_QKV) {
    static_assert(R == 32, "paired epilogue: a pair lies 16 columns apart");
    if (tid < 16) {
#pragma unroll
      for (int m = 0; m < M; ++m) qrow[m] = qkv_row(e, min(m, g.M - 1));
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int c = kp + j * KS;
    w[j] = c < nc ? *reinterpret_cast<const u32x4*>(wr + 64 * c) : u32x4{0, 0, 0, 0};
  }
  if (gate_closed(g.live)) return;
  gemv_stage_x<M, NW>(g, xs);
  if constexpr (KIND == EPI_QKV) {
    if (tid < 16) {
#pragma unroll
      for (int m = 0; m < M; ++m) qp[m] = qkv_prep(e, qrow[m], m, nb * R + tid);
    }
  }
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (int j0 = 0; kp + j0 * KS < nc; j0 += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = kp + (j0 + j) * KS;
      if (c >= nc) break;
      const half8 wv = __builtin_bit_cast(half8, w[j]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const half8 xv = *reinterpret_cast<const half8*>(&xs[m * K + 64 * c + 8 * kl]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const half2v a = {wv[2 * p], wv[2 * p + 1]};
          const half2v b = {xv[2 * p], xv[2 * p + 1]};
          acc[m] = __builtin_amdgcn_fdot2(a, b, acc[m], false);
        }
      }
      const int cn = c + U * KS;
      if (cn < nc) w[j] = *reinterpret_cast<const u32x4*>(wr + 64 * cn);
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) acc[m] += __shfl_xor(acc[m], o, 64);
    if (kl == 0) red[kp][rg * 8 + rr][m] = acc[m];
  }
  __syncthreads();
  if (tid >= R) return;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < KS; ++q) v += red[q][tid][m];
    if (m >= g.M) continue;
    if constexpr (KIND == EPI_QKV) {
      const float v1 = __shfl_down(v, 16, 32);   // column + 16 of the pair
      if (tid < 16) qkv_put<f16>(e, qp[m], v, v1);
    } else {
      gemv_epilogue<KIND>(e, m, nb * R + tid, v);
    }
  }
}

template <int M>
hipError_t gemv_f16_launch(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  const size_t lds = (size_t)M * g.K * sizeof(f16);
  // paired epilogues: 32 rows per workgroup, two waves per row group; residual:
  // 8 rows per workgroup, four waves per row group (four times the workgroups)
  switch (e.kind) {
    case EPI_QKV: TL_LAUNCH((gemv_f16_kernel<M, 8, 2, EPI_QKV>), dim3(g.N / 32), dim3(512), lds, s, g, e); break;
    case EPI_SWIGLU: TL_LAUNCH((gemv_f16_kernel<M, 8, 2, EPI_SWIGLU>), dim3(g.N / 32), dim3(512), lds, s, g, e); break;
    case EPI_RESID: TL_LAUNCH((gemv_f16_kernel<M, 4, 4, EPI_RESID>), dim3(g.N / 8), dim3(256), lds, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int M, int NW>
hipError_t gemv_launch_kind(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  const dim3 grid(g.N / 32);
  const size_t lds = (size_t)M * g.K * sizeof(f16);
  switch (e.kind) {
    case EPI_QKV: TL_LAUNCH((gemv_w4_kernel<M, NW, EPI_QKV>), grid, dim3(NW * 64), lds, s, g, e); break;
    case EPI_RESID: TL_LAUNCH((gemv_w4_kernel<M, NW, EPI_RESID>), grid, dim3(NW * 64), lds, s, g, e); break;
    case EPI_SWIGLU: TL_LAUNCH((gemv_w4_kernel<M, NW, EPI_SWIGLU>), grid, dim3(NW * 64), lds, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NW>
hipError_t gemv_launch_nw(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  switch (g.M) {
    case 1: return gemv_launch_kind<1, NW>(g, e, s);
    case 2: return gemv_launch_kind<2, NW>(g, e, s);
    default: return gemv_launch_kind<4, NW>(g, e, s);
  }
}

}  // namespace

bool gemv_applies(const GemmArgs& g, int kind) {
  const bool w4 = g.Bw4 && !g.B, dense = g.B && !g.Bw4;
  return (w4 || dense) && g.M >= 1 && g.M <= kGemvMaxRows && (g.K % 128) == 0 && (g.N % 32) == 0 &&
         (size_t)kGemvMaxRows * g.K * sizeof(f16) <= 64 * 1024 &&
         (kind == EPI_QKV || kind == EPI_RESID || kind == EPI_SWIGLU);
}

hipError_t launch_gemv(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  if (!gemv_applies(g, e.kind)) return hipErrorInvalidValue;
  if (g.B) {
    switch (g.M) {
      case 1: return gemv_f16_launch<1>(g, e, s);
      case 2: return gemv_f16_launch<2>(g, e, s);
      default: return gemv_f16_launch<4>(g, e, s);
    }
  }
  // INT4: fewer column blocks -> more waves per block, so enough groups are in flight
  return g.N / 32 >= 128 ? gemv_launch_nw<4>(g, e, s) : gemv_launch_nw<8>(g, e, s);
}
