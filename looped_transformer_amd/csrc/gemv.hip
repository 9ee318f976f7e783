// INT4 GEMV for decode at batch 1..4: y = x W^T with W in the W4G128 fragment
// layout and the GEMM epilogues.
//
// At a few rows the product is a stream over the weights (each weight used M
// times), so it runs on the vector units, not on MFMA tiles that would be 1/32
// full.  A workgroup owns one 32-row block of W; its waves take every NW-th
// 128-wide group of K.  In a group's 2 KB fragment block, lane l = r + 32 h of a
// wave reads two coalesced 16-byte words: 64 of row r's 128 codes (k steps
// 0..3 and 4..7, k half h).  The codes become exact fp16 integers (one and/or
// and one packed subtract per pair), dot2 instructions accumulate x * q in fp32,
// and the group's sum is multiplied by its scale, as on the MFMA path.  The two k
// halves meet with one shuffle, the waves through LDS in a fixed order (no split-K
// pass, no atomics), and wave 0 applies the epilogue: a rotary or gate/up pair
// lies 16 columns apart inside the same 32-row block.  The input is either the
// operand-type x or the fp32 residual, normalised by every workgroup as it is
// staged (the RMSNorm then needs no kernel of its own at these sizes).
#include "device_common.h"
#include "epilogue.h"

namespace {

constexpr int kGemvMaxRows = 4;

template <int M, int NW, int KIND>
__global__ __launch_bounds__(NW * 64) void gemv_w4_kernel(GemmArgs g, GemmEpi e) {
  extern __shared__ __attribute__((aligned(16))) f16 xs[];   // [M][K]
  __shared__ float red[NW][M][32];
  const int nb = blockIdx.x, K = g.K, N = g.N, groups = K >> 7;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hk = lane >> 5;
  // the weights of this wave's first group are requested before anything waits
  int gi = wave;
  u32x4 w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0};
  if (gi < groups) {
    const uint32_t* blk = g.Bw4 + ((int64_t)nb * groups + gi) * 512;
    w0 = *reinterpret_cast<const u32x4*>(blk + lane * 4);
    w1 = *reinterpret_cast<const u32x4*>(blk + 256 + lane * 4);
  }
  if (gate_closed(g.live)) return;   // whole workgroup: no barrier passed yet
  if (g.norm_h) {
    // x = RMSNorm(h) * gain, formed here from the fp32 residual: mean of squares
    // per row (fixed-order workgroup sum), then the rows in the operand type
    __shared__ float ssw[NW][M];
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
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  const int col = nb * 32 + r;
  for (; gi < groups; gi += NW) {
    // next group's words in flight while this one is summed
    const int gn = gi + NW;
    u32x4 n0 = {0, 0, 0, 0}, n1 = {0, 0, 0, 0};
    if (gn < groups) {
      const uint32_t* blk = g.Bw4 + ((int64_t)nb * groups + gn) * 512;
      n0 = *reinterpret_cast<const u32x4*>(blk + lane * 4);
      n1 = *reinterpret_cast<const u32x4*>(blk + 256 + lane * 4);
    }
    asm volatile("" ::: "memory");   // keep the prefetch ahead of this group's math
    const float sc = (float)__builtin_bit_cast(f16, g.Bs[(int64_t)gi * N + col]);
    float ga[M];
#pragma unroll
    for (int m = 0; m < M; ++m) ga[m] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t wd = jj < 4 ? w0[jj] : w1[jj - 4];
      // word jj holds k = 16 jj + 8 hk + 0..7 of the group
      const int k0 = gi * 128 + 16 * jj + 8 * hk;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const half8 xv = *reinterpret_cast<const half8*>(&xs[m * K + k0]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const half2v q = w4_pair(wd, p);
          const half2v xp = {xv[2 * p], xv[2 * p + 1]};
          ga[m] = __builtin_amdgcn_fdot2(q, xp, ga[m], false);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = fmaf(ga[m], sc, acc[m]);
    w0 = n0;
    w1 = n1;
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
    for (int w = 0; w < NW; ++w) v += red[w][m][r];
    if (m >= g.M) continue;
    if constexpr (paired(KIND)) {
      const float v1 = __shfl_down(v, 16, 32);   // column col + 16 of the pair
      if (r < 16) epi_pair<f16, KIND>(e, m, col, v, v1);
    } else {
      epi_one<KIND>(e, m, col, v);
    }
  }
}

template <int M, int NW>
hipError_t gemv_launch_kind(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  const dim3 grid(g.N / 32);
  const size_t lds = (size_t)M * g.K * sizeof(f16);
  switch (e.kind) {
    case EPI_QKV: hipLaunchKernelGGL((gemv_w4_kernel<M, NW, EPI_QKV>), grid, dim3(NW * 64), lds, s, g, e); break;
    case EPI_RESID: hipLaunchKernelGGL((gemv_w4_kernel<M, NW, EPI_RESID>), grid, dim3(NW * 64), lds, s, g, e); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemv_w4_kernel<M, NW, EPI_SWIGLU>), grid, dim3(NW * 64), lds, s, g, e); break;
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

bool gemv_w4_applies(const GemmArgs& g, int kind) {
  return g.Bw4 && !g.B && g.M >= 1 && g.M <= kGemvMaxRows && (g.K % 128) == 0 && (g.N % 32) == 0 &&
         (!g.norm_h || (g.K % 4) == 0) &&
         (size_t)kGemvMaxRows * g.K * sizeof(f16) <= 64 * 1024 &&
         (kind == EPI_QKV || kind == EPI_RESID || kind == EPI_SWIGLU);
}

hipError_t launch_gemv_w4(const GemmArgs& g, const GemmEpi& e, hipStream_t s) {
  if (!gemv_w4_applies(g, e.kind)) return hipErrorInvalidValue;
  // fewer column blocks: more waves per block, so enough groups are in flight
  return g.N / 32 >= 128 ? gemv_launch_nw<4>(g, e, s) : gemv_launch_nw<8>(g, e, s);
}
