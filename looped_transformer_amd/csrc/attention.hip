// Causal softmax attention of each row over its own lane's K/V in the cache slot
// of the current block application (one slot per block application: the K/V a
// loop iteration attends to are the ones that same iteration wrote at earlier
// positions).  Row r at position p attends to positions 0..p of its slot; scale
// 1/sqrt(head_dim); one K/V head per query head.
//
// One wave per (row, head).  Keys are streamed in chunks of 64 (one key per lane
// for the score), with a running max / sum (online softmax); the value sum keeps
// two head dimensions per lane.  Serves prefill (rows of one sequence share the
// slot) and decode (one row per lane) alike.
#include "device_common.h"

namespace {

template <class T> struct Vec8;
template <> struct Vec8<f16> { typedef half8 type; };
template <> struct Vec8<bf16> { typedef bf16x8 type; };

template <class T>
__device__ __forceinline__ float dot_row(const float* __restrict__ q, const T* __restrict__ k, int dh) {
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
    typedef typename Vec8<T>::type v8;
    for (int i = 0; i < dh; i += 8) {
      const v8 kv = *reinterpret_cast<const v8*>(k + i);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(q[i + u], (float)kv[u], acc);
    }
  } else {
    for (int i = 0; i < dh; i += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(k + i);
      acc = fmaf(q[i], kv.x, acc);
      acc = fmaf(q[i + 1], kv.y, acc);
      acc = fmaf(q[i + 2], kv.z, acc);
      acc = fmaf(q[i + 3], kv.w, acc);
    }
  }
  return acc;
}

template <class T>
__global__ __launch_bounds__(256) void attn_rows_kernel(const T* __restrict__ q, const RowInfo* __restrict__ rows,
                                                       int n, KVParams kv, T* __restrict__ out, int d,
                                                       float scale) {
  __shared__ float qs[4][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = kv.H, dh = kv.dh;
  const int item = blockIdx.x * 4 + wv;
  if (item >= n * H) return;            // whole wave leaves together
  const int r = item / H, h = item - (item / H) * H;
  const RowInfo ri = rows[r];
  const T* Kp = kv_ptr<T>(kv, ri, 0, h, 0);
  const T* Vp = kv_ptr<T>(kv, ri, 1, h, 0);
  float* qw = qs[wv];
  for (int i = lane; i < dh; i += 64) qw[i] = (float)q[(int64_t)r * d + h * dh + i] * scale;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int npos = ri.pos + 1;
  const bool own = 2 * lane < dh;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = 0; t0 < npos; t0 += 64) {
    const int t = t0 + lane;
    float s = -INFINITY;
    if (t < npos) s = dot_row<T>(qw, Kp + (int64_t)t * dh, dh);
    const float mn = fmaxf(m, wave_max(s));
    const float p = (t < npos) ? expf(s - mn) : 0.f;
    const float corr = expf(m - mn);
    l = l * corr + wave_sum(p);
    o0 *= corr;
    o1 *= corr;
    const int cnt = min(64, npos - t0);
    for (int u = 0; u < cnt; ++u) {
      const float pu = __shfl(p, u, 64);
      if (own) {
        const T* vr = Vp + (int64_t)(t0 + u) * dh + 2 * lane;
        o0 = fmaf(pu, (float)vr[0], o0);
        o1 = fmaf(pu, (float)vr[1], o1);
      }
    }
    m = mn;
  }
  if (own) {
    const float inv = 1.0f / l;
    T* op = out + (int64_t)r * d + h * dh + 2 * lane;
    op[0] = from_f32<T>(o0 * inv);
    op[1] = from_f32<T>(o1 * inv);
  }
}

}  // namespace

hipError_t launch_attention(int dtype, const void* q, const RowInfo* rows, int n, const KVParams& kv, void* out,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int d = kv.H * kv.dh;
  const float scale = 1.0f / sqrtf((float)kv.dh);
  dim3 grid((n * kv.H + 3) / 4);
  switch (dtype) {
    case DT_F32:
      hipLaunchKernelGGL(attn_rows_kernel<float>, grid, dim3(256), 0, s, (const float*)q, rows, n, kv, (float*)out, d,
                         scale);
      break;
    case DT_F16:
      hipLaunchKernelGGL(attn_rows_kernel<f16>, grid, dim3(256), 0, s, (const f16*)q, rows, n, kv, (f16*)out, d, scale);
      break;
    case DT_BF16:
      hipLaunchKernelGGL(attn_rows_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)q, rows, n, kv, (bf16*)out, d,
                         scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
