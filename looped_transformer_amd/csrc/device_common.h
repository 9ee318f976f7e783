// Device-side types and helpers shared by the gfx950 kernels of the runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef __bf16 bf16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// native 16-byte vector (HIP's uint4 is a struct whose copies can block register promotion)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#include "kernels.h"

template <class T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
// fp32 -> T with round-to-nearest-even of the fp32 value.  For 16-bit T the value
// is first pinned in a register: otherwise the compiler may fold the conversion
// into the multiply-add that produced x (a mixed-precision FMA that rounds the
// exact result once, straight to 16 bits), and whether it does depends on the
// surrounding code, so one value could round differently in two kernels.
template <class T> __device__ __forceinline__ T from_f32(float x) {
  if constexpr (sizeof(T) == 2) asm volatile("" : "+v"(x));
  return (T)x;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits
// for every outstanding global load of the thread, which would drain the
// register prefetch of the next K stage at each stage boundary.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave64 reductions (xor butterflies keep every lane holding the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// RMSNorm statistics shared by every kernel that normalises a row (the norm
// kernel, the embedding gather, the split-K residual reduction), so that a row
// gets the same bits whichever of them normalises it: a workgroup of 256 threads
// per row, thread t holding the groups of four columns 4 (t + 256 u), its sum of
// squares accumulated group after group (last element of a group first), then the
// wave sums, then waves 0..3 in order.
__device__ __forceinline__ float sumsq4(float x, float y, float z, float w, float ss) {
  return fmaf(x, x, fmaf(y, y, fmaf(z, z, fmaf(w, w, ss))));
}
__device__ __forceinline__ float row_sum256(float ss) {
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float rms_inv(float sumsq, int d, float eps) {
  return 1.0f / sqrtf(sumsq / (float)d + eps);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Address of K (which = 0) or V (which = 1) for (row's lane, slot, head, row's pos).
// Cache layout of one lane: [slot][K|V][head][position < cap][head_dim].
template <class T>
__device__ __forceinline__ T* kv_ptr(const KVParams& kv, const RowInfo& ri, int which, int head, int pos) {
  const int slot = kv.s0 + kv.s1 * ri.iter;
  const int64_t cap = kv.lane_cap[ri.lane];
  const int64_t off = kv.lane_off[ri.lane] +
                      ((int64_t)(slot * 2 + which) * kv.H + head) * cap * kv.dh + (int64_t)pos * kv.dh;
  return reinterpret_cast<T*>(kv.base) + off;
}

// INT4 kernel layout: a 32-bit word holds 8 consecutive k of one output row as
// offset-binary nibbles (q + 8); element 2i sits in bits [4i, 4i+4), element 2i+1
// in bits [16+4i, 16+4i+4).  ((w >> 4i) & 0x000F000F) | 0x64006400 is then the
// fp16 pair (1024 + q_2i + 8, 1024 + q_2i+1 + 8); subtracting 1032 gives q exactly.
//
// Words are ordered as 32x32x16 MFMA B fragments: one 2 KB block per (32 output
// rows, 128-wide group), made of two 1 KB halves; half hb holds, for each lane
// L = (n mod 32) + 32 h, four words t = 0..3 covering k steps j = 4 hb + t, i.e.
// k = 16 j + 8 h + (0..7) of the group.  A wave thus reads a fragment set for four
// k steps as one contiguous 1 KB load.  Needs N a multiple of 32.
__host__ __device__ __forceinline__ int64_t w4_word_offset(int n, int k8, int groups) {
  const int gi = k8 >> 4, kk = k8 & 15, j = kk >> 1, h = kk & 1;
  const int lane = (n & 31) + 32 * h;
  return ((((int64_t)(n >> 5) * groups + gi) * 2 + (j >> 2)) * 64 + lane) * 4 + (j & 3);
}
__device__ __forceinline__ half2v w4_pair(uint32_t w, int i) {
  uint32_t b = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
  half2v h = __builtin_bit_cast(half2v, b);
  const half2v off = {(f16)1032.0f, (f16)1032.0f};
  return h - off;
}

// All four pairs of a word, q[i] = w4_pair(w, i): the low and the high nibble of
// every byte are split once, then each pair's two nibble bytes are placed under
// 0x64 exponent bytes by one byte permute (v_perm_b32; selector bytes 0-3 pick
// from the second operand, 4-7 from the first).
__device__ __forceinline__ void w4_pairs(uint32_t w, half2v (&q)[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu, e = 0x64646464u;
  const half2v off = {(f16)1032.0f, (f16)1032.0f};
  q[0] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(e, lo, 0x04020400u)) - off;   // bits 0-3, 16-19
  q[1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(e, hi, 0x04020400u)) - off;   // bits 4-7, 20-23
  q[2] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(e, lo, 0x04030401u)) - off;   // bits 8-11, 24-27
  q[3] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(e, hi, 0x04030401u)) - off;   // bits 12-15, 28-31
}

// Early-exit gate: true when the pass has no live row left (every row finished).
// Kernels read it once their first loads are in flight, so its latency overlaps
// theirs instead of delaying every other argument load; the barrier keeps those
// loads from being sunk below the test.  A wave that returns here with loads in
// flight is fine: the end of the program waits for them.
__device__ __forceinline__ bool gate_closed(const int32_t* live) {
  asm volatile("" ::: "memory");
  return live && *live <= 0;
}

// Greedy-token reduction with the runner-up value: (v, i) is the largest value
// with the lowest index on ties, v2 the largest of the others (a repeated maximum
// gives v2 = v).  The result does not depend on the order of pushes and merges.
__device__ __forceinline__ void best2_push(float& v, int& i, float& v2, float nv, int ni) {
  if (nv > v || (nv == v && ni < i)) {
    v2 = v;
    v = nv;
    i = ni;
  } else {
    v2 = fmaxf(v2, nv);
  }
}
__device__ __forceinline__ void best2_merge(float& v, int& i, float& v2, float ov, int oi, float ov2) {
  if (ov > v || (ov == v && oi < i)) {
    v2 = fmaxf(ov2, v);
    v = ov;
    i = oi;
  } else {
    v2 = fmaxf(v2, ov);
  }
}
