// Small kernels of the hot path (embedding gather, RMSNorm, per-iteration
// compaction of active rows, greedy-token reduction, row moves) and the
// load-time kernels (INT4 quantisation into the kernel layout, FP16-body
// dequantisation, canonical export, row permutation).
#include "device_common.h"
#include "launch.h"

namespace {

// ---------------------------------------------------------------- embedding
template <class T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ E, const int32_t* __restrict__ tokens,
                                                   int d, float* __restrict__ h, int32_t* err, int vocab) {
  const int r = blockIdx.x;
  int tok = tokens[r];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0 && err) atomicOr(err, 1);
    tok = 0;
  }
  const T* src = E + (int64_t)tok * d;
  float* dst = h + (int64_t)r * d;
  for (int i = threadIdx.x; i < d; i += 256) dst[i] = (float)src[i];
}

// ---------------------------------------------------------------- RMSNorm
// x = h / sqrt(mean(h^2) + eps) * g with fp32 statistics: one workgroup per row,
// the shared arithmetic of sumsq4 / row_sum256 / rms_inv.  With VPT > 0 (d <=
// 1024 VPT) a thread keeps its VPT groups of 4 values and gains in registers: the
// row and the gain are requested in one round, and each group leaves in one 8- or
// 16-byte store.  VPT = 0 serves any d (multiple of 4), reading the row twice.
template <class T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    const T t[4] = {from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
    uint2 u;
    __builtin_memcpy(&u, t, sizeof(u));
    *reinterpret_cast<uint2*>(p) = u;
  }
}

template <class T, int VPT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, const float* __restrict__ g,
                                                     const int32_t* __restrict__ gather, int n, int d, float eps,
                                                     T* __restrict__ out) {
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  T* o = out + (int64_t)r * d;
  const int src = gather ? gather[r] : r;
  const float* hr = h + (int64_t)src * d;
  if constexpr (VPT > 0) {
    float4 gg[VPT], v[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = min(4 * (tid + 256 * u), d - 4);
      gg[u] = *reinterpret_cast<const float4*>(g + i);
      v[u] = *reinterpret_cast<const float4*>(hr + i);
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < VPT; ++u)
      if (4 * (tid + 256 * u) < d) ss = sumsq4(v[u].x, v[u].y, v[u].z, v[u].w, ss);
    const float inv = rms_inv(row_sum256(ss), d, eps);
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = 4 * (tid + 256 * u);
      if (i < d)
        store4(o + i, v[u].x * inv * gg[u].x, v[u].y * inv * gg[u].y, v[u].z * inv * gg[u].z, v[u].w * inv * gg[u].w);
    }
  } else {
    float ss = 0.f;
    for (int i = 4 * tid; i < d; i += 1024) {
      const float4 v = *reinterpret_cast<const float4*>(hr + i);
      ss = sumsq4(v.x, v.y, v.z, v.w, ss);
    }
    const float inv = rms_inv(row_sum256(ss), d, eps);
    for (int i = 4 * tid; i < d; i += 1024) {
      const float4 v = *reinterpret_cast<const float4*>(hr + i);
      const float4 gg = *reinterpret_cast<const float4*>(g + i);
      store4(o + i, v.x * inv * gg.x, v.y * inv * gg.y, v.z * inv * gg.z, v.w * inv * gg.w);
    }
  }
}

// Embedding gather fused with the first block's RMSNorm: one workgroup per row
// keeps its 4 VPT-wide groups (d <= 1024 VPT) in registers, writes h and then
// x = h / sqrt(mean(h^2) + eps) * g (fp32 statistics, a fixed-order workgroup sum)
// in the operand type, saving the norm kernel's launch and its read of h.
template <class T>
__device__ __forceinline__ float4 load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    T t[4];
    __builtin_memcpy(t, &u, sizeof(u));
    return make_float4((float)t[0], (float)t[1], (float)t[2], (float)t[3]);
  }
}

template <class T, class X, int VPT>
__global__ __launch_bounds__(256) void embed_norm_kernel(const T* __restrict__ E, const int32_t* __restrict__ tokens,
                                                        int d, float* __restrict__ h, int32_t* err, int vocab,
                                                        const float* __restrict__ g, float eps, X* __restrict__ x) {
  const int r = blockIdx.x, tid = threadIdx.x;
  float4 gg[VPT], v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) gg[u] = *reinterpret_cast<const float4*>(g + min(4 * (tid + 256 * u), d - 4));
  int tok = tokens[r];
  if (tok < 0 || tok >= vocab) {
    if (tid == 0 && err) atomicOr(err, 1);
    tok = 0;
  }
  const T* src = E + (int64_t)tok * d;
  float* dst = h + (int64_t)r * d;
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int i = 4 * (tid + 256 * u);
    v[u] = load4(src + min(i, d - 4));
    if (i < d) {
      *reinterpret_cast<float4*>(dst + i) = v[u];
      ss = sumsq4(v[u].x, v[u].y, v[u].z, v[u].w, ss);
    }
  }
  const float inv = rms_inv(row_sum256(ss), d, eps);
  X* xo = x + (int64_t)r * d;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int i = 4 * (tid + 256 * u);
    if (i < d)
      store4(xo + i, v[u].x * inv * gg[u].x, v[u].y * inv * gg[u].y, v[u].z * inv * gg[u].z, v[u].w * inv * gg[u].w);
  }
}

// ---------------------------------------------------------------- compaction
// Stable filter in one workgroup: chunks of 1024 rows, wave ballots + prefix.
__global__ __launch_bounds__(1024) void compact_kernel(const RowInfo* __restrict__ in, int n, int it,
                                                      RowInfo* __restrict__ out, int32_t* __restrict__ dest,
                                                      int32_t* count_out, int32_t* log_out, int32_t* running_out) {
  __shared__ int wave_cnt[16], wave_run[16];
  __shared__ int base_s, run_s;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    base_s = 0;
    run_s = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < n; c0 += 1024) {
    const int i = c0 + threadIdx.x;
    bool keep = false;
    RowInfo ri;
    if (i < n) {
      ri = in[i];
      if (it > 0) ri.iter = it;
      keep = ri.depth > ri.iter;
    }
    const uint64_t mask = __ballot(keep);
    const uint64_t run_mask = __ballot(keep && !ri.done);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) {
      wave_cnt[w] = __popcll(mask);
      wave_run[w] = __popcll(run_mask);
    }
    __syncthreads();
    int off = base_s;
    for (int k = 0; k < w; ++k) off += wave_cnt[k];
    if (i < n) {
      if (keep) {
        const int ni = off + before;
        ri.iter += 1;
        out[ni] = ri;
        dest[i] = ni;
        if (log_out) log_out[ni] = ri.orig;
      } else {
        dest[i] = -1;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0, run = 0;
      for (int k = 0; k < 16; ++k) {
        tot += wave_cnt[k];
        run += wave_run[k];
      }
      base_s += tot;
      run_s += run;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0 && count_out) *count_out = base_s;
  if (threadIdx.x == 0 && running_out) *running_out = run_s;
}

__global__ __launch_bounds__(256) void move_rows_kernel(const float* __restrict__ h, const int32_t* __restrict__ dest,
                                                       const RowInfo* __restrict__ rows, int d,
                                                       float* __restrict__ h_next, float* __restrict__ h_exit) {
  const int i = blockIdx.x;
  const int di = dest[i];
  if (di < 0 && rows[i].done) return;   // exit state already stored by the early-exit probe
  float* dst = di >= 0 ? h_next + (int64_t)di * d : h_exit + (int64_t)rows[i].orig * d;
  const float* src = h + (int64_t)i * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024) *reinterpret_cast<float4*>(dst + c) = *reinterpret_cast<const float4*>(src + c);
}

// Compaction and row move in one kernel, for passes of at most kCompactMoveRows
// rows without early exit.  Workgroup i counts the rows before i that stay (every
// workgroup reads the row list), so row i's destination needs no separate
// compaction kernel.  A kept row goes to rows_out / h_next at that index (and its
// operand-type normalised row of x to x_next, when x is set); a leaving row goes
// to h_exit at its caller index.  The last workgroup writes the kept count.
__global__ __launch_bounds__(256) void compact_move_kernel(const RowInfo* __restrict__ in, int n, int it,
                                                          RowInfo* __restrict__ out, int32_t* count_out,
                                                          int32_t* log_out, const float* __restrict__ h, int d,
                                                          float* __restrict__ h_next, float* __restrict__ h_exit,
                                                          const uint8_t* __restrict__ x, uint8_t* __restrict__ x_next,
                                                          int xrow_bytes) {
  __shared__ int wcnt[4];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  RowInfo ri = in[i];
  int c = 0;
  for (int k = tid; k < i; k += 256) {
    const RowInfo rk = in[k];
    c += rk.depth > (it > 0 ? it : rk.iter) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
  if (lane == 0) wcnt[w] = c;
  __syncthreads();
  const int before = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  if (it > 0) ri.iter = it;
  const bool keep = ri.depth > ri.iter;
  if (tid == 0) {
    if (keep) {
      RowInfo ro = ri;
      ro.iter += 1;
      out[before] = ro;
      if (log_out) log_out[before] = ri.orig;
    }
    if (i == n - 1 && count_out) *count_out = before + (keep ? 1 : 0);
  }
  float* dst = keep ? h_next + (int64_t)before * d : h_exit + (int64_t)ri.orig * d;
  const float* src = h + (int64_t)i * d;
  for (int c4 = tid * 4; c4 < d; c4 += 1024) *reinterpret_cast<float4*>(dst + c4) = *reinterpret_cast<const float4*>(src + c4);
  if (keep && x) {
    const uint8_t* xs = x + (int64_t)i * xrow_bytes;
    uint8_t* xd = x_next + (int64_t)before * xrow_bytes;
    for (int b = tid * 16; b < xrow_bytes; b += 4096) *reinterpret_cast<uint4*>(xd + b) = *reinterpret_cast<const uint4*>(xs + b);
  }
}

__global__ void write_orig_kernel(const RowInfo* rows, int n, int32_t* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = rows[i].orig;
}

// ---------------------------------------------------------------- early exit
// One workgroup per row: relative L2 change (or a precomputed logit margin)
// decides a stable probe; patience consecutive stable probes finish the row, whose
// state is copied out as its exit state.  With save set (hidden rule), the row's h
// then replaces its h_prev row, ready for a probe at the next iteration.
__global__ __launch_bounds__(256) void ee_probe_kernel(RowInfo* __restrict__ rows, int it,
                                                      const float* __restrict__ h, float* h_prev,
                                                      const float* __restrict__ margin, float tau, float margin_thr,
                                                      int patience, int d, float* __restrict__ h_exit,
                                                      int32_t* __restrict__ eff_depth, int32_t* live, int save) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const RowInfo ri = rows[r];
  if (ri.done) return;   // uniform over the workgroup
  const float* hr = h + (int64_t)r * d;
  const bool vec = (d & 3) == 0;
  bool stable;
  if (margin) {
    stable = margin[r] > margin_thr;
  } else {
    const float* pr = h_prev + (int64_t)r * d;
    float dd = 0.f, hh = 0.f;
    if (vec) {
      for (int c = tid; c < (d >> 2); c += 256) {
        const floatx4 a = reinterpret_cast<const floatx4*>(hr)[c];
        const floatx4 b = a - reinterpret_cast<const floatx4*>(pr)[c];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dd = fmaf(b[q], b[q], dd);
          hh = fmaf(a[q], a[q], hh);
        }
      }
    } else {
      for (int c = tid; c < d; c += 256) {
        const float a = hr[c], b = a - pr[c];
        dd = fmaf(b, b, dd);
        hh = fmaf(a, a, hh);
      }
    }
    __shared__ float red[2][4];
    dd = wave_sum(dd);
    hh = wave_sum(hh);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = dd;
      red[1][tid >> 6] = hh;
    }
    __syncthreads();   // every read of the h_prev row is done
    dd = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    hh = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    stable = sqrtf(dd) < tau * sqrtf(hh);
    if (save) {
      float* sv = h_prev + (int64_t)r * d;
      if (vec) {
        for (int c = tid; c < (d >> 2); c += 256)
          reinterpret_cast<floatx4*>(sv)[c] = reinterpret_cast<const floatx4*>(hr)[c];
      } else {
        for (int c = tid; c < d; c += 256) sv[c] = hr[c];
      }
    }
  }
  const int streak = stable ? ri.streak + 1 : 0;
  const bool fin = streak >= patience;
  if (fin) {
    float* dst = h_exit + (int64_t)ri.orig * d;
    if (vec) {
      for (int c = tid; c < (d >> 2); c += 256)
        reinterpret_cast<floatx4*>(dst)[c] = reinterpret_cast<const floatx4*>(hr)[c];
    } else {
      for (int c = tid; c < d; c += 256) dst[c] = hr[c];
    }
  }
  if (tid == 0) {
    rows[r].streak = streak;
    if (fin) {
      rows[r].done = 1;
      eff_depth[ri.orig] = it;
      atomicSub(live, 1);
    }
  }
}

// ---------------------------------------------------------------- greedy token
// One workgroup per row merges the head GEMM's per-tile partials: the greedy
// token (largest logit, lowest index on ties) and, when the tiles also kept their
// runner-up, the top-1 minus top-2 logit margin.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                            const float* __restrict__ pv2, int tiles, int32_t* out,
                                                            int32_t* out2, const int32_t* scatter, float* margin) {
  const int r = blockIdx.x, tid = threadIdx.x;
  float bv = -INFINITY, b2 = -INFINITY;
  int bi = 0x7fffffff;
  const int64_t base = (int64_t)r * tiles;
  for (int t = tid; t < tiles; t += 256)
    best2_merge(bv, bi, b2, pv[base + t], pi[base + t], pv2 ? pv2[base + t] : -INFINITY);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64), ov2 = __shfl_xor(b2, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    best2_merge(bv, bi, b2, ov, oi, ov2);
  }
  __shared__ float sv[4], sv2[4];
  __shared__ int si[4];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    sv2[tid >> 6] = b2;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) best2_merge(bv, bi, b2, sv[w], si[w], sv2[w]);
    if (out) out[r] = bi;
    if (out2) out2[scatter ? scatter[r] : r] = bi;
    if (margin) margin[r] = bv - b2;
  }
}

// ---------------------------------------------------------------- store-h cache
// One 64-lane workgroup per (row, head); lane i owns elements 2i and 2i + 1 of the
// head (one packed byte in mode 3).
__device__ __forceinline__ uint8_t* hcache_row(const HCacheParams& hp, const RowInfo& ri, int slot) {
  const int64_t cap = hp.lane_cap[ri.lane];
  uint8_t* lane = hp.base + hp.lane_off[ri.lane] * hp.unit;
  if (hp.mode != 4) return lane + ((int64_t)slot * cap + ri.pos) * hp.rb;
  const int A = hp.n_bound + hp.n_loop;
  if (slot < A) return lane + ((int64_t)slot * cap + ri.pos) * hp.rbA;
  return lane + (int64_t)A * cap * hp.rbA + ((int64_t)(slot - A) * cap + ri.pos) * hp.rbD;
}

// Symmetric codes of one head's values (v0, v1 per lane): the wave's absmax
// gives s = fp16(max / levels), q = clamp(rint(v / s)).
__device__ __forceinline__ f16 hcache_codes(float v0, float v1, float levels, int& q0, int& q1) {
  const float am = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const f16 s16 = (f16)(am / levels);
  const float sc = (float)s16;
  q0 = q1 = 0;
  if (sc > 0.f) {
    q0 = (int)fminf(fmaxf(rintf(v0 / sc), -levels), levels);
    q1 = (int)fminf(fmaxf(rintf(v1 / sc), -levels), levels);
  }
  return s16;
}

// Delta mode: reconstruction of elements e, e + 1 of head h at iteration `upto`
// of loop layer l (anchor, then each decoded difference, in fp32, in order).
template <class AT>
__device__ __forceinline__ void hcache_delta_sum(const HCacheParams& hp, const RowInfo& ri, int l, int upto, int e,
                                                 int h, float& x0, float& x1) {
  const int d = hp.H * hp.dh;
  const AT* an = reinterpret_cast<const AT*>(hcache_row(hp, ri, hp.n_bound + l));
  x0 = (float)an[e];
  x1 = (float)an[e + 1];
  for (int i = 2; i <= upto; ++i) {
    const uint8_t* row = hcache_row(hp, ri, hp.n_bound + (i - 1) * hp.n_loop + l);
    const float sc = (float)*reinterpret_cast<const f16*>(row + d + 2 * h);
    x0 += (float)(int8_t)row[e] * sc;
    x1 += (float)(int8_t)row[e + 1] * sc;
  }
}

template <class AT>
__global__ __launch_bounds__(64) void hcache_write_kernel(const AT* __restrict__ x, const RowInfo* __restrict__ rows,
                                                          HCacheParams hp, int skip_done) {
  const int r = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const RowInfo ri = rows[r];
  if (skip_done && ri.done) return;
  const int d = hp.H * hp.dh, e = h * hp.dh + 2 * i;
  const bool own = 2 * i < hp.dh;
  uint8_t* row = hcache_row(hp, ri, hp.slot);
  AT a0{}, a1{};
  if (own) {
    a0 = x[(int64_t)r * d + e];
    a1 = x[(int64_t)r * d + e + 1];
  }
  const bool plain = hp.mode == 1 || (hp.mode == 4 && hp.slot < hp.n_bound + hp.n_loop);
  if (plain) {
    if (own) {
      reinterpret_cast<AT*>(row)[e] = a0;
      reinterpret_cast<AT*>(row)[e + 1] = a1;
    }
    return;
  }
  float v0 = (float)a0, v1 = (float)a1;
  if (hp.mode == 4) {   // code the difference to the previous iteration's reconstruction
    const int t = hp.slot - hp.n_bound, l = t % hp.n_loop, j = t / hp.n_loop + 1;
    float p0 = 0.f, p1 = 0.f;
    if (own) hcache_delta_sum<AT>(hp, ri, l, j - 1, e, h, p0, p1);
    v0 -= p0;
    v1 -= p1;
  }
  int q0, q1;
  const f16 s16 = hcache_codes(v0, v1, hp.mode == 3 ? 7.f : 127.f, q0, q1);
  const int cb = hp.mode == 3 ? d / 2 : d;
  if (own) {
    if (hp.mode == 3) {
      row[e / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    } else {
      row[e] = (uint8_t)(int8_t)q0;
      row[e + 1] = (uint8_t)(int8_t)q1;
    }
  }
  if (i == 0) *reinterpret_cast<f16*>(row + cb + 2 * h) = s16;
}

template <class AT>
__global__ __launch_bounds__(64) void hcache_read_kernel(HCacheParams hp, const RowInfo* __restrict__ rows,
                                                         AT* __restrict__ out) {
  const int r = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  if (2 * i >= hp.dh) return;
  const RowInfo ri = rows[r];
  const int d = hp.H * hp.dh, e = h * hp.dh + 2 * i;
  const uint8_t* row = hcache_row(hp, ri, hp.slot);
  AT* o = out + (int64_t)r * d + e;
  if (hp.mode == 1 || (hp.mode == 4 && hp.slot < hp.n_bound + hp.n_loop)) {
    o[0] = reinterpret_cast<const AT*>(row)[e];
    o[1] = reinterpret_cast<const AT*>(row)[e + 1];
    return;
  }
  if (hp.mode == 4) {
    const int t = hp.slot - hp.n_bound;
    float x0, x1;
    hcache_delta_sum<AT>(hp, ri, t % hp.n_loop, t / hp.n_loop + 1, e, h, x0, x1);
    o[0] = from_f32<AT>(x0);
    o[1] = from_f32<AT>(x1);
    return;
  }
  int q0, q1, cb;
  if (hp.mode == 2) {
    q0 = (int8_t)row[e];
    q1 = (int8_t)row[e + 1];
    cb = d;
  } else {
    const int b = row[e / 2];
    q0 = (b & 0x8) ? (b & 0xF) - 16 : (b & 0xF);
    q1 = (b & 0x80) ? (b >> 4) - 16 : (b >> 4);
    cb = d / 2;
  }
  const float sc = (float)*reinterpret_cast<const f16*>(row + cb + 2 * h);
  o[0] = from_f32<AT>((float)q0 * sc);
  o[1] = from_f32<AT>((float)q1 * sc);
}

// ---------------------------------------------------------------- self-speculative rounds
__global__ void spec_pack_kernel(const int32_t* __restrict__ pending, const int32_t* __restrict__ lanes,
                                 const int32_t* __restrict__ draft, int n, int k, int32_t* __restrict__ in) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * (k + 1)) return;
  const int i = idx / (k + 1), c = idx - i * (k + 1);
  in[idx] = c == 0 ? pending[lanes[i]] : draft[(c - 1) * n + i];
}

__global__ void spec_accept_kernel(const int32_t* __restrict__ draft, const int32_t* __restrict__ g,
                                   const int32_t* __restrict__ lanes, const int32_t* __restrict__ want,
                                   const int32_t* __restrict__ emitted, const int32_t* __restrict__ slot, int n,
                                   int k, int n_tokens, int32_t* __restrict__ out, int32_t* __restrict__ pending,
                                   int32_t* __restrict__ acc) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t* gi = g + (int64_t)i * (k + 1);
  int a = 0;
  while (a < k && draft[a * n + i] == gi[a]) ++a;
  a = min(a, want[i] - 1);
  int32_t* o = out + (int64_t)slot[i] * n_tokens + emitted[i];
  for (int c = 0; c <= a; ++c) o[c] = gi[c];
  pending[lanes[i]] = gi[a];
  acc[i] = a;
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ src, const int32_t* __restrict__ idx,
                                                         int d, float* __restrict__ dst) {
  const int r = blockIdx.x;
  const float* s = src + (int64_t)idx[r] * d;
  float* o = dst + (int64_t)r * d;
  for (int c = threadIdx.x; c < d; c += 256) o[c] = s[c];
}

__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* __restrict__ src, const int32_t* __restrict__ idx,
                                                          int d, float* __restrict__ dst) {
  const int r = blockIdx.x;
  const float* s = src + (int64_t)r * d;
  float* o = dst + (int64_t)idx[r] * d;
  for (int c = threadIdx.x; c < d; c += 256) o[c] = s[c];
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void gather_i32_kernel(const int32_t* src, const int32_t* idx, int n, int32_t* dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[idx[i]];
}

__global__ void scatter_i32_kernel(const int32_t* src, const int32_t* idx, int n, int32_t* dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[idx[i]] = src[i];
}

// ---------------------------------------------------------------- load time
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint32_t* __restrict__ src, const int32_t* __restrict__ perm,
                                                          int words_per_row, uint32_t* __restrict__ dst) {
  const int n = blockIdx.x;
  const uint32_t* s = src + (int64_t)perm[n] * words_per_row;
  uint32_t* o = dst + (int64_t)n * words_per_row;
  for (int c = threadIdx.x; c < words_per_row; c += 256) o[c] = s[c];
}

__global__ __launch_bounds__(256) void permute_bf16_to_f16_kernel(const uint16_t* __restrict__ src,
                                                                 const int32_t* __restrict__ perm, int K,
                                                                 uint16_t* __restrict__ dst) {
  const int n = blockIdx.x;
  const uint16_t* sr = src + (int64_t)(perm ? perm[n] : n) * K;
  uint16_t* o = dst + (int64_t)n * K;
  for (int c = threadIdx.x; c < K; c += 256) {
    const float v = (float)__builtin_bit_cast(bf16, sr[c]);
    o[c] = __builtin_bit_cast(uint16_t, (f16)v);
  }
}

// One wave per (kernel row n, group): s = fp16(max|w| / 7), q = clamp(rint(w / s), -7, 7).
__global__ __launch_bounds__(256) void quant_w4_kernel(const float* __restrict__ w, const int32_t* __restrict__ perm,
                                                      int N, int K, uint32_t* __restrict__ words,
                                                      uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int groups = K >> 7;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)N * groups) return;
  const int n = (int)(item / groups), gi = (int)(item - (int64_t)n * groups);
  const int src = perm ? perm[n] : n;
  const float2 ab = *reinterpret_cast<const float2*>(w + (int64_t)src * K + gi * 128 + 2 * lane);
  const float amax = wave_max(fmaxf(fabsf(ab.x), fabsf(ab.y)));
  const f16 s16 = (f16)__fdiv_rn(amax, 7.0f);
  const float s32 = (float)s16;
  int qa = 0, qb = 0;
  if (s32 > 0.f) {
    qa = (int)fminf(fmaxf(rintf(__fdiv_rn(ab.x, s32)), -7.f), 7.f);
    qb = (int)fminf(fmaxf(rintf(__fdiv_rn(ab.y, s32)), -7.f), 7.f);
  }
  const int sh = 4 * (lane & 3);
  int part = (int)(((uint32_t)(qa + 8) << sh) | ((uint32_t)(qb + 8) << (16 + sh)));
  part |= __shfl_xor(part, 1, 64);
  part |= __shfl_xor(part, 2, 64);
  if ((lane & 3) == 0)
    words[w4_word_offset(n, gi * 16 + (lane >> 2), groups)] = (uint32_t)part;
  if (lane == 0) scales[(int64_t)gi * N + n] = __builtin_bit_cast(uint16_t, s16);
}

__device__ __forceinline__ f16 w4_value(const uint32_t* words, int groups, int n, int k) {
  const uint32_t wd = words[w4_word_offset(n, k >> 3, groups)];
  const int e = k & 7;
  const half2v p = w4_pair(wd, e >> 1);
  return p[e & 1];
}

// FP16 body: fp16(q * s), product in fp32 (exact), one rounding.
__global__ __launch_bounds__(256) void w4_to_f16_kernel(const uint32_t* __restrict__ words, const uint16_t* __restrict__ scales,
                                                       int N, int K, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)N * K) return;
  const int n = (int)(i / K), k = (int)(i - (int64_t)n * K);
  const int groups = K >> 7;
  const float q = (float)w4_value(words, groups, n, k);
  const float s = (float)__builtin_bit_cast(f16, scales[(int64_t)(k >> 7) * N + n]);
  out[i] = __builtin_bit_cast(uint16_t, (f16)(q * s));
}

__global__ __launch_bounds__(256) void w4_export_kernel(const uint32_t* __restrict__ words, const uint16_t* __restrict__ scales,
                                                       const int32_t* __restrict__ perm, int N, int K,
                                                       int8_t* __restrict__ q, uint16_t* __restrict__ s_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)N * K) return;
  const int n = (int)(i / K), k = (int)(i - (int64_t)n * K);
  const int groups = K >> 7;
  const int dst = perm ? perm[n] : n;
  q[(int64_t)dst * K + k] = (int8_t)(int)(float)w4_value(words, groups, n, k);
  if ((k & 127) == 0) s_out[(int64_t)dst * groups + (k >> 7)] = scales[(int64_t)(k >> 7) * N + n];
}

}  // namespace

template <class T>
hipError_t embed_norm_x(const T* E, const int32_t* tokens, int n, int d, float* h, int32_t* err, int vocab,
                        const float* g, float eps, int x_dtype, void* x, hipStream_t s) {
  const int vpt = (d + 1023) / 1024;
#define TL_EN(X, V)                                                                                        \
  TL_LAUNCH((embed_norm_kernel<T, X, V>), dim3(n), dim3(256), 0, s, E, tokens, d, h, err, vocab, g, eps, \
                     (X*)x)
#define TL_EN_X(X)                 \
  switch (vpt) {                   \
    case 1: TL_EN(X, 1); break;    \
    case 2: TL_EN(X, 2); break;    \
    case 3:                        \
    case 4: TL_EN(X, 4); break;    \
    default: TL_EN(X, 8); break;   \
  }
  switch (x_dtype) {
    case DT_F32: TL_EN_X(float) break;
    case DT_F16: TL_EN_X(f16) break;
    case DT_BF16: TL_EN_X(bf16) break;
    default: return hipErrorInvalidValue;
  }
#undef TL_EN_X
#undef TL_EN
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const void* E, const int32_t* tokens, int n, int d, float* h, int32_t* err,
                        int vocab, hipStream_t s, const float* norm_g, float eps, int x_dtype, void* x, bool* x_done) {
  if (x_done) *x_done = false;
  if (n <= 0) return hipSuccess;
  if (norm_g && x && x_done && d >= 4 && (d % 4) == 0 && d <= 8192) {
    hipError_t err2 = hipErrorInvalidValue;
    switch (dtype) {
      case DT_F32: err2 = embed_norm_x<float>((const float*)E, tokens, n, d, h, err, vocab, norm_g, eps, x_dtype, x, s); break;
      case DT_F16: err2 = embed_norm_x<f16>((const f16*)E, tokens, n, d, h, err, vocab, norm_g, eps, x_dtype, x, s); break;
      case DT_BF16: err2 = embed_norm_x<bf16>((const bf16*)E, tokens, n, d, h, err, vocab, norm_g, eps, x_dtype, x, s); break;
      default: break;
    }
    if (err2 == hipSuccess) *x_done = true;
    return err2;
  }
  switch (dtype) {
    case DT_F32: TL_LAUNCH(embed_kernel<float>, dim3(n), dim3(256), 0, s, (const float*)E, tokens, d, h, err, vocab); break;
    case DT_F16: TL_LAUNCH(embed_kernel<f16>, dim3(n), dim3(256), 0, s, (const f16*)E, tokens, d, h, err, vocab); break;
    case DT_BF16: TL_LAUNCH(embed_kernel<bf16>, dim3(n), dim3(256), 0, s, (const bf16*)E, tokens, d, h, err, vocab); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int out_dtype, const float* h, const float* g, const int32_t* gather, int n, int d, float eps,
                          void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d < 4 || (d % 4) != 0) return hipErrorInvalidValue;
  dim3 grid(n);
  const int vpt = d <= 1024 ? 1 : d <= 2048 ? 2 : d <= 4096 ? 4 : d <= 8192 ? 8 : 0;
#define TL_RMS(T, V)                                                                                          \
  TL_LAUNCH((rmsnorm_kernel<T, V>), grid, dim3(256), 0, s, h, g, gather, n, d, eps, (T*)out)
#define TL_RMS_T(T)                      \
  switch (vpt) {                         \
    case 1: TL_RMS(T, 1); break;         \
    case 2: TL_RMS(T, 2); break;         \
    case 4: TL_RMS(T, 4); break;         \
    case 8: TL_RMS(T, 8); break;         \
    default: TL_RMS(T, 0); break;        \
  }
  switch (out_dtype) {
    case DT_F32: TL_RMS_T(float) break;
    case DT_F16: TL_RMS_T(f16) break;
    case DT_BF16: TL_RMS_T(bf16) break;
    default: return hipErrorInvalidValue;
  }
#undef TL_RMS_T
#undef TL_RMS
  return hipGetLastError();
}

hipError_t launch_compact(const RowInfo* rows_in, int n, int it, RowInfo* rows_out, int32_t* dest, int32_t* count_out,
                          int32_t* log_out, int32_t* running_out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(compact_kernel, dim3(1), dim3(1024), 0, s, rows_in, n, it, rows_out, dest, count_out, log_out, running_out);
  return hipGetLastError();
}

hipError_t launch_compact_move(const RowInfo* rows_in, int n, int it, RowInfo* rows_out, int32_t* count_out,
                               int32_t* log_out, const float* h, int d, float* h_next, float* h_exit, const void* x,
                               void* x_next, int xrow_bytes, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > kCompactMoveRows || (d % 4) || (x && (xrow_bytes % 16))) return hipErrorInvalidValue;
  TL_LAUNCH(compact_move_kernel, dim3(n), dim3(256), 0, s, rows_in, n, it, rows_out, count_out, log_out, h, d,
                     h_next, h_exit, static_cast<const uint8_t*>(x), static_cast<uint8_t*>(x_next), xrow_bytes);
  return hipGetLastError();
}

hipError_t launch_move_rows(const float* h, const int32_t* dest, const RowInfo* rows, int n, int d, float* h_next,
                            float* h_exit, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(move_rows_kernel, dim3(n), dim3(256), 0, s, h, dest, rows, d, h_next, h_exit);
  return hipGetLastError();
}

hipError_t launch_write_orig(const RowInfo* rows, int n, int32_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(write_orig_kernel, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, out);
  return hipGetLastError();
}

hipError_t launch_ee_probe(RowInfo* rows, int n, int it, const float* h, float* h_prev, bool save_prev, const float* margin,
                           float tau, float margin_thr, int patience, int d, float* h_exit, int32_t* eff_depth,
                           int32_t* live, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(ee_probe_kernel, dim3(n), dim3(256), 0, s, rows, it, h, h_prev, margin, tau,
                     margin_thr, patience, d, h_exit, eff_depth, live, (save_prev && !margin) ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const float* pv, const int32_t* pi, const float* pv2, int n, int tiles, int32_t* out,
                                int32_t* out2, const int32_t* scatter, float* margin, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(argmax_reduce_kernel, dim3(n), dim3(256), 0, s, pv, pi, pv2, tiles, out, out2, scatter, margin);
  return hipGetLastError();
}

hipError_t launch_hcache_write(int dtype, const void* x, const RowInfo* rows, int n, const HCacheParams& hp,
                               bool skip_done, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(n, hp.H);
  switch (dtype) {
    case DT_F32:
      TL_LAUNCH(hcache_write_kernel<float>, grid, dim3(64), 0, s, (const float*)x, rows, hp, (int)skip_done);
      break;
    case DT_F16:
      TL_LAUNCH(hcache_write_kernel<f16>, grid, dim3(64), 0, s, (const f16*)x, rows, hp, (int)skip_done);
      break;
    case DT_BF16:
      TL_LAUNCH(hcache_write_kernel<bf16>, grid, dim3(64), 0, s, (const bf16*)x, rows, hp, (int)skip_done);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_hcache_read(int dtype, const HCacheParams& hp, const RowInfo* rows, int n, void* out,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(n, hp.H);
  switch (dtype) {
    case DT_F32: TL_LAUNCH(hcache_read_kernel<float>, grid, dim3(64), 0, s, hp, rows, (float*)out); break;
    case DT_F16: TL_LAUNCH(hcache_read_kernel<f16>, grid, dim3(64), 0, s, hp, rows, (f16*)out); break;
    case DT_BF16: TL_LAUNCH(hcache_read_kernel<bf16>, grid, dim3(64), 0, s, hp, rows, (bf16*)out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_spec_pack(const int32_t* pending, const int32_t* lanes, const int32_t* draft, int n, int k,
                            int32_t* in, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(spec_pack_kernel, dim3((n * (k + 1) + 255) / 256), dim3(256), 0, s, pending, lanes, draft, n, k, in);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const int32_t* draft, const int32_t* g, const int32_t* lanes, const int32_t* want,
                              const int32_t* emitted, const int32_t* slot, int n, int k, int n_tokens,
                              int32_t* out, int32_t* pending, int32_t* acc, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(spec_accept_kernel, dim3((n + 255) / 256), dim3(256), 0, s, draft, g, lanes, want, emitted, slot, n,
                     k, n_tokens, out, pending, acc);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float* src, const int32_t* idx, int n, int d, float* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(gather_rows_kernel, dim3(n), dim3(256), 0, s, src, idx, d, dst);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* src, const int32_t* idx, int n, int d, float* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(scatter_rows_kernel, dim3(n), dim3(256), 0, s, src, idx, d, dst);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_gather_i32(const int32_t* src, const int32_t* idx, int n, int32_t* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(gather_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, idx, n, dst);
  return hipGetLastError();
}

hipError_t launch_scatter_i32(const int32_t* src, const int32_t* idx, int n, int32_t* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TL_LAUNCH(scatter_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, idx, n, dst);
  return hipGetLastError();
}

hipError_t launch_permute_rows(int elem_bytes, const void* src, const int32_t* perm, int N, int K, void* dst,
                               hipStream_t s) {
  if ((int64_t)K * elem_bytes % 4 != 0) return hipErrorInvalidValue;
  const int wpr = (int)((int64_t)K * elem_bytes / 4);
  TL_LAUNCH(permute_rows_kernel, dim3(N), dim3(256), 0, s, (const uint32_t*)src, perm, wpr, (uint32_t*)dst);
  return hipGetLastError();
}

hipError_t launch_permute_bf16_to_f16(const uint16_t* src, const int32_t* perm, int N, int K, uint16_t* dst,
                                      hipStream_t s) {
  TL_LAUNCH(permute_bf16_to_f16_kernel, dim3(N), dim3(256), 0, s, src, perm, K, dst);
  return hipGetLastError();
}

hipError_t launch_quant_w4(const float* w, const int32_t* perm, int N, int K, uint32_t* words, uint16_t* scales,
                           hipStream_t s) {
  const int64_t items = (int64_t)N * (K / 128);
  TL_LAUNCH(quant_w4_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, w, perm, N, K, words, scales);
  return hipGetLastError();
}

hipError_t launch_w4_to_f16(const uint32_t* words, const uint16_t* scales, int N, int K, uint16_t* out, hipStream_t s) {
  const int64_t tot = (int64_t)N * K;
  TL_LAUNCH(w4_to_f16_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, words, scales, N, K, out);
  return hipGetLastError();
}

hipError_t launch_w4_export(const uint32_t* words, const uint16_t* scales, const int32_t* perm, int N, int K, int8_t* q,
                            uint16_t* s_out, hipStream_t s) {
  const int64_t tot = (int64_t)N * K;
  TL_LAUNCH(w4_export_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, words, scales, perm, N, K,
                     q, s_out);
  return hipGetLastError();
}
