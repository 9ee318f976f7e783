// GEMM epilogues shared by the GEMM kernels: applied to one output value (or one
// rotary / gate-up pair of values G columns apart) of row r, column c.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace {

// The rotary pair (x1, x2) = (v0 cos - v1 sin, v1 cos + v0 sin) with its fused
// multiply-adds written out, so that every kernel that rotates a pair rounds it
// the same way.
__device__ __forceinline__ float rot_x1(float v0, float v1, float cs, float sn) { return fmaf(v0, cs, -(v1 * sn)); }
__device__ __forceinline__ float rot_x2(float v0, float v1, float cs, float sn) { return fmaf(v1, cs, v0 * sn); }

template <class AT, int KIND>
__device__ __forceinline__ void epi_pair(const GemmEpi& e, int r, int c, float v0, float v1) {
  if constexpr (KIND == EPI_QKV) {
    const int d = e.d, dh = e.dh, G = e.pair_g;
    const int sect = c / d;
    const int cc = c - sect * d;
    const int head = cc / dh;
    const int cd = cc - head * dh;
    const RowInfo ri = e.rows[r];
    if (e.skip_done && ri.done) return;   // finished by early exit: its later cache slots stay unwritten
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
    const float x1 = rot_x1(v0, v1, cs, sn);
    const float x2 = rot_x2(v0, v1, cs, sn);
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

// epi_pair's QKV epilogue split by when its operands can be read, for kernels that
// know their output rows and columns before the product: qkv_row reads a row's
// cache coordinates, qkv_prep (once those are in) the lane's slot-table entries
// and the rotary factors of one (row, column pair) and resolves the destination,
// qkv_put forms and stores the pair as epi_pair does.  Issued ahead of the main
// loop, the dependent loads overlap the product instead of following it.
struct QkvRow {
  int32_t lane, pos, iter, skip;
};
__device__ __forceinline__ QkvRow qkv_row(const GemmEpi& e, int r) {
  const RowInfo* ri = e.rows + r;
  return QkvRow{ri->lane, ri->pos, ri->iter, e.skip_done && ri->done};
}
struct QkvPrep {
  int64_t off;   // element offset of the pair's first value in q_out (sect 0) or the cache
  int32_t sect;  // 0 q, 1 k, 2 v; -1: nothing to store
  float cs, sn;
};
__device__ __forceinline__ QkvPrep qkv_prep(const GemmEpi& e, const QkvRow& q, int r, int c) {
  const int d = e.d, dh = e.dh, G = e.pair_g;
  const int sect = c / d;
  const int cc = c - sect * d;
  const int head = cc / dh;
  const int cd = cc - head * dh;
  QkvPrep p{0, q.skip ? -1 : sect, 0.f, 0.f};
  const int64_t cap = e.kv.lane_cap[q.lane];
  const int slot = e.kv.s0 + e.kv.s1 * q.iter;
  const int64_t kv0 = e.kv.lane_off[q.lane] + (int64_t)q.pos * dh;   // + ((slot * 2 + which) * H + head) * cap * dh
  if (sect == 2) {
    p.off = kv0 + ((int64_t)(slot * 2 + 1) * e.kv.H + head) * cap * dh + cd;
    return p;
  }
  const int half = dh >> 1;
  const int ci = cd / G;
  const int n0 = (ci >> 1) * G + (cd - ci * G);
  p.cs = e.rope_cos[(int64_t)q.pos * half + n0];
  p.sn = e.rope_sin[(int64_t)q.pos * half + n0];
  p.off = (sect == 0 ? (int64_t)r * d + head * dh : kv0 + ((int64_t)(slot * 2) * e.kv.H + head) * cap * dh) + n0;
  return p;
}
template <class AT>
__device__ __forceinline__ void qkv_put(const GemmEpi& e, const QkvPrep& p, float v0, float v1) {
  if (p.sect < 0) return;
  if (p.sect == 2) {
    AT* vp = reinterpret_cast<AT*>(e.kv.base) + p.off;
    vp[0] = from_f32<AT>(v0);
    vp[e.pair_g] = from_f32<AT>(v1);
    return;
  }
  const float x1 = rot_x1(v0, v1, p.cs, p.sn);
  const float x2 = rot_x2(v0, v1, p.cs, p.sn);
  AT* dst = (p.sect == 0 ? reinterpret_cast<AT*>(e.q_out) : reinterpret_cast<AT*>(e.kv.base)) + p.off;
  dst[0] = from_f32<AT>(x1);
  dst[e.dh >> 1] = from_f32<AT>(x2);
}

}  // namespace
