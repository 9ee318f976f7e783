// GEMM epilogues shared by the GEMM kernels: applied to one output value (or one
// rotary / gate-up pair of values G columns apart) of row r, column c.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace {

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

}  // namespace
