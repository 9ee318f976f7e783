/*
 * Seeded synthetic inputs for the looped transformer: weights, token ids and
 * per-lane / per-token loop counts.  This file holds random-number generation
 * and storage-type rounding only; none of the model's arithmetic lives here.
 * Both the CPU oracle and the GPU library consume what it produces.
 *
 * Generator (one definition, used for every draw):
 *   key(seed, stream) = mix64(mix64(seed + G) ^ (stream * C))
 *   draw(seed, stream, i) = mix64(key + (i + 1) * G)
 * where mix64 is the SplitMix64 finaliser (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), G is the golden
 * gamma 0x9E3779B97F4A7C15 and C = 0xD1B54A32D192ED03.  Being counter based,
 * any element can be drawn independently, so tensors are filled in parallel.
 *
 * Normals: Box-Muller (Box & Muller, 1958) on the pair (draw(2k), draw(2k+1)),
 * u1 = ((a >> 11) + 1) * 2^-53 in (0, 1], u2 = (b >> 11) * 2^-53 in [0, 1);
 * element 2k gets r*cos(2*pi*u2), element 2k+1 gets r*sin(2*pi*u2), with
 * r = sqrt(-2 ln u1), all in double; the value std*z is rounded to fp32 and
 * then (for 16-bit storage) to fp16 or bf16 with round-to-nearest-even.
 *
 * Bounded integers: Lemire's multiply-shift on the top 32 bits,
 * ((draw >> 32) * n) >> 32, which lies in [0, n).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <immintrin.h>

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL
#define SYN_C 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + SYN_GAMMA) ^ (stream * SYN_C));
}

static inline uint64_t draw_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SYN_GAMMA);
}

uint64_t syn_draw(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw_at(stream_key(seed, stream), i);
}

static inline double normal_at(uint64_t key, uint64_t idx) {
  uint64_t k = idx >> 1;
  uint64_t a = draw_at(key, 2 * k), b = draw_at(key, 2 * k + 1);
  double u1 = (double)((a >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(b >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (idx & 1) ? r * sin(t) : r * cos(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline uint16_t f32_to_f16_rne(float f) {
  /* F16C hardware conversion, round to nearest even. */
  __m128 v = _mm_set_ss(f);
  __m128i h = _mm_cvtps_ph(v, _MM_FROUND_TO_NEAREST_INT);
  return (uint16_t)_mm_extract_epi16(h, 0);
}

/* Normal(0, std) draws. out_kind: 0 = fp32, 1 = fp16 bits, 2 = bf16 bits. */
void syn_normal(uint64_t seed, uint64_t stream, uint64_t n, double std, int out_kind, void* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    float v = (float)(std * normal_at(key, (uint64_t)i));
    if (out_kind == 0) ((float*)out)[i] = v;
    else if (out_kind == 1) ((uint16_t*)out)[i] = f32_to_f16_rne(v);
    else ((uint16_t*)out)[i] = f32_to_bf16_rne(v);
  }
}

/* Uniform integers in [lo, lo + n_range). */
void syn_uniform_int(uint64_t seed, uint64_t stream, uint64_t n, int32_t lo, uint32_t n_range, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    uint64_t x = draw_at(key, (uint64_t)i) >> 32;
    out[i] = lo + (int32_t)((x * (uint64_t)n_range) >> 32);
  }
}

/* Poisson(lam) by inversion of its CDF in double on one 53-bit uniform per element. */
void syn_poisson(uint64_t seed, uint64_t stream, uint64_t n, double lam, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (uint64_t i = 0; i < n; ++i) {
    double u = (double)(draw_at(key, i) >> 11) * 0x1.0p-53;
    double p = exp(-lam), c = p;
    int32_t k = 0;
    while (u >= c && k < 1000) {
      ++k;
      p *= lam / (double)k;
      c += p;
    }
    out[i] = k;
  }
}

/* Storage rounding helpers exposed for tests of the generator itself. */
void syn_f32_to_f16(const float* in, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_f16_rne(in[i]);
}
void syn_f32_to_bf16(const float* in, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
