/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no Mixture-of-Experts arithmetic: it only turns
 * (seed, tensor id, element index) into numbers.  Both the CPU oracle and the
 * GPU path are fed from the arrays it writes, so their inputs are identical
 * bit for bit.
 *
 * Generator definition (every element is independent of every other, so any
 * slice of a tensor can be generated on its own):
 *   key(seed, tid) = mix64(seed * 0x9E3779B97F4A7C15 + tid * 0xD1B54A32D192ED03 + 1)
 *   bits(i)        = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   uniform(i)     = ((bits(i) >> 11) + 1) * 2^-53            in (0, 1]
 * mix64 is the SplitMix64 output function (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).
 *   normal(i)      : Box-Muller on the pair p = i / 2, with u1 = uniform(2p),
 *                    u2 = uniform(2p + 1); r = sqrt(-2 ln u1);
 *                    even i -> r cos(2 pi u2), odd i -> r sin(2 pi u2).
 * Values are scaled in double, rounded to fp32 (round to nearest even), and
 * for bf16 rounded again from that fp32 value to bf16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid) {
  return mix64(seed * 0x9E3779B97F4A7C15ULL + tid * 0xD1B54A32D192ED03ULL + 1ULL);
}

static inline double uniform_at(uint64_t key, uint64_t i) {
  uint64_t b = mix64(key + (i + 1ULL) * 0x9E3779B97F4A7C15ULL);
  return (double)((b >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = uniform_at(key, 2 * p);
  double u2 = uniform_at(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[j] = fp32(normal(offset + j) * scale) for j < count. */
void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t count, double scale,
                      float* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static, 65536)
  for (int64_t j = 0; j < (int64_t)count; ++j) out[j] = (float)(normal_at(key, offset + (uint64_t)j) * scale);
}

/* out[j] = bf16(fp32(normal(offset + j) * scale)) as raw bits. */
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t count, double scale,
                       uint16_t* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static, 65536)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = f32_to_bf16_rne((float)(normal_at(key, offset + (uint64_t)j) * scale));
}

/* out[j] = fp32(lo + (hi - lo) * uniform(offset + j)). */
void synth_uniform_f32(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t count, double lo,
                       double hi, float* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static, 65536)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = (float)(lo + (hi - lo) * uniform_at(key, offset + (uint64_t)j));
}

/* Raw 64-bit draws, exposed so tests can pin the generator itself. */
void synth_bits(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t count, uint64_t* out) {
  uint64_t key = stream_key(seed, tid);
  for (uint64_t j = 0; j < count; ++j) out[j] = mix64(key + (offset + j + 1ULL) * 0x9E3779B97F4A7C15ULL);
}

/* Random FP8 E4M3 weight codes built from raw draws alone (no rounding of
 * real values): sign = bit 63, mantissa field = bits 60..62, exponent field
 * = 3 + (number of set bits among bits 0..7), i.e. a binomial spread of
 * magnitudes 2^-4 .. 2^4 around 1 (the exponent never reaches the NaN field). */
void synth_fp8_codes(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t count, uint8_t* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static, 65536)
  for (int64_t j = 0; j < (int64_t)count; ++j) {
    const uint64_t r = mix64(key + (offset + (uint64_t)j + 1ULL) * 0x9E3779B97F4A7C15ULL);
    const uint32_t e = 3u + (uint32_t)__builtin_popcountll(r & 0xFFull);
    out[j] = (uint8_t)(((r >> 63) << 7) | (e << 3) | ((r >> 60) & 7u));
  }
}

/* bf16 bits -> fp32, and fp32 -> bf16 bits (round to nearest even); helpers
 * for callers that hold bf16 as uint16 arrays. */
void synth_f32_to_bf16(const float* in, uint16_t* out, uint64_t n) {
#pragma omp parallel for schedule(static, 65536)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}

/* Plain sequential SplitMix64 (state += golden gamma; output = mix64(state)),
 * exposed so tests can check mix64 against the published output sequence. */
void synth_splitmix64(uint64_t state, uint64_t count, uint64_t* out) {
  for (uint64_t j = 0; j < count; ++j) {
    state += 0x9E3779B97F4A7C15ULL;
    out[j] = mix64(state);
  }
}
