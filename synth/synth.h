/*
 * synth.h -- seeded, counter-based generator of synthetic inputs.
 *
 * This header is the single definition of the random inputs that both the CPU
 * oracle harness and the GPU harness consume.  It holds none of the MoE block's
 * arithmetic: it only turns (seed, stream, index) into a number.
 *
 * Generator: SplitMix64 in counter mode (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), with the 64-bit output mixer
 * published by S. Vigna in splitmix64.c.  The state for draw n of a stream is
 * key + (n+1)*GAMMA; the output is mix64(state).
 *
 * Normal deviates use the Irwin-Hall construction: the sum of eight independent
 * 16-bit uniforms, centred and scaled.  Everything up to the final scaling is
 * exact integer arithmetic; the integer is converted to float exactly (it is
 * below 2^24) and multiplied once by a float scale factor.  One IEEE multiply
 * is correctly rounded on every conforming host and GPU, so the host and the
 * device produce bit-identical values.  The scale factor itself is computed on
 * the host (synth_normal_scale) and passed to the device as a float.
 *
 * The Irwin-Hall(8) law has the first two moments of N(0, sigma^2), kurtosis
 * 2.85 instead of 3, and support bounded at +-4.9 sigma.
 *
 * Uniform deviates take the top 24 bits of one draw, u = m * 2^-24 (exact), and
 * map them to [lo, hi) with one subtract, one multiply and one add (no fused
 * multiply-add: translation units that include this header are compiled with
 * floating-point contraction disabled).
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

/* Variance of the sum of eight independent uniforms on {0..65535}:
 * 8 * (65536^2 - 1) / 12. */
#define SYNTH_IH8_VAR 2863311530.0
#define SYNTH_IH8_MEAN 262140 /* 8 * 65535 / 2 */

/* Stream kinds: the top 16 bits of a stream id. */
enum {
  SYNTH_K_ROUTER_W = 1,
  SYNTH_K_ROUTER_B = 2,
  SYNTH_K_X = 3,
  SYNTH_K_GATE = 4,
  SYNTH_K_UP = 5,
  SYNTH_K_DOWN = 6,
  SYNTH_K_GAMMA = 7,
  SYNTH_K_PERM = 8,
  SYNTH_K_GUMBEL = 9,
  SYNTH_K_Z = 10
};

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream id from (kind, layer, item).  item is an expert index, or 0xFFFF for
 * the shared expert, or 0 for per-layer tensors. */
SYNTH_FN uint64_t synth_stream(uint32_t kind, uint32_t layer, uint32_t item) {
  return ((uint64_t)(kind & 0xFFFFu) << 48) | ((uint64_t)(layer & 0xFFFFu) << 32) |
         (uint64_t)item;
}

/* Per-stream key: decorrelates streams and seeds. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed * SYNTH_GAMMA + 0x2545F4914F6CDD1DULL) ^
                     synth_mix64(stream + SYNTH_GAMMA));
}

/* Draw number n (n >= 0) of the stream with the given key. */
SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t n) {
  return synth_mix64(key + (n + 1) * SYNTH_GAMMA);
}

/* Centred Irwin-Hall(8) integer for element idx: in [-262140, 262140]. */
SYNTH_FN int32_t synth_ih8(uint64_t key, uint64_t idx) {
  uint64_t r0 = synth_draw(key, 2 * idx);
  uint64_t r1 = synth_draw(key, 2 * idx + 1);
  uint32_t s = (uint32_t)(r0 & 0xFFFFu) + (uint32_t)((r0 >> 16) & 0xFFFFu) +
               (uint32_t)((r0 >> 32) & 0xFFFFu) + (uint32_t)(r0 >> 48) +
               (uint32_t)(r1 & 0xFFFFu) + (uint32_t)((r1 >> 16) & 0xFFFFu) +
               (uint32_t)((r1 >> 32) & 0xFFFFu) + (uint32_t)(r1 >> 48);
  return (int32_t)s - SYNTH_IH8_MEAN;
}

/* Normal deviate with standard deviation sigma, where scale is the float
 * returned by synth_normal_scale(sigma). */
SYNTH_FN float synth_normal(uint64_t key, uint64_t idx, float scale) {
  return (float)synth_ih8(key, idx) * scale;
}

/* Uniform deviate on [lo, hi). */
SYNTH_FN float synth_uniform(uint64_t key, uint64_t idx, float lo, float hi) {
  uint32_t m = (uint32_t)(synth_draw(key, idx) >> 40); /* 24 bits */
  float u = (float)m * 0x1p-24f;
  float span = hi - lo;
  float t = span * u;
  return lo + t;
}

/* Round an f32 to bf16 (round to nearest, ties to even); NaN stays NaN. */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  if ((v.u & 0x7F800000u) == 0x7F800000u && (v.u & 0x007FFFFFu))
    return (uint16_t)((v.u >> 16) | 0x0040u);
  uint32_t lsb = (v.u >> 16) & 1u;
  uint32_t r = v.u + 0x7FFFu + lsb;
  return (uint16_t)(r >> 16);
}

#endif /* SYNTH_H */
