/*
 * synth_host.c -- host fills for the counter-based generator in synth.h.
 * Every value is a pure function of (seed, stream, index), so the fills may
 * run on any number of threads without changing a single bit.
 */
#include <math.h>
#include <stdint.h>
#include "synth.h"

float synth_normal_scale(double sigma) { return (float)(sigma / sqrt(SYNTH_IH8_VAR)); }

void synth_fill_normal(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                       float scale, float *out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) out[i] = synth_normal(key, start + (uint64_t)i, scale);
}

void synth_fill_uniform(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, float lo,
                        float hi, float *out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) out[i] = synth_uniform(key, start + (uint64_t)i, lo, hi);
}

/* Open-interval uniform in double, (m + 0.5) * 2^-53 with m the top 53 bits of
 * one draw; used by host-only input recipes (permutations, Gumbel noise). */
void synth_fill_unit_f64(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double *out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) {
    uint64_t m = synth_draw(key, start + (uint64_t)i) >> 11;
    out[i] = ((double)m + 0.5) * 0x1p-53;
  }
}

void synth_fill_ih8(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, int32_t *out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) out[i] = synth_ih8(key, start + (uint64_t)i);
}

void synth_f32_to_bf16_array(const float *x, uint64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) out[i] = synth_f32_to_bf16(x[i]);
}
