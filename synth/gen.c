/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module produces the random inputs (initial weights, per-step
 * gradients, zero masks) that both the oracle and the GPU path consume.  It
 * holds no part of the optimizer step's arithmetic: it only turns
 * (seed, stream, step, index) into a float.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based hash:
 * word(key, c) = mix64(key + c * GAMMA), with the published GAMMA and mix
 * constants.  Normals by the Box-Muller transform, evaluated in single
 * precision (the draws are stored as fp32 or narrower; the radius is cut off
 * at about 5.8 sigma by the 24-bit uniform).  Every element depends only on
 * its own index, so any sub-range can be generated independently and the
 * result does not depend on the thread count.  Normals come in Box-Muller pairs: elements 2q and
 * 2q+1 share counter word q+1.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_word(uint64_t key, uint64_t counter) {
    return sm_mix(key + counter * SM_GAMMA);
}

/* Key for one (seed, stream, step) triple. */
uint64_t synth_key(uint64_t seed, uint64_t stream, uint64_t step) {
    uint64_t k = sm_mix(seed + SM_GAMMA);
    k = sm_mix(k ^ (stream * 0xD1B54A32D192ED03ULL + 1));
    k = sm_mix(k ^ (step * 0x8CB92BA72F3D8DD7ULL + 2));
    return k;
}

/* Uniform in the open interval (0, 1) from the top 53 bits. */
static inline double u01_open(uint64_t w) {
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Uniform in [0, 1). */
static inline double u01(uint64_t w) {
    return (double)(w >> 11) * (1.0 / 9007199254740992.0);
}

/* The pair of normals (Z[2q], Z[2q+1]) = r * (cos a, sin a) of Box-Muller
 * pair q, from one word of the counter (two 24-bit uniforms). */
static inline void normal_pair(uint64_t key, uint64_t q, float *z0, float *z1) {
    const float two_pi = 6.28318530717958647692f;
    uint64_t w = sm_word(key, q + 1);
    float u1 = ((float)(uint32_t)(w >> 40) + 0.5f) * (1.0f / 16777216.0f);          /* (0, 1) */
    float u2 = (float)(uint32_t)((w >> 16) & 0xffffffu) * (1.0f / 16777216.0f);  /* [0, 1) */
    float r = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincosf(two_pi * u2, &s, &c);
    *z0 = r * c;
    *z1 = r * s;
}

/*
 * out[j] = (float)(mean + sigma * Z(index0 + j)) for j in [0, n).
 * If zero_frac > 0, element j is exactly 0.0f when an independent uniform
 * drawn from (seed, mask_stream, step, index0 + j) is below zero_frac.
 */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t step,
                      uint64_t index0, int64_t n, double mean, double sigma,
                      double zero_frac, uint64_t mask_stream, float *out) {
    if (n <= 0) return;
    const uint64_t key = synth_key(seed, stream, step);
    const uint64_t mkey = synth_key(seed, mask_stream, step);
    const uint64_t q0 = index0 >> 1, q1 = (index0 + (uint64_t)n - 1) >> 1;
#pragma omp parallel for schedule(static)
    for (int64_t qq = 0; qq <= (int64_t)(q1 - q0); ++qq) {
        uint64_t q = q0 + (uint64_t)qq;
        float z[2];
        normal_pair(key, q, &z[0], &z[1]);
        for (int h = 0; h < 2; ++h) {
            uint64_t i = 2 * q + (uint64_t)h;
            if (i < index0 || i >= index0 + (uint64_t)n) continue;
            double x = mean + sigma * (double)z[h];
            if (zero_frac > 0.0 && u01(sm_word(mkey, i + 1)) < zero_frac) x = 0.0;
            out[i - index0] = (float)x;
        }
    }
}

/* One uniform integer in [0, bound) for (seed, stream, step, index). */
uint64_t synth_uniform_index(uint64_t seed, uint64_t stream, uint64_t step,
                             uint64_t index, uint64_t bound) {
    uint64_t w = sm_word(synth_key(seed, stream, step), index + 1);
    return (uint64_t)(u01(w) * (double)bound);
}
