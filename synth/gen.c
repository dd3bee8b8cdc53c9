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
 * constants.  Normals by the Box-Muller transform in double precision, one
 * normal per pair of words.  Every element depends only on its own index, so
 * any sub-range can be generated independently and the result does not depend
 * on the thread count.
 */
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

static inline double normal_at(uint64_t key, uint64_t i) {
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = u01_open(sm_word(key, 2 * i + 1));
    double u2 = u01(sm_word(key, 2 * i + 2));
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/*
 * out[j] = (float)(mean + sigma * Z(index0 + j)) for j in [0, n).
 * If zero_frac > 0, element j is exactly 0.0f when an independent uniform
 * drawn from (seed, mask_stream, step, index0 + j) is below zero_frac.
 */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t step,
                      uint64_t index0, int64_t n, double mean, double sigma,
                      double zero_frac, uint64_t mask_stream, float *out) {
    const uint64_t key = synth_key(seed, stream, step);
    const uint64_t mkey = synth_key(seed, mask_stream, step);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = index0 + (uint64_t)j;
        double x = mean + sigma * normal_at(key, i);
        if (zero_frac > 0.0 && u01(sm_word(mkey, i + 1)) < zero_frac) x = 0.0;
        out[j] = (float)x;
    }
}

/* One uniform integer in [0, bound) for (seed, stream, step, index). */
uint64_t synth_uniform_index(uint64_t seed, uint64_t stream, uint64_t step,
                             uint64_t index, uint64_t bound) {
    uint64_t w = sm_word(synth_key(seed, stream, step), index + 1);
    return (uint64_t)(u01(w) * (double)bound);
}
