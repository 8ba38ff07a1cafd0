/*
 * Seeded synthetic inputs for the shard step: one counter-based definition,
 * compiled for the host (synth_cpu.c, gcc) and for the GPU (synth_gpu.hip).
 *
 * This module holds none of the optimizer's arithmetic. It only turns
 * (seed, stream, step, global element index) into a value; both the CPU
 * oracle's tests and the GPU path's tests read inputs from it, so each side
 * sees the same bytes without either producing the other's inputs.
 *
 * Bits: SplitMix64's output function (Steele, Lea & Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014), used in counter mode:
 *   word(key, c) = mix64(key + (c + 1) * GAMMA),  GAMMA = 0x9E3779B97F4A7C15.
 * Every element index i owns the four counters 4i .. 4i+3.
 *
 * Approximate normal: the Irwin-Hall sum of twelve 16-bit uniforms taken from
 * words 4i, 4i+1, 4i+2. The sum of twelve integers uniform on [0, 65535] has
 * mean 393210 and standard deviation (65536^2 - 1)^(1/2) ~ 65536, so
 * (sum - 393210) * (sigma / 65536) has mean 0 and standard deviation sigma to
 * one part in 2^33, with support +-6 sigma. It uses only integer operations
 * and one fp32 multiply of an exactly representable integer, so every
 * compiler and device produces the same bits.
 *
 * Word 4i+3 carries the per-element Bernoulli draws: the heavy-tail selector
 * (this element is drawn with tail_sigma instead of sigma) and, on a separate
 * key shared by all contributions, the exact-zero mask.
 *
 * bf16 values are the fp32 value truncated to its upper 16 bits (this is an
 * input quantiser only, unrelated to the rounding the step itself performs).
 */
#ifndef SYNTH_DEF_H
#define SYNTH_DEF_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull
#define SYNTH_SEED_SALT 0x5A5EED00D5EED5A5ull

typedef struct synth_spec {
    uint64_t key;          /* synth_key(seed, stream, step) */
    uint64_t zero_key;     /* key of the shared exact-zero mask (used when zero_thresh != 0) */
    float sigma;           /* standard deviation of the bulk */
    float tail_sigma;      /* standard deviation of the heavy tail */
    uint32_t tail_thresh;  /* element is a tail draw when (word3 >> 32) < tail_thresh */
    uint32_t zero_thresh;  /* element is +0 when (zero word3 >> 32) < zero_thresh */
    int64_t valid_hi;      /* global indices >= valid_hi are padding: value +0 */
} synth_spec;

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_word(uint64_t key, uint64_t counter) {
    return synth_mix64(key + (counter + 1ull) * SYNTH_GAMMA);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream, uint64_t step) {
    uint64_t k = synth_mix64(seed ^ SYNTH_SEED_SALT);
    k = synth_mix64(k + (stream + 1ull) * SYNTH_GAMMA);
    k = synth_mix64(k + (step + 1ull) * SYNTH_GAMMA);
    return k;
}

SYNTH_FN int32_t synth_sum12(uint64_t a, uint64_t b, uint64_t c) {
    int32_t s = 0;
    for (int k = 0; k < 4; ++k) {
        s += (int32_t)((a >> (16 * k)) & 0xFFFFu);
        s += (int32_t)((b >> (16 * k)) & 0xFFFFu);
        s += (int32_t)((c >> (16 * k)) & 0xFFFFu);
    }
    return s - 393210;
}

/* fp32 value of global element index i. */
SYNTH_FN float synth_value_f32(const synth_spec* sp, int64_t i) {
    if (i >= sp->valid_hi) return 0.0f;
    uint64_t c = 4ull * (uint64_t)i;
    if (sp->zero_thresh) {
        uint32_t uz = (uint32_t)(synth_word(sp->zero_key, c + 3ull) >> 32);
        if (uz < sp->zero_thresh) return 0.0f;
    }
    int32_t z = synth_sum12(synth_word(sp->key, c), synth_word(sp->key, c + 1ull),
                            synth_word(sp->key, c + 2ull));
    float sig = sp->sigma;
    if (sp->tail_thresh) {
        uint32_t ut = (uint32_t)(synth_word(sp->key, c + 3ull) >> 32);
        if (ut < sp->tail_thresh) sig = sp->tail_sigma;
    }
    float scale = sig * 0x1p-16f;
    return (float)z * scale;
}

SYNTH_FN uint16_t synth_trunc_bf16(float x) {
    union { float f; uint32_t u; } cv;
    cv.f = x;
    return (uint16_t)(cv.u >> 16);
}

#endif
