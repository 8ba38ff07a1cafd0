/* Host build of the synthetic-input definition in synth_def.h. */
#include "synth_def.h"

uint64_t synth_cpu_key(uint64_t seed, uint64_t stream, uint64_t step) {
    return synth_key(seed, stream, step);
}

/* dst[j] = value of global index (base + j), j in [0, n). */
void synth_cpu_fill_f32(float* dst, int64_t n, int64_t base, const synth_spec* sp) {
    for (int64_t j = 0; j < n; ++j) dst[j] = synth_value_f32(sp, base + j);
}

void synth_cpu_fill_bf16(uint16_t* dst, int64_t n, int64_t base, const synth_spec* sp) {
    for (int64_t j = 0; j < n; ++j) dst[j] = synth_trunc_bf16(synth_value_f32(sp, base + j));
}

/* Values at an explicit list of global indices. */
void synth_cpu_at_f32(float* dst, const int64_t* idx, int64_t n, const synth_spec* sp) {
    for (int64_t j = 0; j < n; ++j) dst[j] = synth_value_f32(sp, idx[j]);
}

void synth_cpu_at_bf16(uint16_t* dst, const int64_t* idx, int64_t n, const synth_spec* sp) {
    for (int64_t j = 0; j < n; ++j) dst[j] = synth_trunc_bf16(synth_value_f32(sp, idx[j]));
}
