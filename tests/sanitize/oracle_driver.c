/* Exercises every function of the CPU oracle on random and special inputs
 * (ragged lengths, signed zeros, subnormals, infinities, NaNs, every block
 * size) so that a build with the compiler's address and undefined-behaviour
 * sanitizers can catch out-of-bounds accesses, overflows and invalid
 * conversions. Correctness is the pin tests' business; this program only has
 * to run clean. Test infrastructure, like the oracle itself. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t ora_f32_to_bf16(float x);
float ora_bf16_to_f32(uint16_t h);
void ora_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n);
void ora_reduce(const uint16_t* const* contribs, int32_t n, int64_t lo, int64_t hi, uint16_t* g);
void ora_adamw_coef(double lr, double beta1, double beta2, double eps, double wd, int64_t t, float* c);
void ora_adamw(const float* c, const uint16_t* g, float* master, float* m, float* v, uint16_t* p, int64_t lo,
               int64_t hi);
void ora_gather(const uint16_t* p, int64_t S, int32_t rank, int64_t lo, int64_t hi, uint16_t* full);
void ora_shard_step(const float* c, const uint16_t* const* contribs, int32_t n, uint16_t* g, float* master, float* m,
                    float* v, uint16_t* p, uint16_t* full, int64_t S, int32_t rank, int64_t lo, int64_t hi);
int ora_time_shard_step(const float* c, const uint16_t* const* contribs, int32_t n, uint16_t* g, float* master,
                        float* m, float* v, uint16_t* p, uint16_t* full, int64_t S, int32_t rank, int64_t len,
                        int32_t nthreads, int32_t reps, double* secs);
void ora_accumulate(const uint16_t* const* contribs, int32_t n, float* acc, int32_t first, int64_t lo, int64_t hi);
double ora_grad_sumsq(const float* acc, float divisor, int64_t lo, int64_t hi, int32_t* nonfinite);
float ora_clip_scale(const double* sumsq, int32_t n_ranks, double max_norm);
void ora_adamw_f32grad(const float* c, const float* acc, float divisor, float scale, int32_t skip, float* master,
                       float* m, float* v, uint16_t* p, int64_t lo, int64_t hi);
void ora_quantize(const uint16_t* p, int64_t n, int32_t bits, int32_t B, uint8_t* q, float* scales);
void ora_dequantize(const uint8_t* q, const float* scales, int64_t n, int32_t bits, int32_t B, uint16_t* out);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

/* A bf16 pattern: mostly small Gaussian-like values, sometimes special ones. */
static uint16_t some_bf16(void) {
    static const uint16_t special[] = {0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F7F, 0x0080};
    uint32_t r = next32();
    if (r % 64 == 0) return special[(r >> 8) % (sizeof special / sizeof special[0])];
    float x = ((float)(int32_t)(next32() & 0xFFFF) - 32768.0f) * 1e-7f;
    return ora_f32_to_bf16(x);
}

static float some_f32(void) {
    uint32_t r = next32();
    if (r % 97 == 0) {
        static const float special[] = {0.0f, -0.0f, 1e-40f, -1e-45f, 3.0e38f, INFINITY, -INFINITY};
        return special[(r >> 8) % 7];
    }
    return ((float)(int32_t)(next32() & 0xFFFF) - 32768.0f) * 1e-6f;
}

int main(void) {
    /* every bf16 pattern round-trips through the conversion helpers */
    for (uint32_t h = 0; h < 65536; ++h) (void)ora_f32_to_bf16(ora_bf16_to_f32((uint16_t)h));
    for (uint32_t k = 0; k < 1u << 20; ++k) {
        uint32_t u = next32() * 2654435761u;
        float x;
        memcpy(&x, &u, sizeof x);
        (void)ora_f32_to_bf16(x);
    }
    const int64_t sizes[] = {0, 1, 7, 8, 9, 255, 256, 257, 1000, 4099};
    for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; ++si) {
        const int64_t S = sizes[si];
        for (int32_t n = 1; n <= 9; n += 4) {
            const size_t A = (size_t)(S > 0 ? S : 1);
            uint16_t** cs = (uint16_t**)malloc(sizeof(uint16_t*) * (size_t)n);
            for (int32_t q = 0; q < n; ++q) {
                cs[q] = (uint16_t*)malloc(A * sizeof(uint16_t));
                for (int64_t j = 0; j < S; ++j) cs[q][j] = some_bf16();
            }
            uint16_t* g = (uint16_t*)malloc(A * 2);
            uint16_t* p = (uint16_t*)malloc(A * 2);
            float* master = (float*)malloc(A * 4);
            float* m = (float*)calloc(A, 4);
            float* v = (float*)calloc(A, 4);
            float* acc = (float*)malloc(A * 4);
            const int32_t world = 3, rank = 2;
            uint16_t* full = (uint16_t*)malloc((size_t)world * A * 2);
            for (int64_t j = 0; j < S; ++j) master[j] = some_f32();
            float c[9];
            ora_adamw_coef(1e-3, 0.9, 0.95, 1e-8, 0.1, 1 + (int64_t)si, c);
            ora_shard_step(c, (const uint16_t* const*)cs, n, g, master, m, v, p, full, S, rank, 0, S);
            ora_reduce((const uint16_t* const*)cs, n, S / 3, S, g);
            ora_adamw(c, g, master, m, v, p, 0, S / 2);
            ora_gather(p, S, rank, 0, S, full);
            double secs[2];
            if (ora_time_shard_step(c, (const uint16_t* const*)cs, n, g, master, m, v, p, full, S, 1, S, 3, 2,
                                    secs) != 0)
                return 2;
            ora_accumulate((const uint16_t* const*)cs, n, acc, 1, 0, S);
            ora_accumulate((const uint16_t* const*)cs, n, acc, 0, 0, S);
            int32_t bad = 0;
            double sumsq[2] = {ora_grad_sumsq(acc, 2.0f, 0, S, &bad), ora_grad_sumsq(acc, 3.0f, 0, S / 2, &bad)};
            const float sc = ora_clip_scale(sumsq, 2, 1.0);
            ora_adamw_f32grad(c, acc, 2.0f, isfinite(sc) ? sc : 1.0f, 0, master, m, v, p, 0, S);
            ora_adamw_f32grad(c, acc, 2.0f, 1.0f, 1, master, m, v, p, 0, S);
            for (int32_t bits = 4; bits <= 8; bits += 4) {
                for (int32_t B = 8; B <= 256; B *= 2) {
                    const int64_t nb = (S + B - 1) / B;
                    uint8_t* q = (uint8_t*)calloc((size_t)(S > 0 ? S : 1), 1);
                    float* scales = (float*)malloc((size_t)(nb > 0 ? nb : 1) * 4);
                    uint16_t* out = (uint16_t*)malloc(A * 2);
                    ora_quantize(p, S, bits, B, q, scales);
                    ora_dequantize(q, scales, S, bits, B, out);
                    /* arbitrary payloads: every code value, any scale */
                    for (int64_t j = 0; j < S; ++j) q[j] = (uint8_t)next32();
                    for (int64_t b = 0; b < nb; ++b) scales[b] = some_f32();
                    ora_dequantize(q, scales, S, bits, B, out);
                    free(q);
                    free(scales);
                    free(out);
                }
            }
            for (int32_t q = 0; q < n; ++q) free(cs[q]);
            free(cs);
            free(g);
            free(p);
            free(master);
            free(m);
            free(v);
            free(acc);
            free(full);
        }
    }
    printf("oracle driver ok\n");
    return 0;
}
