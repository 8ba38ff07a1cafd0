/*
 * Plain CPU oracle for one rank's shard-local optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header or constant table with the
 * HIP library.
 *
 * What it computes, element by element, in the order the sources describe:
 *
 *   reduce  - the averaged gradient a reduce-scatter leaves on the owning rank:
 *             "ZeRO vs FSDP: A Rigorous Dissection..." section 2.1 (reduce-scatter
 *             hands each rank the gradient slice of its optimizer shard) and
 *             "从 Data Parallel 到 ZeRO/FSDP" section "Data Parallel 保证的数学语义"
 *             (all ranks obtain the *average* gradient through AllReduce) plus
 *             section "DDP 为什么单卡仍是 16P" (ring AllReduce = ReduceScatter that
 *             leaves one reduced chunk per rank, then AllGather).
 *   adamw   - mixed-precision AdamW on the owned shard: bf16 parameter, bf16
 *             gradient, fp32 master / first moment / second moment
 *             ("ZeRO vs FSDP..." section 1.1, and the persistent ledger of
 *             "FSDP2's parameter lifecycle..." section "16 bytes per parameter is
 *             where planning starts"). The pages name AdamW but do not write its
 *             update; the update used here is decoupled weight decay with bias
 *             correction (Loshchilov & Hutter, "Decoupled Weight Decay
 *             Regularization", ICLR 2019), decay applied to the master weight
 *             first, eps added outside the square root.
 *   gather  - the updated bf16 shard placed at offset rank*S of the full
 *             parameter buffer, the all-gather half of "ZeRO vs FSDP..." section
 *             2.1 and of "从 Data Parallel 到 ZeRO/FSDP" section "ZeRO Stage 1".
 *
 * Precision. The pages fix the storage dtypes (bf16 param and grad, fp32
 * master/m/v; "从 Data Parallel 到 ZeRO/FSDP" section "Mixed Precision 至少有四个
 * Dtype" asks for each to be written down). The element arithmetic therefore
 * runs in the optimizer dtype, fp32, with one IEEE round-to-nearest per
 * operation in the order written below. Build with -ffp-contract=off and
 * without -ffast-math so that no operation is fused or reordered.
 *
 * bf16 <-> fp32: bf16 is the upper half of an IEEE binary32. Narrowing is
 * IEEE round-to-nearest, ties to even; a NaN narrows to a quiet NaN with its
 * sign; subnormals and signed zeros are kept (no flush to zero).
 */
#define _POSIX_C_SOURCE 199309L
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

/* ---------------------------------------------------------------- bf16 */

static inline uint32_t f32_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return u;
}

static inline float bits_f32(uint32_t u) {
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

/* IEEE round-to-nearest-even of a binary32 to its upper 16 bits. Adding
 * 0x7FFF plus the lowest kept bit carries into the kept half exactly when the
 * dropped half is above one half, or equal to one half with an odd kept half. */
uint16_t ora_f32_to_bf16(float x) {
    uint32_t u = f32_bits(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) /* NaN: keep sign, force quiet bit */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

float ora_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

void ora_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = ora_f32_to_bf16(x[i]);
}

/* ---------------------------------------------------------------- reduce */

/* g[j] for j in [lo, hi): the average over the n contributions, summed in
 * fp32 one add at a time in rank order 0..n-1 starting from +0, divided once
 * by n, rounded to bf16. contribs[q][j] is rank q's bf16 gradient for the
 * owned element j. */
void ora_reduce(const uint16_t* const* contribs, int32_t n, int64_t lo, int64_t hi, uint16_t* g) {
    const float nf = (float)n;
    for (int64_t j = lo; j < hi; ++j) {
        float acc = 0.0f;
        for (int32_t q = 0; q < n; ++q) acc = acc + ora_bf16_to_f32(contribs[q][j]);
        float avg = acc / nf;
        g[j] = ora_f32_to_bf16(avg);
    }
}

/* ---------------------------------------------------------------- AdamW */

/* Scalars of one AdamW step t >= 1, each computed in double from the
 * hyperparameters and rounded once to fp32:
 *   c[0]=beta1  c[1]=1-beta1  c[2]=beta2  c[3]=1-beta2  c[4]=lr  c[5]=eps
 *   c[6]=1-lr*wd (decoupled decay factor)  c[7]=1-beta1^t  c[8]=1-beta2^t */
void ora_adamw_coef(double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                    float* c) {
    c[0] = (float)beta1;
    c[1] = (float)(1.0 - beta1);
    c[2] = (float)beta2;
    c[3] = (float)(1.0 - beta2);
    c[4] = (float)lr;
    c[5] = (float)eps;
    c[6] = (float)(1.0 - lr * wd);
    c[7] = (float)(1.0 - pow(beta1, (double)t));
    c[8] = (float)(1.0 - pow(beta2, (double)t));
}

/* One AdamW step over owned elements [lo, hi). Reads the bf16 gradient g and
 * the fp32 state; writes master, m, v in place and the bf16 parameter p (the
 * bf16 rounding of the new master weight). */
void ora_adamw(const float* c, const uint16_t* g, float* master, float* m, float* v, uint16_t* p,
               int64_t lo, int64_t hi) {
    const float b1 = c[0], omb1 = c[1], b2 = c[2], omb2 = c[3];
    const float lr = c[4], eps = c[5], decay = c[6], bc1 = c[7], bc2 = c[8];
    for (int64_t j = lo; j < hi; ++j) {
        float gf = ora_bf16_to_f32(g[j]);
        float w = master[j] * decay;             /* decoupled weight decay first */
        float mj = b1 * m[j] + omb1 * gf;        /* first moment */
        float vj = b2 * v[j] + omb2 * (gf * gf); /* second moment */
        float mhat = mj / bc1;                   /* bias corrections */
        float vhat = vj / bc2;
        float den = sqrtf(vhat) + eps;           /* eps outside the root */
        w = w - lr * (mhat / den);
        master[j] = w;
        m[j] = mj;
        v[j] = vj;
        p[j] = ora_f32_to_bf16(w);
    }
}

/* ---------------------------------------------------------------- gather */

/* full[rank*S + j] = p[j] for j in [lo, hi); nothing else of full is touched. */
void ora_gather(const uint16_t* p, int64_t S, int32_t rank, int64_t lo, int64_t hi, uint16_t* full) {
    for (int64_t j = lo; j < hi; ++j) full[(int64_t)rank * S + j] = p[j];
}

/* ---------------------------------------------------------------- step */

/* One whole shard step on owned elements [lo, hi): reduce into g, AdamW, then
 * the gather write. The three phases are applied in sequence to the range. */
void ora_shard_step(const float* c, const uint16_t* const* contribs, int32_t n, uint16_t* g,
                    float* master, float* m, float* v, uint16_t* p, uint16_t* full, int64_t S,
                    int32_t rank, int64_t lo, int64_t hi) {
    ora_reduce(contribs, n, lo, hi, g);
    ora_adamw(c, g, master, m, v, p, lo, hi);
    if (full) ora_gather(p, S, rank, lo, hi, full);
}

/* ---------------------------------------------------------------- timing */

typedef struct {
    const float* c;
    const uint16_t* const* contribs;
    int32_t n;
    uint16_t* g;
    float *master, *m, *v;
    uint16_t *p, *full;
    int64_t S;
    int32_t rank;
    int64_t lo, hi;
} ora_job;

static void* ora_job_run(void* arg) {
    ora_job* j = (ora_job*)arg;
    ora_shard_step(j->c, j->contribs, j->n, j->g, j->master, j->m, j->v, j->p, j->full, j->S,
                   j->rank, j->lo, j->hi);
    return NULL;
}

/* Runs ora_shard_step over [0, len) split into nthreads contiguous ranges,
 * reps times; returns the wall-clock seconds of each repetition in secs[]. */
int ora_time_shard_step(const float* c, const uint16_t* const* contribs, int32_t n, uint16_t* g,
                        float* master, float* m, float* v, uint16_t* p, uint16_t* full, int64_t S,
                        int32_t rank, int64_t len, int32_t nthreads, int32_t reps, double* secs) {
    if (nthreads < 1 || reps < 1) return -1;
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    ora_job* jobs = (ora_job*)calloc((size_t)nthreads, sizeof(ora_job));
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return -1;
    }
    for (int32_t k = 0; k < nthreads; ++k) {
        ora_job* j = &jobs[k];
        j->c = c; j->contribs = contribs; j->n = n; j->g = g;
        j->master = master; j->m = m; j->v = v; j->p = p; j->full = full;
        j->S = S; j->rank = rank;
        j->lo = len * k / nthreads;
        j->hi = len * (k + 1) / nthreads;
    }
    for (int32_t r = 0; r < reps; ++r) {
        struct timespec t0, t1;
        clock_gettime(CLOCK_MONOTONIC, &t0);
        if (nthreads == 1) {
            ora_job_run(&jobs[0]);
        } else {
            for (int32_t k = 0; k < nthreads; ++k) pthread_create(&th[k], NULL, ora_job_run, &jobs[k]);
            for (int32_t k = 0; k < nthreads; ++k) pthread_join(th[k], NULL);
        }
        clock_gettime(CLOCK_MONOTONIC, &t1);
        secs[r] = (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
    }
    free(th);
    free(jobs);
    return 0;
}

/* ---------------------------------------------------------------- accumulation and clipping
 *
 * Gradient accumulation over G micro-batches with the gradient shard kept in
 * fp32 ("从 Data Parallel 到 ZeRO/FSDP", section "Gradient Accumulation 会改变生命周期":
 * each micro-step reduce-scatters and accumulates on the shard, the loss is
 * divided by the accumulation steps, and clipping uses the global norm;
 * section "一次 Mixed-precision Adam 为什么接近 16 Bytes/Parameter": the
 * accumulation dtype may be fp32). Each micro-step's averaged gradient is
 * rounded to bf16 (the reduce dtype) and added in fp32; the gradient AdamW
 * uses is the sum divided once by G. Global-norm clipping scales it by
 * min(1, max_norm / (||g|| + 1e-6)), ||g|| being the L2 norm over every
 * rank's shard. A non-finite gradient anywhere skips the optimizer step. */

/* acc[j] = (first ? +0 : acc[j]) + f32(bf16(average of the contributions)) */
void ora_accumulate(const uint16_t* const* contribs, int32_t n, float* acc, int32_t first, int64_t lo,
                    int64_t hi) {
    const float nf = (float)n;
    for (int64_t j = lo; j < hi; ++j) {
        float s = 0.0f;
        for (int32_t q = 0; q < n; ++q) s = s + ora_bf16_to_f32(contribs[q][j]);
        float g = ora_bf16_to_f32(ora_f32_to_bf16(s / nf));
        float base = first ? 0.0f : acc[j];
        acc[j] = base + g;
    }
}

/* The gradient AdamW consumes: g = acc / G, then g * scale. */
static inline float ora_final_grad(float acc, float divisor, float scale) {
    float g = acc / divisor;
    return g * scale;
}

/* Sum of squares of the final gradient (acc / G) over [lo, hi) in double,
 * element order; *nonfinite is set to 1 when any of those values is not
 * finite. */
double ora_grad_sumsq(const float* acc, float divisor, int64_t lo, int64_t hi, int32_t* nonfinite) {
    double s = 0.0;
    for (int64_t j = lo; j < hi; ++j) {
        float g = acc[j] / divisor;
        if (!isfinite(g)) *nonfinite = 1;
        s += (double)g * (double)g;
    }
    return s;
}

/* Clip factor from the squared norms of all ranks' shards (the all-reduced
 * sum, added in rank order), as an fp32 multiplier no larger than 1. */
float ora_clip_scale(const double* sumsq, int32_t n_ranks, double max_norm) {
    double total = 0.0;
    for (int32_t r = 0; r < n_ranks; ++r) total += sumsq[r];
    double coef = max_norm / (sqrt(total) + 1e-6);
    return (float)(coef < 1.0 ? coef : 1.0);
}

/* AdamW from an fp32 accumulated gradient: identical to ora_adamw with the
 * element gradient ora_final_grad(acc[j], divisor, scale) in place of the
 * bf16 gradient; skip != 0 leaves every array unchanged. */
void ora_adamw_f32grad(const float* c, const float* acc, float divisor, float scale, int32_t skip, float* master,
                       float* m, float* v, uint16_t* p, int64_t lo, int64_t hi) {
    if (skip) return;
    const float b1 = c[0], omb1 = c[1], b2 = c[2], omb2 = c[3];
    const float lr = c[4], eps = c[5], decay = c[6], bc1 = c[7], bc2 = c[8];
    for (int64_t j = lo; j < hi; ++j) {
        float gf = ora_final_grad(acc[j], divisor, scale);
        float w = master[j] * decay;
        float mj = b1 * m[j] + omb1 * gf;
        float vj = b2 * v[j] + omb2 * (gf * gf);
        float mhat = mj / bc1;
        float vhat = vj / bc2;
        float den = sqrtf(vhat) + eps;
        w = w - lr * (mhat / den);
        master[j] = w;
        m[j] = mj;
        v[j] = vj;
        p[j] = ora_f32_to_bf16(w);
    }
}

/* ---------------------------------------------------------------- quantized parameter gather
 * ZeRO++ quantizes the parameters that the all-gather moves, down to 4 bits,
 * for up to four times less traffic ("ZeRO vs FSDP...", section 5.2). The
 * pages give no scheme; this is the plain symmetric block-wise reading:
 *
 *   the rank's updated bf16 shard is cut into blocks of B elements (the last
 *   one may be shorter); per block, amax = max |x| over its elements and
 *   scale = amax / qmax in fp32, qmax = 2^(bits-1) - 1 (127 for 8 bits, 7
 *   for 4 bits); each element becomes the integer k = x / scale rounded to
 *   nearest, ties to even, clamped to [-qmax, qmax]. A block whose amax is 0
 *   has scale 0 and every k = 0. A block holding a NaN or an infinity has
 *   scale NaN and every k = 0, so every element of it dequantizes to NaN.
 *   Dequantization: x' = bf16(f32(k) * scale), round-to-nearest-even.
 *
 * Storage: 8 bits -- one two's-complement byte per element; 4 bits -- two
 * elements per byte, element 2i in the low nibble and 2i+1 in the high
 * nibble, each a 4-bit two's-complement value. One fp32 scale per block. */

static int32_t ora_qmax(int32_t bits) { return (1 << (bits - 1)) - 1; }

static void ora_put_code(uint8_t* q, int32_t bits, int64_t j, int32_t k) {
    if (bits == 8) {
        q[j] = (uint8_t)(k & 0xFF);
    } else {
        uint8_t nib = (uint8_t)(k & 0xF);
        if (j & 1)
            q[j >> 1] = (uint8_t)((q[j >> 1] & 0x0F) | (nib << 4));
        else
            q[j >> 1] = (uint8_t)((q[j >> 1] & 0xF0) | nib);
    }
}

static int32_t ora_get_code(const uint8_t* q, int32_t bits, int64_t j) {
    if (bits == 8) return (int32_t)(int8_t)q[j];
    int32_t nib = (j & 1) ? (q[j >> 1] >> 4) : (q[j >> 1] & 0xF);
    return nib >= 8 ? nib - 16 : nib;
}

/* Quantizes p[0, n) in blocks of B: codes into q (n bytes for 8 bits,
 * ceil(n/2) for 4 bits), one scale per block into scales. */
void ora_quantize(const uint16_t* p, int64_t n, int32_t bits, int32_t B, uint8_t* q, float* scales) {
    const int32_t qmax = ora_qmax(bits);
    for (int64_t lo = 0, b = 0; lo < n; lo += B, ++b) {
        const int64_t hi = lo + B < n ? lo + B : n;
        float amax = 0.0f;
        int finite = 1;
        for (int64_t j = lo; j < hi; ++j) {
            float x = ora_bf16_to_f32(p[j]);
            if (!isfinite(x)) finite = 0;
            float a = fabsf(x);
            if (a > amax) amax = a;
        }
        const float scale = finite ? amax / (float)qmax : NAN;
        for (int64_t j = lo; j < hi; ++j) {
            int32_t k = 0;
            if (finite && amax > 0.0f) {
                float r = nearbyintf(ora_bf16_to_f32(p[j]) / scale);
                if (r > (float)qmax) r = (float)qmax;
                if (r < -(float)qmax) r = -(float)qmax;
                k = (int32_t)r;
            }
            ora_put_code(q, bits, j, k);
        }
        scales[b] = scale;
    }
}

/* out[j] = bf16(f32(code j) * scale of its block), j in [0, n). */
void ora_dequantize(const uint8_t* q, const float* scales, int64_t n, int32_t bits, int32_t B, uint16_t* out) {
    for (int64_t j = 0; j < n; ++j) {
        float x = (float)ora_get_code(q, bits, j) * scales[j / B];
        out[j] = ora_f32_to_bf16(x);
    }
}
