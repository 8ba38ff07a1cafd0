/* A plain C11 program that runs shard steps through the library's C ABI
 * alone: no Python and no torch in the process. The HIP runtime's C API
 * provides device memory and the stream; every step of the method runs in
 * libzs.so.
 *
 *   zs_c_step IN OUT
 *
 * IN (little-endian, packed):
 *   int64  n_tensors, world, rank, align, steps, S, layout
 *   int64  numels[n_tensors]
 *   double lr, beta1, beta2, eps, weight_decay
 *   uint16 contributions[steps][world][S]   (bf16 bits; rank q's gradient
 *                                            restricted to the owned elements,
 *                                            in shard order)
 *   float  master[S]                        (initial fp32 master shard; m = v = 0)
 * OUT:
 *   int64  T, S
 *   float  master[S], m[S], v[S]
 *   uint16 grad[S], param[S], full[T]       (full starts as 0x5A5A everywhere)
 *
 * The owned shard lives in one allocation per array in both layouts; with
 * the PER_TENSOR layout every piece points into them at its shard offset and
 * into `full` (the tensors' gathered buffers, packed) at its tensor's offset.
 * Step t (1-based) takes one of three routes, all of which must give the
 * same bytes: t % 3 == 1 the fused call, t % 3 == 2 the unfused calls
 * (FLAT: reduce in two buckets, AdamW, gather), t % 3 == 0 the fused call
 * with its scalars read from device memory. Before the steps, an invalid plan
 * request must fail with ZS_EINVAL and a message. Exit status 0 on success,
 * 1 on any failure (the failing call and zs_last_error() on stderr), 2 on bad
 * usage. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zs.h"

#define ZS_CHECK(call)                                                                    \
    do {                                                                                  \
        zs_status st_ = (call);                                                           \
        if (st_ != ZS_OK) {                                                               \
            fprintf(stderr, "%s failed: status %d: %s\n", #call, (int)st_, zs_last_error()); \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

#define HIP_CHECK(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static void read_exact(FILE* f, void* dst, size_t bytes, const char* what) {
    if (bytes && fread(dst, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read: %s\n", what);
        exit(1);
    }
}

static void write_exact(FILE* f, const void* src, size_t bytes) {
    if (bytes && fwrite(src, 1, bytes, f) != bytes) {
        fprintf(stderr, "short write\n");
        exit(1);
    }
}

static void* host_alloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of host memory\n");
        exit(1);
    }
    return p;
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_CHECK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT (library %s)\n", argv[0], zs_version());
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        perror(argv[1]);
        return 1;
    }
    int64_t hdr[7];
    read_exact(in, hdr, sizeof hdr, "header");
    const int32_t n_tensors = (int32_t)hdr[0], world = (int32_t)hdr[1], rank = (int32_t)hdr[2];
    const int32_t align = (int32_t)hdr[3], steps = (int32_t)hdr[4], layout = (int32_t)hdr[6];
    const int64_t S_file = hdr[5];
    if (n_tensors < 1 || world < 1 || world > ZS_MAX_CONTRIBS || steps < 1 || S_file < 0 ||
        (layout != ZS_LAYOUT_FLAT && layout != ZS_LAYOUT_PER_TENSOR)) {
        fprintf(stderr, "bad header\n");
        return 1;
    }
    int64_t* numels = (int64_t*)host_alloc(sizeof(int64_t) * (size_t)n_tensors);
    read_exact(in, numels, sizeof(int64_t) * (size_t)n_tensors, "numels");
    double h[5];
    read_exact(in, h, sizeof h, "hyperparameters");

    /* the error path: a rank outside [0, world) */
    zs_plan* bad = NULL;
    if (zs_shard_plan(numels, n_tensors, world, world, align, ZS_LAYOUT_FLAT, &bad) != ZS_EINVAL || bad ||
        zs_last_error()[0] == '\0') {
        fprintf(stderr, "an invalid rank was not rejected with ZS_EINVAL and a message\n");
        return 1;
    }
    printf("expected error: %s\n", zs_last_error());

    zs_plan* plan = NULL;
    ZS_CHECK(zs_shard_plan(numels, n_tensors, world, rank, align, layout, &plan));
    const int64_t T = zs_plan_padded_numel(plan), S = zs_plan_shard_numel(plan);
    if (S != S_file || (layout == ZS_LAYOUT_FLAT && T != S * world)) {
        fprintf(stderr, "plan gives S = %lld, T = %lld; the input holds S = %lld\n", (long long)S, (long long)T,
                (long long)S_file);
        return 1;
    }
    const size_t b16 = sizeof(uint16_t) * (size_t)S, b32 = sizeof(float) * (size_t)S;
    uint16_t* contribs_h = (uint16_t*)host_alloc(b16 * (size_t)world * (size_t)steps);
    read_exact(in, contribs_h, b16 * (size_t)world * (size_t)steps, "contributions");
    float* master_h = (float*)host_alloc(b32);
    read_exact(in, master_h, b32, "master");
    fclose(in);

    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    void** contribs_d = (void**)host_alloc(sizeof(void*) * (size_t)world);
    for (int32_t q = 0; q < world; ++q) contribs_d[q] = dev_alloc(b16);
    float* master = (float*)dev_alloc(b32);
    float* m = (float*)dev_alloc(b32);
    float* v = (float*)dev_alloc(b32);
    void* grad = dev_alloc(b16);
    void* param = dev_alloc(b16);
    void* full = dev_alloc(sizeof(uint16_t) * (size_t)T);
    zs_adamw_coefs* coefs_d = (zs_adamw_coefs*)dev_alloc(sizeof(zs_adamw_coefs));
    HIP_CHECK(hipMemcpy(master, master_h, b32, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemset(m, 0, b32));
    HIP_CHECK(hipMemset(v, 0, b32));
    HIP_CHECK(hipMemset(grad, 0, b16));
    HIP_CHECK(hipMemset(param, 0, b16));
    HIP_CHECK(hipMemsetD16((hipDeviceptr_t)full, 0x5A5A, (size_t)T));
    HIP_CHECK(hipDeviceSynchronize());

    /* PER_TENSOR: the pieces' pointers into the shard arrays and the packed
     * gathered buffers, and the bound multi-tensor table */
    void* ws = NULL;
    if (layout == ZS_LAYOUT_PER_TENSOR) {
        zs_piece_ptrs* pieces = (zs_piece_ptrs*)host_alloc(sizeof(zs_piece_ptrs) * (size_t)n_tensors);
        const void** cptr = (const void**)host_alloc(sizeof(void*) * (size_t)n_tensors * (size_t)world);
        for (int32_t i = 0; i < n_tensors; ++i) {
            zs_tensor_info ti;
            ZS_CHECK(zs_plan_tensor(plan, i, &ti));
            const int64_t o = ti.shard_off;
            pieces[i].grad = (char*)grad + 2 * o;
            pieces[i].master = master + o;
            pieces[i].m = m + o;
            pieces[i].v = v + o;
            pieces[i].param = (char*)param + 2 * o;
            pieces[i].full = (char*)full + 2 * ti.flat_off;
            for (int32_t q = 0; q < world; ++q)
                cptr[(size_t)q * (size_t)n_tensors + (size_t)i] = (const char*)contribs_d[q] + 2 * o;
        }
        const int64_t ws_bytes = zs_multi_workspace_bytes(plan, world);
        ws = dev_alloc((size_t)ws_bytes);
        ZS_CHECK(zs_multi_bind(plan, pieces, cptr, world, ws, ws_bytes, stream));
        free(pieces);
        free(cptr);
    }

    const int64_t half = S / 16 * 8; /* first bucket: a multiple of 8 */
    for (int32_t t = 1; t <= steps; ++t) {
        for (int32_t q = 0; q < world; ++q)
            HIP_CHECK(hipMemcpyAsync(contribs_d[q], contribs_h + ((size_t)(t - 1) * (size_t)world + (size_t)q) * (size_t)S,
                                     b16, hipMemcpyHostToDevice, stream));
        const zs_adamw_hparams hp = {h[0], h[1], h[2], h[3], h[4], t};
        const void* const* cs = (const void* const*)contribs_d;
        if (layout == ZS_LAYOUT_PER_TENSOR) {
            if (t % 3 == 1) {
                ZS_CHECK(zs_fused_shard_step_multi(plan, &hp, ws, stream));
            } else if (t % 3 == 2) {
                ZS_CHECK(zs_reduce_shard_multi(plan, ws, stream));
                ZS_CHECK(zs_adamw_shard_step_multi(plan, &hp, ws, stream));
                ZS_CHECK(zs_gather_params_multi(plan, ws, stream));
            } else {
                zs_adamw_coefs c;
                ZS_CHECK(zs_adamw_coefs_compute(&hp, &c));
                HIP_CHECK(hipMemcpyAsync(coefs_d, &c, sizeof c, hipMemcpyHostToDevice, stream));
                ZS_CHECK(zs_fused_shard_step_multi_dc(plan, coefs_d, 1, ws, stream));
            }
        } else if (t % 3 == 1) {
            ZS_CHECK(zs_fused_shard_step(plan, &hp, cs, world, master, m, v, grad, param, full, stream));
        } else if (t % 3 == 2) {
            ZS_CHECK(zs_reduce_shard(plan, cs, world, grad, 0, half, stream));
            ZS_CHECK(zs_reduce_shard(plan, cs, world, grad, half, S - half, stream));
            ZS_CHECK(zs_adamw_shard_step(plan, &hp, grad, master, m, v, param, stream));
            ZS_CHECK(zs_gather_params(plan, param, full, stream));
        } else {
            zs_adamw_coefs c;
            ZS_CHECK(zs_adamw_coefs_compute(&hp, &c));
            HIP_CHECK(hipMemcpyAsync(coefs_d, &c, sizeof c, hipMemcpyHostToDevice, stream));
            ZS_CHECK(zs_fused_shard_step_dc(plan, coefs_d, cs, world, master, m, v, grad, param, full, stream));
        }
        /* the host buffer of the scalars and the contributions are reused */
        HIP_CHECK(hipStreamSynchronize(stream));
    }

    float* out32 = (float*)host_alloc(b32);
    uint16_t* out16 = (uint16_t*)host_alloc(sizeof(uint16_t) * (size_t)T);
    FILE* out = fopen(argv[2], "wb");
    if (!out) {
        perror(argv[2]);
        return 1;
    }
    const int64_t sizes[2] = {T, S};
    write_exact(out, sizes, sizeof sizes);
    const float* state[3] = {master, m, v};
    for (int k = 0; k < 3; ++k) {
        HIP_CHECK(hipMemcpy(out32, state[k], b32, hipMemcpyDeviceToHost));
        write_exact(out, out32, b32);
    }
    HIP_CHECK(hipMemcpy(out16, grad, b16, hipMemcpyDeviceToHost));
    write_exact(out, out16, b16);
    HIP_CHECK(hipMemcpy(out16, param, b16, hipMemcpyDeviceToHost));
    write_exact(out, out16, b16);
    HIP_CHECK(hipMemcpy(out16, full, sizeof(uint16_t) * (size_t)T, hipMemcpyDeviceToHost));
    write_exact(out, out16, sizeof(uint16_t) * (size_t)T);
    if (fclose(out) != 0) {
        perror(argv[2]);
        return 1;
    }

    if (ws) {
        ZS_CHECK(zs_multi_unbind(ws, stream));
        HIP_CHECK(hipFree(ws));
    }
    for (int32_t q = 0; q < world; ++q) HIP_CHECK(hipFree(contribs_d[q]));
    HIP_CHECK(hipFree(master));
    HIP_CHECK(hipFree(m));
    HIP_CHECK(hipFree(v));
    HIP_CHECK(hipFree(grad));
    HIP_CHECK(hipFree(param));
    HIP_CHECK(hipFree(full));
    HIP_CHECK(hipFree(coefs_d));
    HIP_CHECK(hipStreamDestroy(stream));
    zs_plan_destroy(plan);
    free(contribs_d);
    free(contribs_h);
    free(master_h);
    free(out32);
    free(out16);
    free(numels);
    printf("ok: %s layout, %d steps, T = %lld, S = %lld, world = %d, rank = %d\n",
           layout == ZS_LAYOUT_FLAT ? "FLAT" : "PER_TENSOR", steps, (long long)T, (long long)S, world, rank);
    return 0;
}
