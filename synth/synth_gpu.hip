// GPU build of the synthetic-input definition in synth_def.h: fills device
// buffers with the same bits the host build produces. Grid-stride, one
// element per thread per iteration; the launch is bounded by n.
#include <hip/hip_runtime.h>

#include "synth_def.h"

namespace {

__global__ void k_fill_f32(float* __restrict__ dst, int64_t n, int64_t base, synth_spec sp) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        dst[j] = synth_value_f32(&sp, base + j);
}

__global__ void k_fill_bf16(uint16_t* __restrict__ dst, int64_t n, int64_t base, synth_spec sp) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        dst[j] = synth_trunc_bf16(synth_value_f32(&sp, base + j));
}

__global__ void k_fill_u16(uint16_t* __restrict__ dst, int64_t n, uint16_t value) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        dst[j] = value;
}

unsigned grid_for(int64_t n) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

}  // namespace

extern "C" {

int synth_gpu_fill_f32(float* dst, int64_t n, int64_t base, const synth_spec* sp, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n, base,
                       *sp);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int synth_gpu_fill_bf16(uint16_t* dst, int64_t n, int64_t base, const synth_spec* sp, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n,
                       base, *sp);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Constant fill of a bf16 buffer (sentinels for untouched regions).
int synth_gpu_fill_u16(uint16_t* dst, int64_t n, uint16_t value, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_u16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n,
                       value);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
