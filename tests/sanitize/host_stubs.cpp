// Host-only stand-ins for the device side of libzs: the kernel launchers, the
// workspace copy and the offload pipeline. With them the host part of the
// library -- plans, argument validation, the multi-tensor table, the host
// AdamW and its thread pool -- builds with g++ alone and runs under the
// compiler's sanitizers, no GPU involved. Launchers count their calls and
// succeed without touching memory; the workspace copy writes into (host)
// memory so the driver can inspect the table the library built.
#include <atomic>
#include <cstring>

#include "../../fsdp_sharded_mixed_flatten_amd/csrc/zs_internal.h"

namespace zs {

std::atomic<int> g_launches{0};

int launch_reduce(const void* const*, int, void*, int64_t, void*) { return ++g_launches, 0; }
int launch_adamw(const AdamCoef&, const void*, float*, float*, float*, void*, void*, int64_t, void*,
                 const QuantOut*, const AdamCoef*) {
    return ++g_launches, 0;
}
int launch_gather(const void*, void*, int64_t, void*) { return ++g_launches, 0; }
int launch_gather_sources(const void* const*, int, void*, int64_t, void*) { return ++g_launches, 0; }
int launch_fused(const AdamCoef&, const void* const*, int, float*, float*, float*, void*, void*, void*, int64_t,
                 void*, const QuantOut*, const AdamCoef*) {
    return ++g_launches, 0;
}
int launch_quantize(const QuantOut&, const void*, int64_t, void*) { return ++g_launches, 0; }
int launch_dequant(int, int, const void*, const float*, int64_t, int64_t, int, void*, int64_t, void*) {
    return ++g_launches, 0;
}
int launch_accumulate(const void* const*, int, float*, int, int64_t, void*) { return ++g_launches, 0; }
int launch_grad_stats(const float*, float, double*, int32_t*, void*, int64_t, void*) { return ++g_launches, 0; }
int launch_grad_stats_noalloc(const float*, float, double*, int32_t*, int64_t, void*) { return ++g_launches, 0; }
int launch_clip_scale(const double*, const int32_t*, int, double, float*, int32_t*, void*) {
    return ++g_launches, 0;
}
int launch_adamw_accum(const AdamCoef&, const float*, float, const float*, const int32_t*, float*, float*, float*,
                       void*, void*, int64_t, void*, const AdamCoef*) {
    return ++g_launches, 0;
}
int launch_multi(int, const CoefTable*, const void*, const MultiOffsets&, int, int, void*, const AdamCoef*) {
    return ++g_launches, 0;
}
int copy_h2d_sync(void* dst, const void* src, int64_t bytes, void*) {
    std::memcpy(dst, src, (size_t)bytes);
    return 0;
}
int is_pinned_host(const void*) { return 1; }
// The offloaded step on host memory only: the host arithmetic of the real
// pipeline, without the copies.
int offload_adamw(const AdamCoef& c, const void* grad_dev, float* master, float* m, float* v, void*,
                  void* param_host, void*, void*, int64_t len, int64_t, int n_threads, void*) {
    host_adamw(c, static_cast<const uint16_t*>(grad_dev), master, m, v, static_cast<uint16_t*>(param_host), len,
               n_threads);
    return 0;
}
const char* hip_error_text(int) { return "no device in this build"; }

}  // namespace zs
