// CPU-offloaded optimizer step: the bf16 gradient shard goes to host memory,
// the host steps the fp32 state there, and the bf16 parameters come back
// (ZeRO-Offload: "ZeRO vs FSDP: A Rigorous Dissection...", section 2.4). The
// transfers are pipelined with the host arithmetic chunk by chunk, the only
// way the step's PCIe traffic and host-memory traffic can hide behind each
// other ("从 Data Parallel 到 ZeRO/FSDP", section "CPU/NVMe Offload 不是免费显存").
//
// Pipeline, for chunks k = 0, 1, ... of the shard:
//   caller's stream:  D2H grad chunk 0, 1, 2, ...  (all enqueued up front,
//                     each followed by an event)
//   host threads:     wait for chunk k's event, AdamW on chunk k
//   output stream:    H2D param chunk k as soon as its update is done
// so the copy-in of chunk k+1, the update of chunk k and the copy-out of
// chunk k-1 overlap. The caller's stream finally waits for the last copy-out.
// The output stream is one non-blocking stream per device at the default
// priority, created on first use and kept until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>
#include <vector>

#include "zs_internal.h"

namespace zs {
namespace {

struct DeviceCtx {
    hipStream_t out = nullptr;
    std::vector<hipEvent_t> events;  // grown on demand, reused across calls
    hipEvent_t done = nullptr;       // the last call's final copy-out
    bool recorded = false;           // `done` has been recorded at least once
};

std::mutex g_ctx_mu;
std::unordered_map<int, DeviceCtx> g_ctx;

int ensure_ctx(DeviceCtx** out, size_t n_events) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return (int)e;
    std::lock_guard<std::mutex> lk(g_ctx_mu);
    DeviceCtx& c = g_ctx[dev];
    if (!c.out)
        if (hipError_t e = hipStreamCreateWithFlags(&c.out, hipStreamNonBlocking)) return (int)e;
    if (!c.done)
        if (hipError_t e = hipEventCreateWithFlags(&c.done, hipEventDisableTiming)) return (int)e;
    while (c.events.size() < n_events) {
        hipEvent_t ev;
        if (hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) return (int)e;
        c.events.push_back(ev);
    }
    *out = &c;
    return 0;
}

}  // namespace

int is_pinned_host(const void* p) {
    hipPointerAttribute_t a;
    const hipError_t e = hipPointerGetAttributes(&a, p);
    (void)hipGetLastError();  // an unknown (pageable) pointer reports an error: clear it
    if (e != hipSuccess) return 0;
    return a.type == hipMemoryTypeHost ? 1 : 0;
}

int offload_adamw(const AdamCoef& c, const void* grad_dev, float* master, float* m, float* v, void* grad_host,
                  void* param_host, void* param_dev, void* full_own_dev, int64_t len, int64_t chunk, int n_threads,
                  void* stream_v) {
    if (len <= 0) return 0;
    static std::mutex call_mu;  // the per-device events are shared: one offloaded step at a time
    std::lock_guard<std::mutex> serial(call_mu);
    hipStream_t stream = (hipStream_t)stream_v;
    const int64_t n_chunks = (len + chunk - 1) / chunk;
    DeviceCtx* ctx = nullptr;
    if (int e = ensure_ctx(&ctx, (size_t)n_chunks)) return e;
    const char* gd = static_cast<const char*>(grad_dev);
    char* gh = static_cast<char*>(grad_host);
    char* ph = static_cast<char*>(param_host);
    // The previous call's copy-outs may still read its staging buffers, which
    // this call's host arithmetic overwrites; its caller waited for them, but
    // this call may come on another stream: order this stream after them too.
    if (ctx->recorded)
        if (hipError_t e = hipStreamWaitEvent(stream, ctx->done, 0)) return (int)e;
    for (int64_t k = 0; k < n_chunks; ++k) {
        const int64_t off = k * chunk, n = off + chunk < len ? chunk : len - off;
        if (hipError_t e = hipMemcpyAsync(gh + 2 * off, gd + 2 * off, (size_t)(2 * n), hipMemcpyDeviceToHost, stream))
            return (int)e;
        if (hipError_t e = hipEventRecord(ctx->events[(size_t)k], stream)) return (int)e;
    }
    for (int64_t k = 0; k < n_chunks; ++k) {
        const int64_t off = k * chunk, n = off + chunk < len ? chunk : len - off;
        if (hipError_t e = hipEventSynchronize(ctx->events[(size_t)k])) return (int)e;
        host_adamw(c, reinterpret_cast<const uint16_t*>(gh) + off, master + off, m + off, v + off,
                   reinterpret_cast<uint16_t*>(ph) + off, n, n_threads);
        if (param_dev)
            if (hipError_t e = hipMemcpyAsync(static_cast<char*>(param_dev) + 2 * off, ph + 2 * off, (size_t)(2 * n),
                                              hipMemcpyHostToDevice, ctx->out))
                return (int)e;
        if (full_own_dev)
            if (hipError_t e = hipMemcpyAsync(static_cast<char*>(full_own_dev) + 2 * off, ph + 2 * off,
                                              (size_t)(2 * n), hipMemcpyHostToDevice, ctx->out))
                return (int)e;
    }
    if (hipError_t e = hipEventRecord(ctx->done, ctx->out)) return (int)e;
    ctx->recorded = true;
    return (int)hipStreamWaitEvent(stream, ctx->done, 0);
}

}  // namespace zs
