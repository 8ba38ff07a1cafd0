// Host-side AdamW for the CPU-offloaded optimizer step (ZeRO-Offload keeps
// the fp32 optimizer state in host memory and steps it on the CPU: "ZeRO vs
// FSDP: A Rigorous Dissection...", section 2.4).
//
// The element arithmetic is the same IEEE fp32 sequence as the GPU kernels,
// one rounding per operation in the same order (built with
// -ffp-contract=off; sqrtf and division are the correctly rounded SSE/AVX
// instructions), so host and device steps give identical bytes. The loop is
// compiled for AVX-512, AVX2 and baseline x86-64 and picks one at load time.
//
// Work is split over a persistent pool of host threads in contiguous,
// 16-element-aligned ranges; concurrent callers are serialized.
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <math.h>
#include <mutex>
#include <thread>
#include <vector>

#include "zs_internal.h"

namespace zs {
namespace {

inline uint32_t bits_of(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return u;
}

inline float from_bits(uint32_t u) {
    float x;
    std::memcpy(&x, &u, 4);
    return x;
}

// Round-to-nearest-even narrowing to bf16; NaN -> quiet NaN with its sign.
inline uint16_t to_bf16(float f) {
    const uint32_t u = bits_of(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? (uint16_t)((u >> 16) | 0x40u) : (uint16_t)r;
}

// Compiled for AVX-512, AVX2 and baseline x86-64, the variant picked when the
// library loads. ZS_HOST_ONE_ISA builds the baseline only, for runtimes that
// cannot resolve the variants at load time (the thread sanitizer's).
#ifdef ZS_HOST_ONE_ISA
#define ZS_ISA_CLONES
#else
#define ZS_ISA_CLONES __attribute__((target_clones("avx512f", "avx2", "default")))
#endif

ZS_ISA_CLONES void adamw_range(
    const AdamCoef c, const uint16_t* __restrict__ g, float* __restrict__ master, float* __restrict__ m,
    float* __restrict__ v, uint16_t* __restrict__ p, int64_t n) {
    const float b1 = c.b1, omb1 = c.omb1, b2 = c.b2, omb2 = c.omb2;
    const float lr = c.lr, eps = c.eps, decay = c.decay, bc1 = c.bc1, bc2 = c.bc2;
    for (int64_t j = 0; j < n; ++j) {
        const float gf = from_bits((uint32_t)g[j] << 16);
        float w = master[j] * decay;
        const float mn = b1 * m[j] + omb1 * gf;
        const float vn = b2 * v[j] + omb2 * (gf * gf);
        const float mh = mn / bc1;
        const float vh = vn / bc2;
        const float den = sqrtf(vh) + eps;
        w = w - lr * (mh / den);
        master[j] = w;
        m[j] = mn;
        v[j] = vn;
        if (p) p[j] = to_bf16(w);
    }
}

class Pool {
public:
    ~Pool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : threads_) t.join();
    }

    // Runs fn(0) .. fn(n-1), fn(0) on the calling thread; returns when all end.
    void run(int n, const std::function<void(int)>& fn) {
        std::lock_guard<std::mutex> serial(call_mu_);
        grow(n - 1);
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &fn;
            n_job_ = n;
            remaining_ = n - 1;
            ++gen_;
        }
        cv_.notify_all();
        fn(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_cv_.wait(lk, [&] { return remaining_ == 0; });
        job_ = nullptr;
    }

private:
    void grow(int workers) {
        while ((int)threads_.size() < workers) {
            const int id = (int)threads_.size() + 1;
            threads_.emplace_back([this, id] { loop(id); });
        }
    }

    void loop(int id) {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(mu_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            if (id >= n_job_) continue;
            const std::function<void(int)>* fn = job_;
            lk.unlock();
            (*fn)(id);
            lk.lock();
            if (--remaining_ == 0) done_cv_.notify_all();
        }
    }

    std::mutex call_mu_;
    std::mutex mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> threads_;
    const std::function<void(int)>* job_ = nullptr;
    int n_job_ = 0;
    int remaining_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

Pool& pool() {
    static Pool p;
    return p;
}

}  // namespace

void host_adamw(const AdamCoef& c, const uint16_t* g, float* master, float* m, float* v, uint16_t* p, int64_t n,
                int n_threads) {
    if (n <= 0) return;
    if (n_threads < 1) n_threads = 1;
    const int64_t per = ((n + n_threads - 1) / n_threads + 15) / 16 * 16;
    const int used = (int)((n + per - 1) / per);
    const std::function<void(int)> fn = [&](int t) {
        const int64_t lo = (int64_t)t * per;
        const int64_t hi = lo + per < n ? lo + per : n;
        if (lo < hi) adamw_range(c, g + lo, master + lo, m + lo, v + lo, p ? p + lo : nullptr, hi - lo);
    };
    if (used <= 1)
        fn(0);
    else
        pool().run(used, fn);
}

}  // namespace zs
