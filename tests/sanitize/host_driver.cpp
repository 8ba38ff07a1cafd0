// Drives the host part of libzs (built with tests/sanitize/host_stubs.cpp in
// place of the device code) through random plans, every entry point's
// argument validation, the multi-tensor table, the host AdamW thread pool and
// concurrent callers, so that address, undefined-behaviour and thread
// sanitizer builds can check it. Prints "host driver ok" and exits 0 when
// every check holds.
#include <zs.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                                        \
        }                                                                        \
    } while (0)

namespace zs {
extern std::atomic<int> g_launches;
}

namespace {

// Aligned host memory standing in for device buffers (the stubs never touch it).
struct Fake {
    std::vector<unsigned char> mem = std::vector<unsigned char>(1 << 20);
    char* base() { return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(mem.data()) + 255) & ~uintptr_t(255)); }
};

int64_t roundup(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

void random_plans(std::mt19937_64& rng, int count) {
    for (int k = 0; k < count; ++k) {
        const int n = (int)(rng() % 40);
        std::vector<int64_t> numels((size_t)(n ? n : 1));
        for (auto& x : numels) x = (rng() % 8 == 0) ? (int64_t)(rng() % 8) : (int64_t)(rng() % 300000);
        const int32_t world = 1 + (int32_t)(rng() % 300), rank = (int32_t)(rng() % (uint64_t)world);
        zs_plan_options o{};
        o.layout = (int32_t)(rng() % 2);
        o.tensor_align_elems = 1 + (int32_t)(rng() % 256);
        std::vector<int32_t> groups((size_t)numels.size());
        for (auto& g : groups) g = (int32_t)(rng() % ZS_MAX_GROUPS);
        if (o.layout == ZS_LAYOUT_PER_TENSOR) {
            o.persist_below_elems = (rng() % 2) ? (int64_t)(rng() % 5000) : 0;
            o.groups = (rng() % 2) ? groups.data() : nullptr;
        }
        zs_plan* p = nullptr;
        if (zs_shard_plan_ex(numels.data(), n, world, rank, &o, &p) != ZS_OK) {
            CHECK(p == nullptr && std::strlen(zs_last_error()) > 0);
            continue;
        }
        const int64_t T = zs_plan_padded_numel(p), S = zs_plan_shard_numel(p);
        CHECK(zs_plan_persistent_bytes(p) == 16 * S && zs_plan_num_tensors(p) == n);
        int64_t owned = 0, padded = 0;
        for (int32_t i = 0; i < n; ++i) {
            zs_tensor_info t;
            CHECK(zs_plan_tensor(p, i, &t) == ZS_OK);
            CHECK(t.own_lo <= t.own_hi && t.shard_off >= 0 && t.shard_off + (t.own_hi - t.own_lo) <= S);
            owned += t.own_hi - t.own_lo;
            padded += t.padded_numel;
            CHECK(zs_plan_tensor_group(p, i) >= 0 && zs_plan_tensor_replicated(p, i) >= 0);
        }
        zs_tensor_info t;
        CHECK(zs_plan_tensor(p, n, &t) == ZS_EINVAL && zs_plan_tensor(p, -1, &t) == ZS_EINVAL);
        if (o.layout == ZS_LAYOUT_FLAT) {
            CHECK(T == S * world && T % (8 * world) == 0 && owned <= S);
            CHECK(zs_plan_workspace_bytes(p) == 0);
        } else {
            CHECK(owned == S && padded == T);
            CHECK(zs_plan_workspace_bytes(p) > 0 && zs_plan_workspace_bytes(p) % 256 == 0);
        }
        zs_plan_destroy(p);
    }
}

void validation(Fake& fake) {
    char* d = fake.base();
    const int64_t numels[2] = {1000, 77};
    zs_plan* p = nullptr;
    CHECK(zs_shard_plan(numels, 2, 4, 1, 1, ZS_LAYOUT_FLAT, &p) == ZS_OK);
    const int64_t S = zs_plan_shard_numel(p);
    const void* c4[4] = {d, d + 4096, d + 8192, d + 12288};
    float* f = reinterpret_cast<float*>(d + 65536);
    zs_adamw_hparams hp{1e-3, 0.9, 0.95, 1e-8, 0.1, 1};
    const int before = zs::g_launches.load();
    CHECK(zs_reduce_shard(p, c4, 4, d, 0, S, nullptr) == ZS_OK);
    CHECK(zs_reduce_shard(p, c4, 3, d, 0, S, nullptr) == ZS_EINVAL);
    CHECK(zs_reduce_shard(p, c4, 4, d, 4, 8, nullptr) == ZS_ERANGE);
    CHECK(zs_reduce_shard(p, c4, 4, d + 2, 0, 8, nullptr) == ZS_EALIGN);
    CHECK(zs_adamw_shard_step(p, &hp, d, f, f, f, d, nullptr) == ZS_OK);
    CHECK(zs_gather_params(p, d, d, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step(p, &hp, c4, 4, f, f, f, nullptr, nullptr, d, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_bucket(p, &hp, c4, 4, f, f, f, d, d, d, 8, S - 8, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_bucket(p, &hp, c4, 4, f, f, f, d, d, d, 8, S, nullptr) == ZS_ERANGE);
    zs_adamw_hparams bad = hp;
    bad.step = 0;
    CHECK(zs_fused_shard_step(p, &bad, c4, 4, f, f, f, nullptr, nullptr, d, nullptr) == ZS_EINVAL);
    bad = hp;
    bad.lr = std::nan("");
    CHECK(zs_adamw_shard_step(p, &bad, d, f, f, f, d, nullptr) == ZS_EINVAL);
    CHECK(zs_quant_code_bytes(p, 4) == S / 2 && zs_quant_num_scales(p, 256) == (S + 255) / 256);
    CHECK(zs_quantize_shard(p, 4, 256, d, d, f, nullptr) == ZS_OK);
    CHECK(zs_quantize_shard(p, 4, 100, d, d, f, nullptr) == ZS_EINVAL);
    CHECK(zs_fused_shard_step_quant(p, &hp, c4, 4, f, f, f, nullptr, nullptr, 8, 64, d, f, nullptr) == ZS_OK);
    CHECK(zs_dequant_gather(p, 8, 64, d, f, d, nullptr) == ZS_OK);
    CHECK(zs_accumulate_shard(p, c4, 4, f, 0, S, 1, nullptr) == ZS_OK);
    const int64_t wsb = zs_grad_stats_workspace_bytes(p);
    CHECK(wsb > 0 && wsb < 60000);
    CHECK(zs_grad_stats(p, f, 2.0f, reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(d + 8), d + 4096, wsb,
                        nullptr) == ZS_OK);
    CHECK(zs_grad_stats(p, f, 2.0f, reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(d + 8), d + 4096,
                        wsb - 1, nullptr) == ZS_ENOMEM);
    CHECK(zs_grad_stats(p, f, 0.0f, reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(d + 8), d + 4096, wsb,
                        nullptr) == ZS_EINVAL);
    CHECK(zs_clip_scale(reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(d + 8), 1, 1.0, f,
                        reinterpret_cast<int32_t*>(d + 16), nullptr) == ZS_OK);
    CHECK(zs_clip_scale(reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(d + 8), 1, -1.0, f,
                        reinterpret_cast<int32_t*>(d + 16), nullptr) == ZS_EINVAL);
    CHECK(zs_adamw_shard_step_accum(p, &hp, f, 2.0f, f, nullptr, f, f, f, d, d, nullptr) == ZS_OK);
    // the same calls with the scalars in (stand-in) device memory
    zs_adamw_coefs co;
    CHECK(zs_adamw_coefs_compute(&hp, &co) == ZS_OK && co.bias_correction1 > 0.0f);
    const zs_adamw_coefs* cd = reinterpret_cast<const zs_adamw_coefs*>(d + 32768);
    CHECK(zs_fused_shard_step_dc(p, cd, c4, 4, f, f, f, nullptr, nullptr, d, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_dc(p, nullptr, c4, 4, f, f, f, nullptr, nullptr, d, nullptr) == ZS_EINVAL);
    CHECK(zs_adamw_shard_step_dc(p, cd, d, f, f, f, d, nullptr) == ZS_OK);
    CHECK(zs_adamw_shard_step_accum_dc(p, cd, f, 2.0f, nullptr, nullptr, f, f, f, d, nullptr, nullptr) == ZS_OK);
    CHECK(zs::g_launches.load() > before);
    zs_plan_destroy(p);
}

void multi_table(Fake& fake) {
    char* d = fake.base();
    const int64_t numels[5] = {4096 * 3, 512, 1000, 77, 70000};
    const int32_t groups[5] = {0, 1, 0, 1, 0};
    zs_plan_options o{ZS_LAYOUT_PER_TENSOR, 1, 600, groups};
    zs_plan* p = nullptr;
    CHECK(zs_shard_plan_ex(numels, 5, 4, 2, &o, &p) == ZS_OK);
    const int32_t n = zs_plan_num_tensors(p), N = 4;
    std::vector<zs_piece_ptrs> pieces((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        zs_tensor_info t;
        CHECK(zs_plan_tensor(p, i, &t) == ZS_OK);
        float* f = reinterpret_cast<float*>(d + 65536);
        pieces[(size_t)i] = zs_piece_ptrs{d, f, f, f, d, d + 4096};  // full offset by own_lo stays 16-B aligned
    }
    std::vector<const void*> contribs((size_t)(N * n), d);
    const int64_t need = zs_multi_workspace_bytes(p, N);
    CHECK(need > 0 && need == zs_plan_workspace_bytes(p));
    std::vector<unsigned char> ws_mem((size_t)need + 256);
    void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws_mem.data()) + 255) & ~uintptr_t(255));
    CHECK(zs_multi_bind(p, pieces.data(), contribs.data(), N, ws, need - 1, nullptr) == ZS_ENOMEM);
    CHECK(zs_multi_bind(p, pieces.data(), contribs.data(), N, ws, need, nullptr) == ZS_OK);
    // the table: header, then per-chunk piece indices that step through the pieces in order
    uint64_t magic;
    std::memcpy(&magic, ws, 8);
    CHECK(magic != 0);
    int32_t hdr[4];
    std::memcpy(hdr, static_cast<char*>(ws) + 8, sizeof hdr);
    CHECK(hdr[0] == n && hdr[2] == N);
    const int32_t n_chunks = hdr[1];
    int64_t chunks_off;
    std::memcpy(&chunks_off, static_cast<char*>(ws) + 8 + 16 + 16, 8);
    CHECK(chunks_off > 0 && chunks_off + 4 * (int64_t)n_chunks <= need);
    std::vector<int32_t> cp((size_t)n_chunks);
    std::memcpy(cp.data(), static_cast<char*>(ws) + chunks_off, 4 * (size_t)n_chunks);
    int64_t expect = 0;
    for (int32_t i = 0; i < n; ++i) {
        zs_tensor_info t;
        zs_plan_tensor(p, i, &t);
        const int64_t k = (t.own_hi - t.own_lo + 255) / 256;
        for (int64_t c = 0; c < k; ++c) CHECK(cp[(size_t)(expect + c)] == i);
        expect += k;
    }
    CHECK(expect == n_chunks);
    zs_adamw_hparams hps[2] = {{1e-3, 0.9, 0.95, 1e-8, 0.1, 1}, {1e-3, 0.9, 0.95, 1e-8, 0.0, 1}};
    CHECK(zs_fused_shard_step_multi(p, &hps[0], ws, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_multi_groups(p, hps, 2, ws, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_multi_groups(p, hps, 1, ws, nullptr) == ZS_EINVAL);  // group 1 has no hparams
    const zs_adamw_coefs* cd = reinterpret_cast<const zs_adamw_coefs*>(d + 32768);
    CHECK(zs_fused_shard_step_multi_dc(p, cd, 2, ws, nullptr) == ZS_OK);
    CHECK(zs_fused_shard_step_multi_dc(p, cd, 1, ws, nullptr) == ZS_EINVAL);
    CHECK(zs_reduce_shard_multi(p, ws, nullptr) == ZS_OK);
    CHECK(zs_adamw_shard_step_multi(p, &hps[0], ws, nullptr) == ZS_OK);
    CHECK(zs_gather_params_multi(p, ws, nullptr) == ZS_OK);
    CHECK(zs_multi_unbind(ws, nullptr) == ZS_OK);
    std::memcpy(&magic, ws, 8);
    CHECK(magic == 0);
    CHECK(zs_multi_unbind(ws, nullptr) == ZS_EINVAL);
    CHECK(zs_fused_shard_step_multi(p, &hps[0], ws, nullptr) == ZS_EINVAL);
    // a destroyed plan forgets its bindings
    CHECK(zs_multi_bind(p, pieces.data(), contribs.data(), N, ws, need, nullptr) == ZS_OK);
    zs_plan_destroy(p);
    CHECK(zs_multi_unbind(ws, nullptr) == ZS_EINVAL);
}

void host_adamw(std::mt19937_64& rng) {
    zs_adamw_hparams hp{2e-4, 0.9, 0.95, 1e-8, 0.1, 3};
    for (int64_t n : {0, 1, 15, 16, 17, 1000, 100003}) {
        std::vector<uint16_t> g((size_t)n + 8);
        std::vector<float> w0((size_t)n + 4), m0((size_t)n + 4), v0((size_t)n + 4);
        for (int64_t j = 0; j < n; ++j) {
            g[(size_t)j] = (uint16_t)(rng() & 0xFFFF);
            w0[(size_t)j] = (float)((int64_t)(rng() % 2001) - 1000) * 1e-4f;
            m0[(size_t)j] = (float)((int64_t)(rng() % 2001) - 1000) * 1e-6f;
            v0[(size_t)j] = (float)(rng() % 1000) * 1e-9f;
        }
        std::vector<float> w1 = w0, m1 = m0, v1 = v0;
        std::vector<uint16_t> p1((size_t)n + 8);
        CHECK(zs_host_adamw_step(&hp, g.data(), w1.data(), m1.data(), v1.data(), p1.data(), n, 1) == ZS_OK);
        for (int32_t threads : {2, 3, 8, 16}) {
            std::vector<float> w = w0, m = m0, v = v0;
            std::vector<uint16_t> p((size_t)n + 8);
            CHECK(zs_host_adamw_step(&hp, g.data(), w.data(), m.data(), v.data(), p.data(), n, threads) == ZS_OK);
            CHECK(std::memcmp(w.data(), w1.data(), 4 * (size_t)n) == 0);
            CHECK(std::memcmp(m.data(), m1.data(), 4 * (size_t)n) == 0);
            CHECK(std::memcmp(v.data(), v1.data(), 4 * (size_t)n) == 0);
            CHECK(std::memcmp(p.data(), p1.data(), 2 * (size_t)n) == 0);
        }
    }
    std::vector<float> f(64);
    std::vector<uint16_t> h(64);
    CHECK(zs_host_adamw_step(&hp, h.data(), f.data(), f.data(), f.data(), nullptr, 16, 0) == ZS_EINVAL);
    CHECK(zs_host_adamw_step(&hp, h.data(), f.data(), f.data(), f.data(), nullptr, -1, 1) == ZS_EINVAL);
}

void concurrent_callers() {
    std::vector<std::thread> th;
    std::atomic<int> failures{0};
    for (int i = 0; i < 8; ++i) {
        th.emplace_back([i, &failures] {
            std::mt19937_64 rng(1000 + (uint64_t)i);
            for (int rep = 0; rep < 50; ++rep) {
                const int64_t numels[1] = {16};
                zs_plan* p = nullptr;
                const int32_t bad_rank = 1000 + 100 * i + rep;
                if (zs_shard_plan(numels, 1, 4, bad_rank, 1, ZS_LAYOUT_FLAT, &p) != ZS_EINVAL) ++failures;
                const std::string want = "rank = " + std::to_string(bad_rank);
                if (std::string(zs_last_error()).find(want) == std::string::npos) ++failures;
                random_plans(rng, 2);
            }
            zs_adamw_hparams hp{1e-3, 0.9, 0.95, 1e-8, 0.1, 1};
            std::vector<uint16_t> g(20000, 0x3C00);
            std::vector<float> w(20000, 0.5f), m(20000), v(20000);
            if (zs_host_adamw_step(&hp, g.data(), w.data(), m.data(), v.data(), nullptr, 20000, 4) != ZS_OK)
                ++failures;
        });
    }
    for (auto& t : th) t.join();
    CHECK(failures.load() == 0);
}

}  // namespace

int main(int argc, char** argv) {
    const std::string mode = argc > 1 ? argv[1] : "all";
    std::mt19937_64 rng(7);
    Fake fake;
    if (mode == "all") {
        random_plans(rng, 400);
        validation(fake);
        multi_table(fake);
        host_adamw(rng);
    }
    concurrent_callers();
    std::printf("host driver ok (%s)\n", mode.c_str());
    return 0;
}
