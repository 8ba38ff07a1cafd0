// Host side of the C ABI: shard plan, argument validation, error reporting
// and the multi-tensor workspace binding. Every device-touching entry point
// validates all of its arguments before it enqueues anything.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "zs_internal.h"

namespace {

thread_local std::string g_err;

zs_status fail(zs_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

constexpr int64_t kMaxElems = int64_t(1) << 60;
// Largest owned shard: 2^34 - 256 elements. A kernel launch covers at most
// 2^32 - 1 work-items and the step kernels give each work-item 4 elements
// (16 B/param of state alone is then 256 GiB: about all one MI355X holds).
constexpr int64_t kMaxShardElems = (int64_t(1) << 34) - 256;

int64_t roundup(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

zs_status check_ptr(const void* p, const char* what) {
    if (!p) return fail(ZS_EINVAL, "%s is NULL", what);
    if (!aligned16(p)) return fail(ZS_EALIGN, "%s (%p) is not 16-byte aligned", what, p);
    return ZS_OK;
}

zs_status check_opt_ptr(const void* p, const char* what) { return p ? check_ptr(p, what) : ZS_OK; }

zs_status check_plan(const zs_plan* plan) {
    if (!plan) return fail(ZS_EINVAL, "plan is NULL");
    return ZS_OK;
}

zs_status check_hp(const zs_adamw_hparams* hp) {
    if (!hp) return fail(ZS_EINVAL, "hparams is NULL");
    const double v[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
    for (double x : v)
        if (!std::isfinite(x)) return fail(ZS_EINVAL, "hparams hold a non-finite value");
    if (hp->beta1 < 0.0 || hp->beta1 >= 1.0 || hp->beta2 < 0.0 || hp->beta2 >= 1.0)
        return fail(ZS_EINVAL, "beta1 = %g and beta2 = %g must lie in [0, 1)", hp->beta1, hp->beta2);
    if (hp->eps < 0.0) return fail(ZS_EINVAL, "eps = %g is negative", hp->eps);
    if (hp->step < 1) return fail(ZS_EINVAL, "step = %lld, the first AdamW step is 1", (long long)hp->step);
    return ZS_OK;
}

// A device pointer to zs_adamw_coefs scalars.
zs_status check_coefs(const zs_adamw_coefs* coefs) {
    if (!coefs) return fail(ZS_EINVAL, "coefs is NULL");
    if (reinterpret_cast<uintptr_t>(coefs) & 3) return fail(ZS_EALIGN, "coefs must be 4-byte aligned");
    return ZS_OK;
}

zs_status check_contribs(const zs_plan* plan, const void* const* contribs, int32_t n) {
    if (!contribs) return fail(ZS_EINVAL, "contribs is NULL");
    if (n < 1 || n > ZS_MAX_CONTRIBS)
        return fail(ZS_EINVAL, "n_contribs = %d outside [1, %d]", n, ZS_MAX_CONTRIBS);
    if (n % plan->world != 0)
        return fail(ZS_EINVAL, "n_contribs = %d is not a multiple of the plan's world size %d", n, plan->world);
    for (int32_t q = 0; q < n; ++q) {
        if (!contribs[q]) return fail(ZS_EINVAL, "contribs[%d] is NULL (no contribution from rank %d)", q, q);
        if (!aligned16(contribs[q])) return fail(ZS_EALIGN, "contribs[%d] is not 16-byte aligned", q);
    }
    return ZS_OK;
}

// Per-call trace, on when ZS_LOG is set (and not "0"): one line on stderr for
// every call that enqueues work, with a process-wide sequence number, the
// entry point, the plan's world size and rank, the contributions and the
// range it covers, and the stream -- enough to line a stuck or failing step
// up with the other ranks' logs.
bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("ZS_LOG");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}

std::atomic<uint64_t> g_seq{0};

void trace(const char* op, const zs_plan* p, int32_t n_contribs, int64_t off, int64_t len, const void* stream) {
    if (!log_enabled()) return;
    std::fprintf(stderr, "zs %llu %s world=%d rank=%d contribs=%d off=%lld len=%lld stream=%p\n",
                 (unsigned long long)++g_seq, op, p ? p->world : -1, p ? p->rank : -1, n_contribs, (long long)off,
                 (long long)len, stream);
}

zs_status hip_status(int err, const char* what) {
    if (err == 0) return ZS_OK;
    return fail(ZS_EHIP, "%s: HIP error %d (%s)", what, err, zs::hip_error_text(err));
}

// Registry of bound multi-tensor workspaces: which plan and which fields.
struct Binding {
    const zs_plan* plan;
    int32_t flags;
    int32_t n_contribs;
};
std::mutex g_bind_mu;
std::unordered_map<const void*, Binding> g_bind;

}  // namespace

namespace zs {

AdamCoef make_coef(const zs_adamw_hparams& hp) {
    AdamCoef c;
    c.b1 = (float)hp.beta1;
    c.omb1 = (float)(1.0 - hp.beta1);
    c.b2 = (float)hp.beta2;
    c.omb2 = (float)(1.0 - hp.beta2);
    c.lr = (float)hp.lr;
    c.eps = (float)hp.eps;
    c.decay = (float)(1.0 - hp.lr * hp.weight_decay);
    c.bc1 = (float)(1.0 - std::pow(hp.beta1, (double)hp.step));
    c.bc2 = (float)(1.0 - std::pow(hp.beta2, (double)hp.step));
    return c;
}

}  // namespace zs

extern "C" {

const char* zs_last_error(void) { return g_err.c_str(); }

const char* zs_version(void) { return "0.1.0"; }

// ------------------------------------------------------------------ plan

zs_status zs_shard_plan_ex(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t rank,
                           const zs_plan_options* opt, zs_plan** out) {
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    if (!opt) return fail(ZS_EINVAL, "options is NULL");
    const int32_t layout = opt->layout;
    const int32_t tensor_align_elems = opt->tensor_align_elems;
    if (n_tensors < 0) return fail(ZS_EINVAL, "n_tensors = %d is negative", n_tensors);
    if (n_tensors > 0 && !numels) return fail(ZS_EINVAL, "numels is NULL");
    if (world_size < 1) return fail(ZS_EINVAL, "world_size = %d must be >= 1", world_size);
    if (rank < 0 || rank >= world_size)
        return fail(ZS_EINVAL, "rank = %d outside [0, %d)", rank, world_size);
    if (layout != ZS_LAYOUT_FLAT && layout != ZS_LAYOUT_PER_TENSOR)
        return fail(ZS_EINVAL, "unknown layout %d", layout);
    if (layout == ZS_LAYOUT_FLAT && tensor_align_elems < 1)
        return fail(ZS_EINVAL, "tensor_align_elems = %d must be >= 1", tensor_align_elems);
    if (opt->persist_below_elems < 0) return fail(ZS_EINVAL, "persist_below_elems is negative");
    if (layout == ZS_LAYOUT_FLAT && (opt->persist_below_elems > 0 || opt->groups))
        return fail(ZS_EINVAL, "a persistence threshold and groups need a PER_TENSOR plan");
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0 || numels[i] > kMaxElems)
            return fail(ZS_EINVAL, "numels[%d] = %lld out of range", i, (long long)numels[i]);
        if (opt->groups && (opt->groups[i] < 0 || opt->groups[i] >= ZS_MAX_GROUPS))
            return fail(ZS_EINVAL, "groups[%d] = %d outside [0, %d)", i, opt->groups[i], ZS_MAX_GROUPS);
    }

    zs_plan* p = new (std::nothrow) zs_plan();
    if (!p) return fail(ZS_ENOMEM, "out of host memory");
    p->layout = layout;
    p->world = world_size;
    p->rank = rank;
    p->align = layout == ZS_LAYOUT_FLAT ? tensor_align_elems : 1;
    const int64_t granule = int64_t(8) * world_size;  // N shards of whole 16-byte vectors
    try {
        p->tensors.resize((size_t)n_tensors);
        if (layout == ZS_LAYOUT_FLAT) {
            int64_t end = 0;
            for (int32_t i = 0; i < n_tensors; ++i) {
                zs::TensorEntry& t = p->tensors[(size_t)i];
                t.numel = numels[i];
                t.flat_off = roundup(end, p->align);
                t.padded = t.numel;
                end = t.flat_off + t.numel;
                if (end > kMaxElems) {
                    delete p;
                    return fail(ZS_EINVAL, "flat buffer exceeds 2^60 elements");
                }
            }
            p->T = roundup(end, granule);
            p->S = p->T / world_size;
            const int64_t lo = (int64_t)rank * p->S, hi = lo + p->S;
            for (auto& t : p->tensors) {
                const int64_t a = std::max(t.flat_off, lo), b = std::min(t.flat_off + t.numel, hi);
                if (a < b) {
                    t.own_lo = a - t.flat_off;
                    t.own_hi = b - t.flat_off;
                    t.shard_off = a - lo;
                } else {
                    t.own_lo = t.own_hi = 0;
                    t.shard_off = std::min(std::max(t.flat_off - lo, int64_t(0)), p->S);
                }
            }
        } else {
            int64_t full = 0, shard = 0;
            for (int32_t i = 0; i < n_tensors; ++i) {
                zs::TensorEntry& t = p->tensors[(size_t)i];
                t.numel = numels[i];
                t.group = opt->groups ? opt->groups[i] : 0;
                t.replicated = t.numel < opt->persist_below_elems ? 1 : 0;
                t.flat_off = full;
                int64_t Si;
                if (t.replicated) {
                    t.padded = roundup(t.numel, 8);
                    Si = t.padded;
                    t.own_lo = 0;
                } else {
                    t.padded = roundup(t.numel, granule);
                    Si = t.padded / world_size;
                    t.own_lo = (int64_t)rank * Si;
                }
                t.own_hi = t.own_lo + Si;
                t.shard_off = shard;
                full += t.padded;
                shard += Si;
                if (full > kMaxElems) {
                    delete p;
                    return fail(ZS_EINVAL, "packed buffer exceeds 2^60 elements");
                }
            }
            p->T = full;
            p->S = shard;
            if (shard > kMaxShardElems) {  // checked before the chunk list is built
                delete p;
                return fail(ZS_EINVAL, "owned shard of %lld elements exceeds the limit of 2^34 - 256",
                            (long long)shard);
            }
            int64_t n_chunks = 0;
            for (auto& t : p->tensors) {
                t.first_chunk = n_chunks;
                n_chunks += (t.own_hi - t.own_lo + zs::kChunkElems - 1) / zs::kChunkElems;
            }
            // one block per chunk: the launch's work-items must stay below 2^32
            if (n_chunks > (int64_t)UINT32_MAX / zs::kBlockThreads) {
                delete p;
                return fail(ZS_EINVAL, "%lld multi-tensor chunks exceed one launch", (long long)n_chunks);
            }
            p->chunk_piece.reserve((size_t)n_chunks);
            for (int32_t i = 0; i < n_tensors; ++i) {
                const zs::TensorEntry& t = p->tensors[(size_t)i];
                for (int64_t c = 0; c < t.own_hi - t.own_lo; c += zs::kChunkElems) p->chunk_piece.push_back(i);
            }
        }
    } catch (const std::bad_alloc&) {
        delete p;
        return fail(ZS_ENOMEM, "out of host memory");
    }
    if (p->S > kMaxShardElems) {
        const long long S = (long long)p->S;
        delete p;
        return fail(ZS_EINVAL, "owned shard of %lld elements exceeds the limit of 2^34 - 256", S);
    }
    *out = p;
    return ZS_OK;
}

zs_status zs_shard_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t rank,
                        int32_t tensor_align_elems, int32_t layout, zs_plan** out) {
    zs_plan_options o;
    o.layout = layout;
    o.tensor_align_elems = tensor_align_elems;
    o.persist_below_elems = 0;
    o.groups = nullptr;
    return zs_shard_plan_ex(numels, n_tensors, world_size, rank, &o, out);
}

int32_t zs_plan_tensor_group(const zs_plan* p, int32_t i) {
    if (!p || i < 0 || i >= (int32_t)p->tensors.size()) return -1;
    return p->tensors[(size_t)i].group;
}

int32_t zs_plan_tensor_replicated(const zs_plan* p, int32_t i) {
    if (!p || i < 0 || i >= (int32_t)p->tensors.size()) return -1;
    return p->tensors[(size_t)i].replicated;
}

void zs_plan_destroy(zs_plan* plan) {
    if (!plan) return;
    {
        std::lock_guard<std::mutex> lk(g_bind_mu);
        for (auto it = g_bind.begin(); it != g_bind.end();)
            it = it->second.plan == plan ? g_bind.erase(it) : std::next(it);
    }
    delete plan;
}

int64_t zs_plan_padded_numel(const zs_plan* p) { return p ? p->T : -1; }
int64_t zs_plan_shard_numel(const zs_plan* p) { return p ? p->S : -1; }
int64_t zs_plan_persistent_bytes(const zs_plan* p) { return p ? 16 * p->S : -1; }
int32_t zs_plan_num_tensors(const zs_plan* p) { return p ? (int32_t)p->tensors.size() : -1; }
int32_t zs_plan_world_size(const zs_plan* p) { return p ? p->world : -1; }
int32_t zs_plan_rank(const zs_plan* p) { return p ? p->rank : -1; }
int32_t zs_plan_layout(const zs_plan* p) { return p ? p->layout : -1; }

zs_status zs_plan_tensor(const zs_plan* p, int32_t i, zs_tensor_info* out) {
    if (zs_status st = check_plan(p)) return st;
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    if (i < 0 || i >= (int32_t)p->tensors.size())
        return fail(ZS_EINVAL, "tensor index %d outside [0, %zu)", i, p->tensors.size());
    const zs::TensorEntry& t = p->tensors[(size_t)i];
    out->numel = t.numel;
    out->flat_off = t.flat_off;
    out->padded_numel = t.padded;
    out->own_lo = t.own_lo;
    out->own_hi = t.own_hi;
    out->shard_off = t.shard_off;
    return ZS_OK;
}

// ------------------------------------------------------------------ flat step

zs_status zs_reduce_shard(const zs_plan* plan, const void* const* contribs, int32_t n_contribs,
                          void* grad_bf16, int64_t off, int64_t len, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_contribs(plan, contribs, n_contribs)) return st;
    if (zs_status st = check_ptr(grad_bf16, "grad_bf16")) return st;
    if (off < 0 || len < 0 || off % 8 || len % 8 || off > plan->S || len > plan->S - off)
        return fail(ZS_ERANGE, "bucket [%lld, %lld) must be multiples of 8 inside the shard [0, %lld)",
                    (long long)off, (long long)(off + len), (long long)plan->S);
    if (len == 0) return ZS_OK;
    const void* shifted[ZS_MAX_CONTRIBS];
    for (int32_t q = 0; q < n_contribs; ++q) shifted[q] = static_cast<const char*>(contribs[q]) + 2 * off;
    trace("zs_reduce_shard", plan, n_contribs, off, len, stream);
    return hip_status(zs::launch_reduce(shifted, n_contribs, static_cast<char*>(grad_bf16) + 2 * off, len, stream),
                      "reduce launch");
}

namespace {

// The AdamW calls below, after their scalars were validated: by value (c) or
// in device memory (cdev).
zs_status adamw_impl(const zs_plan* plan, const zs::AdamCoef& c, const zs::AdamCoef* cdev, const void* grad_bf16,
                     float* master, float* m, float* v, void* param_bf16, void* stream) {
    if (zs_status st = check_ptr(grad_bf16, "grad_bf16")) return st;
    if (zs_status st = check_ptr(master, "master")) return st;
    if (zs_status st = check_ptr(m, "m")) return st;
    if (zs_status st = check_ptr(v, "v")) return st;
    if (zs_status st = check_ptr(param_bf16, "param_bf16")) return st;
    if (plan->S == 0) return ZS_OK;
    trace(cdev ? "zs_adamw_shard_step_dc" : "zs_adamw_shard_step", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_adamw(c, grad_bf16, master, m, v, param_bf16, nullptr, plan->S, stream, nullptr, cdev),
                      "adamw launch");
}

const zs::AdamCoef* dev_coef(const zs_adamw_coefs* coefs) { return reinterpret_cast<const zs::AdamCoef*>(coefs); }

}  // namespace

zs_status zs_adamw_shard_step(const zs_plan* plan, const zs_adamw_hparams* hp, const void* grad_bf16,
                              float* master, float* m, float* v, void* param_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    return adamw_impl(plan, zs::make_coef(*hp), nullptr, grad_bf16, master, m, v, param_bf16, stream);
}

zs_status zs_adamw_shard_step_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const void* grad_bf16,
                                 float* master, float* m, float* v, void* param_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_coefs(coefs)) return st;
    return adamw_impl(plan, zs::AdamCoef{}, dev_coef(coefs), grad_bf16, master, m, v, param_bf16, stream);
}

zs_status zs_adamw_coefs_compute(const zs_adamw_hparams* hp, zs_adamw_coefs* out) {
    if (zs_status st = check_hp(hp)) return st;
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    const zs::AdamCoef c = zs::make_coef(*hp);
    *out = zs_adamw_coefs{c.b1, c.omb1, c.b2, c.omb2, c.lr, c.eps, c.decay, c.bc1, c.bc2};
    return ZS_OK;
}

zs_status zs_gather_params(const zs_plan* plan, const void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (plan->layout != ZS_LAYOUT_FLAT)
        return fail(ZS_EINVAL, "zs_gather_params needs a FLAT plan; PER_TENSOR plans gather through "
                               "zs_gather_params_multi");
    if (zs_status st = check_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_ptr(full_bf16, "full_bf16")) return st;
    if (plan->S == 0) return ZS_OK;
    char* own = static_cast<char*>(full_bf16) + 2 * (int64_t)plan->rank * plan->S;
    trace("zs_gather_params", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_gather(param_bf16, own, plan->S, stream), "gather launch");
}

// ------------------------------------------------------------------ resharding to a smaller group

namespace {

zs_status check_group(const zs_plan* plan, int32_t k) {
    if (zs_status st = check_plan(plan)) return st;
    if (plan->layout != ZS_LAYOUT_FLAT) return fail(ZS_EINVAL, "reshard slices need a FLAT plan");
    if (k < 1 || k > plan->world || plan->world % k)
        return fail(ZS_EINVAL, "reshard group size %d must divide the world size %d", k, plan->world);
    return ZS_OK;
}

zs_reshard_slice make_slice(const zs_plan* plan, int32_t k) {
    const int32_t per_slice = plan->world / k;
    const int64_t len = plan->T / k;
    zs_reshard_slice s{};
    s.group_size = k;
    s.slice_index = plan->rank % k;
    s.slice_off = (int64_t)s.slice_index * len;
    s.slice_len = len;
    s.first_source = s.slice_index * per_slice;
    s.n_sources = per_slice;
    s.owner_slice = plan->rank / per_slice;
    s.reserved = 0;
    s.own_off = (int64_t)(plan->rank % per_slice) * plan->S;
    s.retained_bytes = 2 * len;
    return s;
}

}  // namespace

zs_status zs_plan_reshard_slice(const zs_plan* plan, int32_t group_size, zs_reshard_slice* out) {
    if (zs_status st = check_group(plan, group_size)) return st;
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    *out = make_slice(plan, group_size);
    return ZS_OK;
}

zs_status zs_gather_params_to_slice(const zs_plan* plan, int32_t group_size, const void* param_bf16,
                                    void* slice_bf16, void* stream) {
    if (zs_status st = check_group(plan, group_size)) return st;
    if (zs_status st = check_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_ptr(slice_bf16, "slice_bf16")) return st;
    if (plan->S == 0) return ZS_OK;
    const zs_reshard_slice s = make_slice(plan, group_size);
    char* own = static_cast<char*>(slice_bf16) + 2 * s.own_off;
    trace("zs_gather_params_to_slice", plan, 0, s.own_off, plan->S, stream);
    return hip_status(zs::launch_gather(param_bf16, own, plan->S, stream), "gather launch");
}

zs_status zs_gather_slice(const zs_plan* plan, int32_t group_size, const void* const* shards, int32_t n_shards,
                          void* slice_bf16, void* stream) {
    if (zs_status st = check_group(plan, group_size)) return st;
    const int32_t need = plan->world / group_size;
    if (!shards) return fail(ZS_EINVAL, "shards is NULL");
    if (n_shards != need)
        return fail(ZS_EINVAL, "a slice of a %d-rank group is %d shards, got %d", group_size, need, n_shards);
    for (int32_t i = 0; i < n_shards; ++i) {
        char what[32];
        std::snprintf(what, sizeof what, "shards[%d]", i);
        if (zs_status st = check_ptr(shards[i], what)) return st;
    }
    if (zs_status st = check_ptr(slice_bf16, "slice_bf16")) return st;
    if (plan->S == 0) return ZS_OK;
    trace("zs_gather_slice", plan, n_shards, 0, plan->T / group_size, stream);
    return hip_status(zs::launch_gather_sources(shards, n_shards, slice_bf16, plan->S, stream), "gather launch");
}

zs_status zs_fused_shard_step(const zs_plan* plan, const zs_adamw_hparams* hp, const void* const* contribs,
                              int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                              void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    return zs_fused_shard_step_bucket(plan, hp, contribs, n_contribs, master, m, v, grad_bf16, param_bf16, full_bf16,
                                      0, plan->S, stream);
}

namespace {

zs_status fused_impl(const zs_plan* plan, const zs::AdamCoef& c, const zs::AdamCoef* cdev,
                     const void* const* contribs, int32_t n_contribs, float* master, float* m, float* v,
                     void* grad_bf16, void* param_bf16, void* full_bf16, int64_t off, int64_t len, void* stream);

}  // namespace

zs_status zs_fused_shard_step_bucket(const zs_plan* plan, const zs_adamw_hparams* hp, const void* const* contribs,
                                     int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                                     void* param_bf16, void* full_bf16, int64_t off, int64_t len, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    return fused_impl(plan, zs::make_coef(*hp), nullptr, contribs, n_contribs, master, m, v, grad_bf16, param_bf16,
                      full_bf16, off, len, stream);
}

zs_status zs_fused_shard_step_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const void* const* contribs,
                                 int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                                 void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_coefs(coefs)) return st;
    return fused_impl(plan, zs::AdamCoef{}, dev_coef(coefs), contribs, n_contribs, master, m, v, grad_bf16,
                      param_bf16, full_bf16, 0, plan->S, stream);
}

namespace {

zs_status fused_impl(const zs_plan* plan, const zs::AdamCoef& c, const zs::AdamCoef* cdev,
                     const void* const* contribs, int32_t n_contribs, float* master, float* m, float* v,
                     void* grad_bf16, void* param_bf16, void* full_bf16, int64_t off, int64_t len, void* stream) {
    if (zs_status st = check_contribs(plan, contribs, n_contribs)) return st;
    if (zs_status st = check_ptr(master, "master")) return st;
    if (zs_status st = check_ptr(m, "m")) return st;
    if (zs_status st = check_ptr(v, "v")) return st;
    if (zs_status st = check_opt_ptr(grad_bf16, "grad_bf16")) return st;
    if (zs_status st = check_opt_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_opt_ptr(full_bf16, "full_bf16")) return st;
    if (full_bf16 && plan->layout != ZS_LAYOUT_FLAT)
        return fail(ZS_EINVAL, "a gather into full_bf16 needs a FLAT plan; PER_TENSOR plans use "
                               "zs_fused_shard_step_multi");
    if (off < 0 || len < 0 || off % 8 || len % 8 || off > plan->S || len > plan->S - off)
        return fail(ZS_ERANGE, "bucket [%lld, %lld) must be multiples of 8 inside the shard [0, %lld)",
                    (long long)off, (long long)(off + len), (long long)plan->S);
    if (len == 0) return ZS_OK;
    const void* shifted[ZS_MAX_CONTRIBS];
    for (int32_t q = 0; q < n_contribs; ++q) shifted[q] = static_cast<const char*>(contribs[q]) + 2 * off;
    auto at16 = [off](void* p) { return p ? static_cast<void*>(static_cast<char*>(p) + 2 * off) : nullptr; };
    char* own = full_bf16 ? static_cast<char*>(full_bf16) + 2 * ((int64_t)plan->rank * plan->S + off) : nullptr;
    trace(cdev ? "zs_fused_shard_step_dc" : "zs_fused_shard_step", plan, n_contribs, off, len, stream);
    return hip_status(zs::launch_fused(c, shifted, n_contribs, master + off, m + off, v + off, at16(grad_bf16),
                                       at16(param_bf16), own, len, stream, nullptr, cdev),
                      "fused launch");
}

}  // namespace

// ------------------------------------------------------------------ quantized parameter gather

namespace {

bool quant_spec_ok(int32_t bits, int32_t block) {
    return (bits == 4 || bits == 8) && block >= zs::kQuantMinBlock && block <= zs::kQuantMaxBlock &&
           (block & (block - 1)) == 0;
}

zs_status check_quant(const zs_plan* plan, int32_t bits, int32_t block) {
    if (zs_status st = check_plan(plan)) return st;
    if (plan->layout != ZS_LAYOUT_FLAT) return fail(ZS_EINVAL, "the quantized gather needs a FLAT plan");
    if (!quant_spec_ok(bits, block))
        return fail(ZS_EINVAL, "bits = %d must be 4 or 8 and block = %d a power of two in [%d, %d]", bits, block,
                    zs::kQuantMinBlock, zs::kQuantMaxBlock);
    return ZS_OK;
}

}  // namespace

int64_t zs_quant_code_bytes(const zs_plan* plan, int32_t bits) {
    if (!plan || (bits != 4 && bits != 8)) return -1;
    return plan->S * bits / 8;
}

int64_t zs_quant_num_scales(const zs_plan* plan, int32_t block) {
    if (!plan || !quant_spec_ok(8, block)) return -1;
    return (plan->S + block - 1) / block;
}

zs_status zs_quantize_shard(const zs_plan* plan, int32_t bits, int32_t block, const void* param_bf16, void* codes,
                            float* scales, void* stream) {
    if (zs_status st = check_quant(plan, bits, block)) return st;
    if (zs_status st = check_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_ptr(codes, "codes")) return st;
    if (zs_status st = check_ptr(scales, "scales")) return st;
    if (plan->S == 0) return ZS_OK;
    const zs::QuantOut q{codes, scales, bits, block};
    trace("zs_quantize_shard", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_quantize(q, param_bf16, plan->S, stream), "quantize launch");
}

zs_status zs_fused_shard_step_quant(const zs_plan* plan, const zs_adamw_hparams* hp, const void* const* contribs,
                                    int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                                    void* param_bf16, int32_t bits, int32_t block, void* codes, float* scales,
                                    void* stream) {
    if (zs_status st = check_quant(plan, bits, block)) return st;
    if (zs_status st = check_hp(hp)) return st;
    if (zs_status st = check_contribs(plan, contribs, n_contribs)) return st;
    if (zs_status st = check_ptr(master, "master")) return st;
    if (zs_status st = check_ptr(m, "m")) return st;
    if (zs_status st = check_ptr(v, "v")) return st;
    if (zs_status st = check_opt_ptr(grad_bf16, "grad_bf16")) return st;
    if (zs_status st = check_opt_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_ptr(codes, "codes")) return st;
    if (zs_status st = check_ptr(scales, "scales")) return st;
    if (plan->S == 0) return ZS_OK;
    const zs::QuantOut q{codes, scales, bits, block};
    trace("zs_fused_shard_step_quant", plan, n_contribs, 0, plan->S, stream);
    return hip_status(zs::launch_fused(zs::make_coef(*hp), contribs, n_contribs, master, m, v, grad_bf16, param_bf16,
                                       nullptr, plan->S, stream, &q),
                      "fused quantized launch");
}

zs_status zs_dequant_gather(const zs_plan* plan, int32_t bits, int32_t block, const void* codes_all,
                            const float* scales_all, void* full_bf16, void* stream) {
    if (zs_status st = check_quant(plan, bits, block)) return st;
    if (zs_status st = check_ptr(codes_all, "codes_all")) return st;
    if (zs_status st = check_ptr(scales_all, "scales_all")) return st;
    if (zs_status st = check_ptr(full_bf16, "full_bf16")) return st;
    if (plan->S == 0) return ZS_OK;
    if ((plan->S / 8 + zs::kBlockThreads - 1) / zs::kBlockThreads > INT32_MAX)
        return fail(ZS_EINVAL, "shard of %lld elements is too long for one dequantizing launch", (long long)plan->S);
    if (plan->world > 65535)  // one launch row per rank: the grid's second dimension
        return fail(ZS_EINVAL, "the dequantizing gather handles at most 65535 ranks, the plan has %d", plan->world);
    trace("zs_dequant_gather", plan, plan->world, 0, plan->S, stream);
    return hip_status(zs::launch_dequant(bits, block, codes_all, scales_all, zs_quant_code_bytes(plan, bits),
                                         zs_quant_num_scales(plan, block), plan->world, full_bf16, plan->S, stream),
                      "dequantize launch");
}

// ------------------------------------------------------------------ CPU-offloaded optimizer step

namespace {

constexpr int32_t kMaxHostThreads = 256;

zs_status check_host_threads(int32_t n_threads) {
    if (n_threads < 1 || n_threads > kMaxHostThreads)
        return fail(ZS_EINVAL, "n_threads = %d outside [1, %d]", n_threads, kMaxHostThreads);
    return ZS_OK;
}

}  // namespace

zs_status zs_host_adamw_step(const zs_adamw_hparams* hp, const void* grad_bf16, float* master, float* m, float* v,
                             void* param_bf16, int64_t n, int32_t n_threads) {
    if (zs_status st = check_hp(hp)) return st;
    if (n < 0) return fail(ZS_EINVAL, "n = %lld is negative", (long long)n);
    if (zs_status st = check_host_threads(n_threads)) return st;
    if (zs_status st = check_ptr(grad_bf16, "grad_bf16")) return st;
    if (zs_status st = check_ptr(master, "master")) return st;
    if (zs_status st = check_ptr(m, "m")) return st;
    if (zs_status st = check_ptr(v, "v")) return st;
    if (zs_status st = check_opt_ptr(param_bf16, "param_bf16")) return st;
    zs::host_adamw(zs::make_coef(*hp), static_cast<const uint16_t*>(grad_bf16), master, m, v,
                   static_cast<uint16_t*>(param_bf16), n, n_threads);
    return ZS_OK;
}

zs_status zs_offload_adamw_step(const zs_plan* plan, const zs_adamw_hparams* hp, const void* grad_bf16_dev,
                                float* master_host, float* m_host, float* v_host, void* grad_bf16_host,
                                void* param_bf16_host, void* param_bf16_dev, void* full_bf16_dev, int64_t chunk_elems,
                                int32_t n_threads, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    if (zs_status st = check_host_threads(n_threads)) return st;
    if (chunk_elems < 1024 || chunk_elems % 8)
        return fail(ZS_EINVAL, "chunk_elems = %lld must be a multiple of 8, at least 1024", (long long)chunk_elems);
    if (zs_status st = check_ptr(grad_bf16_dev, "grad_bf16_dev")) return st;
    if (zs_status st = check_ptr(master_host, "master_host")) return st;
    if (zs_status st = check_ptr(m_host, "m_host")) return st;
    if (zs_status st = check_ptr(v_host, "v_host")) return st;
    if (zs_status st = check_ptr(grad_bf16_host, "grad_bf16_host")) return st;
    if (zs_status st = check_ptr(param_bf16_host, "param_bf16_host")) return st;
    if (zs_status st = check_opt_ptr(param_bf16_dev, "param_bf16_dev")) return st;
    if (zs_status st = check_opt_ptr(full_bf16_dev, "full_bf16_dev")) return st;
    if (full_bf16_dev && plan->layout != ZS_LAYOUT_FLAT)
        return fail(ZS_EINVAL, "a gather into full_bf16_dev needs a FLAT plan");
    if (plan->S == 0) return ZS_OK;
    if (!zs::is_pinned_host(grad_bf16_host) || !zs::is_pinned_host(param_bf16_host))
        return fail(ZS_EINVAL, "grad_bf16_host and param_bf16_host must be page-locked host memory "
                               "(hipHostMalloc, or a pinned tensor)");
    char* own = full_bf16_dev ? static_cast<char*>(full_bf16_dev) + 2 * (int64_t)plan->rank * plan->S : nullptr;
    trace("zs_offload_adamw_step", plan, 0, 0, plan->S, stream);
    return hip_status(zs::offload_adamw(zs::make_coef(*hp), grad_bf16_dev, master_host, m_host, v_host,
                                        grad_bf16_host, param_bf16_host, param_bf16_dev, own, plan->S, chunk_elems,
                                        n_threads, stream),
                      "offloaded step");
}

// ------------------------------------------------------------------ accumulation and clipping

zs_status zs_accumulate_shard(const zs_plan* plan, const void* const* contribs, int32_t n_contribs, float* acc_f32,
                              int64_t off, int64_t len, int32_t first, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_contribs(plan, contribs, n_contribs)) return st;
    if (zs_status st = check_ptr(acc_f32, "acc_f32")) return st;
    if (off < 0 || len < 0 || off % 8 || len % 8 || off > plan->S || len > plan->S - off)
        return fail(ZS_ERANGE, "bucket [%lld, %lld) must be multiples of 8 inside the shard [0, %lld)",
                    (long long)off, (long long)(off + len), (long long)plan->S);
    if (len == 0) return ZS_OK;
    const void* shifted[ZS_MAX_CONTRIBS];
    for (int32_t q = 0; q < n_contribs; ++q) shifted[q] = static_cast<const char*>(contribs[q]) + 2 * off;
    trace("zs_accumulate_shard", plan, n_contribs, off, len, stream);
    return hip_status(zs::launch_accumulate(shifted, n_contribs, acc_f32 + off, first ? 1 : 0, len, stream),
                      "accumulate launch");
}

int64_t zs_grad_stats_workspace_bytes(const zs_plan* plan) {
    if (!plan) return -1;
    const int64_t nb = (plan->S + zs::kStatsChunk - 1) / zs::kStatsChunk;
    return roundup(nb * 8, 256) + roundup(nb * 4, 256) + 256;
}

zs_status zs_grad_stats(const zs_plan* plan, const float* acc_f32, float grad_divisor, double* sumsq_out,
                        int32_t* nonfinite_out, void* workspace, int64_t workspace_bytes, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_ptr(acc_f32, "acc_f32")) return st;
    if (!std::isfinite(grad_divisor) || grad_divisor == 0.0f)
        return fail(ZS_EINVAL, "grad_divisor = %g must be finite and nonzero", (double)grad_divisor);
    if (!sumsq_out || !nonfinite_out) return fail(ZS_EINVAL, "sumsq_out and nonfinite_out must not be NULL");
    if ((reinterpret_cast<uintptr_t>(sumsq_out) & 7) || (reinterpret_cast<uintptr_t>(nonfinite_out) & 3))
        return fail(ZS_EALIGN, "sumsq_out must be 8-byte and nonfinite_out 4-byte aligned");
    if (zs_status st = check_ptr(workspace, "workspace")) return st;
    const int64_t need = zs_grad_stats_workspace_bytes(plan);
    if (workspace_bytes < need)
        return fail(ZS_ENOMEM, "workspace holds %lld bytes, zs_grad_stats needs %lld", (long long)workspace_bytes,
                    (long long)need);
    trace("zs_grad_stats", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_grad_stats(acc_f32, grad_divisor, sumsq_out, nonfinite_out, workspace, plan->S, stream),
                      "grad stats launch");
}

zs_status zs_grad_stats_noalloc(const zs_plan* plan, const float* acc_f32, float grad_divisor, double* sumsq_out,
                                int32_t* nonfinite_out, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_ptr(acc_f32, "acc_f32")) return st;
    if (!std::isfinite(grad_divisor) || grad_divisor == 0.0f)
        return fail(ZS_EINVAL, "grad_divisor = %g must be finite and nonzero", (double)grad_divisor);
    if (!sumsq_out || !nonfinite_out) return fail(ZS_EINVAL, "sumsq_out and nonfinite_out must not be NULL");
    if ((reinterpret_cast<uintptr_t>(sumsq_out) & 7) || (reinterpret_cast<uintptr_t>(nonfinite_out) & 3))
        return fail(ZS_EALIGN, "sumsq_out must be 8-byte and nonfinite_out 4-byte aligned");
    const int64_t need = zs_grad_stats_workspace_bytes(plan);
    if (need > zs::kNoallocScratchBytes)
        return fail(ZS_ENOMEM,
                    "a shard of %lld elements needs %lld bytes of partials, more than the %lld-byte static scratch "
                    "of zs_grad_stats_noalloc (at most %lld elements); use zs_grad_stats with a workspace",
                    (long long)plan->S, (long long)need, (long long)zs::kNoallocScratchBytes,
                    (long long)ZS_GRAD_STATS_NOALLOC_MAX_ELEMS);
    trace("zs_grad_stats_noalloc", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_grad_stats_noalloc(acc_f32, grad_divisor, sumsq_out, nonfinite_out, plan->S, stream),
                      "grad stats launch");
}

zs_status zs_clip_scale(const double* sumsq, const int32_t* nonfinite, int32_t n_ranks, double max_norm,
                        float* scale_out, int32_t* skip_out, void* stream) {
    if (!sumsq || !nonfinite || !scale_out || !skip_out) return fail(ZS_EINVAL, "a pointer argument is NULL");
    if ((reinterpret_cast<uintptr_t>(sumsq) & 7) || (reinterpret_cast<uintptr_t>(nonfinite) & 3) ||
        (reinterpret_cast<uintptr_t>(scale_out) & 3) || (reinterpret_cast<uintptr_t>(skip_out) & 3))
        return fail(ZS_EALIGN, "sumsq needs 8-byte, the others 4-byte alignment");
    if (n_ranks < 1) return fail(ZS_EINVAL, "n_ranks = %d must be >= 1", n_ranks);
    if (!std::isfinite(max_norm) || max_norm <= 0.0) return fail(ZS_EINVAL, "max_norm = %g must be positive", max_norm);
    trace("zs_clip_scale", nullptr, n_ranks, 0, 0, stream);
    return hip_status(zs::launch_clip_scale(sumsq, nonfinite, n_ranks, max_norm, scale_out, skip_out, stream),
                      "clip scale launch");
}

namespace {

zs_status accum_step_impl(const zs_plan* plan, const zs::AdamCoef& c, const zs::AdamCoef* cdev, const float* acc_f32,
                          float grad_divisor, const float* scale, const int32_t* skip, float* master, float* m,
                          float* v, void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_ptr(acc_f32, "acc_f32")) return st;
    if (!std::isfinite(grad_divisor) || grad_divisor == 0.0f)
        return fail(ZS_EINVAL, "grad_divisor = %g must be finite and nonzero", (double)grad_divisor);
    if ((scale && (reinterpret_cast<uintptr_t>(scale) & 3)) || (skip && (reinterpret_cast<uintptr_t>(skip) & 3)))
        return fail(ZS_EALIGN, "scale and skip must be 4-byte aligned");
    if (zs_status st = check_ptr(master, "master")) return st;
    if (zs_status st = check_ptr(m, "m")) return st;
    if (zs_status st = check_ptr(v, "v")) return st;
    if (zs_status st = check_opt_ptr(param_bf16, "param_bf16")) return st;
    if (zs_status st = check_opt_ptr(full_bf16, "full_bf16")) return st;
    if (full_bf16 && plan->layout != ZS_LAYOUT_FLAT)
        return fail(ZS_EINVAL, "a gather into full_bf16 needs a FLAT plan");
    if (plan->S == 0) return ZS_OK;
    char* own = full_bf16 ? static_cast<char*>(full_bf16) + 2 * (int64_t)plan->rank * plan->S : nullptr;
    trace(cdev ? "zs_adamw_shard_step_accum_dc" : "zs_adamw_shard_step_accum", plan, 0, 0, plan->S, stream);
    return hip_status(zs::launch_adamw_accum(c, acc_f32, grad_divisor, scale, skip, master, m, v, param_bf16, own,
                                             plan->S, stream, cdev),
                      "adamw accum launch");
}

}  // namespace

zs_status zs_adamw_shard_step_accum(const zs_plan* plan, const zs_adamw_hparams* hp, const float* acc_f32,
                                    float grad_divisor, const float* scale, const int32_t* skip, float* master,
                                    float* m, float* v, void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    return accum_step_impl(plan, zs::make_coef(*hp), nullptr, acc_f32, grad_divisor, scale, skip, master, m, v,
                           param_bf16, full_bf16, stream);
}

zs_status zs_adamw_shard_step_accum_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const float* acc_f32,
                                       float grad_divisor, const float* scale, const int32_t* skip, float* master,
                                       float* m, float* v, void* param_bf16, void* full_bf16, void* stream) {
    if (zs_status st = check_plan(plan)) return st;
    if (zs_status st = check_coefs(coefs)) return st;
    return accum_step_impl(plan, zs::AdamCoef{}, dev_coef(coefs), acc_f32, grad_divisor, scale, skip, master, m, v,
                           param_bf16, full_bf16, stream);
}

// ------------------------------------------------------------------ multi-tensor

namespace {

struct MultiLayout {
    int64_t pieces_off, contribs_off, chunks_off, total;
};

MultiLayout multi_layout(const zs_plan* p, int32_t n_contribs) {
    auto al = [](int64_t x) { return roundup(x, 256); };
    MultiLayout L;
    const int64_t n = (int64_t)p->tensors.size();
    L.pieces_off = al((int64_t)sizeof(zs::MultiHeader));
    L.contribs_off = al(L.pieces_off + n * (int64_t)sizeof(zs::PieceDev));
    L.chunks_off = al(L.contribs_off + n * (int64_t)n_contribs * (int64_t)sizeof(void*));
    L.total = al(L.chunks_off + (int64_t)p->chunk_piece.size() * (int64_t)sizeof(int32_t));
    return L;
}

zs::MultiOffsets multi_offsets(const zs_plan* p, int32_t n_contribs) {
    const MultiLayout L = multi_layout(p, n_contribs);
    return zs::MultiOffsets{L.pieces_off, L.contribs_off, L.chunks_off};
}

zs_status check_multi_plan(const zs_plan* plan) {
    if (zs_status st = check_plan(plan)) return st;
    if (plan->layout != ZS_LAYOUT_PER_TENSOR)
        return fail(ZS_EINVAL, "multi-tensor calls need a PER_TENSOR plan");
    return ZS_OK;
}

zs_status lookup_binding(const zs_plan* plan, const void* ws, int32_t need, Binding* out) {
    if (!ws) return fail(ZS_EINVAL, "workspace is NULL");
    std::lock_guard<std::mutex> lk(g_bind_mu);
    auto it = g_bind.find(ws);
    if (it == g_bind.end()) return fail(ZS_EINVAL, "workspace %p was never bound by zs_multi_bind", ws);
    if (it->second.plan != plan) return fail(ZS_EINVAL, "workspace %p was bound to another plan", ws);
    if ((it->second.flags & need) != need)
        return fail(ZS_EINVAL, "workspace %p lacks fields this call needs (bound 0x%x, needed 0x%x)", ws,
                    it->second.flags, need);
    *out = it->second;
    return ZS_OK;
}

// The fused multi-tensor step: one pass, or, from
// ZS_FUSED_TWO_PASS_MIN_CONTRIBS contributions on with the grad pieces
// bound, the reduce into the grad pieces and then AdamW writing the
// parameter and gathered pieces (the same bytes; faster at those sizes, as
// for the flat step).
int launch_fused_multi(const zs_plan* plan, const Binding& b, const zs::CoefTable* ct, const void* workspace,
                       void* stream, const zs::AdamCoef* cdev) {
    const zs::MultiOffsets off = multi_offsets(plan, b.n_contribs);
    const int n_chunks = (int)plan->chunk_piece.size();
    if ((b.flags & zs::kHasGrad) && b.n_contribs >= ZS_FUSED_TWO_PASS_MIN_CONTRIBS) {
        if (int e = zs::launch_multi(zs::kOpReduce, nullptr, workspace, off, n_chunks, b.n_contribs, stream)) return e;
        return zs::launch_multi(zs::kOpAdamwGather, ct, workspace, off, n_chunks, b.n_contribs, stream, cdev);
    }
    return zs::launch_multi(zs::kOpFused, ct, workspace, off, n_chunks, b.n_contribs, stream, cdev);
}

}  // namespace

int64_t zs_plan_workspace_bytes(const zs_plan* plan) {
    if (!plan) return -1;
    if (plan->layout != ZS_LAYOUT_PER_TENSOR) return 0;
    return multi_layout(plan, plan->world).total;
}

int64_t zs_multi_workspace_bytes(const zs_plan* plan, int32_t n_contribs) {
    if (!plan || plan->layout != ZS_LAYOUT_PER_TENSOR || n_contribs < 0 || n_contribs > ZS_MAX_CONTRIBS) return -1;
    return multi_layout(plan, n_contribs).total;
}

zs_status zs_multi_bind(const zs_plan* plan, const zs_piece_ptrs* pieces, const void* const* contribs,
                        int32_t n_contribs, void* workspace, int64_t workspace_bytes, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    if (!pieces && !plan->tensors.empty()) return fail(ZS_EINVAL, "pieces is NULL");
    if (zs_status st = check_ptr(workspace, "workspace")) return st;
    if (n_contribs < 0 || n_contribs > ZS_MAX_CONTRIBS || n_contribs % plan->world != 0)
        return fail(ZS_EINVAL, "n_contribs = %d must be 0 or a multiple of the world size %d, at most %d",
                    n_contribs, plan->world, ZS_MAX_CONTRIBS);
    if (n_contribs > 0 && !contribs) return fail(ZS_EINVAL, "contribs is NULL");
    const MultiLayout L = multi_layout(plan, n_contribs);
    if (workspace_bytes < L.total)
        return fail(ZS_ENOMEM, "workspace holds %lld bytes, the binding needs %lld", (long long)workspace_bytes,
                    (long long)L.total);

    const int32_t n = (int32_t)plan->tensors.size();
    // Which fields are bound: decided by the first non-empty piece, and every
    // other non-empty piece must agree.
    int32_t flags = -1;
    for (int32_t i = 0; i < n; ++i) {
        const zs::TensorEntry& t = plan->tensors[(size_t)i];
        if (t.own_hi == t.own_lo) continue;
        const zs_piece_ptrs& pc = pieces[i];
        int32_t f = 0;
        if (pc.grad) f |= zs::kHasGrad;
        if (pc.master || pc.m || pc.v) {
            if (!(pc.master && pc.m && pc.v))
                return fail(ZS_EINVAL, "piece %d binds only part of master/m/v", i);
            f |= zs::kHasState;
        }
        if (pc.param) f |= zs::kHasParam;
        if (pc.full) f |= zs::kHasFull;
        if (flags < 0) flags = f;
        if (f != flags) return fail(ZS_EINVAL, "piece %d binds a different set of fields than piece 0", i);
        const void* ptrs[6] = {pc.grad, pc.master, pc.m, pc.v, pc.param, pc.full};
        const char* names[6] = {"grad", "master", "m", "v", "param", "full"};
        for (int k = 0; k < 6; ++k)
            if (ptrs[k] && !aligned16(ptrs[k])) return fail(ZS_EALIGN, "piece %d: %s is not 16-byte aligned", i, names[k]);
        if (pc.full && ((t.own_lo * 2) & 15))
            return fail(ZS_EALIGN, "piece %d: owned offset of the gathered tensor is not 16-byte aligned", i);
        for (int32_t q = 0; q < n_contribs; ++q) {
            const void* c = contribs[(int64_t)q * n + i];
            if (!c) return fail(ZS_EINVAL, "contribution of rank %d for piece %d is NULL", q, i);
            if (!aligned16(c)) return fail(ZS_EALIGN, "contribution of rank %d for piece %d is not aligned", q, i);
        }
    }
    if (flags < 0) flags = 0;
    if (n_contribs > 0) flags |= zs::kHasContribs;

    std::vector<char> host;
    try {
        host.assign((size_t)L.total, 0);
    } catch (const std::bad_alloc&) {
        return fail(ZS_ENOMEM, "out of host memory");
    }
    zs::MultiHeader* h = reinterpret_cast<zs::MultiHeader*>(host.data());
    h->magic = zs::kMultiMagic;
    h->n_pieces = n;
    h->n_chunks = (int32_t)plan->chunk_piece.size();
    h->n_contribs = n_contribs;
    h->flags = flags;
    h->pieces_off = L.pieces_off;
    h->contribs_off = L.contribs_off;
    h->chunks_off = L.chunks_off;
    zs::PieceDev* pd = reinterpret_cast<zs::PieceDev*>(host.data() + L.pieces_off);
    const void** cd = reinterpret_cast<const void**>(host.data() + L.contribs_off);
    for (int32_t i = 0; i < n; ++i) {
        const zs::TensorEntry& t = plan->tensors[(size_t)i];
        const zs_piece_ptrs& pc = pieces[i];
        pd[i].grad = pc.grad;
        pd[i].master = pc.master;
        pd[i].m = pc.m;
        pd[i].v = pc.v;
        pd[i].param = pc.param;
        pd[i].full_own = pc.full ? static_cast<char*>(pc.full) + 2 * t.own_lo : nullptr;
        pd[i].len = t.own_hi - t.own_lo;
        pd[i].group = t.group;
        pd[i].first_chunk = (int32_t)t.first_chunk;
        for (int32_t q = 0; q < n_contribs; ++q) cd[(int64_t)i * n_contribs + q] = contribs[(int64_t)q * n + i];
    }
    std::memcpy(host.data() + L.chunks_off, plan->chunk_piece.data(), plan->chunk_piece.size() * sizeof(int32_t));
    trace("zs_multi_bind", plan, n_contribs, 0, plan->S, stream);
    if (zs_status st = hip_status(zs::copy_h2d_sync(workspace, host.data(), L.total, stream), "workspace copy"))
        return st;
    std::lock_guard<std::mutex> lk(g_bind_mu);
    g_bind[workspace] = Binding{plan, flags, n_contribs};
    return ZS_OK;
}

zs_status zs_multi_unbind(void* workspace, void* stream) {
    if (!workspace) return fail(ZS_EINVAL, "workspace is NULL");
    {
        std::lock_guard<std::mutex> lk(g_bind_mu);
        if (g_bind.erase(workspace) == 0) return fail(ZS_EINVAL, "workspace %p is not bound", workspace);
    }
    const uint64_t zero = 0;  // clear the table's magic: later launches on it do nothing
    trace("zs_multi_unbind", nullptr, 0, 0, 0, stream);
    return hip_status(zs::copy_h2d_sync(workspace, &zero, sizeof zero, stream), "workspace clear");
}

zs_status zs_reduce_shard_multi(const zs_plan* plan, const void* workspace, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasContribs | zs::kHasGrad, &b)) return st;
    trace("zs_reduce_shard_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(zs::launch_multi(zs::kOpReduce, nullptr, workspace, multi_offsets(plan, b.n_contribs), (int)plan->chunk_piece.size(), b.n_contribs, stream),
                      "multi reduce launch");
}

zs_status zs_adamw_shard_step_multi(const zs_plan* plan, const zs_adamw_hparams* hp, const void* workspace,
                                    void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasGrad | zs::kHasState, &b)) return st;
    zs::CoefTable ct;
    for (auto& e : ct.c) e = zs::make_coef(*hp);
    trace("zs_adamw_shard_step_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(zs::launch_multi(zs::kOpAdamw, &ct, workspace, multi_offsets(plan, b.n_contribs), (int)plan->chunk_piece.size(), b.n_contribs, stream),
                      "multi adamw launch");
}

zs_status zs_gather_params_multi(const zs_plan* plan, const void* workspace, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasParam | zs::kHasFull, &b)) return st;
    trace("zs_gather_params_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(zs::launch_multi(zs::kOpGather, nullptr, workspace, multi_offsets(plan, b.n_contribs), (int)plan->chunk_piece.size(), b.n_contribs, stream),
                      "multi gather launch");
}

zs_status zs_fused_shard_step_multi(const zs_plan* plan, const zs_adamw_hparams* hp, const void* workspace,
                                    void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    if (zs_status st = check_hp(hp)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasContribs | zs::kHasState, &b)) return st;
    zs::CoefTable ct;
    for (auto& e : ct.c) e = zs::make_coef(*hp);
    trace("zs_fused_shard_step_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(launch_fused_multi(plan, b, &ct, workspace, stream, nullptr), "multi fused launch");
}

namespace {

zs_status group_table(const zs_plan* plan, const zs_adamw_hparams* hps, int32_t n_groups, zs::CoefTable* ct) {
    if (!hps) return fail(ZS_EINVAL, "hparams array is NULL");
    if (n_groups < 1 || n_groups > ZS_MAX_GROUPS)
        return fail(ZS_EINVAL, "n_groups = %d outside [1, %d]", n_groups, ZS_MAX_GROUPS);
    for (const auto& t : plan->tensors)
        if (t.group >= n_groups)
            return fail(ZS_EINVAL, "the plan uses group %d but only %d sets of hyperparameters were given", t.group,
                        n_groups);
    for (int32_t g = 0; g < n_groups; ++g)
        if (zs_status st = check_hp(&hps[g])) return st;
    for (int32_t g = 0; g < ZS_MAX_GROUPS; ++g) ct->c[g] = zs::make_coef(hps[g < n_groups ? g : 0]);
    return ZS_OK;
}

}  // namespace

zs_status zs_adamw_shard_step_multi_groups(const zs_plan* plan, const zs_adamw_hparams* hps, int32_t n_groups,
                                           const void* workspace, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    zs::CoefTable ct;
    if (zs_status st = group_table(plan, hps, n_groups, &ct)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasGrad | zs::kHasState, &b)) return st;
    trace("zs_adamw_shard_step_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(zs::launch_multi(zs::kOpAdamw, &ct, workspace, multi_offsets(plan, b.n_contribs), (int)plan->chunk_piece.size(), b.n_contribs, stream),
                      "multi adamw launch");
}

zs_status zs_fused_shard_step_multi_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, int32_t n_groups,
                                       const void* workspace, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    if (zs_status st = check_coefs(coefs)) return st;
    if (n_groups < 1 || n_groups > ZS_MAX_GROUPS)
        return fail(ZS_EINVAL, "n_groups = %d outside [1, %d]", n_groups, ZS_MAX_GROUPS);
    for (const auto& t : plan->tensors)
        if (t.group >= n_groups)
            return fail(ZS_EINVAL, "the plan uses group %d but only %d sets of scalars were given", t.group, n_groups);
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasContribs | zs::kHasState, &b)) return st;
    const zs::CoefTable unused{};
    trace("zs_fused_shard_step_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(launch_fused_multi(plan, b, &unused, workspace, stream, dev_coef(coefs)), "multi fused launch");
}

zs_status zs_fused_shard_step_multi_groups(const zs_plan* plan, const zs_adamw_hparams* hps, int32_t n_groups,
                                           const void* workspace, void* stream) {
    if (zs_status st = check_multi_plan(plan)) return st;
    zs::CoefTable ct;
    if (zs_status st = group_table(plan, hps, n_groups, &ct)) return st;
    Binding b;
    if (zs_status st = lookup_binding(plan, workspace, zs::kHasContribs | zs::kHasState, &b)) return st;
    trace("zs_fused_shard_step_multi", plan, b.n_contribs, 0, plan->S, stream);
    return hip_status(launch_fused_multi(plan, b, &ct, workspace, stream, nullptr), "multi fused launch");
}

}  // extern "C"
