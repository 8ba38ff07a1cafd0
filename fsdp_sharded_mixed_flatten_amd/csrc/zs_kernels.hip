// HIP kernels of the shard-local step for CDNA4 (gfx950).
//
// Every kernel here is an HBM stream: per owned element the fused step reads
// 2N + 12 bytes (N bf16 contributions, fp32 master/m/v) and writes 14 (fp32
// master/m/v, the bf16 parameter), with ~100 fp32 instructions, far below the
// fp32 ridge of MI355X, so nothing is compute-bound and nothing uses MFMA.
//
// Design points, each measured on MI355X:
//   * One tile per block, the grid covering the shard once. Blocks dispatch in
//     index order, so the resident blocks stream one compact window that
//     advances through every array and DRAM rows stay open; a persistent
//     grid-stride grid scatters its blocks over the arrays and ran 20-25%
//     slower.
//   * 64-thread blocks plus an occupancy throttle: each block reserves
//     dynamic LDS it never touches, capping the resident waves per CU. With
//     reads and writes mixed, fewer waves in flight keep fewer DRAM rows in
//     play (+6-8% on the fused kernel).
//   * Lanes own 4 consecutive elements where bf16 and fp32 arrays mix (fp32 as
//     one 16-byte dwordx4, bf16 as one 8-byte dwordx2: every wave access is a
//     contiguous, fully used 1 KiB / 512 B span) and 8 elements in bf16-only
//     kernels (one dwordx4).
//   * Each lane issues the loads of a group of ranks, and of the state arrays,
//     before consuming any, so many independent loads are in flight.
//   * Every access is nontemporal (each access class was swept; the cached
//     variants were slower). Rows a whole wave writes go out as buffer stores
//     that also set sc1, which only a buffer access can express from HIP
//     (2-5% faster for the kernels that mix reads and writes).
//   * Writes that interleave with heavy read traffic cost several times their
//     share of bytes, so at large N the fused entry point runs as a nearly
//     read-only reduce followed by AdamW writing the gathered slice directly.
//   * The element arithmetic is the IEEE fp32 sequence of the C ABI contract
//     (no FMA contraction: built with -ffp-contract=off; IEEE division and
//     correctly rounded square root, the HIP defaults; denormals kept), so
//     results are bit-identical to a plain sequential implementation.
#include <hip/hip_runtime.h>

#include <mutex>

#include "zs_internal.h"

namespace zs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ launch shape
// Every value below was measured against its neighbours on MI355X at the
// model shapes (Qwen2.5-3B N=4, Llama-7B N=8, Llama-70B N=64) and, for the
// world-size rules, at the Llama-7B shape cut for N = 1 to 128.

constexpr int kBlock = kBlockThreads;
// Ranks whose loads a lane issues together (16 or 32 measured within noise).
constexpr int kGroup = 8;
// Units of work per lane: 8 elements (reduce) or 4 elements (the others);
// two or four units per lane measured slower in every kernel.
constexpr int kReduceU = 1;
constexpr int kAdamwU = 1;
constexpr int kFusedU = 1;
// Occupancy throttle: bytes of untouched dynamic LDS per block (160 KiB per
// CU), which caps the resident 64-thread blocks per CU.
//   fused step, N > 4: 16 KiB (ten waves per CU; at N=8 12 KiB 2% slower,
//   20 KiB the same, 24 KiB 7% slower), except the compiled 16 and 32 rank
//   loops: 24 KiB (1.4-3% faster than 16 or 20 KiB); the runtime rank loop,
//   which holds two register sets of loads, loses 2-14% at 24 KiB;
constexpr unsigned kFusedLds = 16u << 10;
constexpr unsigned kFusedMidLds = 24u << 10;
//   fused step at 4 or fewer ranks, whose lighter reads leave room for more
//   resident waves: eleven per CU (14 KiB) measured 1.4% faster than ten or
//   thirteen at the Qwen2.5-3B shape;
constexpr unsigned kFusedNarrowLds = 14u << 10;
//   and at 1 or 2 ranks 12 KiB (up to 1.7% faster than 14 KiB);
constexpr unsigned kFusedTinyLds = 12u << 10;
//   fused step writing quantized codes (more registers): 12 KiB, 3% faster
//   than 14 or 16 KiB at the Qwen2.5-3B and Llama-7B shapes;
constexpr unsigned kFusedQuantLds = 12u << 10;
//   accumulation micro-steps (read 2N+4 bytes, write 4 per element): 16 KiB
//   (8 to 40 KiB measured at the Llama-7B and -70B shapes; 24 KiB the same
//   at N=64 and slower at N = 8 and 24, 32 KiB and more lose 8-11% at N=64),
//   12 KiB at 3 or 4 ranks (2-3% faster than 8 KiB with the nt sc1 stores,
//   16 KiB 10% slower) and 8 KiB at 1 or 2 (5-13% faster than 12 KiB).
//   Lanes of 8 elements (16-byte contribution loads, two 16-byte
//   accumulator accesses 32 bytes apart) ran 1.3-2x slower: each wave
//   access then covers half of every line it touches;
constexpr unsigned kAccumLds = 16u << 10;
constexpr unsigned kAccumNarrowLds = 12u << 10;
constexpr unsigned kAccumTinyLds = 8u << 10;
//   reduce: 4 KiB per rank up to 16 KiB below kMidN ranks (16 KiB 2-7%
//   faster than 8 KiB at N = 8, 12, 16 and 24; a light kernel needs more
//   waves in flight: 16 KiB ran 79% slower than 4 KiB at N=1 and 33%
//   slower than 8 KiB at N=2), 24 KiB from kMidN (2-7% faster than 16 or
//   32 KiB at N = 32, 40 and 48) and 32 KiB from kWideN ranks on, about
//   five waves per CU (at N=64 3-8% faster than 8 KiB, 0.2-1.6% than
//   24 KiB; 48 KiB and up lose);
constexpr unsigned kReduceLds = 16u << 10;
constexpr unsigned kReduceLdsPerRank = 4u << 10;
constexpr unsigned kReduceMidLds = 24u << 10;
constexpr unsigned kReduceWideLds = 32u << 10;
constexpr int kMidN = 32;
constexpr int kWideN = 64;
//   AdamW (from the grad shard or the accumulator): 12 KiB (1-3% faster than
//   8 or 16 KiB at all three shapes with the nt sc1 stores);
constexpr unsigned kAdamwLds = 12u << 10;
//   gather copies and the bf16 codes of a shard: 4 KiB (3.5% faster than 8;
//   0 and 2 KiB the same as 4, 16 KiB 50% slower);
constexpr unsigned kGatherLds = 4u << 10;
//   multi-tensor kernels: 12 KiB for reduce and AdamW (10 and 14 KiB slower;
//   for the reduce 8, 16, 24 and 32 KiB at N = 8, 24 and 64 too; the reduce
//   at 1 or 2 ranks takes 4 KiB, 44-52% faster, and at 3 or 4 ranks 8 KiB,
//   15% faster), 14 KiB for the fused step (12 KiB 2% slower, 16 the same, 18 and 20 KiB
//   slower at the Llama-7B wrap-stress shape) and 8 KiB for the gather (12%
//   faster than 12 KiB, 2% faster than 4 KiB or none);
constexpr unsigned kMultiLds = 12u << 10;
constexpr unsigned kMultiFusedLds = 14u << 10;
constexpr unsigned kMultiFusedTinyLds = 10u << 10;  // 1 or 2 ranks: 4-6% faster than 14 KiB
constexpr unsigned kMultiGatherLds = 8u << 10;
constexpr unsigned kMultiReduceLds = 12u << 10;
constexpr unsigned kMultiReduceNarrowLds = 8u << 10;
constexpr unsigned kMultiReduceTinyLds = 4u << 10;
//   dequantizing gather, a nearly pure write stream: 4 KiB (2% faster than
//   none, 2 or 3 KiB at the Llama-7B and Qwen2.5-3B shapes, 5 KiB 0.5%
//   slower; 6 KiB and up 13-20% slower, larger throttles up to 2x). Its
//   lanes decode four 8-element units each.
constexpr unsigned kDequantLds = 4u << 10;
constexpr int kDequantU = 4;
// World size from which the fused entry point runs the reduce into the grad
// shard, then AdamW + gather, when the caller provides the grad buffer. At
// the Llama-7B shape the two passes are 3.7% faster at N=52 (mean of five
// buffer sets), 3-6% at N=56, 11% at N=64 and 14% at N=128 (at the
// Llama-70B shape every one-pass layout measured 7-25% slower at N=64);
// from 33 to 48 ranks the two forms average within 1.6% of each other
// either way round, and below 32 the one pass wins (5-7% at N=16 and 24).
constexpr int kSplitMinN = ZS_FUSED_TWO_PASS_MIN_CONTRIBS;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, IEEE round to nearest even; NaN -> quiet NaN, sign kept.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) { return bf16_rne(a) | (bf16_rne(b) << 16); }

// The same rounding for values known not to be NaN (infinities included).
__device__ __forceinline__ uint32_t pack2_finite(float a, float b) {
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    return ((ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16) | (((ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16) << 16);
}

// ------------------------------------------------------------------ AdamW element

__device__ __forceinline__ void adamw_elem(const AdamCoef& c, float gf, float& w, float& m, float& v) {
    float wd = w * c.decay;
    float mn = c.b1 * m + c.omb1 * gf;
    float vn = c.b2 * v + c.omb2 * (gf * gf);
    float mh = mn / c.bc1;
    float vh = vn / c.bc2;
    float den = sqrtf(vh) + c.eps;
    w = wd - c.lr * (mh / den);
    m = mn;
    v = vn;
}

__device__ __forceinline__ void adamw_unit(const AdamCoef& c, u32x2 g, f32x4& w, f32x4& m, f32x4& v) {
    float w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    float m0 = m.x, m1 = m.y, m2 = m.z, m3 = m.w;
    float v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
    adamw_elem(c, lo_bf16(g.x), w0, m0, v0);
    adamw_elem(c, hi_bf16(g.x), w1, m1, v1);
    adamw_elem(c, lo_bf16(g.y), w2, m2, v2);
    adamw_elem(c, hi_bf16(g.y), w3, m3, v3);
    w = f32x4{w0, w1, w2, w3};
    m = f32x4{m0, m1, m2, m3};
    v = f32x4{v0, v1, v2, v3};
}

__device__ __forceinline__ u32x2 to_bf16x4(const f32x4& w) {
    u32x2 p;
    p.x = pack2(w.x, w.y);
    p.y = pack2(w.z, w.w);
    return p;
}

// ------------------------------------------------------------------ memory helpers

// Every access goes through a global-address-space pointer. Pointers read
// from a device table (the multi-tensor pieces) are generic to the compiler,
// which would emit flat memory instructions for them; flat loads count
// against both wait counters and serialize the grouped loads. Every buffer
// here is global memory.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load((gptr<const T>)p); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T x) { __builtin_nontemporal_store(x, (gptr<T>)p); }

// Plain (cached) global load, for table records.
template <typename T>
__device__ __forceinline__ T ld_g(const T* p) { return *(gptr<const T>)p; }

// The step's AdamW scalars: the launch's own (by value), or, when `dev` is
// set, the ones in device memory at the time the kernel runs (so a captured
// graph can be replayed with new scalars). Uniform across the grid.
__device__ __forceinline__ AdamCoef pick_coef(const AdamCoef& c, const AdamCoef* dev) {
    if (!dev) return c;
    AdamCoef d;
    d.b1 = ld_g(&dev->b1);
    d.omb1 = ld_g(&dev->omb1);
    d.b2 = ld_g(&dev->b2);
    d.omb2 = ld_g(&dev->omb2);
    d.lr = ld_g(&dev->lr);
    d.eps = ld_g(&dev->eps);
    d.decay = ld_g(&dev->decay);
    d.bc1 = ld_g(&dev->bc1);
    d.bc2 = ld_g(&dev->bc2);
    return d;
}

// Rows: lane L of the wave accesses unit L of a row of kBlock consecutive
// units, which starts at p - L. Such an access can go through a buffer
// resource based at the row's first unit (the same address in every lane,
// taken into scalar registers) and bounded by the row's bytes, with the
// lane's byte offset as its vector offset; a buffer access carries the full
// cache-policy field, a global one written in HIP only nt.
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer: 32-bit data format

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const T* p) {
    static_assert(kBlock == 64, "a row is one wave: blocks are single waves");
    const uintptr_t row = reinterpret_cast<uintptr_t>(p - threadIdx.x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(row >> 32));
    void* base = reinterpret_cast<void*>(((uintptr_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, kBlock * (int)sizeof(T), kBufferWord3);
}

// Row stores: nontemporal with sc1 set. At the Llama-7B shape this is 2-3%
// faster for the fused step and up to 4% for AdamW than the global
// nontemporal store (nt alone, which a buffer store with nt alone times the
// same as); sc1 without nt is slower than both.
constexpr int kStreamAux = 2 | 16;  // nt | sc1

template <typename T>
__device__ __forceinline__ void st_lane(T* p, T x) {
    const __amdgpu_buffer_rsrc_t r = row_rsrc(p);
    const int off = (int)(threadIdx.x * sizeof(T));
    if constexpr (sizeof(T) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, kStreamAux);
    else {
        static_assert(sizeof(T) == 8, "rows of 8- or 16-byte units");
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, kStreamAux);
    }
}

// Row loads of 16-byte units, nontemporal: the N-way reduce's contribution
// reads (0.2-1.2% faster at N=64 than global loads; sc0 or sc1 added change
// nothing, sc0|sc1 without nt is 5% slower). The fused step and the
// accumulation micro-step measured the same or slower with them (the
// accumulation 1% slower at N=64 with its contributions loaded this way, 4%
// at N=8 with its accumulator too) and keep global loads.
__device__ __forceinline__ u32x4 ld_lane(const u32x4* p) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(p), (int)(threadIdx.x * 16), 0, 2));
}

// Cache policy per access class: read-once inputs and the read-modify-write
// optimizer state are nontemporal loads (each class was swept; every cached
// variant was slower); rows written by a whole wave (the state, the grad and
// parameter outputs, gather copies) are st_lane stores, other writes (codes,
// scales, the multi-tensor gather and reduce, whose lanes write two chunks)
// nontemporal global stores.
template <typename T>
__device__ __forceinline__ T ld_in(const T* p) { return ld_nt(p); }
template <typename T>
__device__ __forceinline__ T ld_state(const T* p) { return ld_nt(p); }
template <typename T>
__device__ __forceinline__ void st_out(T* p, T x) { st_nt(p, x); }

template <int CAP>
struct Ptrs {
    const void* p[CAP];
};

// ------------------------------------------------------------------ rank sums
//
// The N contributions of a lane's units are summed in fp32, one add at a time
// in rank order 0..N-1 starting from +0. Loads are issued a group of G ranks
// at a time for all U units of the lane before any of them is consumed, so
// every lane keeps G*U independent loads in flight (a plain rank loop makes
// the compiler wait for each load before issuing the next).

template <typename V>
struct Lanes;
template <>
struct Lanes<u32x2> {
    static constexpr int E = 4;  // bf16 elements per vector
};
template <>
struct Lanes<u32x4> {
    static constexpr int E = 8;
};

template <typename V>
__device__ __forceinline__ void acc_add(float* a, const V& x) {
    a[0] = a[0] + lo_bf16(x.x);
    a[1] = a[1] + hi_bf16(x.x);
    a[2] = a[2] + lo_bf16(x.y);
    a[3] = a[3] + hi_bf16(x.y);
    if constexpr (Lanes<V>::E == 8) {
        a[4] = a[4] + lo_bf16(x.z);
        a[5] = a[5] + hi_bf16(x.z);
        a[6] = a[6] + lo_bf16(x.w);
        a[7] = a[7] + hi_bf16(x.w);
    }
}

// Loads ranks [q0, q0 + G) of the U units u[k] with ok[k] into x.
template <typename V, int U, int G, bool ROW>
__device__ __forceinline__ void load_group(const void* const* p, int q0, const int64_t* u, const bool* ok,
                                           V (*x)[U]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (ok[k]) {
                const V* src = reinterpret_cast<const V*>(p[q0 + g]) + u[k];
                if constexpr (ROW)
                    x[g][k] = ld_lane(src);
                else
                    x[g][k] = ld_in(src);
            }
}

// Adds a loaded group into a[k][*], rank by rank.
template <typename V, int U, int G>
__device__ __forceinline__ void add_group(const V (*x)[U], const bool* ok, float (*a)[Lanes<V>::E]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (ok[k]) acc_add<V>(a[k], x[g][k]);
}

// Adds ranks [q0, q0 + G) into a[k][*] for the U units u[k] with ok[k].
template <typename V, int U, int G, bool ROW>
__device__ __forceinline__ void sum_group(const void* const* p, int q0, const int64_t* u, const bool* ok,
                                          float (*a)[Lanes<V>::E]) {
    V x[G][U];
    load_group<V, U, G, ROW>(p, q0, u, ok, x);
    add_group<V, U, G>(x, ok, a);
}

// Full rank sum. Compile-time N: groups of min(N, kGroup), fully unrolled.
// Runtime N: groups of kGroup with the next group's loads issued before the
// current group is added (two register sets in turn, so a lane keeps up to
// 2 * kGroup loads in flight; a plain loop waits for each group before
// issuing the next: 5.0 TB/s against 6.6 for the N=48 reduce), then 4, 2
// and 1 ranks. Either way the adds run in rank order 0..N-1. ROW: the units
// are rows (u[k] is the row's first unit plus the lane), loaded with
// ld_lane.
template <typename V, int U, int N, bool ROW = false>
__device__ __forceinline__ void rank_sum(const void* const* p, int n_rt, const int64_t* u, const bool* ok,
                                         float (*a)[Lanes<V>::E]) {
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
        for (int e = 0; e < Lanes<V>::E; ++e) a[k][e] = 0.0f;
    if constexpr (N > 0) {
        constexpr int G = N < kGroup ? N : kGroup;
        static_assert(N % G == 0, "world sizes with compiled loops are powers of two");
#pragma unroll
        for (int q0 = 0; q0 < N; q0 += G) sum_group<V, U, G, ROW>(p, q0, u, ok, a);
    } else {
        constexpr int G = kGroup;
        int q0 = 0;
        if (n_rt >= G) {
            V x[G][U], y[G][U];
            load_group<V, U, G, ROW>(p, 0, u, ok, x);
            q0 = G;
            bool y_pending = false;  // which set holds the loaded, not yet added group
            while (q0 + G <= n_rt) {
                load_group<V, U, G, ROW>(p, q0, u, ok, y);
                add_group<V, U, G>(x, ok, a);
                q0 += G;
                y_pending = true;
                if (q0 + G > n_rt) break;
                load_group<V, U, G, ROW>(p, q0, u, ok, x);
                add_group<V, U, G>(y, ok, a);
                q0 += G;
                y_pending = false;
            }
            if (y_pending)
                add_group<V, U, G>(y, ok, a);
            else
                add_group<V, U, G>(x, ok, a);
        }
        if (q0 + 4 <= n_rt) {
            sum_group<V, U, 4, ROW>(p, q0, u, ok, a);
            q0 += 4;
        }
        if (q0 + 2 <= n_rt) {
            sum_group<V, U, 2, ROW>(p, q0, u, ok, a);
            q0 += 2;
        }
        if (q0 < n_rt) sum_group<V, U, 1, ROW>(p, q0, u, ok, a);
    }
}

// The average: one division by N (compile-time N: a division by a power of
// two, which the compiler turns into the exact multiplication by 1/N).
template <int N>
__device__ __forceinline__ float div_n(float x, float nf) {
    if constexpr (N > 0)
        return x / (float)N;
    else
        return x / nf;
}

template <int N>
__device__ __forceinline__ u32x2 avg_bf16x4(const float* a, float nf) {
    u32x2 g;
    g.x = pack2(div_n<N>(a[0], nf), div_n<N>(a[1], nf));
    g.y = pack2(div_n<N>(a[2], nf), div_n<N>(a[3], nf));
    return g;
}

// ------------------------------------------------------------------ tiles
//
// A tile is kBlock lanes x U units; a lane's units sit at base, base + kBlock,
// ... (in units of the tile's vector type), where base is the tile's first
// unit plus the lane's index (the row layout st_lane stores); units at or past
// `limit` are skipped. Optional outputs are nullptr when not written (uniform
// per block).

// reduce in units of 8 elements (bf16 only)
template <int N, int U>
__device__ __forceinline__ void reduce8_tile(const void* const* cp, int n_rt, float nf, u32x4* __restrict__ out,
                                             int64_t base, int64_t limit) {
    int64_t u[U];
    bool ok[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        u[k] = base + (int64_t)k * kBlock;
        ok[k] = u[k] < limit;
    }
    float a[U][8];
    rank_sum<u32x4, U, N, true>(cp, n_rt, u, ok, a);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (!ok[k]) continue;
        u32x4 o;
        o.x = pack2(div_n<N>(a[k][0], nf), div_n<N>(a[k][1], nf));
        o.y = pack2(div_n<N>(a[k][2], nf), div_n<N>(a[k][3], nf));
        o.z = pack2(div_n<N>(a[k][4], nf), div_n<N>(a[k][5], nf));
        o.w = pack2(div_n<N>(a[k][6], nf), div_n<N>(a[k][7], nf));
        st_lane(out + u[k], o);
    }
}

// ------------------------------------------------------------------ block quantization
//
// Symmetric block-wise codes of the updated bf16 shard (ZeRO++'s quantized
// parameter gather): per block of B elements, scale = amax / qmax in fp32 and
// code = rne(x / scale) clamped to [-qmax, qmax]; amax == 0 gives scale 0 and
// codes 0, a non-finite element gives scale NaN and codes 0. A lane holds E
// consecutive elements, so a block spans B / E consecutive lanes of the wave
// and its amax is a butterfly max over them. Every lane of the wave must call
// this (the cross-lane exchange), with ok == false where it holds no elements.

// Butterfly over groups of `lanes` consecutive lanes (a power of two <= 64):
// afterwards every lane of a group holds the group's largest amax and the OR
// of its flags. Within a row of 16 lanes the exchange is DPP (quad
// permutations, then the half-row and row mirrors); across rows it is
// gfx950's permlane swaps; no LDS round trip. All 64 lanes must execute it.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ void group_max_or(float& amax, int& bad, int lanes) {
    auto merge = [&](int o_amax, int o_bad) {
        const float o = __int_as_float(o_amax);
        amax = o > amax ? o : amax;
        bad |= o_bad;
    };
    if (lanes > 1) merge(dpp_i<0xB1>(__float_as_int(amax)), dpp_i<0xB1>(bad));    // quad_perm [1,0,3,2]
    if (lanes > 2) merge(dpp_i<0x4E>(__float_as_int(amax)), dpp_i<0x4E>(bad));    // quad_perm [2,3,0,1]
    if (lanes > 4) merge(dpp_i<0x141>(__float_as_int(amax)), dpp_i<0x141>(bad));  // row_half_mirror
    if (lanes > 8) merge(dpp_i<0x140>(__float_as_int(amax)), dpp_i<0x140>(bad));  // row_mirror
    if (lanes > 16) {  // rows 0<->1, 2<->3: each lane sees its partner in one of the two results
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(amax), __float_as_int(amax), false, false);
        const auto b = __builtin_amdgcn_permlane16_swap(bad, bad, false, false);
        merge(a[0], b[0]);
        merge(a[1], b[1]);
    }
    if (lanes > 32) {  // halves of the wave
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(amax), __float_as_int(amax), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(bad, bad, false, false);
        merge(a[0], b[0]);
        merge(a[1], b[1]);
    }
}

// The codes of one lane (QB*E bits, low element first) and its block's scale.
struct QuantWord {
    uint32_t lo, hi;
    float scale;
};

template <int QB, int E>
__device__ __forceinline__ QuantWord quant_compute(const uint32_t* w, bool ok, int block) {
    constexpr float qmax = (float)((1 << (QB - 1)) - 1);
    const int lanes = block / E;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = (e & 1) ? hi_bf16(w[e >> 1]) : lo_bf16(w[e >> 1]);
    float amax = 0.0f;
    int bad = 0;
    if (ok) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float a = fabsf(x[e]);
            bad |= !__builtin_isfinite(x[e]);
            amax = a > amax ? a : amax;
        }
    }
    group_max_or(amax, bad, lanes);
    QuantWord q;
    q.scale = bad ? __builtin_nanf("") : amax / qmax;
    const bool zero = bad || !(amax > 0.0f);
    q.lo = 0u;
    q.hi = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // Branch-free: a zero or NaN scale gives an inf/NaN quotient that the
        // select below discards.
        float r = rintf(x[e] / q.scale);
        r = r > qmax ? qmax : r;
        r = r < -qmax ? -qmax : r;
        const int k = zero ? 0 : (int)r;
        const uint32_t c = (uint32_t)k & ((1u << QB) - 1u);
        if (QB * e < 32)
            q.lo |= c << (QB * e);
        else
            q.hi |= c << (QB * e - 32);
    }
    return q;
}

// Stores a lane's codes, and its block's scale from the block's first lane.
template <int QB, int E>
__device__ __forceinline__ void quant_emit(const QuantWord& q, int64_t unit, const QuantOut& qo) {
    const int lanes = qo.block / E;
    const int64_t first = unit * E;  // first element of the lane
    char* cb = static_cast<char*>(qo.codes) + first * QB / 8;
    if constexpr (QB * E == 64)
        st_out(reinterpret_cast<u32x2*>(cb), u32x2{q.lo, q.hi});
    else if constexpr (QB * E == 32)
        st_out(reinterpret_cast<uint32_t*>(cb), q.lo);
    else
        st_out(reinterpret_cast<uint16_t*>(cb), (uint16_t)q.lo);
    if ((threadIdx.x & (lanes - 1)) == 0) st_out(qo.scales + first / qo.block, q.scale);
}

// AdamW from a bf16 grad; writes the bf16 parameter to `param` and/or `full`
template <int U, int QB = 0>
__device__ __forceinline__ void adamw_tile(const AdamCoef& c, const u32x2* __restrict__ g, f32x4* __restrict__ master,
                                           f32x4* __restrict__ m, f32x4* __restrict__ v, u32x2* __restrict__ param,
                                           u32x2* __restrict__ full, int64_t base, int64_t limit,
                                           const QuantOut& qo = QuantOut{}) {
    int64_t u[U];
    bool ok[U];
    u32x2 gv[U], pv[U];
    f32x4 wv[U], mv[U], vv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        u[k] = base + (int64_t)k * kBlock;
        ok[k] = u[k] < limit;
        pv[k] = u32x2{0u, 0u};
        if (ok[k]) {
            gv[k] = ld_in(g + u[k]);
            wv[k] = ld_state(master + u[k]);
            mv[k] = ld_state(m + u[k]);
            vv[k] = ld_state(v + u[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (!ok[k]) continue;
        adamw_unit(c, gv[k], wv[k], mv[k], vv[k]);
        pv[k] = to_bf16x4(wv[k]);
    }
    // Codes are computed by every lane before any store is issued.
    QuantWord qw[QB != 0 ? U : 1];
    if constexpr (QB != 0) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t w[2] = {pv[k].x, pv[k].y};
            qw[k] = quant_compute<QB, 4>(w, ok[k], qo.block);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (!ok[k]) continue;
        st_lane(master + u[k], wv[k]);
        st_lane(m + u[k], mv[k]);
        st_lane(v + u[k], vv[k]);
        if (param) st_lane(param + u[k], pv[k]);
        if (full) st_lane(full + u[k], pv[k]);
        if constexpr (QB != 0) quant_emit<QB, 4>(qw[k], u[k], qo);
    }
}

template <typename V, int U>
__device__ __forceinline__ void copy_tile(const V* __restrict__ src, V* __restrict__ dst, int64_t base,
                                          int64_t limit) {
    V x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t u = base + (int64_t)k * kBlock;
        if (u < limit) x[k] = ld_in(src + u);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t u = base + (int64_t)k * kBlock;
        if (u < limit) st_lane(dst + u, x[k]);
    }
}

// reduce + AdamW + gather write in registers
template <int N, int U, int QB = 0>
__device__ __forceinline__ void fused_tile(const AdamCoef& c, const void* const* cp, int n_rt, float nf,
                                           f32x4* __restrict__ master, f32x4* __restrict__ m,
                                           f32x4* __restrict__ v, u32x2* __restrict__ grad,
                                           u32x2* __restrict__ param, u32x2* __restrict__ full,
                                           int64_t base, int64_t limit, const QuantOut& qo = QuantOut{}) {
    int64_t u[U];
    bool ok[U];
    f32x4 wv[U], mv[U], vv[U];
    u32x2 gv[U], pv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        u[k] = base + (int64_t)k * kBlock;
        ok[k] = u[k] < limit;
        pv[k] = u32x2{0u, 0u};
        if (ok[k]) {
            wv[k] = ld_state(master + u[k]);
            mv[k] = ld_state(m + u[k]);
            vv[k] = ld_state(v + u[k]);
        }
    }
    float a[U][4];
    rank_sum<u32x2, U, N>(cp, n_rt, u, ok, a);
    if constexpr (QB == 0) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!ok[k]) continue;
            const u32x2 g = avg_bf16x4<N>(a[k], nf);
            adamw_unit(c, g, wv[k], mv[k], vv[k]);
            st_lane(master + u[k], wv[k]);
            st_lane(m + u[k], mv[k]);
            st_lane(v + u[k], vv[k]);
            const u32x2 p = to_bf16x4(wv[k]);
            if (grad) st_lane(grad + u[k], g);
            if (param) st_lane(param + u[k], p);
            if (full) st_lane(full + u[k], p);
        }
    } else {
        // Codes are computed by every lane before any store is issued.
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!ok[k]) continue;
            gv[k] = avg_bf16x4<N>(a[k], nf);
            adamw_unit(c, gv[k], wv[k], mv[k], vv[k]);
            pv[k] = to_bf16x4(wv[k]);
        }
        QuantWord qw[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t w[2] = {pv[k].x, pv[k].y};
            qw[k] = quant_compute<QB, 4>(w, ok[k], qo.block);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!ok[k]) continue;
            st_lane(master + u[k], wv[k]);
            st_lane(m + u[k], mv[k]);
            st_lane(v + u[k], vv[k]);
            if (grad) st_lane(grad + u[k], gv[k]);
            if (param) st_lane(param + u[k], pv[k]);
            if (full) st_lane(full + u[k], pv[k]);
            quant_emit<QB, 4>(qw[k], u[k], qo);
        }
    }
}

// ------------------------------------------------------------------ flat kernels
// One tile per block; the grid covers the shard once.

__device__ __forceinline__ int64_t tile_base(int units_per_lane) {
    return (int64_t)blockIdx.x * kBlock * units_per_lane + threadIdx.x;
}

template <int N, int CAP, int U>
__global__ __launch_bounds__(kBlock) void k_reduce(Ptrs<CAP> cp, int n_rt, float nf, u32x4* __restrict__ out,
                                                   int64_t n8) {
    reduce8_tile<N, U>(cp.p, n_rt, nf, out, tile_base(U), n8);
}

template <int U, int QB>
__global__ __launch_bounds__(kBlock) void k_adamw(AdamCoef c, const AdamCoef* __restrict__ cdev,
                                                  const u32x2* __restrict__ g, f32x4* __restrict__ master,
                                                  f32x4* __restrict__ m, f32x4* __restrict__ v,
                                                  u32x2* __restrict__ param, u32x2* __restrict__ full, int64_t n4,
                                                  QuantOut qo) {
    adamw_tile<U, QB>(pick_coef(c, cdev), g, master, m, v, param, full, tile_base(U), n4, qo);
}

__global__ __launch_bounds__(kBlock) void k_gather(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n8) {
    copy_tile<u32x4, 1>(src, dst, tile_base(1), n8);
}

template <int N, int CAP, int U, int QB>
__global__ __launch_bounds__(kBlock) void k_fused(AdamCoef c, const AdamCoef* __restrict__ cdev, Ptrs<CAP> cp,
                                                  int n_rt, float nf, f32x4* __restrict__ master,
                                                  f32x4* __restrict__ m, f32x4* __restrict__ v,
                                                  u32x2* __restrict__ grad, u32x2* __restrict__ param,
                                                  u32x2* __restrict__ full, int64_t n4, QuantOut qo) {
    fused_tile<N, U, QB>(pick_coef(c, cdev), cp.p, n_rt, nf, master, m, v, grad, param, full, tile_base(U), n4,
                         qo);
}

// The receiving side of a gather into a k-way slice: blockIdx.y is the source
// whose S-element shard a block copies (8 elements per lane) to dst + y*S.
__global__ __launch_bounds__(kBlock) void k_gather_sources(Ptrs<ZS_MAX_CONTRIBS> src, u32x4* __restrict__ dst,
                                                           int64_t n8) {
    const int q = blockIdx.y;
    copy_tile<u32x4, 1>(reinterpret_cast<const u32x4*>(src.p[q]), dst + (int64_t)q * n8, tile_base(1), n8);
}

// Codes of a bf16 shard, 8 elements per lane.
template <int QB>
__global__ __launch_bounds__(kBlock) void k_quant(const u32x4* __restrict__ p, QuantOut qo, int64_t n8) {
    const int64_t u = tile_base(1);
    const bool ok = u < n8;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (ok) {
        const u32x4 x = ld_in(p + u);
        w[0] = x.x;
        w[1] = x.y;
        w[2] = x.z;
        w[3] = x.w;
    }
    const QuantWord q = quant_compute<QB, 8>(w, ok, qo.block);
    if (ok) quant_emit<QB, 8>(q, u, qo);
}

// The receiving side of the quantized gather: blockIdx.y is the rank whose
// payload a block decodes; a lane decodes U units of 8 elements (units
// kBlock apart), each one 16-byte store. A block's kBlock * U units start on
// a quantization-block boundary (8 * kBlock * U elements is a multiple of
// every block size), so the scales they use are the n_sc consecutive words
// from s0 on: the block loads them once into LDS instead of every lane
// loading its units' scales (32 lanes of a wave reading the same word, four
// times over: 5% slower at the Llama-7B shape). WIDE (every rank's code
// payload a multiple of 16 bytes, so each block's codes start on a 16-byte
// boundary): the block's codes arrive as 16-byte loads, one or two per lane,
// and are handed to the lanes that decode them through LDS; otherwise each
// lane loads its own units' 4 or 8 code bytes (1.7% slower at int4, 4.6% at
// int8 in a probe at the Llama-7B shape).
template <int QB, int U, bool WIDE>
__global__ __launch_bounds__(kBlock) void k_dequant(const char* __restrict__ codes_all,
                                                    const float* __restrict__ scales_all, int64_t code_bytes,
                                                    int64_t n_scales, int block_shift, u32x4* __restrict__ full,
                                                    int64_t s8) {
    static_assert(8 * kBlock * U >= kQuantMaxBlock, "a block's span covers whole quantization blocks");
    constexpr int kWords = QB / 4;                     // code words per 8-element unit
    constexpr int kPieces = kBlock * U * kWords / 4;   // 16-byte pieces of a block's codes
    static_assert(kPieces % kBlock == 0, "whole 16-byte pieces per lane");
    __shared__ float sl[kBlock * U];
    __shared__ u32x4 cl[WIDE ? kPieces : 1];
    const int64_t r = blockIdx.y;
    const int64_t ub = (int64_t)blockIdx.x * kBlock * U;  // the block's first unit
    const char* cb = codes_all + r * code_bytes;
    const float* sb = scales_all + r * n_scales;
    const int n_sc = (kBlock * U * 8) >> block_shift;
    const int64_t s0 = (ub * 8) >> block_shift;
    uint32_t lo[U], hi[U];
    float sv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int j = threadIdx.x + k * kBlock;
        sv[k] = j < n_sc && s0 + j < n_scales ? ld_in(sb + s0 + j) : 0.0f;
    }
    if constexpr (WIDE) {
        // the shard's units end on a piece boundary: a piece is wholly inside or outside
        const u32x4* src = reinterpret_cast<const u32x4*>(cb) + ub * kWords / 4;
        const int64_t pieces_left = (s8 - ub) * kWords / 4;
#pragma unroll
        for (int h = 0; h < kPieces / kBlock; ++h) {
            const int pc = threadIdx.x + h * kBlock;
            cl[pc] = pc < pieces_left ? ld_in(src + pc) : u32x4{0u, 0u, 0u, 0u};
        }
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t u = ub + threadIdx.x + k * kBlock;
            if (u >= s8) continue;
            if constexpr (QB == 8) {
                const u32x2 c = ld_in(reinterpret_cast<const u32x2*>(cb + u * 8));
                lo[k] = c.x;
                hi[k] = c.y;
            } else {
                lo[k] = ld_in(reinterpret_cast<const uint32_t*>(cb + u * 4));
                hi[k] = 0u;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) sl[threadIdx.x + k * kBlock] = sv[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int j = threadIdx.x + k * kBlock;
        const int64_t u = ub + j;
        if (u >= s8) continue;
        if constexpr (WIDE) {
            const uint32_t* words = reinterpret_cast<const uint32_t*>(cl);
            lo[k] = words[j * kWords];
            hi[k] = kWords == 2 ? words[j * kWords + 1] : 0u;
        }
        const float sc = sl[(j * 8) >> block_shift];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int q;
            if constexpr (QB == 8) {
                const uint32_t w = e < 4 ? lo[k] : hi[k];
                q = (int32_t)(w << (24 - 8 * (e & 3))) >> 24;  // signed byte: one v_bfe_i32
            } else {
                q = (int32_t)(lo[k] << (28 - 4 * e)) >> 28;  // signed 4-bit field: one v_bfe_i32
            }
            x[e] = (float)q * sc;
        }
        // A code is finite, so a product is NaN only when the block's scale is
        // NaN (the whole unit is replaced below) or infinite with a zero code
        // (the default NaN, which the rounding keeps a NaN): round without the
        // per-element NaN path.
        u32x4 o;
        o.x = pack2_finite(x[0], x[1]);
        o.y = pack2_finite(x[2], x[3]);
        o.z = pack2_finite(x[4], x[5]);
        o.w = pack2_finite(x[6], x[7]);
        if (sc != sc) o = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        st_lane(full + r * s8 + u, o);
    }
}

// ------------------------------------------------------------------ multi-tensor kernel

// AdamW and the fused step over the pieces: one block per chunk; a chunk is
// one tile (kBlock lanes x kMultiU units of 4 elements) of one piece. The
// piece supplies every pointer and its hyperparameter group; the
// contributions of piece i are cps[i * N .. i * N + N).
template <int OP, int N>
__global__ __launch_bounds__(kBlock) void k_multi(CoefTable ct, const AdamCoef* __restrict__ cdev,
                                                  const MultiHeader* __restrict__ hdr, MultiOffsets off, int n_rt,
                                                  float nf) {
    static_assert(OP == kOpAdamw || OP == kOpAdamwGather || OP == kOpFused,
                  "reduce and gather have kernels of their own");
    if (hdr->magic != kMultiMagic) return;  // not a bound table (e.g. reused memory): touch nothing
    const char* ws = reinterpret_cast<const char*>(hdr);
    const int32_t piece = reinterpret_cast<const int32_t*>(ws + off.chunks)[blockIdx.x];
    const PieceDev pc = reinterpret_cast<const PieceDev*>(ws + off.pieces)[piece];
    const AdamCoef c = pick_coef(ct.c[pc.group], cdev ? cdev + pc.group : nullptr);
    const int flags = hdr->flags;
    // the chunk's range in its piece; piece lengths are multiples of 8
    const int64_t start = (int64_t)((int32_t)blockIdx.x - pc.first_chunk) * kChunkElems;
    const int64_t len = pc.len - start < kChunkElems ? pc.len - start : kChunkElems;
    const int64_t u0 = start >> 2;
    const int64_t base = u0 + threadIdx.x;
    const int64_t limit = u0 + (len >> 2);
    if constexpr (OP == kOpAdamw || OP == kOpAdamwGather) {
        u32x2* full = OP == kOpAdamwGather && (flags & kHasFull) ? reinterpret_cast<u32x2*>(pc.full_own) : nullptr;
        adamw_tile<kMultiU>(c, reinterpret_cast<const u32x2*>(pc.grad), reinterpret_cast<f32x4*>(pc.master),
                            reinterpret_cast<f32x4*>(pc.m), reinterpret_cast<f32x4*>(pc.v),
                            (flags & kHasParam) ? reinterpret_cast<u32x2*>(pc.param) : nullptr, full, base, limit);
    } else {
        const void* const* cps =
            reinterpret_cast<const void* const*>(ws + off.contribs) + (int64_t)piece * (N > 0 ? N : n_rt);
        fused_tile<N, kMultiU>(c, cps, n_rt, nf, reinterpret_cast<f32x4*>(pc.master), reinterpret_cast<f32x4*>(pc.m),
                               reinterpret_cast<f32x4*>(pc.v),
                               (flags & kHasGrad) ? reinterpret_cast<u32x2*>(pc.grad) : nullptr,
                               (flags & kHasParam) ? reinterpret_cast<u32x2*>(pc.param) : nullptr,
                               (flags & kHasFull) ? reinterpret_cast<u32x2*>(pc.full_own) : nullptr, base, limit);
    }
}

// Multi-tensor gather (bf16 copy, no arithmetic): one chunk per block would
// move only 1 KiB after its table lookups, so a block covers kGatherRows rows
// of chunks with 8 elements (one 16-byte access) per lane; each lane looks up
// its own chunk and piece, all rows' lookups and loads are issued before any
// store.
constexpr int kGatherLanesPerChunk = kChunkElems / 8;
constexpr int kGatherChunksPerRow = kBlock / kGatherLanesPerChunk;
constexpr int kGatherRows = 4;
constexpr int kGatherChunksPerBlock = kGatherChunksPerRow * kGatherRows;
static_assert(kChunkElems % 8 == 0 && kBlock % kGatherLanesPerChunk == 0, "gather lanes must tile the wave");

__global__ __launch_bounds__(kBlock) void k_multi_gather(const MultiHeader* __restrict__ hdr, MultiOffsets moff,
                                                         int n_chunks) {
    if (hdr->magic != kMultiMagic) return;
    const char* ws = reinterpret_cast<const char*>(hdr);
    const int32_t* cpiece = reinterpret_cast<const int32_t*>(ws + moff.chunks);
    const PieceDev* pieces = reinterpret_cast<const PieceDev*>(ws + moff.pieces);
    const int lane = threadIdx.x;
    const int64_t first = (int64_t)blockIdx.x * kGatherChunksPerBlock + lane / kGatherLanesPerChunk;
    const int off = (lane % kGatherLanesPerChunk) * 8;
    // phase 1: every row's chunk and piece (rows past the end take chunk 0 and are dropped)
    int32_t chunk[kGatherRows], piece[kGatherRows];
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r) {
        const int64_t c = first + (int64_t)r * kGatherChunksPerRow;
        chunk[r] = c < n_chunks ? (int32_t)c : 0;
        piece[r] = ld_g(cpiece + chunk[r]);
    }
    // phase 2: the pieces' records. A lane past its chunk's end reads the
    // chunk's first vector instead (always inside the piece) and stores nothing,
    // so the loads below need no branch.
    const char* src[kGatherRows];
    char* dst[kGatherRows];
    int64_t len[kGatherRows];
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r) {
        const PieceDev* pc = pieces + piece[r];
        const int64_t start = (int64_t)(chunk[r] - ld_g(&pc->first_chunk)) * kChunkElems;
        const int64_t rest = ld_g(&pc->len) - start;
        const int64_t c = first + (int64_t)r * kGatherChunksPerRow;
        len[r] = c < n_chunks ? (rest < kChunkElems ? rest : kChunkElems) : 0;
        const int o = off < len[r] ? off : 0;
        src[r] = static_cast<const char*>(ld_g(&pc->param)) + 2 * (start + o);
        dst[r] = static_cast<char*>(ld_g(&pc->full_own)) + 2 * (start + off);
    }
    // phase 3: loads, then stores
    u32x4 x[kGatherRows];
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r) x[r] = ld_in(reinterpret_cast<const u32x4*>(src[r]));
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r)
        if (off < len[r]) st_out(reinterpret_cast<u32x4*>(dst[r]), x[r]);
}

// Multi-tensor reduce in the same shape: 8 elements (16-byte loads) per lane,
// two chunks per row of the wave, kReduceRows rows per block; the rows' table
// lookups are batched, then each row sums its N contributions in rank order.
constexpr int kReduceRows = 2;
constexpr int kReduceChunksPerBlock = kGatherChunksPerRow * kReduceRows;

template <int N>
__global__ __launch_bounds__(kBlock) void k_multi_reduce(const MultiHeader* __restrict__ hdr, MultiOffsets moff,
                                                         int n_chunks, int n_rt, float nf) {
    if (hdr->magic != kMultiMagic) return;
    const char* ws = reinterpret_cast<const char*>(hdr);
    const int32_t* cpiece = reinterpret_cast<const int32_t*>(ws + moff.chunks);
    const PieceDev* pieces = reinterpret_cast<const PieceDev*>(ws + moff.pieces);
    const void* const* cps = reinterpret_cast<const void* const*>(ws + moff.contribs);
    const int nq = N > 0 ? N : n_rt;
    const int lane = threadIdx.x;
    const int64_t first = (int64_t)blockIdx.x * kReduceChunksPerBlock + lane / kGatherLanesPerChunk;
    const int off = (lane % kGatherLanesPerChunk) * 8;
    int32_t chunk[kReduceRows], piece[kReduceRows];
#pragma unroll
    for (int r = 0; r < kReduceRows; ++r) {
        const int64_t c = first + (int64_t)r * kGatherChunksPerRow;
        chunk[r] = c < n_chunks ? (int32_t)c : 0;
        piece[r] = ld_g(cpiece + chunk[r]);
    }
    char* grad[kReduceRows];
    int64_t start[kReduceRows], len[kReduceRows];
#pragma unroll
    for (int r = 0; r < kReduceRows; ++r) {
        const PieceDev* pc = pieces + piece[r];
        grad[r] = static_cast<char*>(ld_g(&pc->grad));
        start[r] = (int64_t)(chunk[r] - ld_g(&pc->first_chunk)) * kChunkElems;
        const int64_t rest = ld_g(&pc->len) - start[r];
        const int64_t c = first + (int64_t)r * kGatherChunksPerRow;
        len[r] = c < n_chunks ? (rest < kChunkElems ? rest : kChunkElems) : 0;
    }
#pragma unroll
    for (int r = 0; r < kReduceRows; ++r) {
        // a lane past its chunk's end sums the chunk's first vector (inside the
        // piece) and stores nothing
        const bool ok = off < len[r];
        const int64_t u = (start[r] + (ok ? off : 0)) / 8;
        const bool t = true;
        float a[1][8];
        rank_sum<u32x4, 1, N>(cps + (int64_t)piece[r] * nq, n_rt, &u, &t, a);
        if (ok) {
            u32x4 o;
            o.x = pack2(div_n<N>(a[0][0], nf), div_n<N>(a[0][1], nf));
            o.y = pack2(div_n<N>(a[0][2], nf), div_n<N>(a[0][3], nf));
            o.z = pack2(div_n<N>(a[0][4], nf), div_n<N>(a[0][5], nf));
            o.w = pack2(div_n<N>(a[0][6], nf), div_n<N>(a[0][7], nf));
            st_out(reinterpret_cast<u32x4*>(grad[r]) + u, o);
        }
    }
}

// ------------------------------------------------------------------ accumulation and clipping

// One micro-step: acc += f32(bf16(average)) in units of 4 elements; FIRST
// starts from +0 instead of reading acc.
template <int N, int U, bool FIRST>
__device__ __forceinline__ void accum_tile(const void* const* cp, int n_rt, float nf, f32x4* __restrict__ acc,
                                           int64_t base, int64_t limit) {
    int64_t u[U];
    bool ok[U];
    f32x4 av[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        u[k] = base + (int64_t)k * kBlock;
        ok[k] = u[k] < limit;
        av[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (!FIRST && ok[k]) av[k] = ld_state(acc + u[k]);
    }
    float a[U][4];
    rank_sum<u32x2, U, N>(cp, n_rt, u, ok, a);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (!ok[k]) continue;
        const u32x2 g = avg_bf16x4<N>(a[k], nf);
        f32x4 r;
        r.x = av[k].x + lo_bf16(g.x);
        r.y = av[k].y + hi_bf16(g.x);
        r.z = av[k].z + lo_bf16(g.y);
        r.w = av[k].w + hi_bf16(g.y);
        st_lane(acc + u[k], r);
    }
}

template <int N, int CAP, bool FIRST>
__global__ __launch_bounds__(kBlock) void k_accum(Ptrs<CAP> cp, int n_rt, float nf, f32x4* __restrict__ acc,
                                                  int64_t n4) {
    accum_tile<N, kFusedU, FIRST>(cp.p, n_rt, nf, acc, tile_base(kFusedU), n4);
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ int wave_or(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x |= __shfl_xor(x, off, 64);
    return x;
}

// Block sum over a fixed partition: lane sums, then a wave tree, then (for
// blocks of several waves) the wave sums in order.
__device__ __forceinline__ void block_reduce(double& s, int& bad) {
    s = wave_sum(s);
    bad = wave_or(bad);
    if constexpr (kBlock > 64) {
        __shared__ double ws[kBlock / 64];
        __shared__ int wb[kBlock / 64];
        const int w = threadIdx.x / 64;
        if ((threadIdx.x & 63) == 0) {
            ws[w] = s;
            wb[w] = bad;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            s = 0.0;
            bad = 0;
            for (int i = 0; i < kBlock / 64; ++i) {
                s += ws[i];
                bad |= wb[i];
            }
        }
    }
}

// Stage 1: block b reduces elements [b*kStatsChunk, (b+1)*kStatsChunk) of the
// final gradient acc/divisor: partial sum of squares (double) and a flag.
__global__ __launch_bounds__(kBlock) void k_stats(const f32x4* __restrict__ acc, float divisor, int64_t n4,
                                                  double* __restrict__ part, int32_t* __restrict__ flags) {
    const int64_t u0 = (int64_t)blockIdx.x * (kStatsChunk / 4);
    const int64_t u1 = u0 + kStatsChunk / 4 < n4 ? u0 + kStatsChunk / 4 : n4;
    double s = 0.0;
    int bad = 0;
    for (int64_t u = u0 + threadIdx.x; u < u1; u += kBlock) {
        const f32x4 x = ld_in(acc + u);
        const float g[4] = {x.x / divisor, x.y / divisor, x.z / divisor, x.w / divisor};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bad |= !__builtin_isfinite(g[e]);
            s = s + (double)g[e] * (double)g[e];
        }
    }
    block_reduce(s, bad);
    if (threadIdx.x == 0) {
        part[blockIdx.x] = s;
        flags[blockIdx.x] = bad;
    }
}

// Stage 2 (one block of kFinalThreads): thread i sums partials i, i + 1024,
// ... in order, then a fixed tree within each wave and the wave sums in
// order: a fixed partition, so reruns give identical bits.
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void k_stats_final(const double* __restrict__ part,
                                                               const int32_t* __restrict__ flags, int64_t nb,
                                                               double* __restrict__ sumsq_out,
                                                               int32_t* __restrict__ nonfinite_out) {
    double s = 0.0;
    int bad = 0;
    for (int64_t i = threadIdx.x; i < nb; i += kFinalThreads) {
        s = s + part[i];
        bad |= flags[i];
    }
    s = wave_sum(s);
    bad = wave_or(bad);
    __shared__ double ws[kFinalThreads / 64];
    __shared__ int wb[kFinalThreads / 64];
    const int w = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) {
        ws[w] = s;
        wb[w] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        int b = 0;
        for (int i = 0; i < kFinalThreads / 64; ++i) {
            t += ws[i];
            b |= wb[i];
        }
        *sumsq_out = t;
        *nonfinite_out = b ? 1 : 0;
    }
}

// One thread: the all-reduced norm (ranks added in order) to an fp32 factor.
__global__ void k_clip_scale(const double* __restrict__ sumsq, const int32_t* __restrict__ nonfinite, int n,
                             double max_norm, float* __restrict__ scale_out, int32_t* __restrict__ skip_out) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    double total = 0.0;
    int bad = 0;
    for (int r = 0; r < n; ++r) {
        total = total + sumsq[r];
        bad |= nonfinite[r];
    }
    const double coef = max_norm / (sqrt(total) + 1e-6);
    *scale_out = (float)(coef < 1.0 ? coef : 1.0);
    *skip_out = bad ? 1 : 0;
}

// AdamW from the fp32 accumulator: element gradient (acc / divisor) * scale.
template <int U>
__device__ __forceinline__ void adamw_accum_tile(const AdamCoef& c, const f32x4* __restrict__ acc, float divisor,
                                                 float scale, f32x4* __restrict__ master, f32x4* __restrict__ m,
                                                 f32x4* __restrict__ v, u32x2* __restrict__ param,
                                                 u32x2* __restrict__ full, int64_t base, int64_t limit) {
    f32x4 av[U], wv[U], mv[U], vv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t u = base + (int64_t)k * kBlock;
        if (u < limit) {
            av[k] = ld_in(acc + u);
            wv[k] = ld_state(master + u);
            mv[k] = ld_state(m + u);
            vv[k] = ld_state(v + u);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t u = base + (int64_t)k * kBlock;
        if (u >= limit) continue;
        float w[4] = {wv[k].x, wv[k].y, wv[k].z, wv[k].w};
        float mm[4] = {mv[k].x, mv[k].y, mv[k].z, mv[k].w};
        float vv4[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
        const float ac[4] = {av[k].x, av[k].y, av[k].z, av[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g = (ac[e] / divisor) * scale;
            adamw_elem(c, g, w[e], mm[e], vv4[e]);
        }
        const f32x4 wn{w[0], w[1], w[2], w[3]};
        st_lane(master + u, wn);
        st_lane(m + u, f32x4{mm[0], mm[1], mm[2], mm[3]});
        st_lane(v + u, f32x4{vv4[0], vv4[1], vv4[2], vv4[3]});
        const u32x2 p = to_bf16x4(wn);
        if (param) st_lane(param + u, p);
        if (full) st_lane(full + u, p);
    }
}

template <int U>
__global__ __launch_bounds__(kBlock) void k_adamw_accum(AdamCoef c, const AdamCoef* __restrict__ cdev,
                                                        const f32x4* __restrict__ acc, float divisor,
                                                        const float* __restrict__ scale_p,
                                                        const int32_t* __restrict__ skip_p,
                                                        f32x4* __restrict__ master, f32x4* __restrict__ m,
                                                        f32x4* __restrict__ v, u32x2* __restrict__ param,
                                                        u32x2* __restrict__ full, int64_t n4) {
    if (skip_p && *skip_p) return;  // uniform: the whole grid skips the step
    const float scale = scale_p ? *scale_p : 1.0f;
    adamw_accum_tile<U>(pick_coef(c, cdev), acc, divisor, scale, master, m, v, param, full, tile_base(U), n4);
}

// ------------------------------------------------------------------ launch helpers

// Blocks of a tile launch over `units` lane-units, `per_lane` units per lane.
unsigned grid_for(int64_t units, int per_lane) {
    const int64_t per_block = (int64_t)kBlock * per_lane;
    int64_t blocks = (units + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

unsigned reduce_lds(int n) {
    if (n >= kWideN) return kReduceWideLds;
    if (n >= kMidN) return kReduceMidLds;
    return (unsigned)n * kReduceLdsPerRank < kReduceLds ? (unsigned)n * kReduceLdsPerRank : kReduceLds;
}

template <int N, int CAP>
int launch_reduce_t(const void* const* contribs, int n, void* grad, int64_t len, hipStream_t s) {
    Ptrs<CAP> cp{};
    for (int q = 0; q < n; ++q) cp.p[q] = contribs[q];
    const int64_t n8 = len / 8;
    hipLaunchKernelGGL((k_reduce<N, CAP, kReduceU>), dim3(grid_for(n8, kReduceU)), dim3(kBlock),
                       reduce_lds(n), s, cp, n, (float)n, reinterpret_cast<u32x4*>(grad), n8);
    return (int)hipGetLastError();
}

template <int N, int CAP, int QB>
int launch_fused_q(const AdamCoef& c, const AdamCoef* cdev, const void* const* contribs, int n, float* master,
                   float* m, float* v, void* grad, void* param, void* full, int64_t len, const QuantOut& qo,
                   hipStream_t s) {
    Ptrs<CAP> cp{};
    for (int q = 0; q < n; ++q) cp.p[q] = contribs[q];
    const int64_t n4 = len / 4;
    const unsigned lds = QB != 0 ? kFusedQuantLds
                         : n <= 2 ? kFusedTinyLds
                         : n <= 4 ? kFusedNarrowLds
                         : (N == 16 || N == 32) ? kFusedMidLds
                                                : kFusedLds;
    hipLaunchKernelGGL((k_fused<N, CAP, kFusedU, QB>), dim3(grid_for(n4, kFusedU)), dim3(kBlock), lds, s, c, cdev,
                       cp, n, (float)n, reinterpret_cast<f32x4*>(master), reinterpret_cast<f32x4*>(m),
                       reinterpret_cast<f32x4*>(v), reinterpret_cast<u32x2*>(grad),
                       reinterpret_cast<u32x2*>(param), reinterpret_cast<u32x2*>(full), n4, qo);
    return (int)hipGetLastError();
}

template <int N, int CAP>
int launch_fused_t(const AdamCoef& c, const AdamCoef* cdev, const void* const* contribs, int n, float* master,
                   float* m, float* v, void* grad, void* param, void* full, int64_t len, const QuantOut* q,
                   hipStream_t s) {
    if (!q)
        return launch_fused_q<N, CAP, 0>(c, cdev, contribs, n, master, m, v, grad, param, full, len, QuantOut{}, s);
    if (q->bits == 8)
        return launch_fused_q<N, CAP, 8>(c, cdev, contribs, n, master, m, v, grad, param, full, len, *q, s);
    return launch_fused_q<N, CAP, 4>(c, cdev, contribs, n, master, m, v, grad, param, full, len, *q, s);
}

template <int OP, int N>
int launch_multi_t(const CoefTable& c, const AdamCoef* cdev, const void* ws, const MultiOffsets& off, int n_chunks,
                   int n, hipStream_t s) {
    hipLaunchKernelGGL((k_multi<OP, N>), dim3((unsigned)n_chunks), dim3(kBlock),
                       OP == kOpFused ? (n <= 2 ? kMultiFusedTinyLds : kMultiFusedLds) : kMultiLds, s, c, cdev,
                       reinterpret_cast<const MultiHeader*>(ws), off, n, (float)n);
    return (int)hipGetLastError();
}

template <int N>
int launch_multi_reduce_t(const void* ws, const MultiOffsets& off, int n_chunks, int n, hipStream_t s) {
    hipLaunchKernelGGL((k_multi_reduce<N>),
                       dim3((unsigned)((n_chunks + kReduceChunksPerBlock - 1) / kReduceChunksPerBlock)), dim3(kBlock),
                       n <= 2 ? kMultiReduceTinyLds : n <= 4 ? kMultiReduceNarrowLds : kMultiReduceLds, s,
                       reinterpret_cast<const MultiHeader*>(ws), off, n_chunks, n, (float)n);
    return (int)hipGetLastError();
}

int launch_multi_reduce(const void* ws, const MultiOffsets& off, int n_chunks, int n, hipStream_t s) {
    switch (n) {
        case 1: return launch_multi_reduce_t<1>(ws, off, n_chunks, n, s);
        case 2: return launch_multi_reduce_t<2>(ws, off, n_chunks, n, s);
        case 4: return launch_multi_reduce_t<4>(ws, off, n_chunks, n, s);
        case 8: return launch_multi_reduce_t<8>(ws, off, n_chunks, n, s);
        case 16: return launch_multi_reduce_t<16>(ws, off, n_chunks, n, s);
        // From 32 ranks on the runtime loop: a lane of this kernel loads its
        // own rank pointers (its chunk's piece), and a fully unrolled 32- or
        // 64-rank loop keeps them all live (187 and 458 VGPRs; 9% and 2.9x
        // slower than the runtime loop at the Llama-7B wrap shape).
        default: return launch_multi_reduce_t<0>(ws, off, n_chunks, n, s);
    }
}

template <int OP>
int launch_multi_op(const CoefTable& c, const AdamCoef* cdev, const void* ws, const MultiOffsets& off, int n_chunks,
                    int n, hipStream_t s) {
    switch (n) {
        case 1: return launch_multi_t<OP, 1>(c, cdev, ws, off, n_chunks, n, s);
        case 2: return launch_multi_t<OP, 2>(c, cdev, ws, off, n_chunks, n, s);
        case 4: return launch_multi_t<OP, 4>(c, cdev, ws, off, n_chunks, n, s);
        case 8: return launch_multi_t<OP, 8>(c, cdev, ws, off, n_chunks, n, s);
        case 16: return launch_multi_t<OP, 16>(c, cdev, ws, off, n_chunks, n, s);
        case 32: return launch_multi_t<OP, 32>(c, cdev, ws, off, n_chunks, n, s);
        case 64: return launch_multi_t<OP, 64>(c, cdev, ws, off, n_chunks, n, s);
        default: return launch_multi_t<OP, 0>(c, cdev, ws, off, n_chunks, n, s);
    }
}

template <int N, int CAP>
int launch_accum_t(const void* const* contribs, int n, float* acc, int first, int64_t len, hipStream_t s) {
    Ptrs<CAP> cp{};
    for (int q = 0; q < n; ++q) cp.p[q] = contribs[q];
    const int64_t n4 = len / 4;
    const unsigned lds = n <= 2 ? kAccumTinyLds : n <= 4 ? kAccumNarrowLds : kAccumLds;
    if (first)
        hipLaunchKernelGGL((k_accum<N, CAP, true>), dim3(grid_for(n4, kFusedU)), dim3(kBlock), lds, s, cp, n,
                           (float)n, reinterpret_cast<f32x4*>(acc), n4);
    else
        hipLaunchKernelGGL((k_accum<N, CAP, false>), dim3(grid_for(n4, kFusedU)), dim3(kBlock), lds, s, cp, n,
                           (float)n, reinterpret_cast<f32x4*>(acc), n4);
    return (int)hipGetLastError();
}

template <int QB>
int launch_adamw_q(const AdamCoef& c, const AdamCoef* cdev, const void* grad, float* master, float* m, float* v,
                   void* param, void* full_at_own, int64_t len, const QuantOut& qo, hipStream_t s) {
    const int64_t n4 = len / 4;
    hipLaunchKernelGGL((k_adamw<kAdamwU, QB>), dim3(grid_for(n4, kAdamwU)), dim3(kBlock), kAdamwLds, s, c, cdev,
                       reinterpret_cast<const u32x2*>(grad), reinterpret_cast<f32x4*>(master),
                       reinterpret_cast<f32x4*>(m), reinterpret_cast<f32x4*>(v), reinterpret_cast<u32x2*>(param),
                       reinterpret_cast<u32x2*>(full_at_own), n4, qo);
    return (int)hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ public launchers

int launch_reduce(const void* const* contribs, int n, void* grad, int64_t len, void* stream) {
    if (len <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    switch (n) {
        case 1: return launch_reduce_t<1, 1>(contribs, n, grad, len, s);
        case 2: return launch_reduce_t<2, 2>(contribs, n, grad, len, s);
        case 4: return launch_reduce_t<4, 4>(contribs, n, grad, len, s);
        case 8: return launch_reduce_t<8, 8>(contribs, n, grad, len, s);
        case 16: return launch_reduce_t<16, 16>(contribs, n, grad, len, s);
        case 32: return launch_reduce_t<32, 32>(contribs, n, grad, len, s);
        case 64: return launch_reduce_t<64, 64>(contribs, n, grad, len, s);
        default: return launch_reduce_t<0, ZS_MAX_CONTRIBS>(contribs, n, grad, len, s);
    }
}

int launch_adamw(const AdamCoef& c, const void* grad, float* master, float* m, float* v, void* param,
                 void* full_at_own, int64_t len, void* stream, const QuantOut* q, const AdamCoef* cdev) {
    if (len <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    if (!q) return launch_adamw_q<0>(c, cdev, grad, master, m, v, param, full_at_own, len, QuantOut{}, s);
    if (q->bits == 8) return launch_adamw_q<8>(c, cdev, grad, master, m, v, param, full_at_own, len, *q, s);
    return launch_adamw_q<4>(c, cdev, grad, master, m, v, param, full_at_own, len, *q, s);
}

int launch_quantize(const QuantOut& q, const void* param, int64_t len, void* stream) {
    if (len <= 0) return 0;
    const int64_t n8 = len / 8;
    hipStream_t s = (hipStream_t)stream;
    if (q.bits == 8)
        hipLaunchKernelGGL(k_quant<8>, dim3(grid_for(n8, 1)), dim3(kBlock), kGatherLds, s,
                           reinterpret_cast<const u32x4*>(param), q, n8);
    else
        hipLaunchKernelGGL(k_quant<4>, dim3(grid_for(n8, 1)), dim3(kBlock), kGatherLds, s,
                           reinterpret_cast<const u32x4*>(param), q, n8);
    return (int)hipGetLastError();
}

int launch_dequant(int bits, int block, const void* codes_all, const float* scales_all, int64_t code_bytes,
                   int64_t n_scales, int n_ranks, void* full, int64_t S, void* stream) {
    if (S <= 0 || n_ranks <= 0) return 0;
    const int64_t s8 = S / 8;
    int shift = 0;
    while ((1 << shift) < block) ++shift;
    const dim3 grid(grid_for(s8, kDequantU), (unsigned)n_ranks);
    hipStream_t s = (hipStream_t)stream;
    const char* cb = static_cast<const char*>(codes_all);
    u32x4* out = reinterpret_cast<u32x4*>(full);
    // 16-byte code loads need every rank's payload to start 16-byte aligned
    // (codes_all itself is 16-byte aligned)
    const bool wide = code_bytes % 16 == 0;
    if (bits == 8 && wide)
        hipLaunchKernelGGL((k_dequant<8, kDequantU, true>), grid, dim3(kBlock), kDequantLds, s, cb, scales_all,
                           code_bytes, n_scales, shift, out, s8);
    else if (bits == 8)
        hipLaunchKernelGGL((k_dequant<8, kDequantU, false>), grid, dim3(kBlock), kDequantLds, s, cb, scales_all,
                           code_bytes, n_scales, shift, out, s8);
    else if (wide)
        hipLaunchKernelGGL((k_dequant<4, kDequantU, true>), grid, dim3(kBlock), kDequantLds, s, cb, scales_all,
                           code_bytes, n_scales, shift, out, s8);
    else
        hipLaunchKernelGGL((k_dequant<4, kDequantU, false>), grid, dim3(kBlock), kDequantLds, s, cb, scales_all,
                           code_bytes, n_scales, shift, out, s8);
    return (int)hipGetLastError();
}

int launch_gather(const void* param, void* full_at_own, int64_t len, void* stream) {
    if (len <= 0) return 0;
    const int64_t n8 = len / 8;
    hipLaunchKernelGGL(k_gather, dim3(grid_for(n8, 1)), dim3(kBlock), kGatherLds, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(param), reinterpret_cast<u32x4*>(full_at_own), n8);
    return (int)hipGetLastError();
}

int launch_gather_sources(const void* const* srcs, int n, void* dst, int64_t len, void* stream) {
    if (len <= 0 || n <= 0) return 0;
    const int64_t n8 = len / 8;
    for (int q0 = 0; q0 < n; q0 += ZS_MAX_CONTRIBS) {
        const int cnt = n - q0 < ZS_MAX_CONTRIBS ? n - q0 : ZS_MAX_CONTRIBS;
        Ptrs<ZS_MAX_CONTRIBS> sp{};
        for (int q = 0; q < cnt; ++q) sp.p[q] = srcs[q0 + q];
        hipLaunchKernelGGL(k_gather_sources, dim3(grid_for(n8, 1), (unsigned)cnt), dim3(kBlock), kGatherLds,
                           (hipStream_t)stream, sp, reinterpret_cast<u32x4*>(dst) + (int64_t)q0 * n8, n8);
        if (int e = (int)hipGetLastError()) return e;
    }
    return 0;
}

int launch_fused(const AdamCoef& c, const void* const* contribs, int n, float* master, float* m, float* v,
                 void* grad, void* param, void* full_at_own, int64_t len, void* stream, const QuantOut* q,
                 const AdamCoef* cdev) {
    if (len <= 0) return 0;
    if (kSplitMinN > 0 && n >= kSplitMinN && grad) {
        // Large N: a nearly read-only reduce, then AdamW writing the outputs.
        // Same bytes in every buffer as the one-pass kernel.
        if (int e = launch_reduce(contribs, n, grad, len, stream)) return e;
        return launch_adamw(c, grad, master, m, v, param, full_at_own, len, stream, q, cdev);
    }
    hipStream_t s = (hipStream_t)stream;
    void* f = full_at_own;
    switch (n) {
        case 1: return launch_fused_t<1, 1>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 2: return launch_fused_t<2, 2>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 4: return launch_fused_t<4, 4>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 8: return launch_fused_t<8, 8>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 16: return launch_fused_t<16, 16>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 32: return launch_fused_t<32, 32>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        case 64: return launch_fused_t<64, 64>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
        default:
            return launch_fused_t<0, ZS_MAX_CONTRIBS>(c, cdev, contribs, n, master, m, v, grad, param, f, len, q, s);
    }
}

int launch_multi(int op, const CoefTable* c, const void* workspace, const MultiOffsets& off, int n_chunks,
                 int n_contribs, void* stream, const AdamCoef* cdev) {
    if (n_chunks <= 0) return 0;
    const CoefTable cc = c ? *c : CoefTable{};
    hipStream_t s = (hipStream_t)stream;
    switch (op) {
        case kOpReduce: return launch_multi_reduce(workspace, off, n_chunks, n_contribs, s);
        case kOpAdamw: return launch_multi_t<kOpAdamw, 1>(cc, cdev, workspace, off, n_chunks, 1, s);
        case kOpAdamwGather: return launch_multi_t<kOpAdamwGather, 1>(cc, cdev, workspace, off, n_chunks, 1, s);
        case kOpGather:
            hipLaunchKernelGGL(k_multi_gather, dim3((unsigned)((n_chunks + kGatherChunksPerBlock - 1) /
                                                               kGatherChunksPerBlock)),
                               dim3(kBlock), kMultiGatherLds, s, reinterpret_cast<const MultiHeader*>(workspace),
                               off, n_chunks);
            return (int)hipGetLastError();
        default: return launch_multi_op<kOpFused>(cc, cdev, workspace, off, n_chunks, n_contribs, s);
    }
}

int launch_accumulate(const void* const* contribs, int n, float* acc, int first, int64_t len, void* stream) {
    if (len <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    switch (n) {
        case 1: return launch_accum_t<1, 1>(contribs, n, acc, first, len, s);
        case 2: return launch_accum_t<2, 2>(contribs, n, acc, first, len, s);
        case 4: return launch_accum_t<4, 4>(contribs, n, acc, first, len, s);
        case 8: return launch_accum_t<8, 8>(contribs, n, acc, first, len, s);
        case 16: return launch_accum_t<16, 16>(contribs, n, acc, first, len, s);
        case 32: return launch_accum_t<32, 32>(contribs, n, acc, first, len, s);
        case 64: return launch_accum_t<64, 64>(contribs, n, acc, first, len, s);
        default: return launch_accum_t<0, ZS_MAX_CONTRIBS>(contribs, n, acc, first, len, s);
    }
}

// The workspace holds nb doubles, then (256-byte aligned) nb int32 flags.
int launch_grad_stats(const float* acc, float divisor, double* sumsq_out, int32_t* nonfinite_out, void* workspace,
                      int64_t len, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int64_t nb = (len + kStatsChunk - 1) / kStatsChunk;
    double* part = reinterpret_cast<double*>(workspace);
    int32_t* flags = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + ((nb * 8 + 255) / 256) * 256);
    if (nb > 0)
        hipLaunchKernelGGL(k_stats, dim3((unsigned)nb), dim3(kBlock), 0, s, reinterpret_cast<const f32x4*>(acc),
                           divisor, len / 4, part, flags);
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(kFinalThreads), 0, s, part, flags, nb, sumsq_out, nonfinite_out);
    return (int)hipGetLastError();
}

// Partials of zs_grad_stats_noalloc, for callers that cannot allocate device
// memory. Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept.
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int launch_grad_stats_noalloc(const float* acc, float divisor, double* sumsq_out, int32_t* nonfinite_out,
                              int64_t len, void* stream) {
    // the copy of the array on the GPU the kernels run on: the stream's device
    // (the current device for the null stream)
    hipDevice_t dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            // looked up once per device, with that device current
            int cur = 0;
            e = hipGetDevice(&cur);
            if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
            if (e == hipSuccess) e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t r = hipSetDevice(cur);
                if (e == hipSuccess) e = r;
            }
            if (e != hipSuccess) {
                g_scratch_ptr[dev] = nullptr;
                return (int)e;
            }
        }
        ptr = g_scratch_ptr[dev];
    }
    // k_stats writes every partial and flag before k_stats_final reads them,
    // so nothing of a previous call's contents needs clearing.
    return launch_grad_stats(acc, divisor, sumsq_out, nonfinite_out, ptr, len, stream);
}

int launch_clip_scale(const double* sumsq, const int32_t* nonfinite, int n_ranks, double max_norm, float* scale_out,
                      int32_t* skip_out, void* stream) {
    hipLaunchKernelGGL(k_clip_scale, dim3(1), dim3(64), 0, (hipStream_t)stream, sumsq, nonfinite, n_ranks, max_norm,
                       scale_out, skip_out);
    return (int)hipGetLastError();
}

int launch_adamw_accum(const AdamCoef& c, const float* acc, float divisor, const float* scale, const int32_t* skip,
                       float* master, float* m, float* v, void* param, void* full_at_own, int64_t len, void* stream,
                       const AdamCoef* cdev) {
    if (len <= 0) return 0;
    const int64_t n4 = len / 4;
    hipLaunchKernelGGL((k_adamw_accum<kAdamwU>), dim3(grid_for(n4, kAdamwU)), dim3(kBlock), kAdamwLds,
                       (hipStream_t)stream, c, cdev, reinterpret_cast<const f32x4*>(acc), divisor, scale, skip,
                       reinterpret_cast<f32x4*>(master), reinterpret_cast<f32x4*>(m), reinterpret_cast<f32x4*>(v),
                       reinterpret_cast<u32x2*>(param), reinterpret_cast<u32x2*>(full_at_own), n4);
    return (int)hipGetLastError();
}

int copy_h2d_sync(void* dst, const void* src, int64_t bytes, void* stream) {
    hipError_t e = hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return (int)e;
    return (int)hipStreamSynchronize((hipStream_t)stream);
}

const char* hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace zs
