// Internal declarations shared by the host side (plan, C ABI) and the HIP
// kernel launchers. Not part of the public ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/zs.h"

namespace zs {

// fp32 scalars of one AdamW step, each rounded once from double. The same
// layout as the public zs_adamw_coefs.
struct AdamCoef {
    float b1, omb1, b2, omb2, lr, eps, decay, bc1, bc2;
};
static_assert(sizeof(AdamCoef) == sizeof(zs_adamw_coefs), "AdamCoef mirrors zs_adamw_coefs");

AdamCoef make_coef(const zs_adamw_hparams& hp);

// Per-group AdamW scalars, passed by value to the multi-tensor kernel.
struct CoefTable {
    AdamCoef c[ZS_MAX_GROUPS];
};

struct TensorEntry {
    int32_t group = 0;       // hyperparameter group
    int32_t replicated = 0;  // 1: held whole by every rank (persistence threshold)
    int64_t numel;
    int64_t flat_off;  // FLAT: start in the flat buffer; PER_TENSOR: packed start of padded tensor
    int64_t padded;    // PER_TENSOR: T_i; FLAT: numel
    int64_t own_lo, own_hi;  // owned range, tensor-local coordinates
    int64_t shard_off;       // start of the owned range in the packed shard
    int64_t first_chunk = 0; // PER_TENSOR: index of the owned piece's first multi-tensor chunk
};

}  // namespace zs

struct zs_plan {
    int32_t layout;
    int32_t world;
    int32_t rank;
    int32_t align;
    int64_t T;  // padded flat length (PER_TENSOR: sum of T_i)
    int64_t S;  // owned elements (PER_TENSOR: sum of S_i)
    std::vector<zs::TensorEntry> tensors;
    // Multi-tensor chunks (kChunkElems owned elements each, the last of a
    // piece shorter), in order: the piece each one belongs to.
    std::vector<int32_t> chunk_piece;
};

namespace zs {

// Launch shape shared by the host (chunk table) and the kernels: one 64-lane
// wave per block (128- to 512-thread blocks measured slower), and one
// 4-element unit per lane in a multi-tensor chunk (2-8 measured slower for
// the fused step).
constexpr int kBlockThreads = 64;  // threads per block of every kernel
constexpr int kMultiU = 1;         // 4-element units per lane in a multi-tensor chunk
// Multi-tensor chunk length (elements): one block per chunk, one tile each.
constexpr int32_t kChunkElems = kBlockThreads * 4 * kMultiU;

// Device-side multi-tensor table, stored at the start of the workspace.
struct MultiHeader {
    uint64_t magic;
    int32_t n_pieces;
    int32_t n_chunks;
    int32_t n_contribs;
    int32_t flags;
    int64_t pieces_off;    // byte offset of PieceDev[n_pieces]
    int64_t contribs_off;  // byte offset of const void*[n_pieces * n_contribs]
    int64_t chunks_off;    // byte offset of int32_t[n_chunks]: each chunk's piece
};

struct PieceDev {
    void* grad;
    float* master;
    float* m;
    float* v;
    void* param;
    void* full_own;  // gathered tensor + r*S_i (already offset)
    int64_t len;          // S_i
    int32_t group;        // index into the kernel's coefficient table
    int32_t first_chunk;  // chunk c of the piece covers [(c - first_chunk) * kChunkElems, ...)
};

enum MultiFlags : int32_t {
    kHasGrad = 1,
    kHasState = 2,
    kHasParam = 4,
    kHasFull = 8,
    kHasContribs = 16,
};

constexpr uint64_t kMultiMagic = 0x7A734D554C544931ull;

// Quantized output of the updated shard (block-wise symmetric codes).
struct QuantOut {
    void* codes;    // this rank's codes: bits/8 bytes per element
    float* scales;  // one fp32 scale per block
    int32_t bits;   // 4 or 8
    int32_t block;  // elements per block: a power of two in [kQuantMinBlock, kQuantMaxBlock]
};
constexpr int32_t kQuantMinBlock = 8;
constexpr int32_t kQuantMaxBlock = 256;

// Launchers (zs_kernels.hip). They return a hipError_t value cast to int.
int launch_reduce(const void* const* contribs, int n, void* grad, int64_t len, void* stream);
// launch_adamw / launch_fused: q (optional) also writes the updated shard's
// codes and scales.
// cdev (optional): read the AdamW scalars from device memory when the kernels
// run instead of taking c (one AdamCoef; one per group for launch_multi).
int launch_adamw(const AdamCoef& c, const void* grad, float* master, float* m, float* v,
                 void* param, void* full_at_own, int64_t len, void* stream, const QuantOut* q = nullptr,
                 const AdamCoef* cdev = nullptr);
int launch_gather(const void* param, void* full_at_own, int64_t len, void* stream);
// n shards of len elements each, srcs[q] copied to dst + q*len (one launch per
// ZS_MAX_CONTRIBS sources).
int launch_gather_sources(const void* const* srcs, int n, void* dst, int64_t len, void* stream);
int launch_fused(const AdamCoef& c, const void* const* contribs, int n, float* master, float* m,
                 float* v, void* grad, void* param, void* full_at_own, int64_t len, void* stream,
                 const QuantOut* q = nullptr, const AdamCoef* cdev = nullptr);
int launch_quantize(const QuantOut& q, const void* param, int64_t len, void* stream);
// Dequantizes n_ranks payloads (codes end to end, code_bytes each; scales end
// to end, n_scales each) into full[r*S, (r+1)*S) for every rank r.
int launch_dequant(int bits, int block, const void* codes_all, const float* scales_all, int64_t code_bytes,
                   int64_t n_scales, int n_ranks, void* full, int64_t S, void* stream);

// Elements one block of the stats kernel reduces (kBlockThreads lanes x 4
// elements x 16 trips).
constexpr int64_t kStatsChunk = (int64_t)kBlockThreads * 4 * 16;

int launch_accumulate(const void* const* contribs, int n, float* acc, int first, int64_t len, void* stream);
int launch_grad_stats(const float* acc, float divisor, double* sumsq_out, int32_t* nonfinite_out, void* workspace,
                      int64_t len, void* stream);
// The same two kernels with their partials in the library's statically
// allocated device array (kNoallocScratchBytes per GPU) instead of a caller
// workspace; the caller has checked that the shard's partials fit.
constexpr int64_t kNoallocScratchBytes = (int64_t)4 << 20;
int launch_grad_stats_noalloc(const float* acc, float divisor, double* sumsq_out, int32_t* nonfinite_out,
                              int64_t len, void* stream);
int launch_clip_scale(const double* sumsq, const int32_t* nonfinite, int n_ranks, double max_norm, float* scale_out,
                      int32_t* skip_out, void* stream);
int launch_adamw_accum(const AdamCoef& c, const float* acc, float divisor, const float* scale, const int32_t* skip,
                       float* master, float* m, float* v, void* param, void* full_at_own, int64_t len, void* stream,
                       const AdamCoef* cdev = nullptr);

// kOpAdamwGather: AdamW writing the parameter and the gathered slice where
// bound (the second pass of the two-pass fused step).
enum MultiOp : int32_t { kOpReduce = 0, kOpAdamw = 1, kOpGather = 2, kOpFused = 3, kOpAdamwGather = 4 };
// Byte offsets of the tables in a bound workspace (the header holds the same
// values; the kernels take them as arguments to save a dependent load).
struct MultiOffsets {
    int64_t pieces;
    int64_t contribs;
    int64_t chunks;
};
int launch_multi(int op, const CoefTable* c, const void* workspace, const MultiOffsets& off, int n_chunks,
                 int n_contribs, void* stream, const AdamCoef* cdev = nullptr);
int copy_h2d_sync(void* dst, const void* src, int64_t bytes, void* stream);

// Host AdamW over n elements with n_threads host threads (zs_host_adamw.cpp);
// p may be nullptr.
void host_adamw(const AdamCoef& c, const uint16_t* g, float* master, float* m, float* v, uint16_t* p, int64_t n,
                int n_threads);
// zs_offload.hip: 1 if p is page-locked host memory known to the HIP runtime.
int is_pinned_host(const void* p);
// CPU-offloaded step of `len` elements in chunks of `chunk`; returns a
// hipError_t value.
int offload_adamw(const AdamCoef& c, const void* grad_dev, float* master, float* m, float* v, void* grad_host,
                  void* param_host, void* param_dev, void* full_own_dev, int64_t len, int64_t chunk, int n_threads,
                  void* stream);
const char* hip_error_text(int err);

}  // namespace zs
