/*
 * zs.h -- C ABI of one rank's shard-local step of ZeRO / FSDP data parallelism
 * on AMD Instinct MI355X (gfx950).
 *
 * The step (sources: the four pages on ZeRO and FSDP):
 *   1. plan    flatten the model's tensors into one flat buffer (FSDP's
 *              FlatParameter: "ZeRO vs FSDP: A Rigorous Dissection for
 *              Distributed Training Engineers", section 3.2) or shard each
 *              tensor on its own (FSDP2's per-parameter sharding, "从 Data
 *              Parallel 到 ZeRO/FSDP", section "ZeRO 与 FSDP 的关系"); pad and
 *              cut into N equal shards, rank r owning shard r ("ZeRO vs FSDP...",
 *              section 2).
 *   2. reduce  average the N ranks' bf16 gradient contributions for the owned
 *              shard, the slice a reduce-scatter leaves on rank r ("ZeRO vs
 *              FSDP...", section 2.1; "从 Data Parallel 到 ZeRO/FSDP", sections
 *              "Data Parallel 保证的数学语义" and "DDP 为什么单卡仍是 16P").
 *   3. AdamW   mixed-precision AdamW on the owned shard's 16 bytes/param of
 *              persistent state: bf16 param, bf16 grad, fp32 master, m and v
 *              ("FSDP2's parameter lifecycle, and the wrap-policy bug...",
 *              section "16 bytes per parameter is where planning starts";
 *              "ZeRO vs FSDP...", section 1.1).
 *   4. gather  write the updated bf16 shard into the full gathered parameter
 *              buffer at its offset, this rank's part of the all-gather
 *              ("ZeRO vs FSDP...", section 2.1; "从 Data Parallel 到 ZeRO/FSDP",
 *              section "ZeRO Stage 1").
 *
 * Arithmetic of steps 2-3, per owned element j (fp32 IEEE operations, one
 * rounding each, in this order; bf16 narrowing is round-to-nearest-even):
 *   acc = +0; for q in 0..N-1: acc += f32(contrib_q[j]);  g = bf16(acc / N)
 *   gf = f32(g); w = master*(1-lr*wd); m = b1*m + (1-b1)*gf;
 *   v = b2*v + (1-b2)*(gf*gf); mhat = m/(1-b1^t); vhat = v/(1-b2^t);
 *   w = w - lr*(mhat/(sqrt(vhat)+eps)); master = w; param = bf16(w)
 * The scalars (1-b1, 1-lr*wd, 1-b1^t, ...) are computed in double on the
 * host and rounded once to fp32.
 *
 * Memory: every device buffer is owned by the caller (normally a PyTorch
 * tensor); the library never allocates, frees or retains device memory. A
 * plan is owned by the library between zs_shard_plan and zs_plan_destroy,
 * is immutable, and may be shared between threads.
 *
 * Dtypes are fixed: contributions, gradients and parameters are bf16 (raw
 * 16-bit patterns), master/m/v are fp32. Every device pointer must be 16-byte
 * aligned.
 *
 * Execution: every zs_* call that touches device memory only validates its
 * arguments on the host and enqueues kernels on `stream` (a hipStream_t; NULL
 * is the default stream). It never synchronizes (exceptions, documented
 * below: zs_multi_bind and zs_multi_unbind, which copy into their workspace,
 * and zs_offload_adamw_step, which waits for the copies its host arithmetic
 * needs); a device-side fault is seen at the caller's next synchronization.
 * Calls on different streams that write the same memory race.
 *
 * Errors: a call that returns anything but ZS_OK has enqueued nothing and
 * changed nothing (except a ZS_EHIP in the middle of zs_offload_adamw_step's
 * pipeline); zs_last_error() then returns a thread-local description.
 *
 * Trace: with ZS_LOG set in the environment (to anything but "0"), every call
 * that enqueues work writes one line to stderr: a process-wide sequence
 * number, the entry point, the plan's world size and rank, the number of
 * contributions, the element range and the stream.
 */
#ifndef ZS_H
#define ZS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of gradient contributions one call accepts. */
#define ZS_MAX_CONTRIBS 256
/* Hyperparameter groups a PER_TENSOR plan can hold. */
#define ZS_MAX_GROUPS 8

typedef enum zs_status {
    ZS_OK = 0,
    ZS_EINVAL = -1, /* bad argument: NULL, out of range, inconsistent sizes */
    ZS_EALIGN = -2, /* a device pointer is not 16-byte aligned */
    ZS_ERANGE = -3, /* bucket [off, off+len) outside the owned shard or not a multiple of 8 */
    ZS_EHIP = -4,   /* the HIP runtime refused a launch or a copy */
    ZS_ENOMEM = -5  /* host allocation failed, or a workspace is too small */
} zs_status;

typedef enum zs_layout {
    ZS_LAYOUT_FLAT = 0,      /* one flat buffer, cut into N equal shards */
    ZS_LAYOUT_PER_TENSOR = 1 /* every tensor padded and cut into N pieces on its own */
} zs_layout;

typedef struct zs_plan zs_plan;

/* AdamW hyperparameters of one step. step is t >= 1 (bias corrections use
 * beta^t); all doubles must be finite, 0 <= beta1, beta2 < 1, eps >= 0. */
typedef struct zs_adamw_hparams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int64_t step;
} zs_adamw_hparams;

/* Where tensor i sits in a plan. Coordinates are elements.
 *   FLAT:       flat_off = start of tensor i in the flat buffer
 *               (a multiple of tensor_align_elems); padded_numel = numel.
 *   PER_TENSOR: flat_off = start of padded tensor i in the packed gathered
 *               buffer (tensors back to back); padded_numel = T_i =
 *               roundup(numel, 8*N).
 * own_lo/own_hi: the owned range of tensor i in tensor-local coordinates
 * (FLAT: clipped to the real elements; PER_TENSOR: [r*S_i, (r+1)*S_i),
 * which may cover padding). Empty when own_lo == own_hi.
 * shard_off: start of that range in the rank's packed shard. */
typedef struct zs_tensor_info {
    int64_t numel;
    int64_t flat_off;
    int64_t padded_numel;
    int64_t own_lo;
    int64_t own_hi;
    int64_t shard_off;
} zs_tensor_info;

/* ------------------------------------------------------------------ plan */

/* Builds the shard plan of n_tensors tensors (numels[i] >= 0 elements each,
 * in flatten order) for rank `rank` of `world_size`.
 *   FLAT: tensor i starts at off_i = roundup(off_{i-1} + numel_{i-1},
 *   tensor_align_elems); the flat length T = roundup(end of last tensor,
 *   8*N) so the shards are equal and whole 16-byte vectors; S = T/N; rank r
 *   owns [r*S, (r+1)*S).
 *   PER_TENSOR: T_i = roundup(numel_i, 8*N), S_i = T_i/N, rank r owns
 *   [r*S_i, (r+1)*S_i) of tensor i; the rank's packed shard concatenates
 *   its pieces (S = sum S_i) and the packed gathered buffer concatenates the
 *   padded tensors (T = sum T_i). tensor_align_elems is ignored.
 * Padding elements are part of the shards; they hold +0 and stay +0 under
 * the step when their contributions are +0 and eps > 0 (with eps = 0 a zero
 * gradient over a zero second moment is 0/0 = NaN, as in any AdamW).
 * The owned shard may hold at most 2^34 - 256 elements (a launch covers at
 * most 2^32 - 1 work-items of 4 elements; 16 B/param of state for that many
 * is 256 GiB, about all one MI355X holds).
 * Host only. On success *out owns a new plan; on error *out is untouched. */
zs_status zs_shard_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t rank,
                        int32_t tensor_align_elems, int32_t layout, zs_plan** out);
void zs_plan_destroy(zs_plan* plan);

/* Plan options beyond zs_shard_plan's arguments. */
typedef struct zs_plan_options {
    int32_t layout;             /* ZS_LAYOUT_FLAT or ZS_LAYOUT_PER_TENSOR */
    int32_t tensor_align_elems; /* FLAT: tensor-start alignment (>= 1); ignored otherwise */
    /* PER_TENSOR only: a tensor with fewer elements than this is not sharded
     * but replicated -- every rank holds the whole tensor, padded to a
     * multiple of 8, reduces all of it and updates it, and its gathered copy
     * is written whole ("ZeRO vs FSDP...", section 7: a persistence threshold
     * keeps small parameters such as norms replicated). 0: shard everything. */
    int64_t persist_below_elems;
    /* PER_TENSOR only: hyperparameter group of each tensor, each in
     * [0, ZS_MAX_GROUPS), or NULL (every tensor in group 0). The *_groups
     * multi-tensor calls take one zs_adamw_hparams per group (e.g. no weight
     * decay for norms and biases). */
    const int32_t* groups;
} zs_plan_options;

/* zs_shard_plan with options; zs_shard_plan(numels, n, N, r, align, layout, out)
 * equals this call with {layout, align, 0, NULL}. A replicated tensor i has
 * padded_numel = roundup(numel, 8), own range [0, padded_numel) and a
 * gathered copy of padded_numel elements; the ledger counts it in full. */
zs_status zs_shard_plan_ex(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t rank,
                           const zs_plan_options* options, zs_plan** out);
/* zs_plan_tensor_group: the hyperparameter group of tensor i.
 * zs_plan_tensor_replicated: 1 if tensor i is replicated, 0 if sharded.
 * Both give -1 on a NULL plan or an index out of range. */
int32_t zs_plan_tensor_group(const zs_plan* plan, int32_t i);
int32_t zs_plan_tensor_replicated(const zs_plan* plan, int32_t i);

/* Queries (host only; a NULL plan gives -1). */
int64_t zs_plan_padded_numel(const zs_plan* plan);     /* T */
int64_t zs_plan_shard_numel(const zs_plan* plan);      /* S */
int64_t zs_plan_persistent_bytes(const zs_plan* plan); /* 16*S: the per-rank ledger */
int32_t zs_plan_num_tensors(const zs_plan* plan);
int32_t zs_plan_world_size(const zs_plan* plan);
int32_t zs_plan_rank(const zs_plan* plan);
int32_t zs_plan_layout(const zs_plan* plan);
zs_status zs_plan_tensor(const zs_plan* plan, int32_t i, zs_tensor_info* out);

/* ------------------------------------------------------------------ flat step
 * In these calls the rank's shard is one packed buffer of S elements.
 * contribs is a HOST array of n_contribs device pointers; contribs[q] is rank
 * q's bf16 gradient for this rank's shard, S elements, element j belonging
 * to global index r*S + j (FLAT). n_contribs is the plan's world size N, or
 * N*R for hybrid sharding (shards cut N ways inside a group, R groups
 * replicating them: HYBRID_SHARD in "ZeRO vs FSDP...", section 3.1, and
 * "FSDP2's parameter lifecycle...", section "Hybrid sharding"): the
 * gradient is then averaged over all N*R data-parallel ranks, in the order
 * the array gives, exactly as one flat group of N*R ranks would average it.
 * n_contribs <= ZS_MAX_CONTRIBS. full_bf16 is the gathered parameter buffer
 * of T elements; only [r*S, (r+1)*S) is written. */

/* Averaged reduce of the bucket [off, off+len) of the shard (reduce-scatter
 * bucketed as gradients become ready: "从 Data Parallel 到 ZeRO/FSDP", section
 * "ReduceScatter 必须尽早释放 Gradient"). Writes grad_bf16[off, off+len).
 * off and len must be multiples of 8 with off + len <= S; len == 0 does
 * nothing. Buckets give the same bytes as one call over the whole shard. */
zs_status zs_reduce_shard(const zs_plan* plan, const void* const* contribs, int32_t n_contribs,
                          void* grad_bf16, int64_t off, int64_t len, void* stream);

/* AdamW over the S owned elements: reads grad_bf16, updates master, m, v in
 * place and writes param_bf16 = bf16(master). */
zs_status zs_adamw_shard_step(const zs_plan* plan, const zs_adamw_hparams* hp, const void* grad_bf16,
                              float* master, float* m, float* v, void* param_bf16, void* stream);

/* full_bf16[r*S + j] = param_bf16[j] for j < S. FLAT plans only. */
zs_status zs_gather_params(const zs_plan* plan, const void* param_bf16, void* full_bf16,
                           void* stream);

/* reduce + AdamW + gather over the shard, bit-identical to zs_reduce_shard
 * over the whole shard, then zs_adamw_shard_step, then zs_gather_params.
 * grad_bf16, param_bf16 and full_bf16 are each optional (NULL: not
 * written); full_bf16 requires a FLAT plan. One kernel pass; with
 * n_contribs >= ZS_FUSED_TWO_PASS_MIN_CONTRIBS and grad_bf16 given, two
 * passes -- the reduce into grad_bf16, then AdamW writing param/full --
 * which keep the read-heavy and write-heavy traffic apart and run faster on
 * MI355X at those sizes. Either form leaves the same bytes. */
#define ZS_FUSED_TWO_PASS_MIN_CONTRIBS 52
zs_status zs_fused_shard_step(const zs_plan* plan, const zs_adamw_hparams* hp,
                              const void* const* contribs, int32_t n_contribs, float* master,
                              float* m, float* v, void* grad_bf16, void* param_bf16,
                              void* full_bf16, void* stream);

/* zs_fused_shard_step over the bucket [off, off+len) of the shard only, with
 * zs_reduce_shard's bucket rules (off and len multiples of 8, off + len <= S,
 * len == 0 does nothing). The buffers are the whole-shard ones: bucket
 * element j is element off + j of every contribution, of master/m/v and of
 * grad_bf16/param_bf16, and is written to full_bf16[r*S + off + j]. Buckets
 * give the same bytes as one call over the whole shard, so the step of a
 * bucket can run as soon as its contributions have arrived, while later
 * buckets are still being exchanged (reduce-scatter bucketed as gradients
 * become ready: "从 Data Parallel 到 ZeRO/FSDP", section "ReduceScatter 必须尽早
 * 释放 Gradient"); without global-norm clipping AdamW needs nothing from
 * the other buckets. */
zs_status zs_fused_shard_step_bucket(const zs_plan* plan, const zs_adamw_hparams* hp,
                                     const void* const* contribs, int32_t n_contribs, float* master, float* m,
                                     float* v, void* grad_bf16, void* param_bf16, void* full_bf16, int64_t off,
                                     int64_t len, void* stream);

/* ------------------------------------------------------------------ resharding to a smaller group
 * FSDP2's reshard_after_forward also takes an integer k: after forward the
 * parameters stay sharded over a group of k ranks instead of all N, e.g.
 * within a node, so the backward all-gather spans only that group ("FSDP2's
 * parameter lifecycle...", section "Reshard policy: pay for the memory, or
 * pay for the communication again"). Here k divides N and the groups are k
 * consecutive ranks; the k members of a group split the gathered flat buffer
 * [0, T) into k equal slices, the member at position j = r mod k keeping
 * slice j: T/k elements, the N-way shards of ranks j*N/k .. (j+1)*N/k - 1 in
 * order. k = N keeps only the own shard (full resharding), k = 1 the whole
 * buffer (no resharding). FLAT plans only. */
typedef struct zs_reshard_slice {
    int32_t group_size;     /* k */
    int32_t slice_index;    /* j = r mod k: the slice this rank keeps */
    int64_t slice_off;      /* j*T/k: its start in the gathered flat buffer */
    int64_t slice_len;      /* T/k elements */
    int32_t first_source;   /* the kept slice is the shards of ranks first_source .. */
    int32_t n_sources;      /* .. first_source + n_sources - 1 (n_sources = N/k) */
    int32_t owner_slice;    /* r div (N/k): the slice that holds this rank's own shard */
    int32_t reserved;       /* 0 */
    int64_t own_off;        /* (r mod (N/k))*S: the own shard's start inside that slice */
    int64_t retained_bytes; /* 2*T/k: bf16 parameter bytes a rank keeps after forward */
} zs_reshard_slice;

/* Fills *out for group size k (1 <= k <= N, N % k == 0). Host only. */
zs_status zs_plan_reshard_slice(const zs_plan* plan, int32_t group_size, zs_reshard_slice* out);

/* The gather write of the step into a k-way slice: the own updated shard
 * (param_bf16, S elements) goes to slice_bf16[own_off + j], where
 * slice_bf16 holds slice owner_slice (T/k elements); nothing else of the
 * buffer is touched. With k = 1 this is zs_gather_params. */
zs_status zs_gather_params_to_slice(const zs_plan* plan, int32_t group_size, const void* param_bf16,
                                    void* slice_bf16, void* stream);

/* The receiving side of the gather into the kept slice: shards is a host
 * array of n_shards = N/k device pointers, shards[i] the updated bf16 shard
 * (S elements) of rank first_source + i; each is written to slice_bf16 at
 * i*S, filling this rank's kept slice (T/k elements). */
zs_status zs_gather_slice(const zs_plan* plan, int32_t group_size, const void* const* shards, int32_t n_shards,
                          void* slice_bf16, void* stream);

/* ------------------------------------------------------------------ multi-tensor
 * Multi-tensor apply over the owned pieces of a PER_TENSOR plan whose
 * per-tensor state lives in separate allocations (FSDP2's per-parameter
 * sharding with one unit per Linear or norm: "FSDP2's parameter lifecycle...",
 * section "Wrap granularity is the lever"). One launch covers every piece,
 * however small.
 *
 * zs_multi_bind writes a device table of the pieces' pointers and a
 * chunk list into a caller-allocated device workspace of at least
 * zs_multi_workspace_bytes(plan, n_contribs) bytes. It enqueues one
 * host-to-device copy on `stream` and then synchronizes that stream, so the
 * host arrays may be freed on return. The per-step calls then read only the
 * workspace; rebind when any pointer changes. Pieces of zero length are
 * skipped. A NULL field disables that read or write for every piece (all
 * pieces must agree on which fields are NULL). */
typedef struct zs_piece_ptrs {
    void* grad;    /* bf16 [S_i]: reduce output, AdamW input */
    float* master; /* fp32 [S_i] */
    float* m;      /* fp32 [S_i] */
    float* v;      /* fp32 [S_i] */
    void* param;   /* bf16 [S_i]: updated bf16 shard piece, or NULL */
    void* full;    /* bf16 [T_i]: gathered tensor i (written at [r*S_i, (r+1)*S_i)), or NULL */
} zs_piece_ptrs;

int64_t zs_multi_workspace_bytes(const zs_plan* plan, int32_t n_contribs);
/* The workspace a binding with the plan's world size of contributions needs:
 * zs_multi_workspace_bytes(plan, world size) for PER_TENSOR plans, 0 for FLAT
 * plans (their calls need none); -1 for a NULL plan. */
int64_t zs_plan_workspace_bytes(const zs_plan* plan);

/* pieces: host array of zs_plan_num_tensors(plan) records. contribs: host
 * array of n_contribs * num_tensors device pointers, contribs[q*n_tensors+i]
 * = rank q's bf16 gradient piece of tensor i (S_i elements), or NULL when
 * n_contribs == 0 (no reduce possible on this binding). As in the flat
 * calls, n_contribs is the world size or a multiple of it (hybrid). */
zs_status zs_multi_bind(const zs_plan* plan, const zs_piece_ptrs* pieces, const void* const* contribs,
                        int32_t n_contribs, void* workspace, int64_t workspace_bytes, void* stream);

/* Forgets a binding and clears the table's tag in the workspace (one 8-byte
 * copy on `stream`, then a synchronization), so the memory can be reused.
 * The kernels check that tag and do nothing on a workspace that holds no
 * bound table. */
zs_status zs_multi_unbind(void* workspace, void* stream);

zs_status zs_reduce_shard_multi(const zs_plan* plan, const void* workspace, void* stream);
zs_status zs_adamw_shard_step_multi(const zs_plan* plan, const zs_adamw_hparams* hp,
                                    const void* workspace, void* stream);
zs_status zs_gather_params_multi(const zs_plan* plan, const void* workspace, void* stream);
/* reduce + AdamW + gather for every piece in one launch; writes grad, param
 * and full only where those fields were bound non-NULL. With grad bound and
 * at least ZS_FUSED_TWO_PASS_MIN_CONTRIBS contributions, two launches
 * instead, as zs_fused_shard_step does: the reduce into the grad pieces,
 * then AdamW writing param and full. Either form leaves the same bytes. */
zs_status zs_fused_shard_step_multi(const zs_plan* plan, const zs_adamw_hparams* hp,
                                    const void* workspace, void* stream);
/* As zs_adamw_shard_step_multi / zs_fused_shard_step_multi with one set of
 * hyperparameters per group: piece i uses hps[group of tensor i]. n_groups
 * must exceed every group id of the plan (<= ZS_MAX_GROUPS). The calls
 * without _groups apply their single hp to every group. */
zs_status zs_adamw_shard_step_multi_groups(const zs_plan* plan, const zs_adamw_hparams* hps, int32_t n_groups,
                                           const void* workspace, void* stream);
zs_status zs_fused_shard_step_multi_groups(const zs_plan* plan, const zs_adamw_hparams* hps, int32_t n_groups,
                                           const void* workspace, void* stream);

/* ------------------------------------------------------------------ quantized parameter gather
 * ZeRO++ moves the gathered parameters as low-bit codes, 4 bits giving up to
 * four times less all-gather traffic ("ZeRO vs FSDP...", section 5.2). Here
 * each rank quantizes its updated bf16 shard block-wise and symmetrically;
 * the all-gather then carries every rank's codes and scales, and every rank
 * (the owner included) decodes all of them into the gathered buffer, so all
 * ranks hold the same dequantized parameters. The fp32 master weights stay
 * exact. FLAT plans only.
 *
 * Per block of `block` consecutive shard elements (the last block of a shard
 * may be shorter): amax = max |x|; scale = fp32(amax / qmax), qmax = 127 for
 * bits = 8 and 7 for bits = 4; code = x / scale (one fp32 division) rounded
 * to nearest, ties to even, clamped to [-qmax, qmax]. amax == 0 gives scale
 * 0 and codes 0; a NaN or infinity in the block gives scale NaN and codes 0.
 * Decoding: x' = bf16_rne(f32(code) * scale).
 * Codes: bits = 8 -- one two's-complement byte per element; bits = 4 -- two
 * elements per byte, the even element in the low nibble. block is a power
 * of two in [8, 256].
 *
 * One rank's payload: zs_quant_code_bytes(plan, bits) code bytes (S*bits/8)
 * and zs_quant_num_scales(plan, block) fp32 scales (ceil(S/block)); -1 on a
 * bad argument. */
int64_t zs_quant_code_bytes(const zs_plan* plan, int32_t bits);
int64_t zs_quant_num_scales(const zs_plan* plan, int32_t block);

/* Codes and scales of a bf16 shard (S elements of param_bf16). */
zs_status zs_quantize_shard(const zs_plan* plan, int32_t bits, int32_t block, const void* param_bf16, void* codes,
                            float* scales, void* stream);

/* zs_fused_shard_step whose gather output is the quantized payload: the
 * reduce and AdamW as there (grad_bf16 and param_bf16 optional), then the
 * updated bf16 shard's codes and scales, bit-identical to
 * zs_quantize_shard of the param_bf16 zs_fused_shard_step writes. */
zs_status zs_fused_shard_step_quant(const zs_plan* plan, const zs_adamw_hparams* hp, const void* const* contribs,
                                    int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                                    void* param_bf16, int32_t bits, int32_t block, void* codes, float* scales,
                                    void* stream);

/* The receiving side: codes_all holds the N ranks' codes end to end (rank q
 * at q * zs_quant_code_bytes), scales_all their scales end to end (rank q at
 * q * zs_quant_num_scales); writes every element of full_bf16[0, T).
 * N <= 65535. */
zs_status zs_dequant_gather(const zs_plan* plan, int32_t bits, int32_t block, const void* codes_all,
                            const float* scales_all, void* full_bf16, void* stream);

/* ------------------------------------------------------------------ CPU-offloaded optimizer step
 * ZeRO-Offload keeps the fp32 optimizer state in host memory and runs the
 * step on the CPU ("ZeRO vs FSDP...", section 2.4); the step then pays PCIe
 * transfers and host memory bandwidth, hidden only as far as they overlap
 * ("从 Data Parallel 到 ZeRO/FSDP", section "CPU/NVMe Offload 不是免费显存").
 * Both calls compute exactly the AdamW of zs_adamw_shard_step (same fp32
 * operations in the same order), so host and device steps give identical
 * bytes. */

/* AdamW on host arrays of n elements with n_threads host threads: reads
 * grad_bf16, updates master/m/v, writes param_bf16 (optional). Synchronous.
 * Host pointers, 16-byte aligned; 1 <= n_threads <= 256. */
zs_status zs_host_adamw_step(const zs_adamw_hparams* hp, const void* grad_bf16, float* master, float* m, float* v,
                             void* param_bf16, int64_t n, int32_t n_threads);

/* Offloaded step of the rank's shard (S elements): the device grad shard
 * (grad_bf16_dev, complete in `stream` order) is copied chunk by chunk into
 * grad_bf16_host; each chunk is stepped on the host (master/m/v_host) as
 * soon as it arrives, and its bf16 parameters (param_bf16_host) are copied
 * back to param_bf16_dev and/or the gathered buffer full_bf16_dev (FLAT, at
 * r*S) on a second stream while the next chunks arrive and update. Later
 * work on `stream` sees the new parameters. grad_bf16_host and
 * param_bf16_host must be page-locked (hipHostMalloc or pinned tensors);
 * chunk_elems is a multiple of 8, at least 1024. The call returns once the
 * host arithmetic is done (it waits on the copies it needs). Calls are
 * serialized process-wide, and each call's work on `stream` is ordered after
 * the previous call's copies to the device (whose staging buffer it reuses),
 * whatever stream that call used. Unlike the other calls, a ZS_EHIP return in the
 * middle of the pipeline may leave a prefix of the chunks updated. */
zs_status zs_offload_adamw_step(const zs_plan* plan, const zs_adamw_hparams* hp, const void* grad_bf16_dev,
                                float* master_host, float* m_host, float* v_host, void* grad_bf16_host,
                                void* param_bf16_host, void* param_bf16_dev, void* full_bf16_dev, int64_t chunk_elems,
                                int32_t n_threads, void* stream);

/* ------------------------------------------------------------------ accumulation and clipping
 * Gradient accumulation over G micro-batches with an fp32 gradient shard,
 * global-norm clipping and a non-finite skip ("从 Data Parallel 到
 * ZeRO/FSDP", section "Gradient Accumulation 会改变生命周期": every micro-step
 * reduce-scatters and accumulates on the shard, the loss is divided by G,
 * clipping uses the norm over all ranks, the overflow decision is shared).
 * The per-rank squared norms are combined by the caller (an all-reduce of
 * one double per rank in a multi-GPU job). Scale and skip stay on the device,
 * so the optimizer step needs no host synchronization. */

/* One micro-step over the bucket [off, off+len) of the shard:
 * acc_f32[j] = (first ? +0 : acc_f32[j]) + f32(bf16(average of the N
 * contributions)), the average computed as in zs_reduce_shard. Same argument
 * rules as zs_reduce_shard. */
zs_status zs_accumulate_shard(const zs_plan* plan, const void* const* contribs, int32_t n_contribs,
                              float* acc_f32, int64_t off, int64_t len, int32_t first, void* stream);

/* Device workspace bytes zs_grad_stats needs for this plan. */
int64_t zs_grad_stats_workspace_bytes(const zs_plan* plan);

/* Over the shard's final gradient g = acc_f32 / grad_divisor (fp32
 * division): *sumsq_out = sum of g^2 in double (a fixed-order reduction, so
 * repeated calls give identical bits) and *nonfinite_out = 1 if any g is NaN
 * or infinite, else 0. sumsq_out (8-byte aligned) and nonfinite_out (4-byte
 * aligned) are device pointers; both are always written. grad_divisor must
 * be finite and nonzero. */
zs_status zs_grad_stats(const zs_plan* plan, const float* acc_f32, float grad_divisor, double* sumsq_out,
                        int32_t* nonfinite_out, void* workspace, int64_t workspace_bytes, void* stream);

/* zs_grad_stats for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same result bits, with the per-block partials in a
 * 4 MiB array the library holds statically on each GPU it runs on (until the
 * process ends) instead of a caller workspace. The call itself allocates
 * nothing and uses the copy on the stream's GPU (the current GPU for the
 * null stream); its first call for a GPU looks up that GPU's copy (call it
 * there once outside a capture). Shards of more than
 * ZS_GRAD_STATS_NOALLOC_MAX_ELEMS elements give ZS_ENOMEM and enqueue
 * nothing. All calls on one GPU share its array: two of them in flight at
 * once (on different streams) race and give wrong sums; calls on one stream
 * are ordered and safe, each overwriting every partial it reads. */
#define ZS_GRAD_STATS_NOALLOC_MAX_ELEMS 1431568384LL
zs_status zs_grad_stats_noalloc(const zs_plan* plan, const float* acc_f32, float grad_divisor, double* sumsq_out,
                                int32_t* nonfinite_out, void* stream);

/* From the squared norms of all n_ranks shards (device array, added in rank
 * order) and their flags (device array): *scale_out = (float) min(1,
 * max_norm / (sqrt(sum) + 1e-6)) and *skip_out = 1 if any flag is set.
 * max_norm must be finite and positive; n_ranks >= 1. */
zs_status zs_clip_scale(const double* sumsq, const int32_t* nonfinite, int32_t n_ranks, double max_norm,
                        float* scale_out, int32_t* skip_out, void* stream);

/* AdamW from the fp32 accumulator: element gradient (acc_f32[j] /
 * grad_divisor) * *scale (scale NULL: 1), then the update of
 * zs_adamw_shard_step. If skip is non-NULL and *skip != 0 nothing is
 * written. param_bf16 and full_bf16 are optional outputs (full_bf16: FLAT
 * plans, written at [r*S, (r+1)*S)). */
zs_status zs_adamw_shard_step_accum(const zs_plan* plan, const zs_adamw_hparams* hp, const float* acc_f32,
                                    float grad_divisor, const float* scale, const int32_t* skip, float* master,
                                    float* m, float* v, void* param_bf16, void* full_bf16, void* stream);

/* ------------------------------------------------------------------ scalars in device memory
 * Kernel arguments are fixed when a stream is captured into a HIP graph, so a
 * replayed step would repeat its step count t (and learning rate). The _dc
 * calls below are the corresponding calls with the AdamW scalars read from
 * device memory when the kernels run: capture the step once, and before each
 * replay write that step's scalars into the buffer (for example a captured
 * copy from page-locked host memory that the host refills). Launch-bound
 * shards gain most: replayed steps avoid the host's launch cost. */

/* The fp32 AdamW scalars of one step, each rounded once from double exactly
 * as the by-value calls compute them:
 *   beta1, 1-beta1, beta2, 1-beta2, lr, eps, 1-lr*wd, 1-beta1^t, 1-beta2^t. */
typedef struct zs_adamw_coefs {
    float beta1;
    float one_minus_beta1;
    float beta2;
    float one_minus_beta2;
    float lr;
    float eps;
    float decay;
    float bias_correction1;
    float bias_correction2;
} zs_adamw_coefs;

/* Host only: the scalars of hp (same validation as the step calls). */
zs_status zs_adamw_coefs_compute(const zs_adamw_hparams* hp, zs_adamw_coefs* out);

/* As zs_fused_shard_step, zs_adamw_shard_step and zs_adamw_shard_step_accum,
 * with coefs a DEVICE pointer (4-byte aligned) to the step's scalars, read by
 * the kernels at run time; results are bit-identical to the by-value call
 * with the hparams the scalars were computed from. The values are not
 * checked: fill the buffer with zs_adamw_coefs_compute's output. */
zs_status zs_fused_shard_step_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const void* const* contribs,
                                 int32_t n_contribs, float* master, float* m, float* v, void* grad_bf16,
                                 void* param_bf16, void* full_bf16, void* stream);
zs_status zs_adamw_shard_step_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const void* grad_bf16,
                                 float* master, float* m, float* v, void* param_bf16, void* stream);
zs_status zs_adamw_shard_step_accum_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, const float* acc_f32,
                                       float grad_divisor, const float* scale, const int32_t* skip, float* master,
                                       float* m, float* v, void* param_bf16, void* full_bf16, void* stream);
/* As zs_fused_shard_step_multi_groups with coefs a DEVICE array of n_groups
 * scalar sets (piece i uses coefs[group of tensor i]). */
zs_status zs_fused_shard_step_multi_dc(const zs_plan* plan, const zs_adamw_coefs* coefs, int32_t n_groups,
                                       const void* workspace, void* stream);

/* ------------------------------------------------------------------ misc */

/* Thread-local text describing the last non-OK status of this thread. */
const char* zs_last_error(void);
/* Library version, "major.minor.patch". */
const char* zs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H */
