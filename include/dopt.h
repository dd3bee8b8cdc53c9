/*
 * dopt.h -- C ABI of the shard-local mixed-precision AdamW step of a ZeRO-1
 * distributed optimizer, for AMD Instinct MI355X (gfx950).
 *
 * One data-parallel rank owns a contiguous 1/N slice ("window") of every
 * bucket of every flat grad buffer; the slice cuts across parameter
 * boundaries.  Per step the library unscales the rank's grads into fp32,
 * detects inf/NaN, takes the L2 norm and the clip coefficient, updates the
 * fp32 master weights and Adam moments (AdamW with bias correction), and
 * writes the 16-bit params back into the rank's param window.  The
 * reduce-scatter before the step and the all-gather after it are the
 * caller's.
 *
 * Pages cited (title, then section):
 *   [DO] "Megatron-LM distrib_optimizer.py 源码精读"
 *   [ZL] "02 · ZeRO 显存账本与 Megatron DistributedOptimizer"
 *   [DP] "Megatron-LM distributed 包深度解析：DDP 梯度同步与 finalize_model_grads 全流程"
 *   [DS] "Megatron-LM与DeepSpeed的分布式训练源码里，模型和优化器到底是怎么切分的？"
 *
 * Conventions
 *   - Every function returns 0 on success or a negative DOPT_ERR_* code;
 *     dopt_last_error() then holds a message (per thread).  No exception or
 *     abort crosses the ABI.
 *   - "host" pointers are CPU memory, "device" pointers are GPU memory
 *     (e.g. from hipMalloc or a PyTorch CUDA tensor).  The library never
 *     allocates or frees device memory; its one device array of its own is
 *     the fixed static scratch of dopt_check_grads_noalloc.
 *   - Device work is enqueued on the caller's HIP stream and is ordered with
 *     the caller's other work on that stream; nothing synchronizes unless a
 *     function says so.
 *   - A dopt_layout is immutable once built and may be shared by threads.
 *     Calls that use one workspace must not overlap in time.
 */
#ifndef DOPT_H
#define DOPT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element types ---- */
enum { DOPT_F32 = 0, DOPT_BF16 = 1, DOPT_F16 = 2 };

/* ---- error codes ---- */
enum {
    DOPT_OK = 0,
    DOPT_ERR_INVALID = -1, /* bad argument (null, out of range, bad dtype, misaligned pointer) */
    DOPT_ERR_ASSERT = -2,  /* a layout invariant of [DO] "最终内存大小断言" does not hold */
    DOPT_ERR_NOMEM = -3,   /* host allocation failed */
    DOPT_ERR_HIP = -4,     /* a HIP runtime call failed (message names it) */
    DOPT_ERR_RANGE = -5    /* query index out of range */
};

/* ---- group kinds of [DO] "五组数据结构 / 分片切片逻辑" and [ZL] §3 ---- */
enum {
    DOPT_GROUP_MODEL_FLOAT16 = 0,
    DOPT_GROUP_MODEL_FP32 = 1,
    DOPT_GROUP_SHARD_FLOAT16 = 2,
    DOPT_GROUP_SHARD_FP32_FROM_FLOAT16 = 3,
    DOPT_GROUP_SHARD_FP32 = 4
};

enum { DOPT_SCALER_CONSTANT = 0, DOPT_SCALER_DYNAMIC = 1 };

#define DOPT_MAX_HGROUPS 16
/* Arena arrays hold a whole number of DOPT_ARENA_ALIGN elements. */
#define DOPT_ARENA_ALIGN 2048
/* Required alignment (bytes) of every device pointer passed in. */
#define DOPT_PTR_ALIGN 256

/* One model parameter, in model (registration, forward) order. */
typedef struct dopt_param_desc {
    int64_t numel;               /* > 0 */
    int32_t param_dtype;         /* DOPT_F32 / DOPT_BF16 / DOPT_F16 */
    int32_t grad_dtype;          /* the grad buffer's element type */
    int32_t requires_new_bucket; /* nonzero: the param gets a bucket of its own */
    int32_t hgroup;              /* optimizer param group, 0 <= hgroup < DOPT_MAX_HGROUPS */
} dopt_param_desc;

/*
 * Sharding of one rank.  With num_instances = I > 1 the data-parallel domain
 * of N ranks is split into I distributed-optimizer instances of N/I ranks
 * each ([ZL] §5 "num_distributed_optimizer_instances：分层 ZeRO"; [DP] §3.1):
 * buckets are padded and split across the N/I ranks of the rank's instance,
 * and the rank's shard is taken at its rank inside the instance (the
 * intra-instance rank of the reduce-scatter call in [DO] §7.1); the optimizer
 * state is cut to 1/(N/I).  Reading: instance i holds the consecutive ranks
 * [i*N/I, (i+1)*N/I), so the intra-instance rank is r mod (N/I).  The
 * all-reduce across instances is the caller's.
 */
typedef struct dopt_shard_cfg {
    int32_t dp_size;             /* N >= 1 */
    int32_t dp_rank;             /* 0 <= r < N */
    int64_t bucket_size;         /* elements; <= 0: no size trigger (one bucket) */
    int32_t pad_for_high_busbw;  /* nonzero: buckets padded to lcm(N',128,2^16), N' the instance size */
    int32_t num_instances;       /* I >= 1 dividing N (0 is taken as 1) */
} dopt_shard_cfg;

typedef struct dopt_sharding_info {
    int32_t dp_size, dp_rank;
    int32_t num_instances;
    int32_t instance_size;       /* N / I: the ranks the optimizer state is split over */
    int32_t instance_index;      /* r / (N / I) */
    int32_t instance_rank;       /* r mod (N / I): the shard this rank owns */
} dopt_sharding_info;

typedef struct dopt_range { int64_t start, end; } dopt_range;

typedef struct dopt_layout dopt_layout;

/*
 * dopt_build_ranges -- the host-side shard-range mapper.
 *
 * Groups the params into one flat buffer per (param dtype, grad dtype) in
 * order of first appearance ([DP] §2.2 (3)); lays each buffer out last param
 * first, starting every param on a multiple of 64 elements and closing a
 * bucket when it reaches bucket_size or for a param that needs its own
 * bucket ([DO] "Bucket 划分算法：逆序遍历 + 尺寸触发"); pads every bucket end to
 * a multiple of lcm(N, 128) (or lcm(N, 128, 2^16)) ([DO] "两级 Padding 机制");
 * checks the size invariants ([DO] "最终内存大小断言"); takes rank r's
 * window of every bucket ([DO] "Bucket 级别的均等切分"); intersects every
 * param with its bucket's window in the four coordinate views of [DO]
 * "Range 类：四种视角的统一抽象"; and forms the shard groups ([DO] group
 * building section; [ZL] §3).
 *
 * It also fixes the device layout the step uses: per buffer, an "arena" of
 * arena_numel elements holding the rank's windows of that buffer's buckets
 * back to back in bucket order (bucket b's window at arena_offset of b).
 * The grad window, the param window, the fp32 master and both Adam moments
 * of a buffer are all arrays in this one index space.
 *
 * params: host, n entries, model order; cfg: host.  *out receives a layout
 * owned by the library; free it with dopt_layout_free.
 * Errors: DOPT_ERR_INVALID (null pointers, n <= 0 or n > INT32_MAX,
 * numel <= 0, more than 2^52 elements over the list, bad dtype or hgroup,
 * N < 1, r outside [0, N), a flat buffer padded beyond 2^60 elements);
 * DOPT_ERR_ASSERT; DOPT_ERR_NOMEM.
 */
int dopt_build_ranges(const dopt_param_desc *params, int64_t n, const dopt_shard_cfg *cfg,
                      dopt_layout **out);

void dopt_layout_free(dopt_layout *layout);

/* ---- read-only layout queries (host; no device work) ---- */

typedef struct dopt_buffer_info {
    int32_t param_dtype, grad_dtype;
    int32_t n_buckets;
    int32_t n_params;
    int64_t numel;          /* padded buffer size ([DO] "最终内存大小断言") */
    int64_t numel_unpadded; /* sum of per-bucket unpadded sizes */
    int64_t window_numel;   /* sum of the rank's window sizes */
    int64_t arena_numel;    /* window_numel rounded up to DOPT_ARENA_ALIGN: size of every arena array */
    int64_t shard_numel;    /* param elements inside the rank's windows */
    int32_t apply_bnd;      /* 1: pass 2 runs k_apply_bnd, which updates boundary tiles (params meeting
                               inside a 2048-element tile) from registers: a window of more than 16384 tiles
                               (grid-stride) that holds one; 0: k_apply */
    int32_t reserved;
} dopt_buffer_info;

typedef struct dopt_bucket_info {
    int64_t offset;         /* bucket start in the buffer */
    int64_t numel;          /* padded bucket size, a multiple of N */
    int64_t numel_unpadded;
    int64_t shard_size;     /* numel / N */
    int64_t window_start;   /* offset + r * shard_size (buffer coordinates) */
    int64_t arena_offset;   /* where the window starts in the arena */
    int32_t n_params;
    int32_t reserved;
} dopt_bucket_info;

/* Four views of one param's shard on this rank ([DO] "Range 类"). */
typedef struct dopt_param_info {
    int32_t buffer, bucket;
    int32_t has_shard;          /* 0: no element of the param is in this rank's window */
    int32_t hgroup;
    int64_t start, end;         /* the param's range in its buffer (param_index_map) */
    dopt_range gbuf_world;      /* shard, buffer coordinates */
    dopt_range gbuf_world_in_bucket; /* shard, bucket coordinates */
    dopt_range gbuf_local;      /* shard, window coordinates */
    dopt_range param;           /* shard, coordinates inside the param */
    int64_t arena_offset;       /* shard start in the arena; -1 without a shard */
    int64_t export_offset;      /* shard start in the model-space export (dopt_state_export); -1 without */
} dopt_param_info;

int32_t dopt_layout_num_buffers(const dopt_layout *layout);
/* How this rank's shard was chosen (instances, intra-instance rank). */
int dopt_layout_sharding(const dopt_layout *layout, dopt_sharding_info *out);
int dopt_layout_buffer(const dopt_layout *layout, int32_t k, dopt_buffer_info *out);
int dopt_layout_bucket(const dopt_layout *layout, int32_t k, int32_t b, dopt_bucket_info *out);
/* Window of rank `rank` of the instance (any rank, not only this one; 0 <=
 * rank < instance size) in bucket b of buffer k, buffer coordinates ([DO]
 * "Bucket 级别的均等切分": all ranks' ranges). */
int dopt_layout_rank_window(const dopt_layout *layout, int32_t k, int32_t b, int32_t rank, dopt_range *out);
int dopt_layout_param(const dopt_layout *layout, int64_t p, dopt_param_info *out);
/* Model-order indices of the params of one group kind and hyper-group; writes
 * at most cap entries to idx (host, may be NULL) and returns the full count,
 * or a negative error code (DOPT_ERR_RANGE for a kind or hyper-group out of
 * range). */
int64_t dopt_layout_group(const dopt_layout *layout, int32_t kind, int32_t hgroup, int64_t *idx, int64_t cap);
/* Param elements on this rank over all buffers (the optimizer-state length
 * of the ledger in [ZL] §2). */
int64_t dopt_layout_state_numel(const dopt_layout *layout);

/* Bytes of device workspace the step needs.  The caller allocates it
 * (DOPT_PTR_ALIGN-aligned), passes it to dopt_init_state and then to every
 * step, and keeps it alive: it carries the step count and the loss-scale
 * state from step to step. */
int64_t dopt_workspace_bytes(const dopt_layout *layout);

/* ---- device arrays of one flat buffer (all in arena coordinates) ---- */
typedef struct dopt_buffer_tensors {
    const void *grad;   /* device, arena_numel x grad dtype: the rank's reduced grads; read only
                           (dopt_reduce_prepare writes it) */
    void *param;        /* device, arena_numel x param dtype: the rank's param windows; written back */
    float *master;      /* device, arena_numel fp32; NULL when the param dtype is fp32 */
    float *exp_avg;     /* device, arena_numel fp32: Adam m */
    float *exp_avg_sq;  /* device, arena_numel fp32: Adam v */
} dopt_buffer_tensors;

typedef struct dopt_scaler_cfg {
    int32_t kind;            /* DOPT_SCALER_CONSTANT or DOPT_SCALER_DYNAMIC */
    int32_t hysteresis;      /* dynamic: overflows tolerated before a backoff (>= 1) */
    int64_t growth_interval; /* dynamic: clean steps between growths (>= 1) */
    double initial_scale;    /* finite, > 0, and 1/initial_scale a finite nonzero fp32 number */
    double growth_factor;    /* dynamic, finite, > 1 */
    double backoff_factor;   /* dynamic, in (0, 1) */
    double min_scale;        /* dynamic, as initial_scale */
} dopt_scaler_cfg;

/*
 * dopt_init_state -- S1 of the step: fp32 master = upcast of the 16-bit
 * param window ([DO] "分片切片逻辑": clone of the shard, as float), Adam
 * moments = 0; fp32-param buffers get no master ([ZL] §3).  Loads the tile
 * tables into the workspace and sets step count 0 and the loss scale to
 * scaler->initial_scale.
 *
 * bufs: host array of dopt_layout_num_buffers() entries holding device
 * pointers; scaler: host; workspace: device, dopt_workspace_bytes() bytes.
 * Synchronizes `stream` before returning (the tables are copied from the
 * layout's host memory).
 * Errors: DOPT_ERR_INVALID (null / misaligned pointers, bad scaler),
 * DOPT_ERR_HIP.
 */
int dopt_init_state(const dopt_layout *layout, const dopt_buffer_tensors *bufs, const dopt_scaler_cfg *scaler,
                    void *workspace, hipStream_t stream);

/* Hyper-parameters of one optimizer param group (AdamW). */
typedef struct dopt_hparams {
    double lr, beta1, beta2, eps, weight_decay;
} dopt_hparams;

/* Result of one step (host copy of the device record). */
typedef struct dopt_stats {
    int32_t found_inf;      /* 1: some unscaled grad was inf or NaN */
    int32_t skipped;        /* 1: no state was changed this step */
    int32_t clip_applied;   /* 1: grads were scaled by clip_coef */
    int32_t reserved;
    double sumsq;           /* sum of squares of the unscaled, pre-clip grads */
    double grad_norm;       /* sqrt(sumsq) */
    double clip_coef;       /* max_grad_norm / (grad_norm + 1e-6); 1.0 when not clipping */
    uint64_t num_zeros;     /* unscaled grad elements equal to zero */
    double loss_scale_used; /* scale the grads of this step carried */
    double loss_scale_next; /* scale for the next step */
    int64_t step_count;     /* successful steps so far (Adam's t) */
} dopt_stats;

/*
 * dopt_step -- one optimizer step on this rank's shard, in the order of
 * [DO] "三层继承体系" (second layer): grads to fp32 + unscale + inf/NaN check,
 * clip by the global norm, then the inner AdamW step and the copy of the
 * masters back to the 16-bit params ([DO] "分片切片逻辑"; [DS] §2 step).
 * Equivalent to dopt_step_prepare followed by dopt_step_apply (and to
 * dopt_step_stats, dopt_step_finalize, dopt_step_apply in that order).  A
 * step with an inf/NaN grad is skipped: master, moments,
 * params and the step count stay as they were, and a dynamic loss scale
 * backs off.  Skipping is not an error.
 *
 * bufs: host array (device pointers); hp: host, n_hgroups entries (one per
 * hyper-group used by the params); max_grad_norm <= 0 disables clipping.
 * out: host, may be NULL; when given, the call synchronizes `stream` and
 * fills it.  Errors: DOPT_ERR_INVALID, DOPT_ERR_HIP.
 */
int dopt_step(const dopt_layout *layout, const dopt_buffer_tensors *bufs, const dopt_hparams *hp,
              int32_t n_hgroups, double max_grad_norm, void *workspace, hipStream_t stream, dopt_stats *out);

/*
 * dopt_step_prepare -- the first half of dopt_step for a single rank: pass 1
 * (unscale, sum of squares, zero count; one launch per flat buffer), then
 * one small launch that does the fixed-order reduction and the finalize
 * below together.  Named after the prepare-grads phase of [DO] "三层继承体系"
 * (second layer).  Arguments and errors as dopt_step; never synchronizes.
 */
int dopt_step_prepare(const dopt_layout *layout, const dopt_buffer_tensors *bufs, const dopt_hparams *hp,
                      int32_t n_hgroups, double max_grad_norm, void *workspace, hipStream_t stream);

/*
 * The step in three parts.  Between dopt_step_stats and dopt_step_finalize a
 * multi-rank caller sums the grad-stats record (dopt_stats_record) over the
 * whole distributed-optimizer group, on the same stream: [DO] "三层继承体系"
 * (third layer) takes the grad norm over all data-parallel ranks.  On one
 * rank no exchange is needed.
 *
 * dopt_step_stats: pass 1 -- unscale, sum of squares and zero count over the
 *   rank's shard elements, reduced in a fixed order into the record.
 * dopt_step_finalize: skip decision (record not finite), norm, clip
 *   coefficient, loss-scale update, step count, per-group AdamW scalars.
 * dopt_step_apply: pass 2 -- clip + AdamW + bias correction + write-back;
 *   returns immediately on the device when the step is skipped.
 */
int dopt_step_stats(const dopt_layout *layout, const dopt_buffer_tensors *bufs, void *workspace,
                    hipStream_t stream);
int dopt_step_finalize(const dopt_layout *layout, const dopt_hparams *hp, int32_t n_hgroups, double max_grad_norm,
                       void *workspace, hipStream_t stream);
int dopt_step_apply(const dopt_layout *layout, const dopt_buffer_tensors *bufs, void *workspace,
                    hipStream_t stream);

/*
 * dopt_reduce_prepare -- the local half of a reduce-scatter with fp32
 * accumulation fused with pass 1 ([DP] §3.2,
 * reduce_scatter_with_fp32_accumulation: low precision on the wire, fp32
 * accumulation on the receiving rank, via all-to-all).  After the all-to-all
 * this rank holds one chunk of its windows from every rank of the group;
 * per arena slot
 *     g = (((0 + c_0) + c_1) + ... + c_{N-1}) * scale      (fp32, chunk order)
 * is written to bufs[k].grad in the buffer's grad dtype (round to nearest
 * even for 16-bit), and pass 1 (unscale, sum of squares, zero count) runs on
 * the stored value in the same pass.  Reading: the pages fix neither the
 * order of the sum nor where averaging happens; the sum runs in source-rank
 * order and `scale` (e.g. 1/N for averaging, else 1) multiplies it once.
 *
 * chunks: host array of one device pointer per buffer; chunk j of buffer k
 * is the arena_numel elements at chunks[k] + j * stride_k, element type
 * wire_dtype, where stride_k = chunk_strides[k] (elements) or, with
 * chunk_strides NULL, arena_numel (the chunks back to back).  A stride may
 * exceed arena_numel (a receive buffer with room between chunks); the caller
 * owns (n_chunks - 1) * stride_k + arena_numel elements at chunks[k], and the
 * library reads only each chunk's arena_numel.  n_chunks must equal dp_size
 * (one chunk per rank).  With hp
 * non-NULL the step's finalize runs too (as in dopt_step_prepare; then call
 * dopt_step_apply); with hp NULL only the grad-stats record is formed (as in
 * dopt_step_stats; then dopt_step_finalize after the cross-rank sum).
 * Errors: DOPT_ERR_INVALID (null or misaligned pointers, bad dtype,
 * n_chunks != dp_size, num_instances > 1, which [DP] §3.2 rules out, a
 * stride below arena_numel, above 2^40 elements or whose bytes are not a
 * multiple of DOPT_PTR_ALIGN, n_chunks strides of 2^62 bytes or more),
 * DOPT_ERR_HIP.
 */
int dopt_reduce_prepare(const dopt_layout *layout, const dopt_buffer_tensors *bufs, const void *const *chunks,
                        const int64_t *chunk_strides, int32_t wire_dtype, int32_t n_chunks, float scale,
                        const dopt_hparams *hp, int32_t n_hgroups, double max_grad_norm, void *workspace,
                        hipStream_t stream);

/* Result of the pre-communication check of one bucket. */
typedef struct dopt_bucket_check {
    double sumsq;     /* sum of squares of the bucket's grads, in double; NaN if any grad is NaN */
    float max_abs;    /* largest |grad|, NaN ignored; inf if any grad is infinite */
    int32_t has_nan;  /* some grad is NaN */
    int32_t has_inf;  /* some grad is +-inf */
    int32_t large;    /* large_threshold > 0 and max_abs > large_threshold */
} dopt_bucket_check;

/*
 * dopt_check_grads -- scan every bucket of flat buffer k of this rank's
 * local grads (the whole buffer, before the reduce-scatter) for NaN, Inf and
 * abnormally large values ([DP] §2.4: check_grads of the bucket group; §3.2:
 * check_for_nan_in_grad, check_for_large_grads).  Readings: the pages do not
 * define "large"; it is any |grad| above large_threshold (a caller input;
 * <= 0 turns it off).  The raw buffer values are checked (no unscaling), and
 * the bucket's padding is part of the scan as it is part of the bucket.
 *
 * grad_buffer: device, the full flat buffer k (numel elements of the
 * buffer's grad dtype, bucket b at its offset).  out: device array of
 * n_buckets records, written stream-ordered.  Each bucket's partials are
 * added in a fixed order, so sumsq is deterministic.  The workspace must have
 * been through dopt_init_state (which loads the bucket tables).
 * Errors: DOPT_ERR_INVALID (null or misaligned pointers), DOPT_ERR_RANGE (k),
 * DOPT_ERR_HIP.
 */
int dopt_check_grads(const dopt_layout *layout, int32_t k, const void *grad_buffer, double large_threshold,
                     dopt_bucket_check *out, void *workspace, hipStream_t stream);

/* Bytes of the library's static device scratch (see dopt_check_grads_noalloc). */
#define DOPT_NOALLOC_SCRATCH_BYTES 16777216

/*
 * dopt_check_grads_noalloc -- dopt_check_grads for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same scan, the same kernels and
 * bit-identical results, with no workspace argument and no dopt_init_state
 * needed.  Its bucket table and per-check-tile partials live in a static
 * device array of DOPT_NOALLOC_SCRATCH_BYTES (16 MiB) that each GPU the
 * library runs on holds until the process ends; the call allocates and frees
 * nothing, copies nothing from the host (the bucket table travels in kernel
 * arguments) and does not synchronize.
 *
 * A buffer needs 16 bytes per 16384-element check tile plus 24 bytes per
 * bucket (256-byte aligned): up to about 17e9 elements.  Larger buffers are
 * refused with DOPT_ERR_INVALID (use dopt_check_grads).  All calls on one GPU
 * share the one array: calls that overlap in time on one GPU (e.g. on two
 * streams) race and must not be issued; calls in stream order are safe.
 *
 * Arguments as dopt_check_grads.  Errors: DOPT_ERR_INVALID (null or
 * misaligned pointers, buffer too large for the scratch), DOPT_ERR_RANGE (k),
 * DOPT_ERR_HIP.
 */
int dopt_check_grads_noalloc(const dopt_layout *layout, int32_t k, const void *grad_buffer, double large_threshold,
                             dopt_bucket_check *out, hipStream_t stream);

/*
 * Sharded optimizer-state checkpoint in model-parameter space.  [DO] "三层继承
 * 体系" (third layer) lists fully reshardable optimizer formats: formats that
 * do not depend on the internal optimizer buffer structure.  The export
 * space of a rank is its param shards in model order, each shard contiguous
 * and in param coordinates (dopt_param_info.param), at
 * dopt_param_info.export_offset; it holds dopt_layout_state_numel()
 * elements.  Any other bucketing, data-parallel size or rank can read the
 * state it owns from the union of all ranks' exports.  Reading: the pages
 * name the formats only; this is the plainest model-space form.
 *
 * dopt_state_export: master (for fp32 params: the param itself), m and v of
 *   every shard element -> three device fp32 arrays of state_numel elements.
 * dopt_state_import: the inverse; also rewrites the param window from the
 *   imported master (round to nearest even for 16-bit params), as the step's
 *   copy-back would.
 * Both are stream-ordered device copies; the workspace must have been
 * through dopt_init_state.  Errors: DOPT_ERR_INVALID, DOPT_ERR_HIP.
 */
int dopt_state_export(const dopt_layout *layout, const dopt_buffer_tensors *bufs, float *master, float *exp_avg,
                      float *exp_avg_sq, void *workspace, hipStream_t stream);
int dopt_state_import(const dopt_layout *layout, const dopt_buffer_tensors *bufs, const float *master,
                      const float *exp_avg, const float *exp_avg_sq, void *workspace, hipStream_t stream);

/* The scalar optimizer state kept in the workspace. */
typedef struct dopt_state_scalars {
    int64_t step_count;          /* successful steps (Adam's t) */
    double loss_scale;
    int64_t growth_tracker;
    int64_t hysteresis_tracker;
} dopt_state_scalars;

/* Read / overwrite the scalar state (host struct); both synchronize `stream`.
 * _set: loss_scale as dopt_scaler_cfg.initial_scale, step_count >= 0, else
 * DOPT_ERR_INVALID before anything is written. */
int dopt_state_scalars_get(const dopt_layout *layout, const void *workspace, hipStream_t stream,
                           dopt_state_scalars *out);
int dopt_state_scalars_set(const dopt_layout *layout, void *workspace, hipStream_t stream,
                           const dopt_state_scalars *in);

/* Byte offset in the workspace of the grad-stats record: two doubles,
 * {sum of squares, zero count}; both are sums over ranks.  A non-finite sum
 * of squares means some rank found an inf/NaN. */
int64_t dopt_stats_record_offset(const dopt_layout *layout);

/* Copy the last step's stats to `out` (host); synchronizes `stream`. */
int dopt_read_stats(const dopt_layout *layout, const void *workspace, hipStream_t stream, dopt_stats *out);

/* Message for the last failing call on this thread (static storage). */
const char *dopt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
