/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, single-threaded C statement of what the shard-local
 * mixed-precision AdamW step of a ZeRO-1 distributed optimizer computes on one
 * data-parallel rank.  It exists to check the product library against; only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the product
 * library (sharded_mixed_precision_amd/), and neither includes the other.
 *
 * Pages cited below (title, then the section used):
 *   [DO]  "Megatron-LM distrib_optimizer.py 源码精读"
 *   [ZL]  "02 · ZeRO 显存账本与 Megatron DistributedOptimizer"
 *   [DP]  "Megatron-LM distributed 包深度解析：DDP 梯度同步与 finalize_model_grads 全流程"
 *   [DS]  "Megatron-LM与DeepSpeed的分布式训练源码里，模型和优化器到底是怎么切分的？"
 *
 * Parity pinned by the -m "not gpu" tests: layout (brute-force ownership,
 * the pages' worked example, invariants), ledger (the pages' byte counts),
 * conversions (exhaustive against an exact-arithmetic / library formulation),
 * AdamW closed forms, skip / loss-scale closed forms.  Parity unpinned: the
 * particular fp32 operation order of the update and the dynamic-scaler
 * constants, which the pages do not fix (both are readings, listed in the
 * design notes).
 */
#ifndef SMP_ORACLE_H
#define SMP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };

enum {
    OR_GROUP_MODEL_FLOAT16 = 0,
    OR_GROUP_MODEL_FP32 = 1,
    OR_GROUP_SHARD_FLOAT16 = 2,
    OR_GROUP_SHARD_FP32_FROM_FLOAT16 = 3,
    OR_GROUP_SHARD_FP32 = 4
};

#define OR_MAX_HGROUPS 16

typedef struct {
    int64_t numel;
    int32_t param_dtype, grad_dtype;
    int32_t requires_new_bucket;
    int32_t hgroup;
} or_param;

typedef struct or_layout or_layout;

/* Layout for rank dp_rank of dp_size.  bucket_size <= 0: no size trigger.
 * Returns 0, or -1 with or_error() set. */
int or_build(const or_param *params, int64_t n, int32_t dp_size, int32_t dp_rank,
             int64_t bucket_size, int32_t pad_busbw, or_layout **out);
/* Same, with the data-parallel domain split into `instances` optimizer instances. */
int or_build_instances(const or_param *params, int64_t n, int32_t dp_size, int32_t dp_rank, int32_t instances,
                       int64_t bucket_size, int32_t pad_busbw, or_layout **out);
void or_free(or_layout *L);
const char *or_error(void);

int32_t or_num_buffers(const or_layout *L);
/* out: param_dtype, grad_dtype, n_buckets, n_params, numel, numel_unpadded,
 *      window_numel, shard_numel */
int or_buffer(const or_layout *L, int32_t k, int64_t out[8]);
/* out: offset, numel, numel_unpadded, shard, window_start, arena_offset, n_params */
int or_bucket(const or_layout *L, int32_t k, int32_t b, int64_t out[7]);
/* out: buffer, bucket, start, end, has_shard, hgroup,
 *      gbuf_world(2), gbuf_world_in_bucket(2), gbuf_local(2), param(2), arena_offset */
int or_param_info(const or_layout *L, int64_t p, int64_t out[15]);
/* Forward-order indices of the params of one group kind and hyper-group. */
int64_t or_group(const or_layout *L, int32_t kind, int32_t hgroup, int64_t *idx, int64_t cap);
/* Arena segments of buffer k, ascending: start, length, param index. */
int64_t or_segments(const or_layout *L, int32_t k, int64_t *start, int64_t *len, int64_t *param, int64_t cap);

/* ---- numeric formats (IEEE 754 binary32 <-> bfloat16 / binary16) ---- */
float or_bf16_to_f32(uint16_t h);
float or_f16_to_f32(uint16_t h);
uint16_t or_f32_to_bf16(float x);
uint16_t or_f32_to_f16(float x);
void or_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n);
void or_f32_to_f16_n(const float *x, uint16_t *y, int64_t n);
void or_bf16_to_f32_n(const uint16_t *x, float *y, int64_t n);
void or_f16_to_f32_n(const uint16_t *x, float *y, int64_t n);

/* ---- local half of the fp32-accumulating reduce-scatter ---- */
/* grad[i] = storage((sum over chunks in order, fp32, from +0) * scale) for
 * window slots i in [lo, hi) of buffer k; chunk j at chunks + j*stride. */
void or_reduce_chunks(const or_layout *L, int32_t k, const void *chunks, int32_t wire_dtype, int32_t n_chunks,
                      int64_t stride, float scale, int64_t lo, int64_t hi, void *grad_out);

/* ---- pre-communication check of whole buckets ---- */
/* Over buffer elements [lo, hi) of bucket b of buffer k: sum of squares,
 * largest |g| (NaN ignored), flags {has_nan, has_inf, max > thr}. */
void or_check_bucket(const or_layout *L, int32_t k, int32_t b, const void *grad, int64_t lo, int64_t hi, double thr,
                     double *out_sumsq, float *out_max, int32_t *out_flags);

/* ---- the step ---- */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
} or_hparams;

typedef struct {
    int32_t dynamic;          /* 0: constant scale */
    int32_t hysteresis;
    int64_t growth_interval;
    double growth_factor, backoff_factor, min_scale;
    double scale;             /* live */
    int64_t growth_tracker;   /* live */
    int64_t hysteresis_tracker; /* live */
} or_scaler;

typedef struct {
    int32_t found_inf, skipped, clip_applied, pad;
    double sumsq, norm, clip_coef;
    uint64_t zeros;
    double scale_used, scale_next;
    int64_t t;                /* successful steps after this one */
} or_stats;

/* The fp32 scalars the elementwise update applies (one set per step). */
typedef struct {
    int32_t skip, clip_on;
    float inv_scale, clip;
    float decay[OR_MAX_HGROUPS], beta1[OR_MAX_HGROUPS], omb1[OR_MAX_HGROUPS];
    float beta2[OR_MAX_HGROUPS], omb2[OR_MAX_HGROUPS], eps[OR_MAX_HGROUPS];
    float step_size[OR_MAX_HGROUPS], sqrt_bc2[OR_MAX_HGROUPS];
} or_scalars;

/* Per-buffer arrays in window-arena coordinates (windows of the buffer's
 * buckets back to back in bucket order). */
typedef struct {
    const void *grad;
    void *param;
    float *master;   /* NULL for fp32-param buffers (the param is its own master) */
    float *m, *v;
} or_arrays;

void or_init_state(const or_layout *L, or_arrays *bufs);
/* S2: unscale, inf/NaN, sum of squares, zeros over the rank's shard elements. */
void or_grad_stats(const or_layout *L, const or_arrays *bufs, float inv_scale, or_stats *st);
/* S2 over arena slots [lo, hi) of buffer k only (a partial of the above). */
void or_grad_stats_range(const or_layout *L, int32_t k, const void *grad, float inv_scale, int64_t lo, int64_t hi,
                         or_stats *st);
/* S3: skip decision, norm, clip, loss-scale update, step count, scalars. */
int or_decide(or_stats *st, or_scaler *sc, int64_t *t, const or_hparams *hp, int32_t nh,
              double max_norm, or_scalars *out);
/* S4: clip + AdamW + write-back over the rank's shard elements. */
void or_apply(const or_layout *L, or_arrays *bufs, const or_scalars *s);
/* S4 on a list of elements (each with its own hyper-group). */
/* S4 restricted to arena slots [lo, hi) of buffer k (the same update per
 * element as or_apply; disjoint ranges may run on different threads). */
void or_apply_range(const or_layout *L, int32_t k, or_arrays *bufs, const or_scalars *s, int64_t lo, int64_t hi);
void or_apply_elems(int32_t param_dtype, int32_t grad_dtype, int64_t n, const int32_t *hgroup,
                    const void *grad, float *master, float *m, float *v, void *param_out,
                    const or_scalars *s);
/* S2..S4 in order. */
int or_step(const or_layout *L, or_arrays *bufs, or_scaler *sc, int64_t *t, const or_hparams *hp,
            int32_t nh, double max_norm, or_stats *out);
float or_inv_scale(const or_scaler *sc);

/* ---- model-space optimizer-state checkpoint ---- */
/* The rank's shards of master (fp32 params: the param), m and v, params in
 * model order, each shard contiguous in param coordinates.  Returns the
 * element count. */
int64_t or_state_export(const or_layout *L, const or_arrays *bufs, float *master, float *m, float *v);
/* Inverse; also writes the 16-bit params from the imported master. */
void or_state_import(const or_layout *L, or_arrays *bufs, const float *master, const float *m, const float *v);

#ifdef __cplusplus
}
#endif
#endif
