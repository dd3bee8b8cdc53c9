/*
 * ORACLE -- test infrastructure only (see oracle.h for scope and the page
 * abbreviations [DO], [ZL], [DP], [DS]).
 *
 * Plain single-threaded C, built with -O2 -ffp-contract=off and no fast-math,
 * so every float operation below rounds once, in the order written.
 */
#include "oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static char g_err[256];
const char *or_error(void) { return g_err; }

static int fail(const char *msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return -1;
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t offset, numel, unpadded, shard, window_start, arena_offset;
    int64_t n_params;
} ob_bucket;

typedef struct {
    int32_t pd, gd;
    int64_t n_params;
    int64_t *params;         /* forward order */
    int32_t n_buckets;
    ob_bucket *buckets;
    int64_t numel, unpadded, window_numel, shard_numel;
    int64_t n_segs;
    int64_t *seg_start, *seg_len, *seg_param; /* ascending arena order */
} ob_buffer;

typedef struct {
    int64_t numel;
    int32_t pd, gd, newb, hgroup;
    int32_t buffer, bucket;
    int64_t start, end;      /* position in its flat buffer */
    int32_t has_shard;
    int64_t world[2], world_in_bucket[2], local[2], prange[2];
    int64_t arena;
} ob_param;

struct or_layout {
    int32_t N, r;
    int32_t n_buffers;
    ob_buffer *buf;
    int64_t n_params;
    ob_param *p;
};

static int64_t gcd64(int64_t a, int64_t b) {
    while (b) { int64_t t = a % b; a = b; b = t; }
    return a;
}
static int64_t lcm64(int64_t a, int64_t b) { return a / gcd64(a, b) * b; }
/* Smallest multiple of d that is >= x. */
static int64_t round_up(int64_t x, int64_t d) { return ((x + d - 1) / d) * d; }

static int dtype_ok(int32_t d) { return d == OR_F32 || d == OR_BF16 || d == OR_F16; }

/*
 * Bucket partition of one flat buffer, following [DO] "Bucket 划分算法：逆序
 * 遍历 + 尺寸触发" and "两级 Padding 机制":
 *   params are visited last-to-first; each start is raised to a multiple of 64
 *   elements; a param that must sit alone first closes a non-empty bucket;
 *   after placing a param, the bucket closes when it has reached bucket_size
 *   elements (measured from the bucket start to the param end) or when the
 *   param must sit alone; the last open bucket closes after the loop.
 *   Closing a bucket at x records x - bucket_start as its unpadded size and
 *   ends it at x raised to a multiple of lcm(N, 128) (lcm(N, 128, 2^16) in
 *   the high-bus-bandwidth mode); the next bucket starts there.
 * Reading: the body of the bucket-closing helper is not printed; it is taken
 * from its three call sites and the size assertions of [DO] "最终内存大小断言".
 */
typedef struct {
    int64_t bucket_start;
    int64_t divisor;
    int32_t n_buckets, cap;
    ob_bucket *b;
    int64_t open_count;
} part_state;

static int64_t close_bucket(part_state *s, int64_t x) {
    if (s->n_buckets == s->cap) {
        s->cap = s->cap ? 2 * s->cap : 16;
        s->b = (ob_bucket *)realloc(s->b, (size_t)s->cap * sizeof(ob_bucket));
    }
    ob_bucket *bk = &s->b[s->n_buckets++];
    memset(bk, 0, sizeof *bk);
    int64_t end = round_up(x, s->divisor);
    bk->offset = s->bucket_start;
    bk->numel = end - s->bucket_start;
    bk->unpadded = x - s->bucket_start;
    bk->n_params = s->open_count;
    s->bucket_start = end;
    s->open_count = 0;
    return end;
}

static int partition_buffer(or_layout *L, ob_buffer *B, int64_t bucket_size, int32_t pad_busbw) {
    part_state s;
    memset(&s, 0, sizeof s);
    s.divisor = lcm64(L->N, 128);
    if (pad_busbw) s.divisor = lcm64(s.divisor, 65536);
    int64_t ps = 0, pe = 0;
    for (int64_t j = B->n_params - 1; j >= 0; --j) {
        ob_param *p = &L->p[B->params[j]];
        ps = round_up(ps, 64);
        if (p->newb && s.open_count > 0) ps = close_bucket(&s, ps);
        pe = ps + p->numel;
        p->start = ps;
        p->end = pe;
        p->bucket = s.n_buckets;
        s.open_count++;
        if ((bucket_size > 0 && pe - s.bucket_start >= bucket_size) || p->newb)
            ps = close_bucket(&s, pe);
        else
            ps = pe;
    }
    if (s.open_count > 0) close_bucket(&s, pe);
    B->n_buckets = s.n_buckets;
    B->buckets = s.b;
    B->numel = s.bucket_start;
    B->unpadded = 0;
    for (int32_t b = 0; b < B->n_buckets; ++b) B->unpadded += B->buckets[b].unpadded;
    /* [DO] "最终内存大小断言" and "Bucket 级别的均等切分": size invariants. */
    if (!(B->unpadded <= B->numel)) return fail("assert: numel_unpadded <= numel");
    if (B->numel % L->N != 0) return fail("assert: numel % dp_size == 0");
    for (int32_t b = 0; b < B->n_buckets; ++b)
        if (B->buckets[b].numel % L->N != 0) return fail("assert: bucket numel % dp_size == 0");
    return 0;
}

/*
 * Rank r's window of a bucket is the r-th of N equal parts of it ([DO]
 * "Bucket 级别的均等切分").  A param's shard on this rank is, by definition,
 * the set of its elements that fall inside the window: the intersection of
 * [start, end) with [window_start, window_start + shard).  The four views of
 * [DO] "Range 类：四种视角的统一抽象" are that same element set expressed in
 * buffer, bucket, window and param coordinates.
 */
static void shard_param(ob_param *p, const ob_bucket *bk) {
    int64_t wlo = bk->window_start, whi = bk->window_start + bk->shard;
    int64_t lo = p->start > wlo ? p->start : wlo;
    int64_t hi = p->end < whi ? p->end : whi;
    if (hi <= lo) { p->has_shard = 0; return; }
    p->has_shard = 1;
    p->world[0] = lo;                    p->world[1] = hi;
    p->world_in_bucket[0] = lo - bk->offset; p->world_in_bucket[1] = hi - bk->offset;
    p->local[0] = lo - wlo;              p->local[1] = hi - wlo;
    p->prange[0] = lo - p->start;        p->prange[1] = hi - p->start;
    p->arena = bk->arena_offset + (lo - wlo);
}

int or_build(const or_param *params, int64_t n, int32_t dp_size, int32_t dp_rank, int64_t bucket_size,
             int32_t pad_busbw, or_layout **out) {
    if (!params || !out || n <= 0) return fail("invalid argument");
    if (dp_size < 1 || dp_rank < 0 || dp_rank >= dp_size) return fail("invalid dp_size/dp_rank");
    or_layout *L = (or_layout *)calloc(1, sizeof *L);
    L->N = dp_size;
    L->r = dp_rank;
    L->n_params = n;
    L->p = (ob_param *)calloc((size_t)n, sizeof(ob_param));
    L->buf = (ob_buffer *)calloc((size_t)n, sizeof(ob_buffer));
    for (int64_t i = 0; i < n; ++i) {
        if (params[i].numel <= 0 || !dtype_ok(params[i].param_dtype) || !dtype_ok(params[i].grad_dtype) ||
            params[i].hgroup < 0 || params[i].hgroup >= OR_MAX_HGROUPS) {
            or_free(L);
            return fail("invalid param descriptor");
        }
        ob_param *p = &L->p[i];
        p->numel = params[i].numel;
        p->pd = params[i].param_dtype;
        p->gd = params[i].grad_dtype;
        p->newb = params[i].requires_new_bucket != 0;
        p->hgroup = params[i].hgroup;
        /* One flat buffer per (param dtype, grad dtype), in order of first
         * appearance ([DP] §2.2 (3)). */
        int32_t k = 0;
        while (k < L->n_buffers && !(L->buf[k].pd == p->pd && L->buf[k].gd == p->gd)) ++k;
        if (k == L->n_buffers) {
            L->buf[k].pd = p->pd;
            L->buf[k].gd = p->gd;
            L->buf[k].params = (int64_t *)malloc((size_t)n * sizeof(int64_t));
            L->n_buffers++;
        }
        p->buffer = k;
        L->buf[k].params[L->buf[k].n_params++] = i;
    }
    for (int32_t k = 0; k < L->n_buffers; ++k) {
        ob_buffer *B = &L->buf[k];
        if (partition_buffer(L, B, bucket_size, pad_busbw) != 0) {
            or_free(L);
            return -1;
        }
        int64_t arena = 0;
        for (int32_t b = 0; b < B->n_buckets; ++b) {
            ob_bucket *bk = &B->buckets[b];
            bk->shard = bk->numel / L->N;
            bk->window_start = bk->offset + (int64_t)L->r * bk->shard;
            bk->arena_offset = arena;
            arena += bk->shard;
        }
        B->window_numel = arena;
        B->seg_start = (int64_t *)malloc((size_t)B->n_params * sizeof(int64_t));
        B->seg_len = (int64_t *)malloc((size_t)B->n_params * sizeof(int64_t));
        B->seg_param = (int64_t *)malloc((size_t)B->n_params * sizeof(int64_t));
        for (int64_t j = 0; j < B->n_params; ++j) {
            ob_param *p = &L->p[B->params[j]];
            shard_param(p, &B->buckets[p->bucket]);
            if (p->has_shard) {
                /* insertion into the ascending segment list */
                int64_t pos = B->n_segs++;
                while (pos > 0 && B->seg_start[pos - 1] > p->arena) {
                    B->seg_start[pos] = B->seg_start[pos - 1];
                    B->seg_len[pos] = B->seg_len[pos - 1];
                    B->seg_param[pos] = B->seg_param[pos - 1];
                    --pos;
                }
                B->seg_start[pos] = p->arena;
                B->seg_len[pos] = p->local[1] - p->local[0];
                B->seg_param[pos] = B->params[j];
                B->shard_numel += p->local[1] - p->local[0];
            }
        }
    }
    *out = L;
    return 0;
}

/*
 * [ZL] §5 (num_distributed_optimizer_instances) and [DP] §3.1: the
 * data-parallel domain of N ranks splits into I instances; the optimizer
 * shards over the N/I ranks of one instance, at the rank's place inside it.
 * Reading: instance i is the consecutive ranks [i*N/I, (i+1)*N/I).
 */
int or_build_instances(const or_param *params, int64_t n, int32_t dp_size, int32_t dp_rank, int32_t instances,
                       int64_t bucket_size, int32_t pad_busbw, or_layout **out) {
    if (instances < 1 || dp_size < 1 || dp_size % instances != 0) return fail("instances must divide dp_size");
    if (dp_rank < 0 || dp_rank >= dp_size) return fail("invalid dp_size/dp_rank");
    int32_t per = dp_size / instances;
    return or_build(params, n, per, dp_rank % per, bucket_size, pad_busbw, out);
}

void or_free(or_layout *L) {
    if (!L) return;
    for (int32_t k = 0; k < L->n_buffers; ++k) {
        free(L->buf[k].params);
        free(L->buf[k].buckets);
        free(L->buf[k].seg_start);
        free(L->buf[k].seg_len);
        free(L->buf[k].seg_param);
    }
    free(L->buf);
    free(L->p);
    free(L);
}

int32_t or_num_buffers(const or_layout *L) { return L->n_buffers; }

int or_buffer(const or_layout *L, int32_t k, int64_t out[8]) {
    if (k < 0 || k >= L->n_buffers) return fail("buffer index out of range");
    const ob_buffer *B = &L->buf[k];
    out[0] = B->pd; out[1] = B->gd; out[2] = B->n_buckets; out[3] = B->n_params;
    out[4] = B->numel; out[5] = B->unpadded; out[6] = B->window_numel; out[7] = B->shard_numel;
    return 0;
}

int or_bucket(const or_layout *L, int32_t k, int32_t b, int64_t out[7]) {
    if (k < 0 || k >= L->n_buffers || b < 0 || b >= L->buf[k].n_buckets) return fail("bucket index out of range");
    const ob_bucket *bk = &L->buf[k].buckets[b];
    out[0] = bk->offset; out[1] = bk->numel; out[2] = bk->unpadded; out[3] = bk->shard;
    out[4] = bk->window_start; out[5] = bk->arena_offset; out[6] = bk->n_params;
    return 0;
}

int or_param_info(const or_layout *L, int64_t i, int64_t out[15]) {
    if (i < 0 || i >= L->n_params) return fail("param index out of range");
    const ob_param *p = &L->p[i];
    out[0] = p->buffer; out[1] = p->bucket; out[2] = p->start; out[3] = p->end;
    out[4] = p->has_shard; out[5] = p->hgroup;
    for (int j = 0; j < 2; ++j) {
        out[6 + j] = p->has_shard ? p->world[j] : 0;
        out[8 + j] = p->has_shard ? p->world_in_bucket[j] : 0;
        out[10 + j] = p->has_shard ? p->local[j] : 0;
        out[12 + j] = p->has_shard ? p->prange[j] : 0;
    }
    out[14] = p->has_shard ? p->arena : -1;
    return 0;
}

/*
 * Group lists of [DO] "五组数据结构 / 分片切片逻辑" and [ZL] §3: params with a
 * shard on this rank, per optimizer param group, in model order; 16-bit params
 * go to the model_float16 / shard_float16 / shard_fp32_from_float16 lists (the
 * last is the fp32 master), fp32 params to model_fp32 / shard_fp32.
 */
int64_t or_group(const or_layout *L, int32_t kind, int32_t hgroup, int64_t *idx, int64_t cap) {
    int64_t c = 0;
    int want16 = (kind == OR_GROUP_MODEL_FLOAT16 || kind == OR_GROUP_SHARD_FLOAT16 ||
                  kind == OR_GROUP_SHARD_FP32_FROM_FLOAT16);
    if (kind < 0 || kind > 4) return -1;
    for (int64_t i = 0; i < L->n_params; ++i) {
        const ob_param *p = &L->p[i];
        if (!p->has_shard || p->hgroup != hgroup) continue;
        int is16 = p->pd != OR_F32;
        if (is16 != want16) continue;
        if (idx && c < cap) idx[c] = i;
        ++c;
    }
    return c;
}

int64_t or_segments(const or_layout *L, int32_t k, int64_t *start, int64_t *len, int64_t *param, int64_t cap) {
    if (k < 0 || k >= L->n_buffers) return -1;
    const ob_buffer *B = &L->buf[k];
    for (int64_t s = 0; s < B->n_segs && s < cap; ++s) {
        if (start) start[s] = B->seg_start[s];
        if (len) len[s] = B->seg_len[s];
        if (param) param[s] = B->seg_param[s];
    }
    return B->n_segs;
}

/* ------------------------------------------------------------------------ */
/* Numeric formats, from the IEEE 754 definitions                           */
/* ------------------------------------------------------------------------ */

static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of a binary32: the upcast appends 16 zero bits. */
float or_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float or_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int32_t e = (h >> 10) & 0x1f;
    uint32_t f = h & 0x3ff;
    if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (f << 13) | (f ? 0x00400000u : 0));
    if (e == 0) {
        float mag = ldexpf((float)f, -24); /* subnormal: f * 2^-24, exact in binary32 */
        return sign ? -mag : mag;
    }
    return bits_f32(sign | ((uint32_t)(e - 15 + 127) << 23) | (f << 13));
}

/*
 * Round a binary32 to the nearest bfloat16, ties to even.  The 16 dropped
 * bits decide: more than half an ulp rounds away from zero, less rounds
 * toward zero, exactly half rounds to the candidate with an even last bit.
 * Rounding up out of the largest finite value gives infinity (the carry runs
 * into the exponent).  NaN maps to a quiet NaN of the same sign.
 */
uint16_t or_f32_to_bf16(float x) {
    uint32_t u = f32_bits(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1;
    return (uint16_t)kept;
}

/*
 * Round a binary32 to the nearest binary16, ties to even, with gradual
 * underflow and overflow to infinity.  Work on the exact value
 * M * 2^(E-23) (M the 24-bit significand): the binary16 spacing at that
 * magnitude is 2^(max(E,-14)-10), so drop the low bits of M below that
 * spacing and round on them.
 */
uint16_t or_f32_to_f16(float x) {
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
    if (a == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
    if (a < 0x00800000u) return sign; /* binary32 subnormal: far below 2^-25 */
    int32_t E = (int32_t)(a >> 23) - 127;
    uint32_t M = (a & 0x7fffffu) | 0x800000u;
    if (E >= 16) return (uint16_t)(sign | 0x7c00u);
    int32_t eq = E > -14 ? E : -14;
    int32_t shift = 13 + eq - E;
    if (shift > 24) return sign;
    uint32_t q = M >> shift;
    uint32_t rem = M & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    if (E >= -14) return (uint16_t)(sign | (uint16_t)((uint32_t)(E + 15) * 1024u + (q - 1024u)));
    return (uint16_t)(sign | (uint16_t)q);
}

void or_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = or_f32_to_bf16(x[i]);
}
void or_f32_to_f16_n(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = or_f32_to_f16(x[i]);
}
void or_bf16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = or_bf16_to_f32(x[i]);
}
void or_f16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = or_f16_to_f32(x[i]);
}

/* A table of the 65536 binary16 values, filled from or_f16_to_f32, so that
 * large stats passes do not decode every element again.  It is filled once,
 * when the library is loaded (before any caller thread can run), and only
 * read afterwards, so callers on several threads share it without a race. */
static float g_f16_table[65536];
__attribute__((constructor)) static void f16_table_init(void) {
    for (uint32_t h = 0; h < 65536u; ++h) g_f16_table[h] = or_f16_to_f32((uint16_t)h);
}

static float load_f32(const void *base, int32_t dt, int64_t i) {
    if (dt == OR_F32) return ((const float *)base)[i];
    uint16_t h = ((const uint16_t *)base)[i];
    return dt == OR_BF16 ? or_bf16_to_f32(h) : g_f16_table[h];
}

static void store_param(void *base, int32_t dt, int64_t i, float x) {
    if (dt == OR_F32) ((float *)base)[i] = x;
    else if (dt == OR_BF16) ((uint16_t *)base)[i] = or_f32_to_bf16(x);
    else ((uint16_t *)base)[i] = or_f32_to_f16(x);
}

/* ------------------------------------------------------------------------ */
/* Local half of the fp32-accumulating reduce-scatter                       */
/* ------------------------------------------------------------------------ */

/*
 * [DP] §3.2 (reduce_scatter_with_fp32_accumulation): the values travel in low
 * precision and are accumulated in fp32 on the receiving rank.  For each
 * window slot i of buffer k (slots [lo, hi) only):
 *   acc = +0; acc = acc + chunk_j[i] for j = 0..n-1 (fp32, in chunk order);
 *   acc = acc * scale; grad[i] = acc stored in the buffer's grad dtype
 *   (round to nearest even for 16-bit).
 * Chunk j starts stride elements after chunk j-1.  Readings: the pages fix
 * neither the summation order nor the place of the averaging factor.
 */
void or_reduce_chunks(const or_layout *L, int32_t k, const void *chunks, int32_t wire_dtype, int32_t n_chunks,
                      int64_t stride, float scale, int64_t lo, int64_t hi, void *grad_out) {
    const ob_buffer *B = &L->buf[k];
    if (hi > B->window_numel) hi = B->window_numel;
    for (int64_t i = lo; i < hi; ++i) {
        float acc = 0.0f;
        for (int32_t j = 0; j < n_chunks; ++j) acc = acc + load_f32(chunks, wire_dtype, (int64_t)j * stride + i);
        acc = acc * scale;
        store_param(grad_out, B->gd, i, acc);
    }
}

/* ------------------------------------------------------------------------ */
/* Pre-communication check of whole buckets                                 */
/* ------------------------------------------------------------------------ */

/*
 * [DP] §2.4 (check_grads) and §3.2 (check_for_nan_in_grad,
 * check_for_large_grads), over the raw values of the buffer elements
 * [lo, hi) that lie in bucket b of buffer k (the bucket's padding included):
 * the sum of squares in double in index order, the largest |g| over the
 * non-NaN values, whether some value is NaN, whether some value is
 * infinite, and whether the largest |g| exceeds thr (thr > 0; reading: the
 * pages do not define "large", the threshold is the caller's).
 * out_flags: has_nan, has_inf, large.
 */
void or_check_bucket(const or_layout *L, int32_t k, int32_t b, const void *grad, int64_t lo, int64_t hi, double thr,
                     double *out_sumsq, float *out_max, int32_t *out_flags) {
    const ob_buffer *B = &L->buf[k];
    const ob_bucket *bk = &B->buckets[b];
    if (lo < bk->offset) lo = bk->offset;
    if (hi > bk->offset + bk->numel) hi = bk->offset + bk->numel;
    double sumsq = 0.0;
    float mx = 0.0f;
    int32_t has_nan = 0, has_inf = 0;
    for (int64_t i = lo; i < hi; ++i) {
        float g = load_f32(grad, B->gd, i);
        double gd = (double)g;
        sumsq += gd * gd;
        if (isnan(g)) {
            has_nan = 1;
            continue;
        }
        if (isinf(g)) has_inf = 1;
        if (fabsf(g) > mx) mx = fabsf(g);
    }
    *out_sumsq = sumsq;
    *out_max = mx;
    out_flags[0] = has_nan;
    out_flags[1] = has_inf;
    out_flags[2] = (thr > 0.0 && (double)mx > thr) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* The step                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * S1, master init: the fp32 master of a 16-bit param shard is that shard
 * upcast ([DO] "分片切片逻辑": clone of the shard, converted to float); the
 * Adam moments start at zero.  An fp32 param is updated in place and has no
 * separate master ([ZL] §3).
 */
void or_init_state(const or_layout *L, or_arrays *bufs) {
    for (int32_t k = 0; k < L->n_buffers; ++k) {
        const ob_buffer *B = &L->buf[k];
        for (int64_t s = 0; s < B->n_segs; ++s) {
            for (int64_t i = B->seg_start[s]; i < B->seg_start[s] + B->seg_len[s]; ++i) {
                if (B->pd != OR_F32) bufs[k].master[i] = load_f32(bufs[k].param, B->pd, i);
                bufs[k].m[i] = 0.0f;
                bufs[k].v[i] = 0.0f;
            }
        }
    }
}

float or_inv_scale(const or_scaler *sc) { return (float)(1.0 / sc->scale); }

/*
 * S2 ([DO] "三层继承体系", second layer: copy grads to fp32 main grads and
 * detect inf/NaN; first layer: grad norm and zero count).  Over the rank's
 * shard elements only, in ascending arena order:
 *   g = fp32(raw) * inv_scale     (one fp32 multiply)
 *   found_inf: some g is not finite
 *   sumsq = sum of g*g, each square and the running sum in double
 *   zeros = count of g == 0
 */
/*
 * S2 restricted to arena slots [lo, hi) of buffer k: the same per-element
 * work as or_grad_stats, returned as a partial (sumsq, zeros, found_inf) so a
 * caller can split one large pass into disjoint ranges and add the partials.
 */
void or_grad_stats_range(const or_layout *L, int32_t k, const void *grad, float inv_scale, int64_t lo, int64_t hi,
                         or_stats *st) {
    double sumsq = 0.0;
    uint64_t zeros = 0;
    int32_t found_inf = 0;
    const ob_buffer *B = &L->buf[k];
    for (int64_t s = 0; s < B->n_segs; ++s) {
        int64_t a = B->seg_start[s], e = B->seg_start[s] + B->seg_len[s];
        if (a < lo) a = lo;
        if (e > hi) e = hi;
        for (int64_t i = a; i < e; ++i) {
            float g = load_f32(grad, B->gd, i) * inv_scale;
            if (!isfinite(g)) found_inf = 1;
            double gd = (double)g;
            sumsq += gd * gd;
            if (g == 0.0f) zeros++;
        }
    }
    st->sumsq = sumsq;
    st->zeros = zeros;
    st->found_inf = found_inf;
}

void or_grad_stats(const or_layout *L, const or_arrays *bufs, float inv_scale, or_stats *st) {
    double sumsq = 0.0;
    uint64_t zeros = 0;
    int32_t found_inf = 0;
    for (int32_t k = 0; k < L->n_buffers; ++k) {
        const ob_buffer *B = &L->buf[k];
        for (int64_t s = 0; s < B->n_segs; ++s) {
            int64_t e = B->seg_start[s] + B->seg_len[s];
            for (int64_t i = B->seg_start[s]; i < e; ++i) {
                float g = load_f32(bufs[k].grad, B->gd, i) * inv_scale;
                if (!isfinite(g)) found_inf = 1;
                double gd = (double)g;
                sumsq += gd * gd;
                if (g == 0.0f) zeros++;
            }
        }
    }
    st->sumsq = sumsq;
    st->zeros = zeros;
    st->found_inf = found_inf;
}

/*
 * S3.  The norm is taken over the whole distributed-optimizer group ([DO]
 * third layer: the grad-stats group override); on one rank that reduction is
 * the identity.  A non-finite grad skips the step: nothing is updated and the
 * step count stays ([DO] second layer).  Readings (the pages name these steps
 * without printing them):
 *   clip coefficient = max_norm / (norm + 1e-6), applied only when below 1;
 *   dynamic loss scale: on overflow the growth count resets and, once the
 *   hysteresis count is used up, the scale is multiplied by the backoff
 *   factor (not below min_scale); otherwise the growth count rises and every
 *   growth_interval clean steps the scale is multiplied by the growth factor
 *   and the hysteresis count is restored;
 *   AdamW with decoupled weight decay and bias correction (Loshchilov &
 *   Hutter, "Decoupled Weight Decay Regularization"; Kingma & Ba, "Adam"),
 *   the optimizer type the pages' assertion admits: per-step scalars are
 *   computed in double and rounded once to fp32.
 */
int or_decide(or_stats *st, or_scaler *sc, int64_t *t, const or_hparams *hp, int32_t nh, double max_norm,
              or_scalars *out) {
    if (nh < 1 || nh > OR_MAX_HGROUPS) return fail("bad hyper-group count");
    memset(out, 0, sizeof *out);
    st->scale_used = sc->scale;
    out->inv_scale = or_inv_scale(sc);
    st->norm = sqrt(st->sumsq);
    st->skipped = st->found_inf;
    if (sc->dynamic) {
        if (st->found_inf) {
            sc->growth_tracker = 0;
            sc->hysteresis_tracker -= 1;
            if (sc->hysteresis_tracker <= 0) {
                double s = sc->scale * sc->backoff_factor;
                sc->scale = s > sc->min_scale ? s : sc->min_scale;
            }
        } else {
            sc->growth_tracker += 1;
            if (sc->growth_tracker == sc->growth_interval) {
                sc->growth_tracker = 0;
                sc->hysteresis_tracker = sc->hysteresis;
                sc->scale = sc->scale * sc->growth_factor;
            }
        }
    }
    st->scale_next = sc->scale;
    out->skip = st->skipped;
    st->clip_coef = 1.0;
    st->clip_applied = 0;
    if (!st->skipped) {
        *t += 1;
        if (max_norm > 0.0) {
            double c = max_norm / (st->norm + 1e-6);
            st->clip_coef = c;
            if (c < 1.0) {
                st->clip_applied = 1;
                out->clip_on = 1;
                out->clip = (float)c;
            }
        }
        for (int32_t h = 0; h < nh; ++h) {
            double tt = (double)*t;
            out->decay[h] = (float)(1.0 - hp[h].lr * hp[h].weight_decay);
            out->beta1[h] = (float)hp[h].beta1;
            out->omb1[h] = (float)(1.0 - hp[h].beta1);
            out->beta2[h] = (float)hp[h].beta2;
            out->omb2[h] = (float)(1.0 - hp[h].beta2);
            out->eps[h] = (float)hp[h].eps;
            out->step_size[h] = (float)(hp[h].lr / (1.0 - pow(hp[h].beta1, tt)));
            out->sqrt_bc2[h] = (float)sqrt(1.0 - pow(hp[h].beta2, tt));
        }
    }
    st->t = *t;
    return 0;
}

/*
 * S4 for one element, fp32 throughout, in this order:
 *   g = fp32(raw) * inv_scale;  g = g * clip (if clipping)
 *   p = p * (1 - lr*wd)                         decoupled weight decay
 *   m = beta1*m + (1-beta1)*g
 *   v = beta2*v + (1-beta2)*(g*g)
 *   p = p - step_size * (m / (sqrt(v)/sqrt(1-beta2^t) + eps)),
 *       step_size = lr / (1-beta1^t)
 * then the master is written back to the 16-bit param with round-to-nearest-
 * even ([DO] "分片切片逻辑", master-to-model copy; [DS] §2 step pseudocode).
 */
static inline void adamw_elem(float raw, float *p, float *m, float *v, const or_scalars *s, int32_t h) {
    float g = raw * s->inv_scale;
    if (s->clip_on) g = g * s->clip;
    float pp = *p * s->decay[h];
    float mm = s->beta1[h] * *m + s->omb1[h] * g;
    float vv = s->beta2[h] * *v + s->omb2[h] * (g * g);
    float d = sqrtf(vv) / s->sqrt_bc2[h] + s->eps[h];
    pp = pp - s->step_size[h] * (mm / d);
    *p = pp;
    *m = mm;
    *v = vv;
}

void or_apply(const or_layout *L, or_arrays *bufs, const or_scalars *s) {
    if (s->skip) return;
    for (int32_t k = 0; k < L->n_buffers; ++k) {
        const ob_buffer *B = &L->buf[k];
        for (int64_t q = 0; q < B->n_segs; ++q) {
            int32_t h = L->p[B->seg_param[q]].hgroup;
            int64_t e = B->seg_start[q] + B->seg_len[q];
            for (int64_t i = B->seg_start[q]; i < e; ++i) {
                float raw = load_f32(bufs[k].grad, B->gd, i);
                if (B->pd == OR_F32) {
                    float *pp = (float *)bufs[k].param + i;
                    adamw_elem(raw, pp, &bufs[k].m[i], &bufs[k].v[i], s, h);
                } else {
                    adamw_elem(raw, &bufs[k].master[i], &bufs[k].m[i], &bufs[k].v[i], s, h);
                    store_param(bufs[k].param, B->pd, i, bufs[k].master[i]);
                }
            }
        }
    }
}

/*
 * S4 restricted to arena slots [lo, hi) of buffer k: the update of or_apply
 * for the shard elements in that range.  Every element's update reads only
 * its own grad, master, m and v and the step's scalars, so a caller may split
 * one large pass into disjoint ranges (on threads) without changing any
 * result.
 */
void or_apply_range(const or_layout *L, int32_t k, or_arrays *bufs, const or_scalars *s, int64_t lo, int64_t hi) {
    if (s->skip) return;
    const ob_buffer *B = &L->buf[k];
    for (int64_t q = 0; q < B->n_segs; ++q) {
        int32_t h = L->p[B->seg_param[q]].hgroup;
        int64_t a = B->seg_start[q], e = B->seg_start[q] + B->seg_len[q];
        if (a < lo) a = lo;
        if (e > hi) e = hi;
        for (int64_t i = a; i < e; ++i) {
            float raw = load_f32(bufs[k].grad, B->gd, i);
            if (B->pd == OR_F32) {
                adamw_elem(raw, (float *)bufs[k].param + i, &bufs[k].m[i], &bufs[k].v[i], s, h);
            } else {
                adamw_elem(raw, &bufs[k].master[i], &bufs[k].m[i], &bufs[k].v[i], s, h);
                store_param(bufs[k].param, B->pd, i, bufs[k].master[i]);
            }
        }
    }
}

void or_apply_elems(int32_t param_dtype, int32_t grad_dtype, int64_t n, const int32_t *hgroup, const void *grad,
                    float *master, float *m, float *v, void *param_out, const or_scalars *s) {
    if (s->skip) return;
    for (int64_t i = 0; i < n; ++i) {
        float raw = load_f32(grad, grad_dtype, i);
        adamw_elem(raw, &master[i], &m[i], &v[i], s, hgroup ? hgroup[i] : 0);
        store_param(param_out, param_dtype, i, master[i]);
    }
}

int or_step(const or_layout *L, or_arrays *bufs, or_scaler *sc, int64_t *t, const or_hparams *hp, int32_t nh,
            double max_norm, or_stats *out) {
    or_scalars s;
    memset(out, 0, sizeof *out);
    or_grad_stats(L, bufs, or_inv_scale(sc), out);
    if (or_decide(out, sc, t, hp, nh, max_norm, &s) != 0) return -1;
    or_apply(L, bufs, &s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Model-space optimizer-state checkpoint                                   */
/* ------------------------------------------------------------------------ */

/*
 * [DO] "三层继承体系", third layer: the DistributedOptimizer class lists the
 * checkpoint formats that are fully reshardable, i.e. do not depend on how
 * the optimizer buffers are laid out; one is in model space.  Reading: the
 * pages give the formats' names only.  Plainest model-space form: walk the
 * params in model order; each param that has a shard on this rank contributes
 * its shard, in param coordinates, as one contiguous run of the export; per
 * element the export holds the fp32 master (the param itself for fp32
 * params), m and v.  Any layout (other N, rank or bucketing) recovers its own
 * shards from the union of all ranks' exports by param coordinates.
 * Returns the number of exported elements.
 */
int64_t or_state_export(const or_layout *L, const or_arrays *bufs, float *master, float *m, float *v) {
    int64_t x = 0;
    for (int64_t i = 0; i < L->n_params; ++i) {
        const ob_param *p = &L->p[i];
        if (!p->has_shard) continue;
        const or_arrays *b = &bufs[p->buffer];
        const float *pm = p->pd == OR_F32 ? (const float *)b->param : b->master;
        for (int64_t j = 0; j < p->prange[1] - p->prange[0]; ++j, ++x) {
            master[x] = pm[p->arena + j];
            m[x] = b->m[p->arena + j];
            v[x] = b->v[p->arena + j];
        }
    }
    return x;
}

/*
 * Inverse of or_state_export.  Loading the master also refreshes the 16-bit
 * model param from it (round to nearest even), the same copy-back the
 * update ends with ([DO] "三层继承体系", second layer).
 */
void or_state_import(const or_layout *L, or_arrays *bufs, const float *master, const float *m, const float *v) {
    int64_t x = 0;
    for (int64_t i = 0; i < L->n_params; ++i) {
        const ob_param *p = &L->p[i];
        if (!p->has_shard) continue;
        or_arrays *b = &bufs[p->buffer];
        for (int64_t j = 0; j < p->prange[1] - p->prange[0]; ++j, ++x) {
            const int64_t e = p->arena + j;
            if (p->pd == OR_F32) {
                ((float *)b->param)[e] = master[x];
            } else {
                b->master[e] = master[x];
                store_param(b->param, p->pd, e, master[x]);
            }
            b->m[e] = m[x];
            b->v[e] = v[x];
        }
    }
}
