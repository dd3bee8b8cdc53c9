/*
 * Driver for running the C oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with gcc).
 * Reads the same layout cases as mapper_driver.cpp from stdin; for each it
 * prints the oracle's layout queries and, for windows of at most 1 << 20
 * slots, a checksum of three steps (the third with a +inf grad), a state
 * export / import round trip, the local fp32-accumulating reduce and the
 * whole-bucket check on seeded data.  It reads nothing but the oracle.
 */
#include <inttypes.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void) { /* SplitMix64 */
    uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

/* a value in [-a, a) */
static float draw(float a) { return a * ((float)(next_u32() >> 8) / 8388608.0f - 1.0f); }

static uint64_t fnv(uint64_t h, const void *p, size_t n) {
    const unsigned char *c = (const unsigned char *)p;
    for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001b3ull;
    return h;
}

static size_t esize(int32_t dt) { return dt == OR_F32 ? 4 : 2; }

static void fill(int32_t dt, void *dst, int64_t n, float a) {
    for (int64_t i = 0; i < n; ++i) {
        const float x = draw(a);
        if (dt == OR_F32) ((float *)dst)[i] = x;
        else if (dt == OR_BF16) ((uint16_t *)dst)[i] = or_f32_to_bf16(x);
        else ((uint16_t *)dst)[i] = or_f32_to_f16(x);
    }
}

static void dump_layout(const or_layout *L, int64_t n_params) {
    const int32_t nb = or_num_buffers(L);
    printf("buffers %d\n", nb);
    for (int32_t k = 0; k < nb; ++k) {
        int64_t b8[8];
        const int rc = or_buffer(L, k, b8);
        printf("buf %d %d", k, rc);
        for (int i = 0; i < 8; ++i) printf(" %" PRId64, b8[i]);
        printf("\n");
        for (int32_t b = 0; b < (int32_t)b8[2]; ++b) {
            int64_t k7[7];
            printf("bkt %d %d %d", k, b, or_bucket(L, k, b, k7));
            for (int i = 0; i < 7; ++i) printf(" %" PRId64, k7[i]);
            printf("\n");
        }
        const int64_t ns = or_segments(L, k, NULL, NULL, NULL, 0);
        int64_t *st = malloc(sizeof(int64_t) * (size_t)(ns + 1)), *ln = malloc(sizeof(int64_t) * (size_t)(ns + 1));
        int64_t *pr = malloc(sizeof(int64_t) * (size_t)(ns + 1));
        or_segments(L, k, st, ln, pr, ns);
        uint64_t h = fnv(1469598103934665603ull, st, sizeof(int64_t) * (size_t)ns);
        h = fnv(h, ln, sizeof(int64_t) * (size_t)ns);
        h = fnv(h, pr, sizeof(int64_t) * (size_t)ns);
        printf("segs %d %" PRId64 " %016" PRIx64 "\n", k, ns, h);
        free(st);
        free(ln);
        free(pr);
    }
    for (int64_t p = 0; p < n_params; ++p) {
        int64_t q[15];
        printf("par %" PRId64 " %d", p, or_param_info(L, p, q));
        for (int i = 0; i < 15; ++i) printf(" %" PRId64, q[i]);
        printf("\n");
    }
    for (int32_t kind = 0; kind <= OR_GROUP_SHARD_FP32; ++kind)
        for (int32_t hg = 0; hg < OR_MAX_HGROUPS; ++hg) {
            const int64_t n = or_group(L, kind, hg, NULL, 0);
            if (n <= 0) continue;
            int64_t *idx = malloc(sizeof(int64_t) * (size_t)n);
            or_group(L, kind, hg, idx, n);
            printf("grp %d %d %" PRId64 " %016" PRIx64 "\n", kind, hg, n,
                   fnv(1469598103934665603ull, idx, sizeof(int64_t) * (size_t)n));
            free(idx);
        }
}

typedef struct {
    int32_t pd, gd;
    int64_t win, numel;
    void *grad, *param;
    float *master, *m, *v;
} bufmem;

static uint64_t hash_state(const bufmem *bm, int32_t nb) {
    uint64_t h = 1469598103934665603ull;
    for (int32_t k = 0; k < nb; ++k) {
        const bufmem *b = &bm[k];
        h = fnv(h, b->param, esize(b->pd) * (size_t)b->win);
        if (b->master) h = fnv(h, b->master, 4 * (size_t)b->win);
        h = fnv(h, b->m, 4 * (size_t)b->win);
        h = fnv(h, b->v, 4 * (size_t)b->win);
    }
    return h;
}

static void run_numeric(const or_layout *L) {
    const int32_t nb = or_num_buffers(L);
    bufmem *bm = calloc((size_t)nb, sizeof(bufmem));
    or_arrays *arr = calloc((size_t)nb, sizeof(or_arrays));
    int64_t state_n = 0;
    for (int32_t k = 0; k < nb; ++k) {
        int64_t b8[8];
        or_buffer(L, k, b8);
        bufmem *b = &bm[k];
        b->pd = (int32_t)b8[0];
        b->gd = (int32_t)b8[1];
        b->numel = b8[4];
        b->win = b8[6];
        state_n += b8[7];
        /* zeroed: arena slots that hold no param element are never written */
        const size_t w = (size_t)(b->win > 0 ? b->win : 1);
        b->grad = calloc(w, esize(b->gd));
        b->param = calloc(w, esize(b->pd));
        b->master = b->pd == OR_F32 ? NULL : calloc(w, 4);
        b->m = calloc(w, 4);
        b->v = calloc(w, 4);
        fill(b->pd, b->param, b->win, 0.05f);
        arr[k].grad = b->grad;
        arr[k].param = b->param;
        arr[k].master = b->master;
        arr[k].m = b->m;
        arr[k].v = b->v;
    }
    or_init_state(L, arr);
    or_hparams hp[3] = {{1e-3, 0.9, 0.999, 1e-8, 0.01}, {3e-4, 0.8, 0.99, 1e-6, 0.0}, {2e-3, 0.95, 0.9999, 1e-8, 0.1}};
    or_scaler sc;
    memset(&sc, 0, sizeof sc);
    sc.dynamic = 1;
    sc.hysteresis = 1;
    sc.growth_interval = 2;
    sc.growth_factor = 2.0;
    sc.backoff_factor = 0.5;
    sc.min_scale = 1.0;
    sc.scale = 1024.0;
    sc.hysteresis_tracker = 1;
    int64_t t = 0;
    for (int step = 0; step < 3; ++step) {
        for (int32_t k = 0; k < nb; ++k) fill(bm[k].gd, bm[k].grad, bm[k].win, 0.5f);
        int injected = 0;
        for (int32_t k = 0; step == 2 && k < nb && !injected; ++k) { /* +inf in the middle of a shard */
            const int64_t ns = or_segments(L, k, NULL, NULL, NULL, 0);
            if (ns <= 0) continue;
            int64_t *st0 = malloc(sizeof(int64_t) * (size_t)ns), *ln = malloc(sizeof(int64_t) * (size_t)ns);
            or_segments(L, k, st0, ln, NULL, ns);
            const int64_t i = st0[ns / 2] + ln[ns / 2] / 2;
            if (bm[k].gd == OR_F32) ((float *)bm[k].grad)[i] = INFINITY;
            else ((uint16_t *)bm[k].grad)[i] = bm[k].gd == OR_BF16 ? 0x7f80 : 0x7c00;
            injected = 1;
            free(st0);
            free(ln);
        }
        or_stats st;
        const int rc = or_step(L, arr, &sc, &t, hp, 3, 1.0, &st);
        printf("step %d rc %d inf %d skip %d clip %d sumsq %a zeros %" PRIu64 " scale %a t %" PRId64
               " state %016" PRIx64 "\n",
               step, rc, st.found_inf, st.skipped, st.clip_applied, st.sumsq, st.zeros, st.scale_next, t,
               hash_state(bm, nb));
        if (step == 2)
            printf("overflow %s\n", (injected ? (st.found_inf && st.skipped) : !st.found_inf) ? "ok" : "BAD");
    }
    /* model-space export, then import into the same arrays */
    const size_t sn = (size_t)(state_n > 0 ? state_n : 1);
    float *xm = malloc(4 * sn), *xa = malloc(4 * sn), *xv = malloc(4 * sn);
    const int64_t got = or_state_export(L, arr, xm, xa, xv);
    const uint64_t before = hash_state(bm, nb);
    or_state_import(L, arr, xm, xa, xv);
    printf("export %" PRId64 " %" PRId64 " %016" PRIx64 " same %d\n", got, state_n,
           fnv(fnv(fnv(1469598103934665603ull, xm, 4 * (size_t)got), xa, 4 * (size_t)got), xv, 4 * (size_t)got),
           hash_state(bm, nb) == before);
    free(xm);
    free(xa);
    free(xv);
    /* local reduce of 3 bf16 chunks into buffer 0's grad window */
    if (nb > 0 && bm[0].win > 0) {
        const int64_t w = bm[0].win;
        uint16_t *ch = malloc(2 * (size_t)(3 * w));
        fill(OR_BF16, ch, 3 * w, 0.25f);
        or_reduce_chunks(L, 0, ch, OR_BF16, 3, w, 1.0f / 3.0f, 0, w, bm[0].grad);
        printf("reduce %016" PRIx64 "\n", fnv(1469598103934665603ull, bm[0].grad, esize(bm[0].gd) * (size_t)w));
        free(ch);
        /* whole-bucket check of buffer 0, one NaN planted in its first bucket */
        int64_t b8[8];
        or_buffer(L, 0, b8);
        void *g = calloc((size_t)bm[0].numel, esize(bm[0].gd));
        fill(bm[0].gd, g, bm[0].numel, 2.0f);
        if (bm[0].gd == OR_F32) ((float *)g)[bm[0].numel / 3] = NAN;
        else ((uint16_t *)g)[bm[0].numel / 3] = 0x7fc0;
        for (int32_t b = 0; b < (int32_t)b8[2]; ++b) {
            int64_t k7[7];
            or_bucket(L, 0, b, k7);
            double ss = 0.0;
            float mx = 0.0f;
            int32_t fl[3] = {0, 0, 0}; /* has_nan, has_inf, large */
            or_check_bucket(L, 0, b, g, k7[0], k7[0] + k7[1], 1.5, &ss, &mx, fl);
            printf("check %d %a %a %d %d %d\n", b, ss, (double)mx, fl[0], fl[1], fl[2]);
        }
        free(g);
    }
    for (int32_t k = 0; k < nb; ++k) {
        free(bm[k].grad);
        free(bm[k].param);
        free(bm[k].master);
        free(bm[k].m);
        free(bm[k].v);
    }
    free(bm);
    free(arr);
}

int main(void) {
    int32_t N = 0, r = 0, busbw = 0, inst = 0;
    int64_t bucket = 0, n = 0;
    while (scanf("%d %d %" SCNd64 " %d %d %" SCNd64, &N, &r, &bucket, &busbw, &inst, &n) == 6 && n > 0) {
        or_param *ps = malloc(sizeof(or_param) * (size_t)n);
        for (int64_t i = 0; i < n; ++i)
            if (scanf("%" SCNd64 " %d %d %d %d", &ps[i].numel, &ps[i].param_dtype, &ps[i].grad_dtype,
                      &ps[i].requires_new_bucket, &ps[i].hgroup) != 5)
                return 2;
        or_layout *L = NULL;
        const int rc = or_build_instances(ps, n, N, r, inst, bucket, busbw, &L);
        printf("case %d %d %" PRId64 " %d %d %" PRId64 " rc %d\n", N, r, bucket, busbw, inst, n, rc);
        if (rc == 0) {
            dump_layout(L, n);
            int64_t win = 0;
            for (int32_t k = 0; k < or_num_buffers(L); ++k) {
                int64_t b8[8];
                or_buffer(L, k, b8);
                win += b8[6];
            }
            if (win <= (1 << 20)) run_numeric(L);
            or_free(L);
        }
        free(ps);
    }
    return 0;
}
