/*
 * Driver for running the C oracle's range functions from several threads
 * under ThreadSanitizer (built by tests/test_sanitizers.py with gcc).  The
 * GPU parity harness splits the statistics of the largest workloads, the
 * local fp32-accumulating reduce and the bucket check over disjoint ranges
 * run on host threads; this program does the same on seeded data with fp16
 * and bf16 grads (fp16 decoding goes through the oracle's shared table) and
 * prints the combined results next to the same ranges run on one thread,
 * which must agree bit for bit.  It reads nothing but the oracle.
 */
#include <inttypes.h>
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define NTHREADS 8
#define NRANGES 37

static uint64_t g_rng = 0x243f6a8885a308d3ull;

static uint32_t next_u32(void) { /* SplitMix64 */
    uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static float draw(float a) { return a * ((float)(next_u32() >> 8) / 8388608.0f - 1.0f); }

typedef struct {
    const or_layout *L;
    int32_t k, wire, n_chunks;
    const uint16_t *grad, *chunks;
    uint16_t *reduced;
    int64_t stride;
    int64_t lo[NRANGES], hi[NRANGES];
    or_stats st[NRANGES];
    double chk_sumsq[NRANGES];
    float chk_max[NRANGES];
    int32_t chk_flags[NRANGES][3];
    int next; /* next range to take; guarded by mu */
    pthread_mutex_t mu;
} job;

static void do_range(job *j, int i) {
    or_grad_stats_range(j->L, j->k, j->grad, 1.0f / 1024.0f, j->lo[i], j->hi[i], &j->st[i]);
    or_reduce_chunks(j->L, j->k, j->chunks, j->wire, j->n_chunks, j->stride, 0.125f, j->lo[i], j->hi[i],
                     j->reduced);
    or_check_bucket(j->L, j->k, 0, j->grad, j->lo[i], j->hi[i], 1.0, &j->chk_sumsq[i], &j->chk_max[i],
                    j->chk_flags[i]);
}

static void *worker(void *arg) {
    job *j = (job *)arg;
    for (;;) {
        pthread_mutex_lock(&j->mu);
        const int i = j->next++;
        pthread_mutex_unlock(&j->mu);
        if (i >= NRANGES) return NULL;
        do_range(j, i);
    }
}

static uint64_t fnv(uint64_t h, const void *p, size_t n) {
    const unsigned char *c = (const unsigned char *)p;
    for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001b3ull;
    return h;
}

static void report(const char *tag, const job *j, int64_t n) {
    double sq = 0.0, csq = 0.0;
    uint64_t z = 0;
    int32_t fi = 0, fl[3] = {0, 0, 0};
    float mx = 0.0f;
    for (int i = 0; i < NRANGES; ++i) {
        sq += j->st[i].sumsq;
        z += j->st[i].zeros;
        fi |= j->st[i].found_inf;
        csq += j->chk_sumsq[i];
        if (j->chk_max[i] > mx) mx = j->chk_max[i];
        for (int q = 0; q < 3; ++q) fl[q] |= j->chk_flags[i][q];
    }
    printf("%s k %d sumsq %a zeros %" PRIu64 " inf %d reduced %016" PRIx64 " check %a %a %d %d %d\n", tag, j->k, sq,
           z, fi, fnv(1469598103934665603ull, j->reduced, (size_t)n * 2), csq, (double)mx, fl[0], fl[1], fl[2]);
}

int main(void) {
    /* three layouts: fp16 grads (the table), bf16 grads, and an odd N */
    const int32_t dts[3] = {OR_F16, OR_BF16, OR_F16};
    const int32_t Ns[3] = {8, 4, 96}, ranks[3] = {3, 1, 50};
    for (int c = 0; c < 3; ++c) {
        or_param ps[9];
        const int64_t sizes[9] = {70001, 129, 4096, 33333, 1, 65536, 777, 12000, 5};
        for (int i = 0; i < 9; ++i) {
            memset(&ps[i], 0, sizeof ps[i]);
            ps[i].numel = sizes[i];
            ps[i].param_dtype = dts[c];
            ps[i].grad_dtype = dts[c];
        }
        or_layout *L = NULL;
        if (or_build(ps, 9, Ns[c], ranks[c], 0, 0, &L) != 0) {
            printf("build failed: %s\n", or_error());
            return 1;
        }
        int64_t b8[8];
        or_buffer(L, 0, b8);
        const int64_t win = b8[6], numel = b8[4];
        /* grads over the whole buffer (the check scans buckets; the stats
         * read window slots [0, win)); chunks over the window */
        const int64_t n = numel > win ? numel : win;
        uint16_t *grad = (uint16_t *)malloc((size_t)n * 2);
        uint16_t *chunks = (uint16_t *)malloc((size_t)(4 * win) * 2);
        for (int64_t i = 0; i < n; ++i)
            grad[i] = dts[c] == OR_F16 ? or_f32_to_f16(draw(8.0f)) : or_f32_to_bf16(draw(8.0f));
        for (int64_t i = 0; i < 4 * win; ++i)
            chunks[i] = dts[c] == OR_F16 ? or_f32_to_f16(draw(2.0f)) : or_f32_to_bf16(draw(2.0f));
        job par, seq;
        memset(&par, 0, sizeof par);
        par.L = L;
        par.k = 0;
        par.wire = dts[c];
        par.n_chunks = 4;
        par.grad = grad;
        par.chunks = chunks;
        par.stride = win;
        for (int i = 0; i < NRANGES; ++i) {
            par.lo[i] = win * i / NRANGES;
            par.hi[i] = win * (i + 1) / NRANGES;
        }
        seq = par;
        par.reduced = (uint16_t *)calloc((size_t)win + 1, 2);
        seq.reduced = (uint16_t *)calloc((size_t)win + 1, 2);
        pthread_mutex_init(&par.mu, NULL);
        pthread_t th[NTHREADS];
        for (int t = 0; t < NTHREADS; ++t) pthread_create(&th[t], NULL, worker, &par);
        for (int t = 0; t < NTHREADS; ++t) pthread_join(th[t], NULL);
        for (int i = 0; i < NRANGES; ++i) do_range(&seq, i);
        report("threads", &par, win);
        report("serial ", &seq, win);
        pthread_mutex_destroy(&par.mu);
        free(par.reduced);
        free(seq.reduced);
        free(grad);
        free(chunks);
        or_free(L);
    }
    return 0;
}
