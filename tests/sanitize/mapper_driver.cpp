// Driver for running the host range mapper under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with g++; no
// device code is involved).  Reads layout cases from stdin and prints every
// layout query's result, then exercises the argument-error paths.
//
// Input, per case: "N r bucket_size busbw instances n" then n lines
// "numel param_dtype grad_dtype requires_new_bucket hgroup"; a line with
// n = 0 ends the input.
#include <cinttypes>
#include <cstdio>
#include <vector>

#include "dopt.h"

static void dump(const dopt_layout *L) {
    dopt_sharding_info sh;
    const int rs = dopt_layout_sharding(L, &sh);
    printf("sharding %d %d %d %d %d %d %d\n", rs, sh.dp_size, sh.dp_rank, sh.num_instances, sh.instance_size,
           sh.instance_index, sh.instance_rank);
    const int32_t nb = dopt_layout_num_buffers(L);
    printf("buffers %d\n", nb);
    for (int32_t k = 0; k < nb; ++k) {
        dopt_buffer_info bi;
        const int rc = dopt_layout_buffer(L, k, &bi);
        printf("buf %d %d %d %d %d %d %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 "\n", k, rc,
               bi.param_dtype, bi.grad_dtype, bi.n_buckets, bi.n_params, bi.numel, bi.numel_unpadded, bi.window_numel,
               bi.arena_numel, bi.shard_numel);
        for (int32_t b = 0; b < bi.n_buckets; ++b) {
            dopt_bucket_info bk;
            const int rb = dopt_layout_bucket(L, k, b, &bk);
            printf("bkt %d %d %d %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %d\n", k, b,
                   rb, bk.offset, bk.numel, bk.numel_unpadded, bk.shard_size, bk.window_start, bk.arena_offset,
                   bk.n_params);
            const int32_t ranks[3] = {0, sh.instance_size / 2, sh.instance_size - 1};
            for (int32_t rank : ranks) {
                dopt_range w;
                const int rw = dopt_layout_rank_window(L, k, b, rank, &w);
                printf("win %d %d %d %d %" PRId64 " %" PRId64 "\n", k, b, rank, rw, w.start, w.end);
            }
        }
        dopt_bucket_info bk;
        printf("bkt_oob %d\n", dopt_layout_bucket(L, k, bi.n_buckets, &bk));
    }
    dopt_buffer_info bi;
    printf("buf_oob %d %d\n", dopt_layout_buffer(L, nb, &bi), dopt_layout_buffer(L, -1, &bi));
    for (int64_t p = 0;; ++p) {
        dopt_param_info pi;
        const int rc = dopt_layout_param(L, p, &pi);
        if (rc != DOPT_OK) {
            printf("par_end %" PRId64 " %d\n", p, rc);
            break;
        }
        printf("par %" PRId64 " %d %d %d %d %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64
               " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 "\n",
               p, pi.buffer, pi.bucket, pi.has_shard, pi.hgroup, pi.start, pi.end, pi.gbuf_world.start,
               pi.gbuf_world.end, pi.gbuf_world_in_bucket.start, pi.gbuf_world_in_bucket.end, pi.gbuf_local.start,
               pi.gbuf_local.end, pi.param.start, pi.param.end, pi.arena_offset, pi.export_offset);
    }
    for (int32_t kind = 0; kind <= DOPT_GROUP_SHARD_FP32; ++kind)
        for (int32_t hg = 0; hg < DOPT_MAX_HGROUPS; ++hg) {
            const int64_t n = dopt_layout_group(L, kind, hg, nullptr, 0);
            if (n == 0) continue;
            std::vector<int64_t> idx(static_cast<size_t>(n > 0 ? n : 1));
            // a short buffer receives only its capacity
            const int64_t cap = n > 1 ? n - 1 : n;
            const int64_t m = dopt_layout_group(L, kind, hg, idx.data(), cap);
            printf("grp %d %d %" PRId64 " %" PRId64, kind, hg, n, m);
            for (int64_t i = 0; i < cap && i < n; ++i) printf(" %" PRId64, idx[static_cast<size_t>(i)]);
            printf("\n");
        }
    printf("grp_bad %" PRId64 " %" PRId64 "\n", dopt_layout_group(L, 5, 0, nullptr, 0),
           dopt_layout_group(L, 0, DOPT_MAX_HGROUPS, nullptr, 0));
    printf("state %" PRId64 " ws %" PRId64 " rec %" PRId64 "\n", dopt_layout_state_numel(L), dopt_workspace_bytes(L),
           dopt_stats_record_offset(L));
}

static void errors() {
    dopt_param_desc p{1000, DOPT_BF16, DOPT_BF16, 0, 0};
    dopt_layout *L = nullptr;
    dopt_shard_cfg ok{4, 1, 0, 0, 1};
    dopt_shard_cfg bad_n{0, 0, 0, 0, 1}, bad_r{4, 4, 0, 0, 1}, bad_i{4, 1, 0, 0, 3};
    dopt_param_desc bad_numel{0, DOPT_BF16, DOPT_BF16, 0, 0}, bad_dt{10, 7, DOPT_BF16, 0, 0};
    dopt_param_desc bad_hg{10, DOPT_BF16, DOPT_BF16, 0, DOPT_MAX_HGROUPS};
    printf("err %d %d %d %d %d %d %d %d %d\n", dopt_build_ranges(nullptr, 1, &ok, &L), dopt_build_ranges(&p, 0, &ok, &L),
           dopt_build_ranges(&p, 1, nullptr, &L), dopt_build_ranges(&p, 1, &ok, nullptr),
           dopt_build_ranges(&p, 1, &bad_n, &L), dopt_build_ranges(&p, 1, &bad_r, &L),
           dopt_build_ranges(&p, 1, &bad_i, &L), dopt_build_ranges(&bad_numel, 1, &ok, &L),
           dopt_build_ranges(&bad_dt, 1, &ok, &L));
    printf("err_hg %d\n", dopt_build_ranges(&bad_hg, 1, &ok, &L));
    printf("err_msg %d\n", dopt_last_error()[0] != '\0');
    dopt_buffer_info bi;
    printf("null_queries %d %d %" PRId64 "\n", dopt_layout_num_buffers(nullptr), dopt_layout_buffer(nullptr, 0, &bi),
           dopt_layout_state_numel(nullptr));
    dopt_layout_free(nullptr);
}

int main() {
    int32_t N = 0, r = 0, busbw = 0, inst = 0;
    int64_t bucket = 0, n = 0;
    while (scanf("%d %d %" SCNd64 " %d %d %" SCNd64, &N, &r, &bucket, &busbw, &inst, &n) == 6 && n > 0) {
        std::vector<dopt_param_desc> ps(static_cast<size_t>(n));
        for (auto &p : ps)
            if (scanf("%" SCNd64 " %d %d %d %d", &p.numel, &p.param_dtype, &p.grad_dtype, &p.requires_new_bucket,
                      &p.hgroup) != 5)
                return 2;
        const dopt_shard_cfg cfg{N, r, bucket, busbw, inst};
        dopt_layout *L = nullptr;
        const int rc = dopt_build_ranges(ps.data(), n, &cfg, &L);
        printf("case %d %d %" PRId64 " %d %d %" PRId64 " rc %d\n", N, r, bucket, busbw, inst, n, rc);
        if (rc != DOPT_OK) continue;
        dump(L);
        dopt_layout_free(L);
    }
    errors();
    return 0;
}
