// Host-side shard-range mapper: dopt_build_ranges and the layout queries.
//
// Pages cited: [DO] "Megatron-LM distrib_optimizer.py 源码精读";
// [ZL] "02 · ZeRO 显存账本与 Megatron DistributedOptimizer";
// [DP] "Megatron-LM distributed 包深度解析：DDP 梯度同步与 finalize_model_grads 全流程".
#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <numeric>

#include "internal.h"

namespace dopt {

static thread_local std::string g_last_error;

void set_error(int code, const std::string &msg) {
    (void)code;
    g_last_error = msg;
}

int fail(int code, const std::string &msg) {
    set_error(code, msg);
    return code;
}

static int64_t align_up(int64_t x, int64_t d) { return (x + d - 1) / d * d; }

// The largest element count a param list may hold (far above any device
// memory): every padded offset then stays far from the int64 limit.
static constexpr int64_t kMaxListNumel = int64_t(1) << 52;
// The largest padded buffer: each bucket's end is padded to a multiple of
// up to about 2^47 elements (an odd dp_size near 2^31 with the high-busbw
// padding), so many small buckets could otherwise carry offsets past int64.
static constexpr int64_t kMaxBufferNumel = int64_t(1) << 60;

static bool valid_dtype(int32_t d) { return d == DOPT_F32 || d == DOPT_BF16 || d == DOPT_F16; }

// Lay one flat buffer out in buckets ([DO] "Bucket 划分算法：逆序遍历 + 尺寸触发",
// "两级 Padding 机制").  The cursor walks the params from the last one in model
// order to the first (roughly the order their grads become ready in the
// backward pass).  The size trigger compares the running bucket length
// (param end minus bucket start) with bucket_size, so a single param larger
// than bucket_size forms an oversized bucket of its own.
static int lay_out_buffer(dopt_layout &L, Buffer &B, int64_t bucket_size, bool busbw) {
    int64_t divisor = std::lcm<int64_t>(L.N, 128);
    if (busbw) divisor = std::lcm<int64_t>(divisor, int64_t(1) << 16);

    int64_t bucket_start = 0;
    int32_t open = 0;  // params placed in the bucket being filled
    // Ends the open bucket at element x: records its unpadded length, pads its
    // end for an even N-way split and returns where the next bucket begins.
    auto seal = [&](int64_t x) -> int64_t {
        Bucket bk;
        bk.offset = bucket_start;
        bk.unpadded = x - bucket_start;
        const int64_t end = align_up(x, divisor);
        bk.numel = end - bucket_start;
        bk.n_params = open;
        B.buckets.push_back(bk);
        bucket_start = end;
        open = 0;
        return end;
    };

    int64_t cursor = 0, last_end = 0;
    for (auto it = B.params.rbegin(); it != B.params.rend(); ++it) {
        Param &p = L.params[*it];
        cursor = align_up(cursor, 64);  // 128-byte aligned start for 16-bit elements
        if (p.newb && open > 0) cursor = seal(cursor);
        p.start = cursor;
        p.end = cursor + p.numel;
        p.bucket = static_cast<int32_t>(B.buckets.size());
        ++open;
        last_end = p.end;
        const bool full = bucket_size > 0 && (p.end - bucket_start) >= bucket_size;
        cursor = (full || p.newb) ? seal(p.end) : p.end;
        if (cursor > kMaxBufferNumel)
            return fail(DOPT_ERR_INVALID, "the padded buffer holds more than 2^60 elements");
    }
    if (open > 0) seal(last_end);
    if (bucket_start > kMaxBufferNumel)
        return fail(DOPT_ERR_INVALID, "the padded buffer holds more than 2^60 elements");

    B.numel = bucket_start;
    B.unpadded = 0;
    for (const Bucket &bk : B.buckets) B.unpadded += bk.unpadded;
    // [DO] "最终内存大小断言" and "Bucket 级别的均等切分".
    if (B.unpadded > B.numel) return fail(DOPT_ERR_ASSERT, "layout invariant: numel_unpadded <= numel");
    if (B.numel % L.N != 0) return fail(DOPT_ERR_ASSERT, "layout invariant: numel % dp_size == 0");
    for (const Bucket &bk : B.buckets)
        if (bk.numel % L.N != 0) return fail(DOPT_ERR_ASSERT, "layout invariant: bucket numel % dp_size == 0");
    return DOPT_OK;
}

// Rank r's window of every bucket and every param's intersection with it in
// the four views of [DO] "Range 类：四种视角的统一抽象": first in window-local
// coordinates, then shifted to the buffer, to the bucket and into the param.
static void map_windows(dopt_layout &L, Buffer &B) {
    int64_t arena = 0;
    for (Bucket &bk : B.buckets) {
        bk.shard = bk.numel / L.N;
        bk.window_start = bk.offset + int64_t(L.r) * bk.shard;
        bk.arena_offset = arena;
        arena += bk.shard;
    }
    B.window_numel = arena;
    B.arena_numel = align_up(std::max<int64_t>(arena, 1), kTile);
    B.shard_numel = 0;
    B.segs.clear();
    for (int64_t pi : B.params) {
        Param &p = L.params[pi];
        const Bucket &bk = B.buckets[p.bucket];
        const int64_t lo = std::max<int64_t>(0, p.start - bk.window_start);
        const int64_t hi = std::min<int64_t>(bk.shard, p.end - bk.window_start);
        if (hi <= lo) {
            p.has_shard = 0;
            continue;
        }
        p.has_shard = 1;
        p.local = {lo, hi};
        p.world = {lo + bk.window_start, hi + bk.window_start};
        p.world_in_bucket = {p.world.start - bk.offset, p.world.end - bk.offset};
        const int64_t sub = std::max<int64_t>(0, bk.window_start - p.start);
        p.prange = {sub, sub + (hi - lo)};
        p.arena = bk.arena_offset + lo;
        B.shard_numel += hi - lo;
        B.segs.push_back(SegDesc{p.arena, p.arena + (hi - lo), -1, p.hgroup, static_cast<int32_t>(pi)});
    }
    std::sort(B.segs.begin(), B.segs.end(), [](const SegDesc &a, const SegDesc &b) { return a.start < b.start; });
}

// Tile table: for each TILE-element slice of the arena, the run of segments
// that overlap it and whether one segment covers it entirely.
static void build_tiles(Buffer &B) {
    const int64_t n_tiles = B.arena_numel / kTile;
    B.tiles.assign(static_cast<size_t>(n_tiles), TileDesc{0, 0});
    const int64_t ns = static_cast<int64_t>(B.segs.size());
    int64_t s = 0;
    for (int64_t t = 0; t < n_tiles; ++t) {
        const int64_t lo = t * kTile, hi = lo + kTile;
        while (s < ns && B.segs[s].end <= lo) ++s;
        int64_t j = s;
        while (j < ns && B.segs[j].start < hi) ++j;
        const int32_t cnt = static_cast<int32_t>(j - s);
        const bool full = cnt == 1 && B.segs[s].start <= lo && B.segs[s].end >= hi;
        const int32_t flags = full ? (kTileFull | (B.segs[s].hgroup << kTileHgShift)) : 0;
        B.tiles[t] = TileDesc{static_cast<int32_t>(s), cnt | flags};
    }
    const int64_t stats_one_pass = (n_tiles + kStatsUnroll - 1) / kStatsUnroll;
    const int64_t stats_max = B.gd == DOPT_F32 ? kStatsMaxBlocksF32 : kStatsMaxBlocks;
    B.stats_grid = static_cast<int32_t>(n_tiles <= kOneTileGridMax ? stats_one_pass
                                                                   : std::min<int64_t>(stats_one_pass, stats_max));
    // pass 2's boundary bitmap (see TileBits)
    B.bits.on = 0;
    B.bits.hg = 0;
    std::fill(std::begin(B.bits.w), std::end(B.bits.w), 0u);
    bool one_hg = true;
    for (const SegDesc &sg : B.segs) one_hg = one_hg && sg.hgroup == B.segs.front().hgroup;
    if (one_hg && n_tiles <= kBitmapTiles) {
        B.bits.on = 1;
        B.bits.hg = B.segs.empty() ? 0 : B.segs.front().hgroup;
        for (int64_t t = 0; t < n_tiles; ++t)
            if (!(B.tiles[t].seg_count & kTileFull)) B.bits.w[t >> 5] |= 1u << (t & 31);
    }
    const int64_t G = B.stats_grid, per_iter = G * kStatsUnroll;
    const int64_t n_groups = (n_tiles + per_iter - 1) / per_iter * G;
    B.stats_tiles.assign(static_cast<size_t>(n_groups * kStatsUnroll), TileDesc{0, 0});
    for (int64_t q = 0; q < n_groups; ++q)
        for (int64_t u = 0; u < kStatsUnroll; ++u) {
            const int64_t t = q % G + (q / G) * per_iter + u * G;
            if (t < n_tiles) B.stats_tiles[static_cast<size_t>(q * kStatsUnroll + u)] = B.tiles[static_cast<size_t>(t)];
        }
    // the fused reduce + pass 1: one tile per workgroup on small windows
    B.reduce_grid = static_cast<int32_t>(n_tiles <= kOneTileGridMax ? n_tiles
                                                                    : std::min<int64_t>(n_tiles, kReduceMaxBlocks));
    B.reduce_launches = static_cast<int32_t>(n_tiles <= kOneTileGridMax ? 1
                                                                        : (n_tiles + kRangeTiles - 1) / kRangeTiles);
    B.apply_grid = static_cast<int32_t>(n_tiles <= kApplyOneTileMax ? n_tiles
                                                                   : std::min<int64_t>(n_tiles, kApplyMaxBlocks));
    B.apply_bnd = false;
    if (B.apply_grid < n_tiles)
        for (const TileDesc &td : B.tiles) B.apply_bnd = B.apply_bnd || !(td.seg_count & kTileFull);
    B.copy_grid = static_cast<int32_t>(n_tiles <= kOneTileGridMax ? n_tiles
                                                                  : std::min<int64_t>(n_tiles, kCopyMaxBlocks));
}

static int build(const dopt_param_desc *params, int64_t n, const dopt_shard_cfg *cfg, dopt_layout &L) {
    L.dp_size = cfg->dp_size;
    L.dp_rank = cfg->dp_rank;
    L.num_instances = cfg->num_instances > 0 ? cfg->num_instances : 1;
    L.N = L.dp_size / L.num_instances;  // ranks of one distributed-optimizer instance
    L.r = L.dp_rank % L.N;              // this rank inside its instance
    // param indices are kept in 32 bits in the segment table
    if (n > INT32_MAX) return fail(DOPT_ERR_INVALID, "more than INT32_MAX params");
    L.params.resize(static_cast<size_t>(n));
    int64_t total = 0;
    for (int64_t i = 0; i < n; ++i) {
        const dopt_param_desc &d = params[i];
        if (d.numel <= 0 || d.numel > kMaxListNumel || !valid_dtype(d.param_dtype) || !valid_dtype(d.grad_dtype) ||
            d.hgroup < 0 || d.hgroup >= DOPT_MAX_HGROUPS)
            return fail(DOPT_ERR_INVALID, "param " + std::to_string(i) + ": bad numel, dtype or hgroup");
        total += d.numel;
        if (total > kMaxListNumel)
            return fail(DOPT_ERR_INVALID, "the params hold more than 2^52 elements in total");
        Param &p = L.params[i];
        p.numel = d.numel;
        p.pd = d.param_dtype;
        p.gd = d.grad_dtype;
        p.newb = d.requires_new_bucket != 0;
        p.hgroup = d.hgroup;
        L.max_hgroup = std::max(L.max_hgroup, d.hgroup);
        // one flat buffer per (param dtype, grad dtype), first appearance first ([DP] §2.2 (3))
        size_t k = 0;
        while (k < L.buffers.size() && !(L.buffers[k].pd == p.pd && L.buffers[k].gd == p.gd)) ++k;
        if (k == L.buffers.size()) {
            L.buffers.emplace_back();
            L.buffers.back().pd = p.pd;
            L.buffers.back().gd = p.gd;
        }
        p.buffer = static_cast<int32_t>(k);
        L.buffers[k].params.push_back(i);
    }
    int64_t ws = kWsPartials;
    int32_t partials = 0, reduce_partials = 0;
    for (Buffer &B : L.buffers) {
        int rc = lay_out_buffer(L, B, cfg->bucket_size, cfg->pad_for_high_busbw != 0);
        if (rc != DOPT_OK) return rc;
        map_windows(L, B);
        build_tiles(B);
        B.partial_base = partials;
        partials += B.stats_grid;
        B.reduce_partial_base = reduce_partials;
        reduce_partials += B.reduce_grid * B.reduce_launches;
        L.state_numel += B.shard_numel;
    }
    L.total_partials = partials;
    L.total_reduce_partials = reduce_partials;
    // model-space export: the shards in model order, back to back
    int64_t xoff = 0;
    for (Param &p : L.params) {
        if (!p.has_shard) continue;
        p.xoff = xoff;
        xoff += p.local.end - p.local.start;
    }
    for (Buffer &B : L.buffers)
        for (SegDesc &s : B.segs) s.xoff = L.params[s.param].xoff;
    ws += align_up(int64_t(std::max(partials, reduce_partials)) * 16, 256);
    for (Buffer &B : L.buffers) {
        B.ws_tiles = ws;
        ws += align_up(int64_t(B.tiles.size()) * int64_t(sizeof(TileDesc)), 256);
        B.ws_stats_tiles = ws;
        ws += align_up(int64_t(B.stats_tiles.size()) * int64_t(sizeof(TileDesc)), 256);
        B.ws_segs = ws;
        ws += align_up(std::max<int64_t>(int64_t(B.segs.size()), 1) * int64_t(sizeof(SegDesc)), 256);
        // whole-bucket check: the bucket table and one 16-byte partial per check tile
        B.chk.clear();
        B.chk_tile.clear();
        B.chk_tiles = 0;
        for (const Bucket &bk : B.buckets) {
            B.chk.push_back(CheckBucket{bk.offset, bk.numel, B.chk_tiles});
            for (int64_t s = bk.offset; s < bk.offset + bk.numel; s += kCheckTile)
                B.chk_tile.push_back(CheckTile{s, bk.offset + bk.numel});
            B.chk_tiles += (bk.numel + kCheckTile - 1) / kCheckTile;
        }
        B.ws_chk = ws;
        ws += align_up(int64_t(B.chk.size()) * int64_t(sizeof(CheckBucket)), 256);
        B.ws_chk_tile = ws;
        ws += align_up(B.chk_tiles * int64_t(sizeof(CheckTile)), 256);
        B.ws_chk_part = ws;
        ws += align_up(B.chk_tiles * 16, 256);
    }
    L.ws_bytes = ws;
    return DOPT_OK;
}

}  // namespace dopt

using namespace dopt;

extern "C" {

const char *dopt_last_error(void) { return g_last_error.c_str(); }

int dopt_build_ranges(const dopt_param_desc *params, int64_t n, const dopt_shard_cfg *cfg, dopt_layout **out) {
    if (!params || !cfg || !out || n <= 0) return fail(DOPT_ERR_INVALID, "null argument or n <= 0");
    *out = nullptr;
    if (cfg->dp_size < 1 || cfg->dp_rank < 0 || cfg->dp_rank >= cfg->dp_size)
        return fail(DOPT_ERR_INVALID, "dp_rank must satisfy 0 <= dp_rank < dp_size");
    if (cfg->num_instances < 0 || (cfg->num_instances > 0 && cfg->dp_size % cfg->num_instances != 0))
        return fail(DOPT_ERR_INVALID, "num_instances must be >= 1 and divide dp_size");
    dopt_layout *L = new (std::nothrow) dopt_layout();
    if (!L) return fail(DOPT_ERR_NOMEM, "out of host memory");
    int rc;
    try {
        rc = build(params, n, cfg, *L);
    } catch (const std::bad_alloc &) {
        rc = fail(DOPT_ERR_NOMEM, "out of host memory");
    }
    if (rc != DOPT_OK) {
        delete L;
        return rc;
    }
    *out = L;
    return DOPT_OK;
}

void dopt_layout_free(dopt_layout *layout) { delete layout; }

int32_t dopt_layout_num_buffers(const dopt_layout *L) { return L ? static_cast<int32_t>(L->buffers.size()) : 0; }

int dopt_layout_sharding(const dopt_layout *L, dopt_sharding_info *out) {
    if (!L || !out) return fail(DOPT_ERR_INVALID, "null argument");
    out->dp_size = L->dp_size;
    out->dp_rank = L->dp_rank;
    out->num_instances = L->num_instances;
    out->instance_size = L->N;
    out->instance_index = L->dp_rank / L->N;
    out->instance_rank = L->r;
    return DOPT_OK;
}

int dopt_layout_buffer(const dopt_layout *L, int32_t k, dopt_buffer_info *out) {
    if (!L || !out) return fail(DOPT_ERR_INVALID, "null argument");
    if (k < 0 || k >= static_cast<int32_t>(L->buffers.size())) return fail(DOPT_ERR_RANGE, "buffer index");
    const Buffer &B = L->buffers[k];
    out->param_dtype = B.pd;
    out->grad_dtype = B.gd;
    out->n_buckets = static_cast<int32_t>(B.buckets.size());
    out->n_params = static_cast<int32_t>(B.params.size());
    out->numel = B.numel;
    out->numel_unpadded = B.unpadded;
    out->window_numel = B.window_numel;
    out->arena_numel = B.arena_numel;
    out->shard_numel = B.shard_numel;
    out->apply_bnd = B.apply_bnd ? 1 : 0;
    out->reserved = 0;
    return DOPT_OK;
}

int dopt_layout_bucket(const dopt_layout *L, int32_t k, int32_t b, dopt_bucket_info *out) {
    if (!L || !out) return fail(DOPT_ERR_INVALID, "null argument");
    if (k < 0 || k >= static_cast<int32_t>(L->buffers.size()) || b < 0 ||
        b >= static_cast<int32_t>(L->buffers[k].buckets.size()))
        return fail(DOPT_ERR_RANGE, "bucket index");
    const Bucket &bk = L->buffers[k].buckets[b];
    out->offset = bk.offset;
    out->numel = bk.numel;
    out->numel_unpadded = bk.unpadded;
    out->shard_size = bk.shard;
    out->window_start = bk.window_start;
    out->arena_offset = bk.arena_offset;
    out->n_params = bk.n_params;
    out->reserved = 0;
    return DOPT_OK;
}

int dopt_layout_rank_window(const dopt_layout *L, int32_t k, int32_t b, int32_t rank, dopt_range *out) {
    if (!L || !out) return fail(DOPT_ERR_INVALID, "null argument");
    if (k < 0 || k >= static_cast<int32_t>(L->buffers.size()) || b < 0 ||
        b >= static_cast<int32_t>(L->buffers[k].buckets.size()) || rank < 0 || rank >= L->N)
        return fail(DOPT_ERR_RANGE, "bucket or rank index");
    const Bucket &bk = L->buffers[k].buckets[b];
    out->start = bk.offset + int64_t(rank) * bk.shard;
    out->end = out->start + bk.shard;
    return DOPT_OK;
}

int dopt_layout_param(const dopt_layout *L, int64_t p, dopt_param_info *out) {
    if (!L || !out) return fail(DOPT_ERR_INVALID, "null argument");
    if (p < 0 || p >= static_cast<int64_t>(L->params.size())) return fail(DOPT_ERR_RANGE, "param index");
    const Param &q = L->params[p];
    std::memset(out, 0, sizeof *out);
    out->buffer = q.buffer;
    out->bucket = q.bucket;
    out->has_shard = q.has_shard;
    out->hgroup = q.hgroup;
    out->start = q.start;
    out->end = q.end;
    if (q.has_shard) {
        out->gbuf_world = q.world;
        out->gbuf_world_in_bucket = q.world_in_bucket;
        out->gbuf_local = q.local;
        out->param = q.prange;
    }
    out->arena_offset = q.has_shard ? q.arena : -1;
    out->export_offset = q.has_shard ? q.xoff : -1;
    return DOPT_OK;
}

// [DO] group-building section; [ZL] §3: 16-bit params feed model_float16,
// shard_float16 (the param-window view) and shard_fp32_from_float16 (the fp32
// master); fp32 params feed model_fp32 and shard_fp32.  Only params with a
// shard on this rank are listed.
int64_t dopt_layout_group(const dopt_layout *L, int32_t kind, int32_t hgroup, int64_t *idx, int64_t cap) {
    if (!L) return fail(DOPT_ERR_INVALID, "null layout");
    if (kind < DOPT_GROUP_MODEL_FLOAT16 || kind > DOPT_GROUP_SHARD_FP32) return fail(DOPT_ERR_RANGE, "group kind");
    if (hgroup < 0 || hgroup >= DOPT_MAX_HGROUPS) return fail(DOPT_ERR_RANGE, "hyper-group");
    const bool lowp = kind == DOPT_GROUP_MODEL_FLOAT16 || kind == DOPT_GROUP_SHARD_FLOAT16 ||
                      kind == DOPT_GROUP_SHARD_FP32_FROM_FLOAT16;
    int64_t count = 0;
    for (size_t i = 0; i < L->params.size(); ++i) {
        const Param &q = L->params[i];
        if (!q.has_shard || q.hgroup != hgroup || (q.pd != DOPT_F32) != lowp) continue;
        if (idx && count < cap) idx[count] = static_cast<int64_t>(i);
        ++count;
    }
    return count;
}

int64_t dopt_layout_state_numel(const dopt_layout *L) { return L ? L->state_numel : 0; }

int64_t dopt_workspace_bytes(const dopt_layout *L) { return L ? L->ws_bytes : 0; }

int64_t dopt_stats_record_offset(const dopt_layout *L) { return L ? kWsRecord : 0; }

}  // extern "C"
