// Internal layout structures shared by the host mapper (mapper.cpp) and the
// step driver / kernels (step.hip).  Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "dopt.h"

namespace dopt {

// Work unit of the device passes: one tile = TILE consecutive arena elements,
// handled by one 256-thread workgroup, 8 consecutive elements per thread.
constexpr int kBlock = 256;
constexpr int kVec = 8;
constexpr int kTile = kBlock * kVec;
static_assert(kTile == DOPT_ARENA_ALIGN, "arena alignment must equal the tile size");

// Workgroups per launch.  Small windows get one workgroup per tile (pass 2,
// the fused reduce, the state copy) or per kStatsUnroll tiles (pass 1), so no
// workgroup does more iterations than another; large ones a fixed grid,
// grid-stride over the tiles.  The grid is a function of the layout only, so
// the reduction order, and hence the sum of squares, does not depend on the
// device it runs on.  The large-window grids were chosen by measurement on
// MI355X: fewer workgroups than the chip could hold keep fewer DRAM rows open
// at a time, which the read-modify-write and copy passes preferred; the
// read-only pass 1 ran fastest with many more workgroups than the chip holds
// at once (each then takes few batches), bounded by the cost of adding their
// partials in the one-workgroup finish.
constexpr int kStatsMaxBlocks = 16384;
// fp32 grads keep 8 16-byte loads in flight per lane (two per tile), which
// one workgroup per CU turns into the full read rate (Llama-3-8B rank: pass 1
// + finish 0.56-0.57 ms at 256 workgroups, 0.60 ms at 16384); 16-bit grads,
// with 4 loads in flight, need the many-workgroup grid above.
constexpr int kStatsMaxBlocksF32 = 256;
constexpr int kReduceMaxBlocks = 1024;  // the fused reduce + pass 1
// The fused reduce and the state copy of a large window are launched once per
// kRangeTiles tiles (each launch grid-strides over its own range; the reduce's
// launches write partials of their own).  Over thousands of iterations the
// workgroups of one long launch drift apart and the pass's concurrent accesses
// spread over more DRAM rows.  Measured on MI355X at 1.0e9 slots, in one
// process: the reduce of 8 bf16 chunks 5.58 TB/s in ranges of 2^15 tiles,
// 5.53 at 2^16, 5.45 at 2^14, 5.19 in one launch; the state export 6.11 /
// 6.02 / 5.24-5.77 TB/s and the import 6.04-6.08 / 6.08 / 5.33-5.65 TB/s at
// 2^15 / 2^16 / one launch.  Pass 2 gained 2-4% the same way on plain
// allocations but nothing on the searched placements it runs on, so it keeps
// one launch.
constexpr int64_t kRangeTiles = 32768;
constexpr int kApplyMaxBlocks = 256;
constexpr int kCopyMaxBlocks = 256;  // state export / import
constexpr int64_t kOneTileGridMax = 8192;  // tiles up to which a window counts as small
// Pass 2 keeps one workgroup per tile up to this many tiles (measured on
// GPT-2-small-shaped windows of 10K and 15K tiles: 6.6% and 1.6% faster
// steps than 256 workgroups; even at 30K tiles).
constexpr int64_t kApplyOneTileMax = 16384;
// Grad windows above this size are streamed through pass 1 with
// nontemporal loads (the MI355X last-level cache is 256 MB).
constexpr int64_t kStreamingReadBytes = int64_t(192) << 20;
// Tiles in flight per workgroup iteration of pass 1 (more bytes outstanding
// per wave for a pass that only reads).
constexpr int kStatsUnroll = 4;

// Tile descriptor: the param segments that overlap the tile.  seg_count
// holds the number of overlapping segments in its low 24 bits; when one
// segment covers the whole tile, kTileFull is set and bits 24-28 hold that
// segment's hyper-group (so the full-tile path needs no segment lookup).
constexpr int32_t kTileFull = 1 << 30;
constexpr int kTileHgShift = 24;
constexpr int32_t kTileHgMask = 0x1f;
constexpr int32_t kTileCountMask = (1 << kTileHgShift) - 1;
static_assert(DOPT_MAX_HGROUPS <= kTileHgMask + 1, "hyper-group field too narrow");
struct TileDesc {
    int32_t seg_first;
    int32_t seg_count;
};

// Pass 2's boundary bitmap, passed by value: for a buffer of at most
// kBitmapTiles tiles whose shards are all in one hyper-group `hg`, bit t is
// set when tile t is not fully covered by one param's shard; a tile whose bit
// is clear is then known to be full without a descriptor load.  on == 0: no
// bitmap (read every tile's descriptor).
constexpr int kBitmapTiles = 8192;
struct TileBits {
    int32_t on, hg;
    uint32_t w[kBitmapTiles / 32];
};

// Pre-communication check of whole buckets: a check tile is kCheckTile
// elements from the bucket start (bucket sizes are multiples of 128
// elements, so an 8-element vector is either wholly inside a bucket or past
// its end); one partial per check tile.
constexpr int64_t kCheckTile = 8 * kTile;
constexpr int kCheckMaxBlocks = 4096;
struct CheckBucket {
    int64_t offset, numel, tile_base;  // tile_base: index of the bucket's first check tile
};
struct CheckTile {
    int64_t start, end;  // the tile's first element and its bucket's end (buffer coordinates)
};

// A param's shard in arena coordinates, [start, end), and where it sits in
// the model-space state export.
struct SegDesc {
    int64_t start, end;
    int64_t xoff;
    int32_t hgroup, param;
};

struct Bucket {
    int64_t offset = 0, numel = 0, unpadded = 0, shard = 0, window_start = 0, arena_offset = 0;
    int32_t n_params = 0;
};

struct Param {
    int64_t numel = 0;
    int32_t pd = 0, gd = 0, newb = 0, hgroup = 0;
    int32_t buffer = 0, bucket = 0;
    int64_t start = 0, end = 0;
    int32_t has_shard = 0;
    dopt_range world{0, 0}, world_in_bucket{0, 0}, local{0, 0}, prange{0, 0};
    int64_t arena = -1;
    int64_t xoff = -1;  // offset of the shard in the model-space export
};

struct Buffer {
    int32_t pd = 0, gd = 0;
    std::vector<int64_t> params;  // model order
    std::vector<Bucket> buckets;
    int64_t numel = 0, unpadded = 0, window_numel = 0, arena_numel = 0, shard_numel = 0;
    std::vector<SegDesc> segs;
    std::vector<TileDesc> tiles;
    // pass 1's copy of the tile table, in the order its workgroups read it:
    // group q = k*G + b (workgroup b, k-th iteration, G = stats_grid) holds
    // the descriptors of tiles b + k*G*kStatsUnroll + u*G, u < kStatsUnroll
    // (empty descriptors past the last tile)
    std::vector<TileDesc> stats_tiles;
    TileBits bits{0, 0, {}};
    int32_t stats_grid = 0, apply_grid = 0, copy_grid = 0, reduce_grid = 0;
    int32_t reduce_launches = 0;  // the fused reduce's launches (kRangeTiles tiles each)
    bool apply_bnd = false;       // pass 2 in k_apply_bnd: a grid-stride window with boundary tiles
    int32_t partial_base = 0, reduce_partial_base = 0;  // first partial slot of pass 1 / the fused reduce
    int64_t ws_tiles = 0, ws_stats_tiles = 0, ws_segs = 0;  // byte offsets in the workspace
    std::vector<CheckBucket> chk;       // per bucket, for dopt_check_grads
    std::vector<CheckTile> chk_tile;    // per check tile
    int64_t chk_tiles = 0;
    int64_t ws_chk = 0, ws_chk_tile = 0, ws_chk_part = 0;
};

// Workspace map (byte offsets).
constexpr int64_t kWsState = 0;       // persistent scaler / step-count state
constexpr int64_t kWsStepRec = 256;   // per-step scalars for the apply pass
constexpr int64_t kWsStats = 1280;    // dopt_stats of the last step
constexpr int64_t kWsRecord = 1536;   // grad-stats record {sumsq, zeros}
constexpr int64_t kWsPartials = 1792; // per-workgroup partials of pass 1

void set_error(int code, const std::string &msg);
int fail(int code, const std::string &msg);

}  // namespace dopt

struct dopt_layout {
    int32_t dp_size = 1, dp_rank = 0, num_instances = 1;
    int32_t N = 1, r = 0;  // ranks the state is split over (the instance size) and this rank among them
    int32_t max_hgroup = 0;
    std::vector<dopt::Param> params;
    std::vector<dopt::Buffer> buffers;
    int64_t state_numel = 0;
    int32_t total_partials = 0, total_reduce_partials = 0;
    int64_t ws_bytes = 0;
};
